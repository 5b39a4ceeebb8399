"""GPU litmus of the tagged-word dependency protocol (include/mk.h, mk_litmus).

The decode step never fences: a consumer accepts a 64-bit word once its tag
carries the current round, and relies on the value half arriving together
with the tag (a single aligned 8-byte store).  Pairs of workgroups on
different XCDs (and, as a control, on the same XCD) exchange many rounds of
tagged blocks with the step kernel's own store/load primitives; every value
that arrives with a current tag must be exactly the one stored with it, and
every poll must complete.  The run also reports the round-trip latency."""
import numpy as np
import pytest

from decode_megakernel_02_amd import mk

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n_pairs,same_xcd", [(127, False), (128, True), (255, False)])
@pytest.mark.parametrize("words", [64, 1024])
def test_tagged_words_arrive_whole(n_pairs, same_xcd, words):
    rounds = 200
    mism, tmo, trips, ticks, xp, xq = mk.mk_litmus(n_pairs, rounds, words)
    assert tmo == 0, f"{tmo} polls timed out"
    assert mism == 0, f"{mism} values arrived with a current tag but not the stored value"
    assert trips == n_pairs * rounds
    cross = int(np.sum(xp != xq))
    if same_xcd:
        assert cross == 0, "pairs expected on one XCD"
    else:
        assert cross == n_pairs, "pairs expected on different XCDs"
    us = ticks.astype(np.float64) * 0.01 / rounds
    print(f"pairs {n_pairs} words {words} {'same' if same_xcd else 'cross'}-XCD: round trip "
          f"median {np.median(us):.2f} us, max {np.max(us):.2f} us")
