"""The decode loop captured as a HIP graph (mk_graph_create / mk_graph_launch)
against the same greedy steps issued one launch at a time: every replay must
give bit-identical logits, tokens, positions and KV cache.  Replays are
separated by the program's own eager GPU work and synchronisations."""
import numpy as np
import pytest

import synth
from tests import helpers as H

pytestmark = pytest.mark.gpu


def _start(dec, first, P):
    dec.kv.zero_()
    dec.tokens.copy_(dec.torch.as_tensor(first))
    dec.positions.fill_(P)


@pytest.mark.parametrize("steps_per_graph", [1, 3])
@pytest.mark.parametrize("multikernel", [True, False], ids=["per-op", "single-launch"])
def test_graph_replays_match_eager_steps(multikernel, steps_per_graph):
    import torch
    from decode_megakernel_02_amd import mk
    shape, B, P, n_total = synth.TINY, 2, 8, 6
    dec = H.GpuDecoder(shape, synth.make_weights(shape), B, P + n_total + 2)
    s = mk.current_stream()
    first = synth.make_first_tokens(shape.vocab, B)
    g = None
    try:
        step = mk.mk_decode_step_multikernel if multikernel else mk.mk_decode_step
        _start(dec, first, P)
        ref = []
        for i in range(n_total):
            step(dec.h, dec.tokens, dec.positions, dec.kv, dec.logits, s)
            mk.mk_greedy_advance(dec.h, dec.logits, dec.tokens, dec.positions, s)
            if (i + 1) % steps_per_graph == 0:
                torch.cuda.synchronize()
                ref.append((dec.logits.cpu().numpy().copy(), dec.tokens.cpu().numpy().copy(),
                            dec.positions.cpu().numpy().copy()))
        ref_kv = dec.kv.cpu().numpy().copy()
        assert mk.mk_get_device_error(dec.h) is None

        _start(dec, first, P)
        torch.cuda.synchronize()
        flags = mk.MK_GRAPH_MULTIKERNEL if multikernel else 0
        try:
            g = mk.mk_graph_create(dec.h, dec.tokens, dec.positions, dec.kv, dec.logits, steps_per_graph, flags)
        except mk.MkError as e:
            if not multikernel and e.code == mk.MK_ERR_HIP:
                pytest.skip(f"the runtime refuses to capture the cooperative single-launch step: {e}")
            raise
        for r, (lg, tok, pos) in enumerate(ref):
            mk.mk_graph_launch(g, s)
            torch.cuda.synchronize()
            other = torch.arange(4096, device="cuda", dtype=torch.float32).mul_(0.5).sum().item()  # eager work
            assert other == 0.5 * 4095 * 4096 / 2
            np.testing.assert_array_equal(dec.logits.cpu().numpy(), lg, err_msg=f"replay {r}")
            np.testing.assert_array_equal(dec.tokens.cpu().numpy(), tok, err_msg=f"replay {r}")
            np.testing.assert_array_equal(dec.positions.cpu().numpy(), pos, err_msg=f"replay {r}")
        np.testing.assert_array_equal(dec.kv.cpu().numpy(), ref_kv)
        assert mk.mk_get_device_error(dec.h) is None
    finally:
        if g is not None:
            mk.mk_graph_destroy(g)
        dec.close()
    if steps_per_graph == 1:
        # teacher-forced against the oracle: replay r saw the tokens replay r - 1 wrote
        run = H.Run([], [], [])
        toks, pos = np.asarray(first, dtype=np.int32), np.full(B, P, dtype=np.int32)
        for lg, tok, npos in ref:
            run.tokens.append(toks)
            run.positions.append(pos)
            run.logits.append(lg)
            toks, pos = tok, npos
        stats = H.compare(run, H.oracle_replay(shape, synth.make_weights(shape), B, P + n_total + 2, run), "graph")
        print("graph replays vs oracle", stats)


def test_empty_launch_graph_and_eager_empty_launches_touch_nothing():
    import torch
    from decode_megakernel_02_amd import mk
    shape = synth.TINY
    dec = H.GpuDecoder(shape, synth.make_weights(shape), 1, 16)
    s = mk.current_stream()
    g = None
    try:
        dec.logits.fill_(3.0)
        dec.tokens.fill_(5)
        dec.positions.fill_(7)
        g = mk.mk_graph_create(dec.h, dec.tokens, dec.positions, dec.kv, dec.logits, 2, mk.MK_GRAPH_EMPTY)
        for _ in range(3):
            mk.mk_graph_launch(g, s)
        ncu = torch.cuda.get_device_properties(0).multi_processor_count
        mk.mk_empty_launches(97, ncu, mk.MK_STEP_THREADS, s)
        torch.cuda.synchronize()
        assert torch.all(dec.logits == 3.0) and torch.all(dec.tokens == 5) and torch.all(dec.positions == 7)
        assert torch.all(dec.kv == 0)
    finally:
        if g is not None:
            mk.mk_graph_destroy(g)
        dec.close()
