"""MK_FLAG_DEBUG_NAN: with the step's untagged scratch (down-projection accumulators, logits, the
value halves of the tagged words, every LDS word) overwritten with NaN before each step, the
logits stay finite and equal to those of a handle without the mode, bit for bit, on every path:
no word is read before this step writes it."""
import dataclasses

import numpy as np
import pytest

import synth
from tests import helpers as H

pytestmark = pytest.mark.gpu

DEBUG_NAN = 8  # MK_FLAG_DEBUG_NAN


def greedy_run(shape, weights, batch, P, steps, flags, path):
    import torch
    from decode_megakernel_02_amd import mk
    max_seq = P + steps + 1
    kv = synth.make_kv_cache(shape, batch, max_seq, P)
    dec = H.GpuDecoder(shape, weights, batch, max_seq, kv_init=kv, flags=flags)
    s = mk.current_stream()
    out = []
    try:
        dec.tokens.copy_(torch.as_tensor(synth.make_first_tokens(shape.vocab, batch)))
        dec.positions.fill_(P)
        for _ in range(steps):
            if path == "fused":
                mk.mk_decode_step_greedy(dec.h, dec.tokens, dec.positions, dec.kv, dec.logits, s)
            else:
                fn = mk.mk_decode_step if path == "single" else mk.mk_decode_step_multikernel
                fn(dec.h, dec.tokens, dec.positions, dec.kv, dec.logits, s)
                mk.mk_greedy_advance(dec.h, dec.logits, dec.tokens, dec.positions, s)
            torch.cuda.synchronize()
            out.append(dec.logits.cpu().numpy().copy())
        assert mk.mk_get_device_error(dec.h) is None
        out.append(dec.kv_host().copy())
    finally:
        dec.close()
    return out


@pytest.mark.parametrize("path", ["single", "fused", "per-op"])
@pytest.mark.parametrize("shape,batch", [(synth.TINY, 2),
                                         (dataclasses.replace(synth.LLAMA_1B, n_layers=2, vocab=4096), 1),
                                         (dataclasses.replace(synth.LLAMA_1B, n_layers=2, vocab=4096), 4)],
                         ids=["tiny-b2", "1b-dims-b1", "1b-dims-b4"])
def test_nan_filled_scratch_is_never_read(shape, batch, path):
    w = synth.make_weights(shape)
    ref = greedy_run(shape, w, batch, 40, 3, 0, path)
    got = greedy_run(shape, w, batch, 40, 3, DEBUG_NAN, path)
    for i, (a, b) in enumerate(zip(ref, got)):
        if i < len(ref) - 1:
            assert np.all(np.isfinite(b)), f"step {i}: NaN logits (a read before write)"
        np.testing.assert_array_equal(b, a, err_msg=f"item {i}")
