"""GPU parity of the FP8-weight mode (MK_FLAG_FP8_WEIGHTS) against the oracle's
FP8 path: both quantise every projection matrix and the LM head to OCP E4M3
codes with one fp32 scale per matrix, so the products use identical weights
and the logits agree to fp32 accumulation error (bound 1e-3, well inside the
usual parity bar; a code that differed would show as ~1e-3 or more)."""
import dataclasses

import numpy as np
import pytest

import synth
from tests import helpers as H

pytestmark = pytest.mark.gpu

FP8 = 4  # MK_FLAG_FP8_WEIGHTS


def prefill_and_decode(shape, weights, batch, prompt_len, n_decode, multikernel, **kw):
    max_seq = prompt_len + n_decode
    prompt = synth.make_prompts(shape.vocab, batch, prompt_len)
    dec = H.GpuDecoder(shape, weights, batch, max_seq, flags=FP8, **kw)
    try:
        run = H.Run([], [], [])
        for i in range(prompt_len):
            toks, pos = prompt[:, i], np.full(batch, i, dtype=np.int32)
            run.tokens.append(toks.copy())
            run.positions.append(pos.copy())
            run.logits.append(dec.step(toks, pos, multikernel))
        g = dec.greedy(np.argmax(run.logits[-1], axis=1), np.full(batch, prompt_len), n_decode, multikernel)
        run.tokens += g.tokens
        run.positions += g.positions
        run.logits += g.logits
    finally:
        dec.close()
    return run, max_seq


@pytest.mark.parametrize("multikernel", [False, True], ids=["megakernel", "multikernel"])
@pytest.mark.parametrize("batch", [1, 4])
def test_tiny_fp8_matches_oracle(batch, multikernel):
    shape = synth.TINY
    w = synth.make_weights(shape)
    run, max_seq = prefill_and_decode(shape, w, batch, 12, 4, multikernel)
    ref = H.oracle_replay(shape, w, batch, max_seq, run, fp8=True)
    stats = H.compare(run, ref, f"tiny fp8 b{batch}")
    print("tiny fp8", batch, multikernel, stats)
    assert stats["max_abs"] < 1e-3


def test_llama1b_dims_fp8_matches_oracle():
    """1B dimensions (2 layers, 4096-row vocabulary): the batch-1 path with
    two-unit FP8 rows, and the chunked down projection."""
    shape = dataclasses.replace(synth.LLAMA_1B, n_layers=2, vocab=4096)
    w = synth.make_weights(shape)
    run, max_seq = prefill_and_decode(shape, w, 1, 6, 3, False)
    ref = H.oracle_replay(shape, w, 1, max_seq, run, fp8=True)
    stats = H.compare(run, ref, "1B dims fp8")
    print("1B dims fp8", stats)
    assert stats["max_abs"] < 1e-3


def test_fp8_and_bf16_handles_differ_but_stay_close():
    shape = synth.TINY
    w = synth.make_weights(shape)
    out = []
    for flags in (0, FP8):
        dec = H.GpuDecoder(shape, w, 1, 4, flags=flags)
        try:
            out.append(dec.step([5], [0]))
        finally:
            dec.close()
    d = np.abs(out[0] - out[1]).max()
    assert 1e-6 < d < 0.5 * np.abs(out[0]).max()
