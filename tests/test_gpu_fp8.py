"""GPU parity of the FP8-weight mode (MK_FLAG_FP8_WEIGHTS) against the oracle's
FP8 path: both quantise every projection matrix and the LM head to OCP E4M3
codes with one fp32 scale per output row, so the products use identical weights
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
    ref = H.oracle_replay(shape, w, batch, max_seq, run, fp8="row")
    stats = H.compare(run, ref, f"tiny fp8 b{batch}")
    print("tiny fp8", batch, multikernel, stats)
    assert stats["max_abs"] < 1e-3


def test_llama1b_dims_fp8_matches_oracle():
    """1B dimensions (2 layers, 4096-row vocabulary): the batch-1 path with
    two-unit FP8 rows, and the chunked down projection."""
    shape = dataclasses.replace(synth.LLAMA_1B, n_layers=2, vocab=4096)
    w = synth.make_weights(shape)
    run, max_seq = prefill_and_decode(shape, w, 1, 6, 3, False)
    ref = H.oracle_replay(shape, w, 1, max_seq, run, fp8="row")
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


def test_rows_of_very_different_magnitude_keep_their_precision():
    """Rows of every matrix scaled by 2^-k (k uniform in 0..12, exact in bf16): with one scale
    per matrix the small rows would fall into the E4M3 subnormals.  Each logit's error, divided
    by its LM-head row's factor, must stay small against the per-row oracle and is far larger
    against a per-matrix oracle, so the GPU path really scales by row."""
    shape = synth.TINY
    w = synth.make_weights(shape)
    rng = np.random.default_rng(21)

    def spread(bits):
        k = rng.integers(0, 13, size=bits.shape[0])
        f = (bits.astype(np.uint32) << 16).view(np.float32) * np.ldexp(np.float32(1), -k)[:, None].astype(np.float32)
        return (f.view(np.uint32) >> 16).astype(np.uint16), np.ldexp(1.0, -k)

    for L in w["layers"]:
        for kind in ["wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down"]:
            L[kind] = spread(L[kind])[0]
    w["embed"], factor = spread(w["embed"])
    run, max_seq = prefill_and_decode(shape, w, 1, 6, 2, False)
    per_row = H.oracle_replay(shape, w, 1, max_seq, run, fp8="row")
    per_mat = H.oracle_replay(shape, w, 1, max_seq, run, fp8="matrix")
    e_row = max(float(np.max(np.abs(g - r)[0] / factor)) for g, r in zip(run.logits, per_row))
    e_mat = max(float(np.max(np.abs(g - r)[0] / factor)) for g, r in zip(run.logits, per_mat))
    print("row-normalised logit error: per-row oracle", e_row, "per-matrix oracle", e_mat)
    assert e_row < 1e-3
    assert e_mat > 30 * e_row and e_mat > 1e-3
