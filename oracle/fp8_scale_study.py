"""FP8 E4M3 weight quantisation: one scale per output row against one per matrix.

Test infrastructure, like the rest of oracle/: a CPU-only study that calls the oracle
and the seeded generators, nothing else.  It prints a Markdown table; the committed copy
is fp8_scale_study.md beside this file.

Two weight families at the 1B shape (hidden 2048, 32/8 heads of 64, FFN 8192, vocabulary
128256):
  * "gaussian": the seeded N(0, 0.02) bf16 weights every test and benchmark uses;
  * "row-spread": the same weights with each row multiplied by exp(N(0, 1)), rounded to
    bf16, standing in for trained weights whose row norms differ (no trained checkpoint
    is available);
  * "wide row-spread": factors exp(N(0, 16)), rows spread over about 2^+-17, so that under
    one scale per matrix many rows fall into the E4M3 subnormals or to zero.
Per matrix: y = W x over the quantised W, x ~ N(0, 1); each row's error divided by that
row's norm, RMS and largest over the rows.  End to end:
the 1B-dimension model with 2 layers and a 4096-token vocabulary, 4 decode steps from a
synthetic token, largest |logit| difference against the bf16 model.

    python -m oracle.fp8_scale_study > oracle/fp8_scale_study.md
"""
from __future__ import annotations

import dataclasses
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import oracle  # noqa: E402
import synth  # noqa: E402

KINDS = ["wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down"]


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """float64 -> bf16 bits, round to nearest even (finite inputs)."""
    u = a.astype(np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def as_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def spread_rows(bits: np.ndarray, rng, sigma: float = 1.0) -> np.ndarray:
    f = sigma * rng.standard_normal(bits.shape[0])
    return bf16_bits(as_f64(bits) * np.exp(f)[:, None])


def row_errs(y, ref, W):
    """Each row's error over that row's norm (x ~ N(0, 1), so y_r ~ N(0, |w_r|^2)): RMS and
    largest over the rows, every row counted alike whatever its magnitude.  All-zero rows
    (none here) would be skipped."""
    n = np.linalg.norm(as_f64(W), axis=1)
    e = np.abs(y - ref)[n > 0] / n[n > 0]
    return float(np.sqrt(np.mean(e * e))), float(np.max(e))


def matrix_rows(shape, threads):
    w = synth.make_weights(dataclasses.replace(shape, n_layers=1, vocab=8192), threads=threads)
    mats = {k: w["layers"][0][k] for k in KINDS}
    mats["lm_head (8192 rows)"] = w["embed"]
    return mats


def end_to_end(shape, family, threads):
    m = dataclasses.replace(shape, n_layers=2, vocab=4096)
    w = synth.make_weights(m, threads=threads)
    if family == "row-spread":
        rng = np.random.default_rng(5)
        for L in w["layers"]:
            for k in KINDS:
                L[k] = spread_rows(L[k], rng)
        w["embed"] = spread_rows(w["embed"], rng)
    out = {}
    for mode in (False, "matrix", "row"):
        orc = oracle.Oracle(m, w, 1, 8, fp8=mode)
        kv = np.zeros(orc.kv_cache_bytes() // 2, dtype=np.uint16)
        out[mode] = [orc.decode_step(kv, [t], [p], threads) for p, t in enumerate([11, 1234, 77, 3001])]
    res = {}
    for mode in ("matrix", "row"):
        d = max(float(np.max(np.abs(a - b))) for a, b in zip(out[mode], out[False]))
        top = sum(int(np.argmax(a) == np.argmax(b)) for a, b in zip(out[mode], out[False]))
        res[mode] = (d, top)
    scale = max(float(np.max(np.abs(a))) for a in out[False])
    return res, scale


def main():
    threads = synth.default_threads()
    shape = synth.LLAMA_1B
    x_rng = np.random.default_rng(1)
    print("| family | matrix | rows x cols | RMS row error, scale per matrix | per row | largest row error, per matrix | per row |")
    print("|---|---|---|---|---|---|---|")
    mats = matrix_rows(shape, threads)
    for family, sigma in (("gaussian", 0.0), ("row-spread", 1.0), ("wide row-spread", 4.0)):
        rng = np.random.default_rng(4)
        for name, W in mats.items():
            if sigma > 0:
                W = spread_rows(W, rng, sigma)
            x = x_rng.standard_normal(W.shape[1])
            ref = oracle.gemv(W, x, threads)
            em = row_errs(oracle.gemv_fp8(W, x, threads), ref, W)
            er = row_errs(oracle.gemv_fp8_rows(W, x, threads), ref, W)
            print(f"| {family} | {name} | {W.shape[0]} x {W.shape[1]} | {em[0]:.3e} | {er[0]:.3e} | {em[1]:.3e} | {er[1]:.3e} |")
    print()
    print("| family | largest abs. logit error, per matrix | per row | argmax agrees (of 4), per matrix | per row | largest abs. bf16 logit |")
    print("|---|---|---|---|---|---|")
    for family in ("gaussian", "row-spread"):
        res, scale = end_to_end(shape, family, threads)
        print(f"| {family} | {res['matrix'][0]:.3e} | {res['row'][0]:.3e} | {res['matrix'][1]} | {res['row'][1]} | {scale:.3f} |")


if __name__ == "__main__":
    main()
