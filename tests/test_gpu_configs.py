"""GPU parity at the other benchmark shapes: batch 4 and 8, long contexts
(8K and 32K tokens in the cache), the 8B shape (head_dim 128, untied head) and
one GPU's share of the 1B shape under 8-way tensor parallelism (hidden size
2048 with 4 query heads, so n_q_heads * head_dim differs from it).

Each case pre-fills the cache with seeded N(0, 1) bf16 rows (identical bytes on
both sides), runs a few greedy steps through the C ABI and compares every step
with the teacher-forced CPU oracle to the same bar as the other parity tests.
"""
import dataclasses
import os

import numpy as np
import pytest

import synth
from tests import helpers as H

pytestmark = pytest.mark.gpu

THREADS = min(32, os.cpu_count() or 1)


FP8 = 4  # MK_FLAG_FP8_WEIGHTS


def run_and_compare(shape, weights, batch, prompt_lens, steps, label, multikernel=False, n_chunks=0, flags=0,
                    to_the_end=False):
    """to_the_end: the cache holds exactly max(prompt) + steps positions, so the last step of the
    longest row writes and attends to position max_seq - 1."""
    P = np.asarray(prompt_lens, dtype=np.int32)
    max_seq = int(P.max()) + steps + (0 if to_the_end else 1)
    kv = synth.make_kv_cache(shape, batch, max_seq, int(P.max()))
    # rows with shorter prompts: slots [P_b, max) stay unused (the step writes slot P_b and
    # attends to 0..P_b), so the extra filled slots of those rows are never read
    first = synth.make_first_tokens(shape.vocab, batch)
    dec = H.GpuDecoder(shape, weights, batch, max_seq, n_chunks=n_chunks, kv_init=kv, flags=flags)
    try:
        run = dec.greedy(first, P, steps, multikernel)
    finally:
        dec.close()
    if to_the_end:
        assert int(run.positions[-1].max()) == max_seq - 1
    ref = H.oracle_replay(shape, weights, batch, max_seq, run, kv_init=kv, nthreads=THREADS,
                          fp8="row" if flags & FP8 else False)
    stats = H.compare(run, ref, label)
    print(label, stats, flush=True)
    return stats


@pytest.mark.parametrize("batch", [4, 8])
def test_llama1b_batch_shared_position(llama1b, batch):
    shape, weights = llama1b
    run_and_compare(shape, weights, batch, [1024] * batch, 2, f"llama1b b{batch}")


@pytest.mark.parametrize("multikernel", [False, True], ids=["single-launch", "per-op"])
def test_llama1b_batch8_staggered_positions(llama1b, multikernel):
    shape, weights = llama1b
    run_and_compare(shape, weights, 8, [1024 - 37 * b for b in range(8)], 2, "llama1b b8 staggered", multikernel)


@pytest.mark.parametrize("batch", [1, 4])
def test_llama1b_step_at_last_cache_position(llama1b, batch):
    """The last step writes the cache's final slot (position max_seq - 1) and attends to every
    slot; rows of a batch stop one or more positions short of it."""
    shape, weights = llama1b
    run_and_compare(shape, weights, batch, [1022 - 3 * b for b in range(batch)], 2,
                    f"llama1b b{batch} to max_seq - 1", to_the_end=True)


@pytest.mark.parametrize("batch,multikernel", [(1, False), (4, False), (1, True)])
def test_llama1b_fp8_full_shape(llama1b, batch, multikernel):
    """FP8 weights (one scale per output row) at the full 1B shape: 16 layers, the 128256-row
    tied LM head, 1024 tokens in the cache; the oracle quantises the same way."""
    shape, weights = llama1b
    stats = run_and_compare(shape, weights, batch, [1024 - 5 * b for b in range(batch)], 2,
                            f"llama1b fp8 b{batch}" + (" per-op" if multikernel else ""), multikernel, flags=FP8)
    assert stats["max_abs"] < 2e-3


@pytest.mark.timeout(900)
def test_llama8b_fp8():
    shape = synth.LLAMA_8B
    weights = synth.make_weights(shape)
    stats = run_and_compare(shape, weights, 1, [1024], 2, "llama8b fp8", flags=FP8)
    assert stats["max_abs"] < 2e-3


@pytest.mark.parametrize("prompt", [8192, 32768])
def test_llama1b_long_context(llama1b, prompt):
    shape, weights = llama1b
    run_and_compare(shape, weights, 1, [prompt], 2, f"llama1b p{prompt}")


@pytest.mark.timeout(600)
def test_llama8b_head_dim_128():
    shape = synth.LLAMA_8B
    weights = synth.make_weights(shape)
    run_and_compare(shape, weights, 1, [1024], 2, "llama8b")


@pytest.mark.parametrize("n_chunks", [8, 16])
def test_uneven_rows_per_wave(n_chunks):
    """Down-projection chunks of 1024 or 512 rows give each CU 4 or 2 up/gate
    rows per instruction, so half or more of the compute waves have no row in
    those instructions and run ahead of the others; the staged-input buffers
    must still not be refilled while a slower wave reads them."""
    shape = dataclasses.replace(synth.LLAMA_1B, n_layers=2, vocab=4096)
    weights = synth.make_weights(shape)
    run_and_compare(shape, weights, 1, [64], 2, f"llama1b-dims 2 layers, {n_chunks} chunks", n_chunks=n_chunks)


def test_llama1b_dims_nonunit_norm_gains():
    """1B dimensions (2 layers) with RMSNorm gains 1 + N(0, 0.3): the folded
    gains of q/k/v, gate/up and the tied LM head against the oracle."""
    shape = dataclasses.replace(synth.LLAMA_1B, n_layers=2, vocab=4096)
    weights = synth.make_weights(shape, gain_std=0.3)
    stats = run_and_compare(shape, weights, 1, [64], 2, "llama1b-dims 2 layers, gains 1 + N(0, 0.3)")
    assert stats["max_abs"] < 1e-3  # fp32 path: ~1e-5; folded-gain rounding gave ~2e-2


@pytest.mark.parametrize("batch,multikernel", [(1, False), (4, False), (4, True)])
def test_llama1b_tp8_shard(batch, multikernel):
    """The per-GPU shape of an 8-way tensor-parallel 1B model (one KV group,
    F/8, V/8): attention output width 256 against hidden size 2048, so the
    O projection reads a 256-wide input and the up/gate instructions hold a
    single row pair."""
    shape = synth.LLAMA_1B_TP8_SHARD
    weights = synth.make_weights(shape)
    run_and_compare(shape, weights, batch, [1024 - 5 * b for b in range(batch)], 2,
                    f"llama1b tp8 shard b{batch}" + (" multikernel" if multikernel else ""), multikernel)
