"""mk_decode_step_greedy: the decode step with greedy selection fused into the same launch.

Against the two-launch path (mk_decode_step + mk_greedy_advance) from the same start: the
logits of every step are bit-identical (the same op bodies), and so are the tokens and
positions; every token is the lowest-index argmax of its step's logits; the logits follow the
teacher-forced oracle to the usual bar (tokens where the oracle's top two are clearly apart).
Also captured in a graph (MK_GRAPH_FUSED_GREEDY), replays separated by eager work; and heads
built so that the largest logit is tied across rows, waves and CUs (the lowest index wins)."""
import dataclasses

import numpy as np
import pytest

import synth
from tests import helpers as H

pytestmark = pytest.mark.gpu

FP8 = 4  # MK_FLAG_FP8_WEIGHTS


def run_both(shape, weights, batch, prompt_lens, steps, flags=0, kv_fill=True, return_run=False):
    import torch
    from decode_megakernel_02_amd import mk
    P = np.asarray(prompt_lens, dtype=np.int32)
    max_seq = int(P.max()) + steps + 1
    kv = synth.make_kv_cache(shape, batch, max_seq, int(P.max())) if kv_fill else None
    first = synth.make_first_tokens(shape.vocab, batch)
    dec = H.GpuDecoder(shape, weights, batch, max_seq, kv_init=kv, flags=flags)
    s = mk.current_stream()
    out = {}
    try:
        for fused in (False, True):
            dec.kv.copy_(H.to_device_u16(kv.reshape(-1)) if kv is not None else torch.zeros_like(dec.kv))
            dec.tokens.copy_(torch.as_tensor(first))
            dec.positions.copy_(torch.as_tensor(P))
            run = H.Run([], [], [])
            for _ in range(steps):
                run.tokens.append(dec.tokens.cpu().numpy().copy())
                run.positions.append(dec.positions.cpu().numpy().copy())
                if fused:
                    mk.mk_decode_step_greedy(dec.h, dec.tokens, dec.positions, dec.kv, dec.logits, s)
                else:
                    mk.mk_decode_step(dec.h, dec.tokens, dec.positions, dec.kv, dec.logits, s)
                    mk.mk_greedy_advance(dec.h, dec.logits, dec.tokens, dec.positions, s)
                torch.cuda.synchronize()
                run.logits.append(dec.logits.cpu().numpy().copy())
            run.tokens.append(dec.tokens.cpu().numpy().copy())
            run.positions.append(dec.positions.cpu().numpy().copy())
            assert mk.mk_get_device_error(dec.h) is None
            out[fused] = run
    finally:
        dec.close()
    a, b = out[False], out[True]
    for i in range(steps):
        np.testing.assert_array_equal(b.logits[i], a.logits[i], err_msg=f"step {i} logits")
        np.testing.assert_array_equal(b.tokens[i + 1], np.argmax(b.logits[i], axis=1), err_msg=f"step {i} argmax")
    for i in range(steps + 1):
        np.testing.assert_array_equal(b.tokens[i], a.tokens[i], err_msg=f"tokens after {i} steps")
        np.testing.assert_array_equal(b.positions[i], a.positions[i], err_msg=f"positions after {i} steps")
    np.testing.assert_array_equal(b.positions[-1], P + steps)
    oracle_run = H.Run(b.tokens[:steps], b.positions[:steps], b.logits)
    ref = H.oracle_replay(shape, weights, batch, max_seq, oracle_run, kv_init=kv, nthreads=16,
                          fp8="row" if flags & FP8 else False)
    stats = H.compare(oracle_run, ref, f"fused greedy {shape.name} b{batch}")
    return (stats, b) if return_run else stats


@pytest.mark.parametrize("batch", [1, 2, 4])
def test_tiny(batch):
    shape = synth.TINY
    print(run_both(shape, synth.make_weights(shape), batch, [20 + 3 * b for b in range(batch)], 6))


def _head_with_every_row_four_times(shape):
    """The seeded weights with an LM head (the tied embedding) in which every row occurs four
    times: row 2k + 1 is a copy of row 2k, and the second half of the vocabulary a copy of the
    first.  Whatever the hidden state, the largest logit is then a four-way tie at rows 2k,
    2k + 1, 2k + V/2 and 2k + V/2 + 1: within one row pair (batched LM head), across the
    waves of one CU (batch 1) and across CUs."""
    w = dict(synth.make_weights(shape))
    key = "embed" if w["lm_head"] is None else "lm_head"
    head = np.ascontiguousarray(w[key]).copy()
    V = shape.vocab
    head[1::2] = head[0::2]
    head[V // 2:] = head[:V // 2]
    w[key] = head
    return w


@pytest.mark.parametrize("batch", [1, 3])
def test_tied_maximum_takes_the_lowest_index(batch):
    """Equal largest logits on several rows, waves and CUs: the fused token is the lowest of them
    (the order np.argmax and the oracle's selection use)."""
    shape = synth.TINY
    V = shape.vocab
    stats, run = run_both(shape, _head_with_every_row_four_times(shape), batch, [20 + 3 * b for b in range(batch)],
                          4, return_run=True)
    print(stats)
    for i, lg in enumerate(run.logits):
        for b in range(batch):
            top = np.flatnonzero(lg[b] == lg[b].max())
            t = top[0]
            assert t % 2 == 0 and t < V // 2 and {t, t + 1, t + V // 2, t + V // 2 + 1} <= set(top.tolist()), (i, b, top)
            assert run.tokens[i + 1][b] == t, (i, b, run.tokens[i + 1][b], top)


@pytest.mark.parametrize("batch", [1, 3])
def test_zero_head_ties_every_row(batch):
    """An all-zero LM head (the tied embedding): every logit of every row is 0, a tie across all
    rows, waves and CUs, so every fused token is 0."""
    shape = synth.TINY
    w = dict(synth.make_weights(shape))
    w["embed"] = np.zeros_like(w["embed"])
    stats, run = run_both(shape, w, batch, [20 + 3 * b for b in range(batch)], 3, return_run=True)
    print(stats)
    for i, lg in enumerate(run.logits):
        assert not lg.any(), i
        np.testing.assert_array_equal(run.tokens[i + 1], np.zeros(batch, dtype=np.int32))


def test_llama1b_full(llama1b):
    shape, weights = llama1b
    print(run_both(shape, weights, 1, [1024], 4))


def test_llama1b_full_batch8_staggered(llama1b):
    shape, weights = llama1b
    print(run_both(shape, weights, 8, [1024 - 37 * b for b in range(8)], 2))


def test_llama1b_dims_fp8():
    shape = dataclasses.replace(synth.LLAMA_1B, n_layers=2, vocab=4096)
    print(run_both(shape, synth.make_weights(shape), 2, [64, 60], 3, flags=FP8))


def test_graph_of_fused_steps_matches_eager():
    import torch
    from decode_megakernel_02_amd import mk
    shape, B, P, n = synth.TINY, 2, 8, 5
    dec = H.GpuDecoder(shape, synth.make_weights(shape), B, P + n + 2)
    s = mk.current_stream()
    first = synth.make_first_tokens(shape.vocab, B)
    g = None

    def start():
        dec.kv.zero_()
        dec.tokens.copy_(torch.as_tensor(first))
        dec.positions.fill_(P)

    try:
        start()
        ref = []
        for _ in range(n):
            mk.mk_decode_step_greedy(dec.h, dec.tokens, dec.positions, dec.kv, dec.logits, s)
            torch.cuda.synchronize()
            ref.append((dec.logits.cpu().numpy().copy(), dec.tokens.cpu().numpy().copy(),
                        dec.positions.cpu().numpy().copy()))
        start()
        torch.cuda.synchronize()
        try:
            g = mk.mk_graph_create(dec.h, dec.tokens, dec.positions, dec.kv, dec.logits, 1, mk.MK_GRAPH_FUSED_GREEDY)
        except mk.MkError as e:
            if e.code == mk.MK_ERR_HIP:
                pytest.skip(f"the runtime refuses to capture the cooperative single-launch step: {e}")
            raise
        for r, (lg, tok, pos) in enumerate(ref):
            mk.mk_graph_launch(g, s)
            torch.cuda.synchronize()
            assert torch.arange(64, device="cuda").sum().item() == 2016  # eager work between replays
            np.testing.assert_array_equal(dec.logits.cpu().numpy(), lg, err_msg=f"replay {r}")
            np.testing.assert_array_equal(dec.tokens.cpu().numpy(), tok, err_msg=f"replay {r}")
            np.testing.assert_array_equal(dec.positions.cpu().numpy(), pos, err_msg=f"replay {r}")
        assert mk.mk_get_device_error(dec.h) is None
    finally:
        if g is not None:
            mk.mk_graph_destroy(g)
        dec.close()
