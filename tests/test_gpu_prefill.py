"""Batched prefill (mk_prefill) against the oracle run token by token.

The oracle's decode step at positions 0 .. P-1 with the prompt tokens is the
plain definition of what a prefill computes: the KV cache slots [0, P) and
the logits of position P-1.  Compared here: the logits to the usual bar, the
cache to the decode path's cache bar (max |d| <= 2e-2 max(1, max |ref|), over
90 % of the bf16 values bit-equal: a value near a rounding boundary may round
the other way), and greedy decode steps
continued from the prefilled cache, against the oracle continuing from its own.
"""
import dataclasses

import numpy as np
import pytest

import synth
from tests import helpers as H

pytestmark = pytest.mark.gpu


def bf16_to_f32(a):
    return (a.astype(np.uint32) << 16).view(np.float32)


def prefill_and_compare(shape, batch, P, decode_steps, label):
    import torch
    import oracle
    from decode_megakernel_02_amd import mk
    weights = synth.make_weights(shape)
    max_seq = P + decode_steps + 1
    prompts = synth.make_prompts(shape.vocab, batch, P)
    dec = H.GpuDecoder(shape, weights, batch, max_seq)
    try:
        toks = torch.as_tensor(np.ascontiguousarray(prompts, dtype=np.int32)).cuda()
        mk.mk_prefill(dec.h, dec.dw, toks, P, dec.kv, dec.logits, mk.current_stream())
        torch.cuda.synchronize()
        gpu_logits = dec.logits.cpu().numpy().copy()
        gpu_kv = dec.kv_host().copy()
        nxt = np.argmax(gpu_logits, axis=1).astype(np.int32)
        run = dec.greedy(nxt, np.full(batch, P, dtype=np.int32), decode_steps)
    finally:
        dec.close()
    orc = oracle.Oracle(shape, weights, batch, max_seq)
    cache = np.zeros(synth.kv_cache_shape(shape, batch, max_seq), dtype=np.uint16)
    ref = None
    for t in range(P):
        ref = orc.decode_step(cache, prompts[:, t].astype(np.int32), np.full(batch, t, dtype=np.int32), 8)
    stats = H.compare(H.Run([prompts[:, -1]], [np.full(batch, P - 1)], [gpu_logits]), [ref], label + " prefill")
    g = bf16_to_f32(gpu_kv[..., :P, :])
    o = bf16_to_f32(cache[..., :P, :])
    # the decode path's cache bar: rounding-order differences flip some bf16 roundings
    kv_err = float(np.max(np.abs(g - o)))
    assert kv_err <= 2e-2 * max(1.0, float(np.max(np.abs(o)))), (label, kv_err)
    frac_equal = float(np.mean(gpu_kv[..., :P, :] == cache[..., :P, :]))
    assert frac_equal > 0.9, (label, frac_equal)
    # decode continues from the prefilled cache; the oracle continues from its own
    H.compare(run, H.oracle_replay(shape, weights, batch, max_seq, run, kv_init=cache), label + " decode")
    print(label, stats, "kv max|d|", kv_err, "bit-equal fraction", frac_equal, flush=True)


@pytest.mark.parametrize("batch,P", [(1, 1), (2, 37), (3, 130)])
def test_tiny_prefill_matches_token_by_token_oracle(batch, P):
    prefill_and_compare(synth.TINY, batch, P, 3, f"tiny b{batch} p{P}")


def test_llama1b_dims_prefill():
    """1B dimensions (2 layers, 4096-token vocabulary): 64-row tiles over a
    ragged 100-position prompt, 32 query heads over 8 KV groups."""
    shape = dataclasses.replace(synth.LLAMA_1B, n_layers=2, vocab=4096)
    prefill_and_compare(shape, 2, 100, 2, "llama1b-dims 2 layers p100")


def test_llama8b_dims_prefill_head_dim_128():
    shape = dataclasses.replace(synth.LLAMA_8B, n_layers=1, vocab=4096, hidden=1024, ffn=2048, n_q_heads=8,
                                n_kv_heads=2)
    prefill_and_compare(shape, 1, 70, 2, "head_dim 128, untied, p70")


def test_prefill_rejects_out_of_range_token():
    import torch
    from decode_megakernel_02_amd import mk
    shape = synth.TINY
    dec = H.GpuDecoder(shape, synth.make_weights(shape), 1, 16)
    try:
        toks = torch.tensor([[1, 2, shape.vocab, 3]], dtype=torch.int32, device="cuda")
        with pytest.raises(mk.MkError) as e:
            mk.mk_prefill(dec.h, dec.dw, toks, 4, dec.kv, dec.logits, mk.current_stream())
        assert e.value.code == mk.MK_ERR_INVALID_ARG
        with pytest.raises(mk.MkError):
            mk.mk_prefill(dec.h, dec.dw, toks, 17, dec.kv, dec.logits, mk.current_stream())  # > max_seq
    finally:
        dec.close()


def test_full_llama1b_p1024(llama1b):
    """The benchmarked prefill shape (full 1B, one 1024-token prompt): the prefill's cache and logits
    against the decode step run token by token on the GPU (oracle-pinned at this shape by the parity
    tests), and its last-position logits against one oracle step on the prefilled cache (slots
    0 .. 1022 from the prefill; the oracle computes slot 1023 itself)."""
    import torch
    import oracle
    from decode_megakernel_02_amd import mk
    shape, weights = llama1b
    B, P = 1, 1024
    max_seq = P + 2
    prompts = synth.make_prompts(shape.vocab, B, P)
    dec = H.GpuDecoder(shape, weights, B, max_seq)
    try:
        toks = torch.as_tensor(np.ascontiguousarray(prompts, dtype=np.int32)).cuda()
        mk.mk_prefill(dec.h, dec.dw, toks, P, dec.kv, dec.logits, mk.current_stream())
        torch.cuda.synchronize()
        pf_logits = dec.logits.cpu().numpy().copy()
        pf_kv = dec.kv_host().copy()
        dec.kv.zero_()
        for t in range(P):  # the decode step, token by token
            lg = dec.step(prompts[:, t], np.full(B, t, dtype=np.int32))
        dk_kv = dec.kv_host().copy()
    finally:
        dec.close()
    d = float(np.max(np.abs(pf_logits - lg)))
    assert d <= 1e-2, f"prefill vs token-by-token decode: max|d| {d}"
    g, o = bf16_to_f32(pf_kv[..., :P, :]), bf16_to_f32(dk_kv[..., :P, :])
    assert float(np.max(np.abs(g - o))) <= 2e-2 * max(1.0, float(np.max(np.abs(o))))
    # bf16 roundings of values computed in different summation orders: over 16 layers the fp32
    # differences grow with depth and flip more of them than over two layers (the bound above and
    # the oracle comparison below are the parity checks; this only guards against wholesale error)
    assert float(np.mean(pf_kv[..., :P, :] == dk_kv[..., :P, :])) > 0.8
    orc = oracle.Oracle(shape, weights, B, max_seq)
    cache = pf_kv.copy()
    ref = orc.decode_step(cache, prompts[:, P - 1].astype(np.int32), np.full(B, P - 1, dtype=np.int32), 16)
    stats = H.compare(H.Run([prompts[:, -1]], [np.full(B, P - 1)], [pf_logits]), [ref], "1B P1024 prefill")
    print("1B P1024 prefill: vs decode max|d|", d, "vs oracle", stats, flush=True)


@pytest.mark.timeout(600)
def test_full_llama1b_p8192(llama1b):
    """The long-prompt benchmark shape (full 1B, one 8192-token prompt: 128 query blocks and up
    to 256 key tiles per head in the prefill's attention, the chunked pass when the workspace
    cap applies): logits and cache against the decode step run token by token on the GPU, and the
    last-position logits against one oracle step on the prefilled cache."""
    import torch
    import oracle
    from decode_megakernel_02_amd import mk
    shape, weights = llama1b
    B, P = 1, 8192
    max_seq = P + 2
    prompts = synth.make_prompts(shape.vocab, B, P)
    dec = H.GpuDecoder(shape, weights, B, max_seq)
    try:
        toks = torch.as_tensor(np.ascontiguousarray(prompts, dtype=np.int32)).cuda()
        mk.mk_prefill(dec.h, dec.dw, toks, P, dec.kv, dec.logits, mk.current_stream())
        torch.cuda.synchronize()
        pf_logits = dec.logits.cpu().numpy().copy()
        pf_kv = dec.kv_host().copy()
        dec.kv.zero_()
        s = mk.current_stream()
        dtok = torch.as_tensor(np.ascontiguousarray(prompts[0], dtype=np.int32)).cuda()  # B = 1
        dpos = torch.arange(P, dtype=torch.int32, device="cuda")
        for t in range(P):  # the decode step, token by token, with no host round trip per step
            mk.mk_decode_step(dec.h, dtok[t:t + 1], dpos[t:t + 1], dec.kv, dec.logits, s)
        torch.cuda.synchronize()
        assert mk.mk_get_device_error(dec.h) is None
        lg = dec.logits.cpu().numpy().copy()
        dk_kv = dec.kv_host().copy()
    finally:
        dec.close()
    d = float(np.max(np.abs(pf_logits - lg)))
    assert d <= 1e-2, f"prefill vs token-by-token decode: max|d| {d}"
    g, o = bf16_to_f32(pf_kv[..., :P, :]), bf16_to_f32(dk_kv[..., :P, :])
    assert float(np.max(np.abs(g - o))) <= 2e-2 * max(1.0, float(np.max(np.abs(o))))
    assert float(np.mean(pf_kv[..., :P, :] == dk_kv[..., :P, :])) > 0.8
    orc = oracle.Oracle(shape, weights, B, max_seq)
    cache = pf_kv.copy()
    ref = orc.decode_step(cache, prompts[:, P - 1].astype(np.int32), np.full(B, P - 1, dtype=np.int32), 16)
    stats = H.compare(H.Run([prompts[:, -1]], [np.full(B, P - 1)], [pf_logits]), [ref], "1B P8192 prefill")
    print("1B P8192 prefill: vs decode max|d|", d, "vs oracle", stats, flush=True)
