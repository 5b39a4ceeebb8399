"""The allocation-free prefill (mk_prefill_static, include/mk.h) against the
allocating one (mk_prefill) on the same inputs, two calls in a row with the
second smaller.  Both run the same kernels; the static one goes through the
prompt in chunks sized to its 64 MiB scratch (attention reads the earlier
chunks from the cache), which changes no element's arithmetic: the logits
and the KV cache must be bit-identical."""
import dataclasses

import numpy as np
import pytest

import synth
from tests import helpers as H

pytestmark = pytest.mark.gpu

# Llama-1B layer dimensions, 2 layers and a 4096-token vocabulary: 100 KiB of
# fp32 rows per position, so two batch rows of a 700-token prompt need three
# passes through the 64 MiB scratch
SHAPE = dataclasses.replace(synth.LLAMA_1B, name="1b-dims-2l", n_layers=2, vocab=4096)


def run_pair(dec, weights_dev, prompts, P, seed_logits):
    import torch
    from decode_megakernel_02_amd import mk
    s = mk.current_stream()
    toks = torch.as_tensor(np.ascontiguousarray(prompts[:, :P], dtype=np.int32)).cuda()
    out = {}
    for name, fn in [("static", mk.mk_prefill_static), ("alloc", mk.mk_prefill)]:
        dec.kv.zero_()
        dec.logits.fill_(seed_logits)  # stale values from an earlier call must not survive
        fn(dec.h, weights_dev, toks, P, dec.kv, dec.logits, s)
        torch.cuda.synchronize()
        assert mk.mk_get_device_error(dec.h) is None
        out[name] = (dec.logits.cpu().numpy().copy(), dec.kv_host()[..., :P, :].copy())
    return out


def test_static_prefill_matches_allocating_prefill_twice():
    B, P1, P2 = 2, 700, 90
    weights = synth.make_weights(SHAPE)
    prompts = synth.make_prompts(SHAPE.vocab, B, P1)
    dec = H.GpuDecoder(SHAPE, weights, B, P1 + 8)
    try:
        for P, seed in [(P1, 7.0), (P2, -3.0)]:
            out = run_pair(dec, dec.dw, prompts, P, seed)
            (ls, ks), (la, ka) = out["static"], out["alloc"]
            assert np.all(np.isfinite(ls))
            assert np.array_equal(ls, la), f"P={P}: logits differ, max|d| {np.max(np.abs(ls - la))}"
            assert np.array_equal(ks, ka), f"P={P}: KV cache differs in {np.sum(ks != ka)} values"
            print(f"P={P}: logits and cache bit-identical", flush=True)
    finally:
        dec.close()


def test_static_prefill_reports_bad_token_in_error_record():
    import torch
    from decode_megakernel_02_amd import mk
    B, P = 1, 40
    weights = synth.make_weights(synth.TINY)
    dec = H.GpuDecoder(synth.TINY, weights, B, P + 4)
    try:
        prompts = synth.make_prompts(synth.TINY.vocab, B, P)
        prompts[0, 17] = synth.TINY.vocab + 5
        toks = torch.as_tensor(np.ascontiguousarray(prompts, dtype=np.int32)).cuda()
        mk.mk_prefill_static(dec.h, dec.dw, toks, P, dec.kv, dec.logits, mk.current_stream())
        err = mk.mk_get_device_error(dec.h)
        assert err is not None and err.code == 2 and err.pc == 17 and err.detail == 0
        assert mk.mk_get_device_error(dec.h) is None
    finally:
        dec.close()
