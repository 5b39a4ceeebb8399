"""mk_set_ablation: the measurement build of the single-launch step with one opcode's
arithmetic switched off.  Closed forms where the switched-off op decides the result (LM head
off: every logit 0; QKV off: the K and V rows the step appends are 0), every opcode runs to
completion without a device error, and switching the ablation off again gives the normal
step's logits bit for bit."""
import numpy as np
import pytest

import synth
from tests import helpers as H

pytestmark = pytest.mark.gpu


def test_each_opcode_switched_off():
    shape, B, P = synth.TINY, 2, 9
    w = synth.make_weights(shape)
    max_seq = P + 4
    kv0 = synth.make_kv_cache(shape, B, max_seq, P)
    dec = H.GpuDecoder(shape, w, B, max_seq, kv_init=kv0)
    from decode_megakernel_02_amd import mk
    toks = synth.make_first_tokens(shape.vocab, B)
    pos = np.full(B, P, dtype=np.int32)
    try:
        normal = dec.step(toks, pos)
        kv_shape = synth.kv_cache_shape(shape, B, max_seq)  # [L][2][B][Hkv][max_seq][D]
        for op in range(1, 8):
            dec.kv.copy_(H.to_device_u16(kv0.reshape(-1)))
            mk.mk_set_ablation(dec.h, op)
            lg = dec.step(toks, pos)
            assert mk.mk_get_device_error(dec.h) is None, op
            kv = dec.kv_host().reshape(kv_shape)
            if op == 7:
                assert np.all(lg == 0.0)
            else:
                assert np.all(np.isfinite(lg)), op
                assert not np.array_equal(lg, normal), op
            new_rows = kv[:, :, :, :, P, :] & 0x7FFF  # magnitude bits (RoPE of a zero row may give -0)
            if op == 1:
                assert np.all(new_rows == 0)
            else:
                assert np.any(new_rows != 0), op
        mk.mk_set_ablation(dec.h, 0)
        dec.kv.copy_(H.to_device_u16(kv0.reshape(-1)))
        np.testing.assert_array_equal(dec.step(toks, pos), normal)
        with pytest.raises(mk.MkError):
            mk.mk_set_ablation(dec.h, 8)
    finally:
        dec.close()
