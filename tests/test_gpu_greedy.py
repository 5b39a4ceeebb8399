"""mk_greedy_advance against torch.argmax on the host: lowest index on ties,
positions advanced, odd vocabulary sizes (unaligned rows)."""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("batch,vocab", [(1, 128256), (4, 128256), (8, 1024), (3, 1023), (2, 5)])
def test_greedy_matches_argmax(batch, vocab):
    import torch
    from decode_megakernel_02_amd import mk
    shape = synth.ModelShape("greedy", 1, 256, 4, 2, 64, 688, vocab, 1e-5, 1e4, True)
    h = mk.mk_create(mk.make_config(shape, batch, 64))
    try:
        rng = np.random.default_rng(batch * 7919 + vocab)
        lg = rng.standard_normal((batch, vocab)).astype(np.float32)
        lg[0, vocab // 3] = lg[0, vocab - 1] = lg[0].max() + 1.0  # tie: the lower index wins
        if batch > 1:
            lg[1, :] = 0.5  # all equal: index 0
        pos0 = np.arange(batch, dtype=np.int32) * 3
        d_lg = torch.from_numpy(lg).cuda()
        d_tok = torch.full((batch,), -1, dtype=torch.int32, device="cuda")
        d_pos = torch.from_numpy(pos0.copy()).cuda()
        mk.mk_greedy_advance(h, d_lg, d_tok, d_pos, mk.current_stream())
        torch.cuda.synchronize()
        ref = torch.argmax(torch.from_numpy(lg), dim=1).numpy()
        assert (d_tok.cpu().numpy() == ref).all()
        assert (d_pos.cpu().numpy() == pos0 + 1).all()
        assert ref[0] == vocab // 3
    finally:
        mk.mk_destroy(h)


def test_greedy_repeated_calls_and_nan():
    """Back-to-back calls on one handle (the per-row slice counter must be back
    at zero after each call) and NaN logits: NaN never wins, an all-NaN row
    gives token 0."""
    import torch
    from decode_megakernel_02_amd import mk
    batch, vocab = 3, 128256
    shape = synth.ModelShape("greedy", 1, 256, 4, 2, 64, 688, vocab, 1e-5, 1e4, True)
    h = mk.mk_create(mk.make_config(shape, batch, 64))
    try:
        rng = np.random.default_rng(11)
        d_tok = torch.zeros(batch, dtype=torch.int32, device="cuda")
        d_pos = torch.zeros(batch, dtype=torch.int32, device="cuda")
        for call in range(4):
            lg = rng.standard_normal((batch, vocab)).astype(np.float32)
            lg[0, rng.integers(vocab, size=500)] = np.nan
            lg[2, :] = np.nan
            want = np.nanargmax(np.where(np.isnan(lg[:2]), -np.inf, lg[:2]), axis=1)
            d_lg = torch.from_numpy(lg).cuda()
            mk.mk_greedy_advance(h, d_lg, d_tok, d_pos, mk.current_stream())
            torch.cuda.synchronize()
            got = d_tok.cpu().numpy()
            assert got[0] == want[0] and got[1] == want[1], (call, got, want)
            assert got[2] == 0
            assert (d_pos.cpu().numpy() == call + 1).all()
    finally:
        mk.mk_destroy(h)
