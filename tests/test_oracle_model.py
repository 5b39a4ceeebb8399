"""Pins of the oracle's whole decode step.

* a hand-built 1-layer model whose logits have a closed form (pins the order of
  the sub-steps, both residual adds, SwiGLU's gate/up roles and causal range);
* a degenerate model (all layer matrices zero) whose logits have a closed form;
* an independent full-sequence causal forward (no KV cache, numpy) against
  token-by-token decode (pins the cache logic);
* batch-row independence, GQA head->group mapping, tied == untied with a copied
  head, and argument errors.
"""
import dataclasses
import math

import numpy as np
import pytest
import torch

import oracle
import synth

BF16_ONE = 0x3F80


def f32_to_bf16_bits(x):
    t = torch.tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().astype(np.uint16)


def bits_to_f64(bits):
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


def run_steps(shape, weights, tokens_per_step, positions_per_step, max_seq, cache=None):
    B = len(tokens_per_step[0])
    orc = oracle.Oracle(shape, weights, B, max_seq)
    if cache is None:
        cache = np.zeros(synth.kv_cache_shape(shape, B, max_seq), dtype=np.uint16)
    out = []
    for t, p in zip(tokens_per_step, positions_per_step):
        out.append(orc.decode_step(cache, t, p))
    return out, cache


# ------------------------------------------------------- hand model --------

HAND = synth.ModelShape("hand", 1, 4, 1, 1, 4, 1, 4, 0.0, 10000.0, True)


def hand_weights():
    f = lambda a: f32_to_bf16_bits(np.asarray(a, dtype=np.float32))
    E = f([[1, 1, 1, 1], [1, 0, 0, 0], [0, 1, 0, 0], [0, 0, 1, -1]])
    layer = {
        "attn_norm": np.full(4, BF16_ONE, np.uint16), "mlp_norm": np.full(4, BF16_ONE, np.uint16),
        "wq": f(np.zeros((4, 4))), "wk": f(np.zeros((4, 4))), "wv": f(np.eye(4)),
        "wo": f(0.5 * np.eye(4)),
        "w_gate": f([[1, 0, 0, 0]]), "w_up": f([[0, 2, 0, 0]]), "w_down": f([[1], [0], [0], [-1]]),
    }
    return {"embed": E, "final_norm": np.full(4, BF16_ONE, np.uint16), "lm_head": None,
            "layers": [layer]}


def silu(z):
    return z / (1.0 + math.exp(-z))


def test_hand_model_first_token_closed_form():
    # token 0 = [1,1,1,1] at position 0: attention returns v = x = 1, h = 1.5*1,
    # gate = 1, up = 2, a = 2 silu(1), h = [1.5+a, 1.5, 1.5, 1.5-a]
    (logits,), _ = run_steps(HAND, hand_weights(), [[0]], [[0]], 4)
    a = 2.0 * silu(1.0)
    h = np.array([1.5 + a, 1.5, 1.5, 1.5 - a])
    rms = math.sqrt(np.mean(h ** 2))
    expect = np.array([6.0, 1.5 + a, 1.5, a]) / rms
    np.testing.assert_allclose(logits[0], expect, rtol=1e-12)


def test_hand_model_second_token_attends_both_positions():
    # token 1 = e_0 at position 1: x = [2,0,0,0]; q = 0 so both cached rows weigh 1/2:
    # o = ([1,1,1,1] + [2,0,0,0]) / 2, h = e_0 + o/2 = [1.75, .25, .25, .25]
    (_, logits), cache = run_steps(HAND, hand_weights(), [[0], [1]], [[0], [1]], 4)
    h = np.array([1.75, 0.25, 0.25, 0.25])
    x = h / math.sqrt(np.mean(h ** 2))
    a = silu(x[0]) * 2.0 * x[1]
    h = h + np.array([a, 0, 0, -a])
    xf = h / math.sqrt(np.mean(h ** 2))
    E = np.array([[1, 1, 1, 1], [1, 0, 0, 0], [0, 1, 0, 0], [0, 0, 1, -1]], dtype=np.float64)
    np.testing.assert_allclose(logits[0], E @ xf, rtol=1e-12)
    # the cache now holds V rows [1,1,1,1] and [2,0,0,0] and zero K rows
    np.testing.assert_array_equal(bits_to_f64(cache[0, 1, 0, 0, :2]),
                                  [[1, 1, 1, 1], [2, 0, 0, 0]])
    assert np.all(cache[0, 0] == 0)


# --------------------------------------------------- identity model ---------

def test_zero_layers_model_closed_form():
    m = dataclasses.replace(synth.TINY, name="tiny-zero")
    w = synth.make_weights(m, zero_layers=True)
    toks = [3, 500, 1023]
    (logits,), _ = run_steps(m, w, [toks], [[0, 5, 9]], 16)
    E = bits_to_f64(w["embed"]).reshape(m.vocab, m.hidden)
    for b, t in enumerate(toks):
        e = E[t]
        x = e / math.sqrt(np.mean(e ** 2) + m.rms_eps)
        np.testing.assert_allclose(logits[b], E @ x, rtol=1e-10, atol=1e-12)
        assert oracle.argmax(logits[b]) == t


# ----------------------------------------- full causal recompute (numpy) ----

def full_forward(m, w, tokens):
    """Causal forward over the whole sequence at once, no cache: logits [n][V].
    K and V rows are rounded to bf16 as the cache stores them."""
    n, H, D, Hq, Hkv = len(tokens), m.hidden, m.head_dim, m.n_q_heads, m.n_kv_heads
    M = lambda a: bits_to_f64(a).reshape(a.shape)
    g = lambda a: bits_to_f64(a)

    def norm(X, gain):
        return X / np.sqrt(np.mean(X ** 2, axis=1, keepdims=True) + m.rms_eps) * g(gain)

    pos = np.arange(n)[:, None]
    half = D // 2
    freqs = m.rope_theta ** (-2.0 * np.arange(half) / D)
    ang = pos * freqs[None, :]
    cos, sin = np.cos(ang), np.sin(ang)

    def rope(X):  # X [n][heads*D]
        X = X.reshape(n, -1, D)
        u, v = X[..., :half], X[..., half:]
        c, s = cos[:, None, :], sin[:, None, :]
        return np.concatenate([u * c - v * s, v * c + u * s], axis=-1)

    X = M(w["embed"])[tokens]
    for L in w["layers"]:
        x = norm(X, L["attn_norm"])
        q = rope(x @ M(L["wq"]).T)
        k = rope(x @ M(L["wk"]).T)
        v = (x @ M(L["wv"]).T).reshape(n, Hkv, D)
        k = bits_to_f64(f32_to_bf16_bits(k)).reshape(k.shape)
        v = bits_to_f64(f32_to_bf16_bits(v)).reshape(v.shape)
        o = np.zeros((n, Hq, D))
        mask = np.tril(np.ones((n, n), dtype=bool))
        for hd in range(Hq):
            grp = hd * Hkv // Hq
            s = q[:, hd, :] @ k[:, grp, :].T / math.sqrt(D)
            s = np.where(mask, s, -np.inf)
            p = np.exp(s - s.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            o[:, hd, :] = p @ v[:, grp, :]
        X = X + o.reshape(n, Hq * D) @ M(L["wo"]).T
        x = norm(X, L["mlp_norm"])
        gt, up = x @ M(L["w_gate"]).T, x @ M(L["w_up"]).T
        X = X + (gt / (1.0 + np.exp(-gt)) * up) @ M(L["w_down"]).T
    head = w["embed"] if m.tied else w["lm_head"]
    return norm(X, w["final_norm"]) @ M(head).T


@pytest.mark.parametrize("gain_std", [0.0, 0.1])
def test_incremental_decode_equals_full_causal_recompute(gain_std):
    m = synth.TINY
    w = synth.make_weights(m, seed=99, gain_std=gain_std)
    n = 12
    toks = synth.make_prompts(m.vocab, 1, n, seed=5)[0]
    steps, _ = run_steps(m, w, [[t] for t in toks], [[p] for p in range(n)], n)
    ref = full_forward(m, w, toks)
    for p in range(n):
        # tolerance covers torch's float32-then-bf16 rounding of K/V in the reference
        np.testing.assert_allclose(steps[p][0], ref[p], atol=2e-3, rtol=0)
    # far tighter than any indexing mistake, which moves logits by O(0.1)
    assert max(np.max(np.abs(steps[p][0] - ref[p])) for p in range(n)) < 2e-3


# ------------------------------------------------------- equivalences -------

def test_batch_rows_are_independent():
    m = synth.TINY
    w = synth.make_weights(m, seed=11)
    seqs = synth.make_prompts(m.vocab, 2, 6, seed=8)
    both, _ = run_steps(m, w, [list(seqs[:, i]) for i in range(6)],
                        [[i, i] for i in range(6)], 8)
    for b in range(2):
        one, _ = run_steps(m, w, [[seqs[b, i]] for i in range(6)], [[i] for i in range(6)], 8)
        for i in range(6):
            np.testing.assert_array_equal(both[i][b], one[i][0])


def test_batch_rows_at_different_positions():
    m = synth.TINY
    w = synth.make_weights(m, seed=12)
    cache = synth.make_kv_cache(m, 2, 16, 10, seed=3)
    single = [np.ascontiguousarray(cache[:, :, b:b + 1]) for b in range(2)]
    (both,), _ = run_steps(m, w, [[5, 6]], [[3, 9]], 16, cache=cache.copy())
    for b, (t, p) in enumerate([(5, 3), (6, 9)]):
        (one,), _ = run_steps(m, w, [[t]], [[p]], 16, cache=single[b].copy())
        np.testing.assert_array_equal(both[b], one[0])


def test_gqa_mapping_matches_duplicated_kv_heads():
    # Hq=4, Hkv=2 (heads 0,1 -> group 0; heads 2,3 -> group 1) must equal Hkv=4
    # with each group's K/V rows copied to the heads that read it
    m = synth.TINY
    w = synth.make_weights(m, seed=13)
    D = m.head_dim
    mha = dataclasses.replace(m, name="tiny-mha", n_kv_heads=4)
    w2 = {k: v for k, v in w.items() if k != "layers"}
    w2["layers"] = []
    for L in w["layers"]:
        L2 = dict(L)
        for kind in ("wk", "wv"):
            rows = L[kind].reshape(2, D, m.hidden)
            L2[kind] = np.ascontiguousarray(np.concatenate([rows[0], rows[0], rows[1], rows[1]]))
        w2["layers"].append(L2)
    toks = [[7], [100], [900], [3]]
    pos = [[0], [1], [2], [3]]
    a, _ = run_steps(m, w, toks, pos, 4)
    b, _ = run_steps(mha, w2, toks, pos, 4)
    for i in range(4):
        np.testing.assert_array_equal(a[i], b[i])


def test_untied_head_equal_to_embedding_matches_tied():
    m = synth.TINY
    w = synth.make_weights(m, seed=14)
    mu = dataclasses.replace(m, name="tiny-untied", tied=False)
    wu = dict(w)
    wu["lm_head"] = w["embed"].copy()
    a, _ = run_steps(m, w, [[1], [2]], [[0], [1]], 4)
    b, _ = run_steps(mu, wu, [[1], [2]], [[0], [1]], 4)
    np.testing.assert_array_equal(a[1], b[1])


def test_argument_errors_write_nothing():
    m = synth.TINY
    w = synth.make_weights(m, seed=15)
    orc = oracle.Oracle(m, w, 1, 8)
    cache = np.zeros(synth.kv_cache_shape(m, 1, 8), dtype=np.uint16)
    for tok, pos in [(-1, 0), (m.vocab, 0), (0, -1), (0, 8)]:
        with pytest.raises(ValueError):
            orc.decode_step(cache, [tok], [pos])
    assert np.all(cache == 0)


def test_argmax_lowest_index_on_ties():
    assert oracle.argmax([1.0, 3.0, 3.0, 2.0]) == 1
    assert oracle.argmax([-1.0]) == 0
