"""Pins of the oracle's component functions to closed forms, invariants and
library routines (numpy / scipy / torch), never to the oracle itself.

Each test names the mistake it is there to catch.
"""
import math

import numpy as np
import pytest
import scipy.special
import torch

import oracle


def bf16_bits_from_f32(x):
    """bf16 RNE bits of float32 values via torch's own conversion."""
    t = torch.tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().astype(np.uint16)


def bits_to_f64(bits):
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


# ---------------------------------------------------------------- bf16 ------

def test_bf16_widen_known_patterns():
    assert oracle.bf16_to_double(0x3F80) == 1.0
    assert oracle.bf16_to_double(0xC000) == -2.0
    assert oracle.bf16_to_double(0x3F81) == 1.0 + 2.0 ** -7
    assert oracle.bf16_to_double(0x0001) == 2.0 ** -133
    assert math.isinf(oracle.bf16_to_double(0x7F80))


def test_bf16_round_matches_torch_on_float32_values():
    # a float32 value is exact in double, so direct rounding must equal torch's RNE
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.normal(0, 1, 20000), rng.normal(0, 1e-3, 2000),
                        rng.normal(0, 300, 2000)]).astype(np.float32)
    ours = np.array([oracle.bf16_round(float(v)) for v in x], dtype=np.uint16)
    assert np.array_equal(ours, bf16_bits_from_f32(x))


def test_bf16_round_ties_to_even_and_no_double_rounding():
    assert oracle.bf16_round(1.0 + 2.0 ** -8) == 0x3F80       # tie -> even (down)
    assert oracle.bf16_round(1.0 + 3 * 2.0 ** -8) == 0x3F82   # tie -> even (up)
    # just above the tie by less than a float32 ulp: rounding via float32 would see an
    # exact tie and go down; the exact value must round up
    assert oracle.bf16_round(1.0 + 2.0 ** -8 + 2.0 ** -40) == 0x3F81
    assert oracle.bf16_round(-1.5) == 0xBFC0
    assert oracle.bf16_round(0.0) == 0 and oracle.bf16_round(-0.0) == 0x8000
    assert oracle.bf16_round(1e39) == 0x7F80


# ------------------------------------------------------------- RMSNorm ------

def test_rmsnorm_constant_vector_closed_form():
    # h = c * 1 -> c / sqrt(c^2 + eps) * g_i ; catches sum-vs-mean, missing eps, gain index
    n, c, eps = 64, 0.37, 1e-5
    gains = bf16_bits_from_f32(np.linspace(0.5, 1.5, n))
    out = oracle.rmsnorm(np.full(n, c), gains, eps)
    expect = c / math.sqrt(c * c + eps) * bits_to_f64(gains)
    np.testing.assert_allclose(out, expect, rtol=1e-14)


def test_rmsnorm_known_mean_square():
    n = 8
    h = np.zeros(n)
    h[0], h[3] = 3.0, 4.0  # mean square 25/8
    out = oracle.rmsnorm(h, np.full(n, 0x3F80, dtype=np.uint16), 0.0)
    np.testing.assert_allclose(out, h / math.sqrt(25 / 8), rtol=1e-15)


def test_rmsnorm_zero_vector_and_scale_invariance():
    g = np.full(16, 0x3F80, dtype=np.uint16)
    assert np.all(oracle.rmsnorm(np.zeros(16), g, 1e-5) == 0)
    rng = np.random.default_rng(1)
    h = rng.normal(size=16)
    np.testing.assert_allclose(oracle.rmsnorm(1e3 * h, g, 1e-5), oracle.rmsnorm(h, g, 0.0),
                               rtol=1e-9)


# ---------------------------------------------------------------- GEMV ------

@pytest.mark.parametrize("rows,cols,threads", [(1, 1, 1), (7, 33, 1), (300, 129, 4)])
def test_gemv_matches_numpy(rows, cols, threads):
    rng = np.random.default_rng(rows * 1000 + cols)
    W = bf16_bits_from_f32(rng.normal(0, 0.02, (rows, cols)))
    x = rng.normal(size=cols)
    ref = bits_to_f64(W).reshape(rows, cols) @ x
    np.testing.assert_allclose(oracle.gemv(W, x, threads), ref, rtol=1e-12, atol=1e-15)


def test_gemv_uses_rows_not_columns():
    # transposed-operand mistake: non-square, row r picks column c only via W[r][c]
    W = np.zeros((2, 3), dtype=np.uint16)
    W[0, 2] = 0x3F80  # 1.0
    W[1, 0] = 0x4000  # 2.0
    np.testing.assert_array_equal(oracle.gemv(W, [10.0, 20.0, 30.0]), [30.0, 20.0])


# ---------------------------------------------------------------- RoPE ------

def test_rope_position_zero_is_identity():
    rng = np.random.default_rng(2)
    v = rng.normal(size=64)
    np.testing.assert_array_equal(oracle.rope(v, 0, 10000.0), v)


def test_rope_unit_vectors_closed_form():
    # e_i -> cos(a_i) e_i + sin(a_i) e_{i+D/2};  e_{i+D/2} -> -sin(a_i) e_i + cos(a_i) e_{i+D/2}
    # with a_i = p * theta^(-2i/D): pins pairing (i, i+D/2), frequency and sign
    D, theta, p = 8, 10000.0, 5
    for i in range(D // 2):
        a = p * theta ** (-2.0 * i / D)
        e = np.zeros(D)
        e[i] = 1.0
        exp1 = np.zeros(D)
        exp1[i], exp1[i + D // 2] = math.cos(a), math.sin(a)
        np.testing.assert_allclose(oracle.rope(e, p, theta), exp1, atol=1e-15)
        e = np.zeros(D)
        e[i + D // 2] = 1.0
        exp2 = np.zeros(D)
        exp2[i], exp2[i + D // 2] = -math.sin(a), math.cos(a)
        np.testing.assert_allclose(oracle.rope(e, p, theta), exp2, atol=1e-15)


def test_rope_preserves_pair_norms_and_relative_dot():
    rng = np.random.default_rng(3)
    D = 64
    q, k = rng.normal(size=D), rng.normal(size=D)
    r = oracle.rope(q, 1234, 500000.0)
    half = D // 2
    np.testing.assert_allclose(r[:half] ** 2 + r[half:] ** 2, q[:half] ** 2 + q[half:] ** 2,
                               rtol=1e-12)
    # <R(m) q, R(n) k> depends only on m - n
    d1 = oracle.rope(q, 40, 10000.0) @ oracle.rope(k, 17, 10000.0)
    d2 = oracle.rope(q, 1040, 10000.0) @ oracle.rope(k, 1017, 10000.0)
    assert abs(d1 - d2) < 1e-9


def test_rope_composition():
    # R(a) R(b) = R(a + b): rotating at p1 then p2 equals rotating at p1 + p2
    rng = np.random.default_rng(4)
    v = rng.normal(size=16)
    two = oracle.rope(oracle.rope(v, 7, 10000.0), 11, 10000.0)
    np.testing.assert_allclose(two, oracle.rope(v, 18, 10000.0), atol=1e-12)


# ----------------------------------------------------------- attention ------

def test_attention_single_key_returns_value():
    rng = np.random.default_rng(5)
    D = 64
    K = bf16_bits_from_f32(rng.normal(size=(1, D)))
    V = bf16_bits_from_f32(rng.normal(size=(1, D)))
    out = oracle.attention(rng.normal(size=D) * 10, K, V)
    np.testing.assert_array_equal(out, bits_to_f64(V[0]))


def test_attention_equal_keys_average_values():
    rng = np.random.default_rng(6)
    D, n = 64, 5
    K = np.tile(bf16_bits_from_f32(rng.normal(size=(1, D))), (n, 1))
    V = bf16_bits_from_f32(rng.normal(size=(n, D)))
    out = oracle.attention(rng.normal(size=D), K, V)
    np.testing.assert_allclose(out, bits_to_f64(V).reshape(n, D).mean(axis=0), rtol=1e-12)


def test_attention_two_keys_scale_closed_form():
    # scores a, b -> weight of key 0 = 1 / (1 + exp((b - a)/sqrt(D))): pins the 1/sqrt(D) scale
    D = 16
    q = np.zeros(D)
    q[0] = 1.0
    K = np.zeros((2, D), dtype=np.uint16)
    K[0, 0] = 0x4040  # 3.0
    K[1, 0] = 0xBF80  # -1.0
    V = np.zeros((2, D), dtype=np.uint16)
    V[0, 1] = 0x3F80  # value row 0 -> e_1
    V[1, 2] = 0x3F80  # value row 1 -> e_2
    out = oracle.attention(q, K, V)
    w0 = 1.0 / (1.0 + math.exp((-1.0 - 3.0) / math.sqrt(D)))
    np.testing.assert_allclose(out[1], w0, rtol=1e-14)
    np.testing.assert_allclose(out[2], 1.0 - w0, rtol=1e-13)


def test_attention_matches_scipy_softmax():
    rng = np.random.default_rng(7)
    D, n = 64, 37
    q = rng.normal(size=D) * 2
    K = bf16_bits_from_f32(rng.normal(size=(n, D)))
    V = bf16_bits_from_f32(rng.normal(size=(n, D)))
    Kf, Vf = bits_to_f64(K).reshape(n, D), bits_to_f64(V).reshape(n, D)
    ref = scipy.special.softmax(Kf @ q / math.sqrt(D)) @ Vf
    np.testing.assert_allclose(oracle.attention(q, K, V), ref, rtol=1e-12, atol=1e-14)


def test_attention_large_scores_stay_finite():
    # max subtraction: exp of raw scores this large would overflow
    D = 4
    q = np.array([1000.0, 0, 0, 0])
    K = bf16_bits_from_f32(np.array([[10.0, 0, 0, 0], [9.0, 0, 0, 0]]))
    V = bf16_bits_from_f32(np.array([[1.0, 0, 0, 0], [0, 1.0, 0, 0]]))
    out = oracle.attention(q, K, V)
    assert np.all(np.isfinite(out))
    np.testing.assert_allclose(out[:2], scipy.special.softmax([5000.0, 4500.0]), atol=1e-15)


# ---------------------------------------------------------------- SiLU ------

def test_silu_closed_forms():
    assert oracle.silu(0.0) == 0.0
    assert abs(oracle.silu(1.0) - 0.7310585786300049) < 1e-15
    assert abs(oracle.silu(-1.0) + 0.2689414213699951) < 1e-15
    assert abs(oracle.silu(40.0) - 40.0) < 1e-12
    assert abs(oracle.silu(-40.0)) < 1e-15
    assert abs(oracle.silu(2.0) - 2.0 * scipy.special.expit(2.0)) < 1e-15
