"""Pins of the oracle's FP8 weight path (OCP E4M3 codes, one fp32 scale per
matrix): code values from the format's definition, rounding against a brute
force search over every finite code, the scale rule, a lossless quantisation
that must reproduce the bf16 products exactly, and the error bound of a lossy
one.  The GPU library's FP8 mode is compared against this path elsewhere."""
import math

import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.filterwarnings("ignore")

# (code, value) written out from the format: sign, 4-bit exponent (bias 7), 3-bit mantissa,
# exponent 0 = subnormals m * 2^-9
KNOWN = [(0x00, 0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6), (0x30, 0.5),
         (0x38, 1.0), (0x39, 1.125), (0x3F, 1.875), (0x40, 2.0), (0x77, 240.0), (0x7E, 448.0),
         (0x80, -0.0), (0xB8, -1.0), (0xFE, -448.0)]


def finite_table():
    codes = [c for c in range(256) if (c & 0x7F) != 0x7F]
    return np.array(codes), np.array([oracle.e4m3_to_double(c) for c in codes])


def test_e4m3_known_codes_and_nan():
    for code, value in KNOWN:
        got = oracle.e4m3_to_double(code)
        assert got == value and math.copysign(1, got) == math.copysign(1, value), hex(code)
    assert math.isnan(oracle.e4m3_to_double(0x7F)) and math.isnan(oracle.e4m3_to_double(0xFF))


def test_e4m3_positive_codes_increase():
    v = [oracle.e4m3_to_double(c) for c in range(0x7F)]
    assert all(b > a for a, b in zip(v, v[1:]))


def brute_round(x, codes, values):
    if abs(x) >= 448:
        return 0xFE if x < 0 else 0x7E
    d = np.abs(values - x)
    best = np.flatnonzero(d == d.min())
    if len(best) > 1:  # a tie between two neighbours: the even mantissa
        best = [b for b in best if codes[b] % 2 == 0] or list(best)
    c = int(codes[best[0]])
    if values[best[0]] == 0:  # +0 / -0 by the sign of x
        c = 0x80 if math.copysign(1, x) < 0 else 0x00
    return c


def test_e4m3_round_matches_brute_force():
    codes, values = finite_table()
    rng = np.random.default_rng(5)
    xs = list(rng.standard_normal(3000) * 30) + list(rng.standard_normal(1000) * 2.0 ** -7)
    pos = np.sort(np.unique(values[values > 0]))
    xs += list((pos[1:] + pos[:-1]) / 2)  # exact midpoints: ties
    xs += [-(a + b) / 2 for a, b in zip(pos[1:], pos[:-1])]
    xs += list(pos) + [0.0, -0.0, 447.9, 448.0, 460.0, 470.0, 1e9, -1e9, 2.0 ** -10, 2.0 ** -11]
    for x in xs:
        assert oracle.e4m3_round(float(x)) == brute_round(float(x), codes, values), x


def test_fp8_scale_rule():
    w = np.array([0x3F00, 0xBF80, 0x0000], dtype=np.uint16)  # 0.5, -1.0, 0
    assert oracle.fp8_scale(w) == np.float32(1.0) / np.float32(448.0)
    assert oracle.fp8_scale(np.zeros(7, dtype=np.uint16)) == 1.0


def lossless_matrix(rng, rows, cols, k):
    """bf16 weights s * v(code) with s = 2^-k and one entry at +-448 s, so that the
    quantiser's scale is exactly s and every weight is its own quantisation."""
    codes, values = finite_table()
    v = values[rng.integers(len(values), size=(rows, cols))]
    v.flat[rng.integers(rows * cols)] = 448.0
    w = (v * 2.0 ** -k).astype(np.float32)
    bits = (w.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal((bits.astype(np.uint32) << 16).view(np.float32), w)  # exact in bf16
    return bits


def test_lossless_quantisation_reproduces_bf16_products():
    rng = np.random.default_rng(9)
    W = lossless_matrix(rng, 37, 300, 11)
    assert oracle.fp8_scale(W) == 2.0 ** -11
    x = rng.standard_normal(300)
    np.testing.assert_array_equal(oracle.gemv_fp8(W, x, 3), oracle.gemv(W, x, 1))


def test_lossy_quantisation_within_half_a_step():
    rng = np.random.default_rng(10)
    W = synth.make_weights(synth.TINY)["layers"][0]["wq"]
    x = np.abs(rng.standard_normal(W.shape[1]))
    s = oracle.fp8_scale(W)
    w = (W.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    # |w - s*q| <= half the spacing: 2^-4 |w| for normals, s * 2^-10 for subnormals
    bound = (np.abs(w) * 2.0 ** -4 + s * 2.0 ** -10) @ x
    d = np.abs(oracle.gemv_fp8(W, x) - oracle.gemv(W, x))
    assert np.all(d <= bound * (1 + 1e-12))
    assert d.max() > 0


def test_model_with_lossless_fp8_weights_equals_bf16_model():
    """Every projection matrix and the tied LM head go through the FP8 path: with
    weights that the quantiser reproduces exactly the logits are bit-identical."""
    shape = synth.TINY
    w = synth.make_weights(shape)
    rng = np.random.default_rng(12)
    w["embed"] = lossless_matrix(rng, *w["embed"].shape, 10)
    for L in w["layers"]:
        for kind in ["wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down"]:
            L[kind] = lossless_matrix(rng, *L[kind].shape, 11)
    max_seq = 8
    outs = []
    for fp8 in (False, True):
        orc = oracle.Oracle(shape, w, 1, max_seq, fp8=fp8)
        kv = np.zeros(orc.kv_cache_bytes() // 2, dtype=np.uint16)
        lg = [orc.decode_step(kv, [t], [p]) for p, t in enumerate([3, 17, 900])]
        outs.append((lg, kv))
    for a, b in zip(outs[0][0], outs[1][0]):
        np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(outs[0][1], outs[1][1])


def test_model_fp8_differs_from_bf16_on_ordinary_weights():
    shape = synth.TINY
    w = synth.make_weights(shape)
    lg = []
    for fp8 in (False, True):
        orc = oracle.Oracle(shape, w, 1, 4, fp8=fp8)
        kv = np.zeros(orc.kv_cache_bytes() // 2, dtype=np.uint16)
        lg.append(orc.decode_step(kv, [5], [0]))
    d = np.abs(lg[0] - lg[1]).max()
    assert 1e-6 < d < 0.5 * np.abs(lg[0]).max()


@pytest.mark.parametrize("lossy", ["wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down", "embed"])
def test_each_matrix_goes_through_the_quantiser(lossy):
    """All weights lossless except one kind (ordinary N(0, 0.02) values there):
    the FP8 logits must then differ from the bf16 ones, so that kind is quantised
    (embed: the tied LM head; the embedding lookup itself stays bf16)."""
    shape = synth.TINY
    w = synth.make_weights(shape)
    rng = np.random.default_rng(13)
    if lossy != "embed":
        w["embed"] = lossless_matrix(rng, *w["embed"].shape, 10)
    for L in w["layers"]:
        for kind in ["wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down"]:
            if kind != lossy:
                L[kind] = lossless_matrix(rng, *L[kind].shape, 11)
    lg = []
    for fp8 in (False, True):
        orc = oracle.Oracle(shape, w, 1, 4, fp8=fp8)
        kv = np.zeros(orc.kv_cache_bytes() // 2, dtype=np.uint16)
        orc.decode_step(kv, [7], [0])
        lg.append(orc.decode_step(kv, [11], [1]))
    assert np.abs(lg[0] - lg[1]).max() > 1e-7


def test_per_row_scale_is_lossless_on_scaled_e4m3_rows():
    """Rows a_r * e_k with e_k E4M3 values (largest 448) and a_r powers of two from 1 to 2^-12: with
    its own scale s_r = a_r every row quantises exactly, so the per-row GEMV equals the bf16 GEMV;
    one scale for the whole matrix pushes the small rows into subnormals and loses them."""
    codes, values = finite_table()
    rng = np.random.default_rng(11)
    fin = values[np.isfinite(values) & (np.abs(values) >= 2.0 ** -6)]  # normal E4M3 values
    rows, cols = 13, 96
    e = rng.choice(fin, size=(rows, cols))
    e[:, 0] = 448.0  # every row's largest magnitude is 448
    a = 2.0 ** -np.arange(rows)
    Wf = (a[:, None] * e).astype(np.float32)
    W = (Wf.view(np.uint32) >> 16).astype(np.uint16)  # exact in bf16: E4M3 values have 4 significant bits
    assert np.array_equal((W.astype(np.uint32) << 16).view(np.float32), Wf)
    x = rng.standard_normal(cols)
    exact = oracle.gemv(W, x)
    per_row = oracle.gemv_fp8_rows(W, x)
    assert np.allclose(per_row, exact, rtol=0, atol=1e-12 * np.max(np.abs(exact)))
    per_mat = oracle.gemv_fp8(W, x)
    assert np.max(np.abs(per_mat[-3:] - exact[-3:])) > 1e-3 * np.max(np.abs(exact[-3:]))


def test_per_row_scale_error_bound():
    """|y_r - exact_r| <= s_r * sum_k |x_k| * (half the E4M3 spacing at |w_rk| / s_r)."""
    w = synth.make_weights(synth.TINY)["layers"][0]["w_gate"][:40]
    x = np.random.default_rng(3).standard_normal(w.shape[1])
    exact = oracle.gemv(w, x)
    got = oracle.gemv_fp8_rows(w, x)
    wf = (w.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    for r in range(w.shape[0]):
        s = oracle.fp8_scale(w[r:r + 1])
        q = np.abs(np.float32(wf[r]) / np.float32(s)).astype(np.float64)
        e = np.where(q >= 2.0 ** -6, np.floor(np.log2(np.maximum(q, 2.0 ** -6))), -6)
        half = np.ldexp(1.0, (e - 3).astype(int)) / 2
        bound = s * np.sum(np.abs(x) * half) * (1 + 1e-6) + 1e-12
        assert abs(got[r] - exact[r]) <= bound, (r, got[r] - exact[r], bound)


@pytest.mark.parametrize("mb,wb", [(0x3D98, 0x3BE4), (0x3E5C, 0x365C), (0x3EA2, 0x38F3)])
def test_quotient_is_taken_in_fp32(mb, wb):
    """The quantiser divides in fp32 (w / s with s an fp32 value).  These bf16 pairs (found by a
    search over random pairs) are ones where the fp32 quotient lands on a rounding midpoint
    that the exact quotient misses, so the two give neighbouring E4M3 codes: a quantiser that
    divided in double would fail here."""
    codes, values = finite_table()
    W = np.array([[mb, wb]], dtype=np.uint16)
    m, w = (W.astype(np.uint32) << 16).view(np.float32)[0]
    s = np.float32(m) / np.float32(448.0)
    assert oracle.fp8_scale(W) == s
    q32 = float(np.float32(w) / s)
    q64 = float(w) / float(s)
    c32, c64 = brute_round(q32, codes, values), brute_round(q64, codes, values)
    assert c32 != c64
    x = np.array([0.0, 1.0])
    for y in (oracle.gemv_fp8(W, x), oracle.gemv_fp8_rows(W, x)):
        assert y[0] == float(s) * oracle.e4m3_to_double(int(c32))
