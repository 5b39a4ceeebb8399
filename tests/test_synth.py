"""The seeded input generator: determinism, independence and distribution."""
import numpy as np
import pytest

import synth


def _bf16_to_f32(bits):
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32)


def test_deterministic_and_counter_based():
    a = synth.normal_bf16(1234, 7, 10000, std=0.02)
    b = synth.normal_bf16(1234, 7, 10000, std=0.02, threads=3)
    assert np.array_equal(a, b)
    # element i does not depend on how many elements were asked for
    c = synth.normal_bf16(1234, 7, 100, std=0.02, offset=9900)
    assert np.array_equal(a[9900:], c)


def test_streams_and_seeds_differ():
    a = synth.normal_bf16(1, 1, 1000)
    assert not np.array_equal(a, synth.normal_bf16(1, 2, 1000))
    assert not np.array_equal(a, synth.normal_bf16(2, 1, 1000))


def test_normal_moments():
    x = _bf16_to_f32(synth.normal_bf16(5, 3, 400000, std=0.02)).astype(np.float64)
    assert abs(x.mean()) < 3 * 0.02 / np.sqrt(x.size) * 2
    assert abs(x.std() - 0.02) < 0.0003
    # tails: about 0.27% beyond 3 sigma
    frac = np.mean(np.abs(x) > 0.06)
    assert 0.0015 < frac < 0.004


def test_mean_shift_for_gains():
    x = _bf16_to_f32(synth.normal_bf16(5, 4, 100000, std=0.1, mean=1.0)).astype(np.float64)
    assert abs(x.mean() - 1.0) < 0.002 and abs(x.std() - 0.1) < 0.002


def test_uniform_ids_range_and_spread():
    ids = synth.uniform_ids(4321, 0, 200000, 1024)
    assert ids.min() >= 0 and ids.max() < 1024
    counts = np.bincount(ids, minlength=1024)
    assert counts.min() > 100 and counts.max() < 300


def test_make_weights_shapes_and_gains():
    w = synth.make_weights(synth.TINY)
    m = synth.TINY
    assert w["embed"].shape == (m.vocab, m.hidden)
    assert w["lm_head"] is None  # tied
    assert len(w["layers"]) == m.n_layers
    for kind, shape in synth.layer_shapes(m).items():
        assert w["layers"][0][kind].shape == shape
    assert np.all(w["final_norm"] == 0x3F80)
    assert not np.array_equal(w["layers"][0]["wq"], w["layers"][1]["wq"])


def test_weight_byte_count_llama_1b():
    # 1,235,814,400 parameters in the Llama-3.2-1B shape (tied embeddings)
    assert synth.LLAMA_1B.weight_bytes() == 2 * 1235814400


def test_kv_cache_fill():
    m = synth.TINY
    c = synth.make_kv_cache(m, 2, 40, 8)
    assert c.shape == (2, 2, 2, 2, 40, 64)
    assert np.all(c[:, :, :, :, 8:, :] == 0)
    assert np.all(c[:, :, :, :, :8, :] != 0)
    x = _bf16_to_f32(c[:, :, :, :, :8, :]).astype(np.float64)
    assert abs(x.std() - 1.0) < 0.05
