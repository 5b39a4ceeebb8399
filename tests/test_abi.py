"""Host-only checks of the C ABI (no GPU): the library loads and exports every
function include/mk.h declares, the schedule builder covers every output
exactly once for the model shapes and CU counts in use, and argument errors
come back as status codes."""
import ctypes
import os
import re

import pytest

import synth
from decode_megakernel_02_amd import mk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    text = open(os.path.join(ROOT, "include", "mk.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mk_\w+)\s*\(", text)))


def test_header_declarations_match_binding():
    names = header_functions()
    assert names == sorted(mk.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(mk.LIB_PATH)
    for n in header_functions():
        assert hasattr(lib, n), n


def test_status_strings():
    for code in [0, -1, -2, -3, -4, -5, -6]:
        s = mk.mk_status_string(code)
        assert s and s != mk.mk_status_string(12345)


@pytest.mark.parametrize("shape_name,batch,max_seq,ncus", [
    ("TINY", 1, 64, 1), ("TINY", 2, 64, 7), ("TINY", 8, 1024, 256), ("TINY", 3, 40, 64),
    ("LLAMA_1B", 1, 1040, 256), ("LLAMA_1B", 4, 1040, 256), ("LLAMA_1B", 8, 1040, 256),
    ("LLAMA_1B", 1, 32784, 256), ("LLAMA_1B", 1, 1040, 200), ("LLAMA_8B", 1, 1040, 256),
    ("LLAMA_1B_TP8_SHARD", 1, 1040, 256), ("LLAMA_1B_TP8_SHARD", 4, 1040, 256),
])
def test_schedule_is_valid(shape_name, batch, max_seq, ncus):
    shape = getattr(synth, shape_name)
    cfg = mk.make_config(shape, batch, max_seq)
    info = mk.mk_schedule_inspect(cfg, ncus)
    assert info.valid == 1, mk.mk_last_error()
    assert info.n_cus == ncus
    assert info.launches_multikernel == 6 * shape.n_layers + 1
    # every weight byte is streamed once per step; each row segment is padded
    # to whole 512-element units (the down projection's rows are cut into
    # n_chunks segments, on multiples of 8 elements)
    H, F, V, D = shape.hidden, shape.ffn, shape.vocab, shape.head_dim
    pad = lambda k: -(-k // 512) * 512
    rows_h = (shape.n_q_heads + 2 * shape.n_kv_heads) * D + 2 * F  # matrices with H inputs, per layer
    dense = 2 * (shape.n_layers * (rows_h * H + H * shape.n_q_heads * D + H * F) + V * H)
    seg = pad(-(-F // info.n_chunks // 8) * 8) * info.n_chunks
    padded = 2 * (shape.n_layers * (rows_h * pad(H) + H * pad(shape.n_q_heads * D) + H * seg) + V * pad(H))
    assert dense <= info.packed_weight_bytes <= padded
    if H % 512 == 0 and (shape.n_q_heads * D) % 512 == 0 and F % (512 * info.n_chunks) == 0:
        assert info.packed_weight_bytes == dense
    assert info.min_stream_bytes_per_wave >= 0
    assert info.max_stream_bytes_per_wave * 8 * ncus >= info.packed_weight_bytes


@pytest.mark.parametrize("shape_name,batch,chunks", [
    ("LLAMA_1B", 1, 4), ("LLAMA_1B", 2, 2), ("LLAMA_1B", 4, 2), ("LLAMA_1B", 5, 4), ("LLAMA_1B", 8, 4),
    ("LLAMA_8B", 1, 4), ("LLAMA_8B", 4, 4), ("TINY", 3, 2), ("LLAMA_1B_TP8_SHARD", 1, 4),
])
def test_default_down_chunks(shape_name, batch, chunks):
    """n_chunks = 0 picks 2 down-projection chunks for 2 to 4 batch rows with ffn <= 8192, else 4;
    an explicit count is kept."""
    shape = getattr(synth, shape_name)
    assert mk.mk_schedule_inspect(mk.make_config(shape, batch, 1040), 256).n_chunks == chunks
    assert mk.mk_schedule_inspect(mk.make_config(shape, batch, 1040, n_chunks=3), 256).n_chunks == 3


@pytest.mark.parametrize("shape_name,bound", [("LLAMA_1B", 1.1), ("LLAMA_8B", 1.12)])
def test_schedule_balances_weight_streams(shape_name, bound):
    """The eight compute waves of a CU get nearly equal weight streams at the
    full-size shapes."""
    info = mk.mk_schedule_inspect(mk.make_config(getattr(synth, shape_name), 1, 1040), 256)
    mean = info.packed_weight_bytes / (256 * 8)
    assert info.max_stream_bytes_per_wave <= bound * mean


@pytest.mark.parametrize("field,value", [
    ("head_dim", 96), ("batch", 9), ("batch", 0), ("n_kv_heads", 3), ("hidden", 100), ("max_seq", 0),
    ("n_chunks", 17),
])
def test_unsupported_configs_are_rejected(field, value):
    cfg = mk.make_config(synth.TINY, 1, 64)
    setattr(cfg, field, value)
    info = mk.MkScheduleInfo()
    rc = mk.lib().mk_schedule_inspect(ctypes.byref(cfg), 8, ctypes.byref(info))
    assert rc in (mk.MK_ERR_UNSUPPORTED_SHAPE, mk.MK_ERR_INVALID_ARG), (field, value, rc)
    assert mk.mk_last_error()


def test_null_arguments():
    L = mk.lib()
    assert L.mk_create(None, None) == mk.MK_ERR_INVALID_ARG
    h = ctypes.c_void_p(1)
    assert L.mk_create(None, ctypes.byref(h)) == mk.MK_ERR_INVALID_ARG
    assert h.value is None
    assert L.mk_schedule_inspect(None, 8, None) == mk.MK_ERR_INVALID_ARG
    assert L.mk_destroy(None) == mk.MK_OK
    assert L.mk_decode_step(None, None, None, None, None, None) == mk.MK_ERR_INVALID_ARG
    assert L.mk_prefill(None, None, None, 0, None, None, None) == mk.MK_ERR_INVALID_ARG
    assert L.mk_decode_step_multikernel(None, None, None, None, None, None) == mk.MK_ERR_INVALID_ARG
    assert L.mk_load_weights(None, None, None) == mk.MK_ERR_INVALID_ARG
    assert L.mk_greedy_advance(None, None, None, None, None) == mk.MK_ERR_INVALID_ARG
    # the read probe checks its arguments before any device call
    sink = ctypes.c_void_p(64)
    assert L.mk_read_probe(None, 16, sink, 1, None) == mk.MK_ERR_INVALID_ARG
    assert L.mk_read_probe(ctypes.c_void_p(256), 24, sink, 1, None) == mk.MK_ERR_INVALID_ARG
    assert L.mk_read_probe(ctypes.c_void_p(264), 16, sink, 1, None) == mk.MK_ERR_INVALID_ARG
    assert L.mk_read_probe(ctypes.c_void_p(256), 16, sink, 0, None) == mk.MK_ERR_INVALID_ARG
    assert L.mk_read_probe(ctypes.c_void_p(256), 16, sink, 4097, None) == mk.MK_ERR_INVALID_ARG
    # launch probe and graph entry points check their arguments before any device call
    assert L.mk_empty_launches(0, 1, 64, None) == mk.MK_ERR_INVALID_ARG
    assert L.mk_empty_launches(1, 0, 64, None) == mk.MK_ERR_INVALID_ARG
    assert L.mk_empty_launches(1, 1, 1025, None) == mk.MK_ERR_INVALID_ARG
    g = ctypes.c_void_p(1)
    assert L.mk_graph_create(None, None, None, None, None, 1, 0, ctypes.byref(g)) == mk.MK_ERR_INVALID_ARG
    assert g.value is None
    assert L.mk_graph_create(None, None, None, None, None, 1, 0, None) == mk.MK_ERR_INVALID_ARG
    assert L.mk_graph_launch(None, None) == mk.MK_ERR_INVALID_ARG
    assert L.mk_graph_destroy(None) == mk.MK_OK


def test_kv_cache_bytes():
    for shape, B, S in [(synth.TINY, 2, 64), (synth.LLAMA_1B, 1, 1040), (synth.LLAMA_8B, 4, 2048)]:
        cfg = mk.make_config(shape, B, S)
        n = 1
        for d in synth.kv_cache_shape(shape, B, S):
            n *= d
        assert mk.mk_kv_cache_bytes(cfg) == 2 * n
    bad = mk.make_config(synth.TINY, 0, 64)
    assert mk.mk_kv_cache_bytes(bad) == 0


@pytest.mark.parametrize("shape_name,batch,ncus", [("TINY", 1, 256), ("TINY", 3, 7), ("LLAMA_1B", 1, 256),
                                                  ("LLAMA_1B", 4, 64)])
def test_validator_rejects_planted_schedule_defects(shape_name, batch, ncus):
    """A duplicate, a hole and a queue that waits on its own later work are each rejected, the last
    one both by the stage-order check and, with that check off, by the dependency simulation."""
    shape = getattr(synth, shape_name)
    cfg = mk.make_config(shape, batch, 256)
    assert mk.mk_schedule_selftest(cfg, ncus, 0) == mk.MK_OK
    expect = {1: "produced 2 times", 2: "produced 0 times", 3: "not in stage order", 4: "deadlock"}
    for mutation, text in expect.items():
        rc = mk.mk_schedule_selftest(cfg, ncus, mutation)
        assert rc == mk.MK_ERR_UNSUPPORTED_SHAPE, (mutation, rc)
        assert text in mk.mk_last_error(), (mutation, mk.mk_last_error())


def test_validator_selftest_argument_errors():
    cfg = mk.make_config(synth.TINY, 1, 64)
    assert mk.mk_schedule_selftest(cfg, 0, 0) == mk.MK_ERR_INVALID_ARG
    assert mk.mk_schedule_selftest(cfg, 4, 9) == mk.MK_ERR_INVALID_ARG
    assert mk.lib().mk_schedule_selftest(None, 4, 0) == mk.MK_ERR_INVALID_ARG
