"""ctypes binding of the decode library's C ABI (include/mk.h).

Argument marshalling only: every step of the decode path runs in the HIP
kernels of libmk.so.  Functions keep the C names; torch tensors (device
memory) are passed as raw pointers.  If libmk.so has not been built, loading
fails with an error instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, List, Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmk.so")

MK_OK = 0
MK_ERR_INVALID_ARG = -1
MK_ERR_UNSUPPORTED_SHAPE = -2
MK_ERR_HIP = -3
MK_ERR_OOM = -4
MK_ERR_STATE = -5
MK_ERR_DEVICE = -6

_P = ctypes.c_void_p


class MkConfig(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("hidden", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("ffn", ctypes.c_int32),
                ("vocab", ctypes.c_int32), ("rms_eps", ctypes.c_float), ("rope_theta", ctypes.c_float),
                ("tied_embeddings", ctypes.c_int32), ("batch", ctypes.c_int32), ("max_seq", ctypes.c_int32),
                ("device", ctypes.c_int32), ("n_cus", ctypes.c_int32), ("n_splits", ctypes.c_int32),
                ("n_chunks", ctypes.c_int32), ("flags", ctypes.c_uint32)]


class MkWeights(ctypes.Structure):
    _fields_ = [("embed", _P), ("final_norm", _P), ("lm_head", _P)] + [
        (n, ctypes.POINTER(_P)) for n in
        ["attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w_gate", "w_up", "w_down"]]


class MkDeviceError(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint32) for n in ["code", "workgroup", "pc", "opcode", "wave", "detail"]]


class MkScheduleInfo(ctypes.Structure):
    _fields_ = [("n_cus", ctypes.c_int32), ("n_splits", ctypes.c_int32), ("n_chunks", ctypes.c_int32),
                ("max_insts_per_cu", ctypes.c_int32), ("total_insts", ctypes.c_int64),
                ("packed_weight_bytes", ctypes.c_int64), ("max_stream_bytes_per_wave", ctypes.c_int64),
                ("min_stream_bytes_per_wave", ctypes.c_int64), ("launches_multikernel", ctypes.c_int32),
                ("valid", ctypes.c_int32)]


EXPORTS = ["mk_create", "mk_load_weights", "mk_kv_cache_bytes", "mk_decode_step", "mk_decode_step_multikernel",
           "mk_decode_step_greedy", "mk_set_ablation",
           "mk_destroy", "mk_status_string", "mk_last_error", "mk_get_device_error", "mk_get_profile",
           "mk_schedule_inspect", "mk_get_trace", "mk_greedy_advance", "mk_read_probe", "mk_empty_launches",
           "mk_graph_create", "mk_graph_launch", "mk_graph_destroy", "mk_prefill", "mk_schedule_selftest", "mk_litmus", "mk_set_spin_limit",
           "mk_debug_stage", "mk_prefill_static"]
MK_FLAG_PROFILE = 1
MK_FLAG_TRACE = 2
MK_FLAG_FP8_WEIGHTS = 4
MK_FLAG_DEBUG_NAN = 8
MK_GRAPH_MULTIKERNEL = 1
MK_GRAPH_EMPTY = 2
MK_GRAPH_FUSED_GREEDY = 4
MK_STEP_THREADS = 640  # threads per workgroup of the step kernels (include/mk.h)
TRACE_SLOTS = 52
PROF_WAVES = 10  # 8 compute waves, the loader and the gather wave per workgroup
PROF_SLOTS = 8

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with decode_megakernel_02_amd/build.py "
                               "(there is no fallback implementation)")
        L = ctypes.CDLL(LIB_PATH)
        H = ctypes.c_void_p  # mk_handle*
        L.mk_create.argtypes = [ctypes.POINTER(MkConfig), ctypes.POINTER(H)]
        L.mk_load_weights.argtypes = [H, ctypes.POINTER(MkWeights), _P]
        L.mk_kv_cache_bytes.argtypes = [ctypes.POINTER(MkConfig)]
        L.mk_kv_cache_bytes.restype = ctypes.c_size_t
        L.mk_decode_step.argtypes = [H, _P, _P, _P, _P, _P]
        L.mk_decode_step_multikernel.argtypes = [H, _P, _P, _P, _P, _P]
        L.mk_decode_step_greedy.argtypes = [H, _P, _P, _P, _P, _P]
        L.mk_set_ablation.argtypes = [H, ctypes.c_int32]
        L.mk_read_probe.argtypes = [_P, ctypes.c_size_t, _P, ctypes.c_int, _P]
        L.mk_destroy.argtypes = [H]
        L.mk_status_string.argtypes = [ctypes.c_int]
        L.mk_status_string.restype = ctypes.c_char_p
        L.mk_last_error.argtypes = [H]
        L.mk_last_error.restype = ctypes.c_char_p
        L.mk_get_device_error.argtypes = [H, ctypes.POINTER(MkDeviceError)]
        L.mk_schedule_inspect.argtypes = [ctypes.POINTER(MkConfig), ctypes.c_int32, ctypes.POINTER(MkScheduleInfo)]
        L.mk_set_spin_limit.argtypes = [H, ctypes.c_uint32]
        L.mk_debug_stage.argtypes = [H, ctypes.c_int32, _P, _P, _P, _P, _P]
        L.mk_litmus.argtypes = [ctypes.c_int, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_uint32, _P]
        L.mk_schedule_selftest.argtypes = [ctypes.POINTER(MkConfig), ctypes.c_int32, ctypes.c_int32]
        L.mk_get_profile.argtypes = [H, _P, ctypes.c_size_t]
        L.mk_get_trace.argtypes = [H, _P, ctypes.c_size_t]
        L.mk_greedy_advance.argtypes = [H, _P, _P, _P, _P]
        L.mk_empty_launches.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, _P]
        L.mk_graph_create.argtypes = [H, _P, _P, _P, _P, ctypes.c_int, ctypes.c_uint32, ctypes.POINTER(ctypes.c_void_p)]
        L.mk_graph_launch.argtypes = [ctypes.c_void_p, _P]
        L.mk_graph_destroy.argtypes = [ctypes.c_void_p]
        L.mk_prefill.argtypes = [H, ctypes.POINTER(MkWeights), _P, ctypes.c_int32, _P, _P, _P]
        L.mk_prefill_static.argtypes = [H, ctypes.POINTER(MkWeights), _P, ctypes.c_int32, _P, _P, _P]
        for name in ["mk_create", "mk_load_weights", "mk_decode_step", "mk_decode_step_multikernel",
                     "mk_decode_step_greedy", "mk_set_ablation", "mk_destroy",
                     "mk_get_device_error", "mk_schedule_inspect", "mk_get_profile", "mk_get_trace",
                     "mk_greedy_advance", "mk_read_probe", "mk_empty_launches", "mk_graph_create",
                     "mk_graph_launch", "mk_graph_destroy", "mk_prefill", "mk_schedule_selftest", "mk_litmus", "mk_set_spin_limit", "mk_debug_stage", "mk_prefill_static"]:
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


class MkError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{mk_status_string(code)} ({code}): {msg}")
        self.code = code


def mk_status_string(code: int) -> str:
    return lib().mk_status_string(code).decode()


def mk_last_error(handle=None) -> str:
    return lib().mk_last_error(handle).decode()


def _check(code: int, handle=None):
    if code != MK_OK:
        raise MkError(code, mk_last_error(handle))


def make_config(shape, batch: int, max_seq: int, device: int = 0, n_cus: int = 0, n_splits: int = 0,
                n_chunks: int = 0, flags: int = 0) -> MkConfig:
    """MkConfig from a model shape object (attributes as in synth.ModelShape)."""
    return MkConfig(shape.n_layers, shape.hidden, shape.n_q_heads, shape.n_kv_heads, shape.head_dim, shape.ffn,
                    shape.vocab, shape.rms_eps, shape.rope_theta, 1 if shape.tied else 0, batch, max_seq, device,
                    n_cus, n_splits, n_chunks, flags)


def mk_create(cfg: MkConfig):
    h = ctypes.c_void_p()
    _check(lib().mk_create(ctypes.byref(cfg), ctypes.byref(h)))
    return h


def mk_kv_cache_bytes(cfg: MkConfig) -> int:
    return int(lib().mk_kv_cache_bytes(ctypes.byref(cfg)))


def mk_schedule_inspect(cfg: MkConfig, n_cus: int) -> MkScheduleInfo:
    info = MkScheduleInfo()
    _check(lib().mk_schedule_inspect(ctypes.byref(cfg), n_cus, ctypes.byref(info)))
    return info


def mk_schedule_selftest(cfg: MkConfig, n_cus: int, mutation: int) -> int:
    """Runs the schedule validator on a schedule with a planted defect (see include/mk.h);
    returns the status code (MK_OK: accepted) without raising."""
    return int(lib().mk_schedule_selftest(ctypes.byref(cfg), n_cus, mutation))


def mk_litmus(n_pairs: int, rounds: int, words: int, spin_limit: int = 1 << 22, device: int = 0):
    """Runs the tagged-word litmus (see include/mk.h); returns (mismatches, timeouts, round_trips,
    per-pair ticks [n_pairs], ping XCC ids [n_pairs], pong XCC ids [n_pairs])."""
    import numpy as np
    res = np.zeros(3 + 3 * n_pairs, dtype=np.uint32)
    _check(lib().mk_litmus(device, n_pairs, rounds, words, spin_limit, res.ctypes.data))
    per = res[3:].reshape(n_pairs, 3)
    return int(res[0]), int(res[1]), int(res[2]), per[:, 0].copy(), per[:, 1].copy(), per[:, 2].copy()


def _ptr(t) -> int:
    return t.data_ptr() if hasattr(t, "data_ptr") else int(t)


def mk_load_weights(handle, weights: Dict[str, object], stream: Optional[int] = None):
    """`weights`: {'embed', 'final_norm', 'lm_head' (or None), 'layers': [dict]} of device tensors (bf16)."""
    layers: List[Dict[str, object]] = weights["layers"]
    L = len(layers)
    arrays = {}
    w = MkWeights()
    w.embed = _ptr(weights["embed"])
    w.final_norm = _ptr(weights["final_norm"])
    w.lm_head = _ptr(weights["lm_head"]) if weights.get("lm_head") is not None else None
    for kind in ["attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w_gate", "w_up", "w_down"]:
        arr = (_P * L)(*[_ptr(layers[l][kind]) for l in range(L)])
        arrays[kind] = arr
        setattr(w, kind, ctypes.cast(arr, ctypes.POINTER(_P)))
    _check(lib().mk_load_weights(handle, ctypes.byref(w), stream), handle)


def _weights_struct(weights: Dict[str, object]):
    layers: List[Dict[str, object]] = weights["layers"]
    L = len(layers)
    keep = []
    w = MkWeights()
    w.embed = _ptr(weights["embed"])
    w.final_norm = _ptr(weights["final_norm"])
    w.lm_head = _ptr(weights["lm_head"]) if weights.get("lm_head") is not None else None
    for kind in ["attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w_gate", "w_up", "w_down"]:
        arr = (_P * L)(*[_ptr(layers[l][kind]) for l in range(L)])
        keep.append(arr)
        setattr(w, kind, ctypes.cast(arr, ctypes.POINTER(_P)))
    return w, keep


def mk_prefill(handle, weights: Dict[str, object], tokens, n_tokens: int, kv_cache, logits,
               stream: Optional[int] = None):
    """Batched prefill of positions 0 .. n_tokens-1 (tokens: device int32 [B][n_tokens]); synchronous."""
    w, keep = _weights_struct(weights)
    _check(lib().mk_prefill(handle, ctypes.byref(w), _ptr(tokens), int(n_tokens), _ptr(kv_cache), _ptr(logits),
                            stream), handle)
    del keep


def mk_prefill_static(handle, weights: Dict[str, object], tokens, n_tokens: int, kv_cache, logits,
                      stream: Optional[int] = None):
    """mk_prefill in the static scratch: no allocation, asynchronous (see include/mk.h)."""
    w, keep = _weights_struct(weights)
    _check(lib().mk_prefill_static(handle, ctypes.byref(w), _ptr(tokens), int(n_tokens), _ptr(kv_cache),
                                   _ptr(logits), stream), handle)
    del keep


def mk_decode_step(handle, tokens, positions, kv_cache, logits, stream: Optional[int] = None):
    _check(lib().mk_decode_step(handle, _ptr(tokens), _ptr(positions), _ptr(kv_cache), _ptr(logits), stream), handle)


def mk_read_probe(buf, sink, n_cus: int, stream: Optional[int] = None):
    """One streaming read of the device tensor `buf` (asynchronous)."""
    _check(lib().mk_read_probe(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), n_cus, stream))


def mk_empty_launches(n_launches: int, n_blocks: int, n_threads: int, stream: Optional[int] = None):
    """n_launches launches of an empty kernel (asynchronous; for timing launch cost)."""
    _check(lib().mk_empty_launches(n_launches, n_blocks, n_threads, stream))


def mk_graph_create(handle, tokens, positions, kv_cache, logits, n_steps: int, flags: int = 0):
    """A HIP graph of n_steps greedy decode steps on these device buffers (see include/mk.h)."""
    g = ctypes.c_void_p()
    _check(lib().mk_graph_create(handle, _ptr(tokens), _ptr(positions), _ptr(kv_cache), _ptr(logits), n_steps, flags,
                                 ctypes.byref(g)), handle)
    return g


def mk_graph_launch(graph, stream: Optional[int] = None):
    _check(lib().mk_graph_launch(graph, stream))


def mk_graph_destroy(graph):
    _check(lib().mk_graph_destroy(graph))


def mk_decode_step_greedy(handle, tokens, positions, kv_cache, logits, stream: Optional[int] = None):
    """mk_decode_step plus greedy selection in one launch: tokens <- argmax(logits), positions += 1."""
    _check(lib().mk_decode_step_greedy(handle, _ptr(tokens), _ptr(positions), _ptr(kv_cache), _ptr(logits),
                                       stream), handle)


def mk_set_ablation(handle, opcode: int):
    """Switch off one opcode's arithmetic in mk_decode_step (0: none); measurement only."""
    _check(lib().mk_set_ablation(handle, opcode), handle)


def mk_decode_step_multikernel(handle, tokens, positions, kv_cache, logits, stream: Optional[int] = None):
    _check(lib().mk_decode_step_multikernel(handle, _ptr(tokens), _ptr(positions), _ptr(kv_cache), _ptr(logits),
                                            stream), handle)


def mk_greedy_advance(handle, logits, tokens, positions, stream: Optional[int] = None):
    _check(lib().mk_greedy_advance(handle, _ptr(logits), _ptr(tokens), _ptr(positions), stream), handle)


def mk_set_spin_limit(handle, spins: int):
    _check(lib().mk_set_spin_limit(handle, spins), handle)


def mk_debug_stage(handle, stage: int, tokens, positions, kv_cache, logits, stream: Optional[int] = None):
    _check(lib().mk_debug_stage(handle, stage, _ptr(tokens), _ptr(positions), _ptr(kv_cache), _ptr(logits), stream),
           handle)


def mk_get_device_error(handle) -> Optional[MkDeviceError]:
    e = MkDeviceError()
    rc = lib().mk_get_device_error(handle, ctypes.byref(e))
    if rc == MK_ERR_DEVICE:
        return e
    _check(rc, handle)
    return None


def mk_get_profile(handle, n_cus: int):
    """Cycle counters of the last step as a numpy array [n_cus][10][8] (uint64)."""
    import numpy as np
    out = np.zeros((n_cus, PROF_WAVES, PROF_SLOTS), dtype=np.uint64)
    _check(lib().mk_get_profile(handle, out.ctypes.data, out.size), handle)
    return out


def mk_get_trace(handle, total_insts: int):
    """Timeline of the last step as a numpy array [total_insts][52] (uint64)."""
    import numpy as np
    out = np.zeros((total_insts, TRACE_SLOTS), dtype=np.uint64)
    _check(lib().mk_get_trace(handle, out.ctypes.data, out.size), handle)
    return out


def mk_destroy(handle):
    _check(lib().mk_destroy(handle))


def current_stream() -> int:
    """hipStream_t of torch's current stream on the current device."""
    import torch
    return torch.cuda.current_stream().cuda_stream
