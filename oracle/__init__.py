"""Python access to the C oracle (oracle/oracle.c).

TEST INFRASTRUCTURE ONLY: imported by tests, the package smoke check and the
bench's CPU-baseline leg.  The decode library never imports it.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

import numpy as np

from . import build as _build

_lib = None
_P = ctypes.c_void_p


class OrcConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in
                ["n_layers", "hidden", "n_q_heads", "n_kv_heads", "head_dim", "ffn", "vocab",
                 "batch", "max_seq", "tied"]] + [("rms_eps", ctypes.c_double),
                                                 ("rope_theta", ctypes.c_double), ("fp8", ctypes.c_int)]


class OrcWeights(ctypes.Structure):
    _fields_ = [("embed", _P), ("final_norm", _P), ("lm_head", _P)] + [
        (n, ctypes.POINTER(_P)) for n in
        ["attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w_gate", "w_up", "w_down"]]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        L = ctypes.CDLL(_build.LIB)
        L.orc_bf16_to_double.argtypes = [ctypes.c_uint16]
        L.orc_bf16_to_double.restype = ctypes.c_double
        L.orc_bf16_round.argtypes = [ctypes.c_double]
        L.orc_bf16_round.restype = ctypes.c_uint16
        L.orc_rmsnorm.argtypes = [_P, _P, ctypes.c_int, ctypes.c_double, _P]
        L.orc_gemv.argtypes = [_P, ctypes.c_int, ctypes.c_int, _P, _P, ctypes.c_int]
        L.orc_rope.argtypes = [_P, ctypes.c_int, ctypes.c_int, ctypes.c_double]
        L.orc_attention.argtypes = [_P, _P, _P, ctypes.c_int, ctypes.c_int, _P]
        L.orc_silu.argtypes = [ctypes.c_double]
        L.orc_silu.restype = ctypes.c_double
        L.orc_kv_cache_bytes.argtypes = [ctypes.POINTER(OrcConfig)]
        L.orc_kv_cache_bytes.restype = ctypes.c_uint64
        L.orc_decode_step.argtypes = [ctypes.POINTER(OrcConfig), ctypes.POINTER(OrcWeights),
                                      _P, _P, _P, _P, ctypes.c_int]
        L.orc_decode_step.restype = ctypes.c_int
        L.orc_e4m3_to_double.argtypes = [ctypes.c_uint8]
        L.orc_e4m3_to_double.restype = ctypes.c_double
        L.orc_e4m3_round.argtypes = [ctypes.c_double]
        L.orc_e4m3_round.restype = ctypes.c_uint8
        L.orc_fp8_scale.argtypes = [_P, ctypes.c_size_t]
        L.orc_fp8_scale.restype = ctypes.c_float
        L.orc_gemv_fp8.argtypes = [_P, ctypes.c_int, ctypes.c_int, _P, _P, ctypes.c_int]
        L.orc_gemv_fp8_rows.argtypes = [_P, ctypes.c_int, ctypes.c_int, _P, _P, ctypes.c_int]
        L.orc_argmax.argtypes = [_P, ctypes.c_int]
        L.orc_argmax.restype = ctypes.c_int
        _lib = L
    return _lib


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def _u16(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    assert a.dtype == np.uint16
    return a


def bf16_to_double(bits: int) -> float:
    return lib().orc_bf16_to_double(int(bits))


def bf16_round(x: float) -> int:
    return int(lib().orc_bf16_round(float(x)))


def rmsnorm(h, gain_bits, eps: float) -> np.ndarray:
    h, g = _f64(h), _u16(gain_bits)
    out = np.empty_like(h)
    lib().orc_rmsnorm(h.ctypes.data, g.ctypes.data, h.size, eps, out.ctypes.data)
    return out


def gemv(W_bits, x, nthreads: int = 1) -> np.ndarray:
    W, x = _u16(W_bits), _f64(x)
    rows, cols = W.shape
    y = np.empty(rows, dtype=np.float64)
    lib().orc_gemv(W.ctypes.data, rows, cols, x.ctypes.data, y.ctypes.data, nthreads)
    return y


def e4m3_to_double(code: int) -> float:
    return lib().orc_e4m3_to_double(int(code))


def e4m3_round(x: float) -> int:
    return int(lib().orc_e4m3_round(float(x)))


def fp8_scale(W_bits) -> float:
    W = _u16(W_bits)
    return float(lib().orc_fp8_scale(W.ctypes.data, W.size))


def gemv_fp8(W_bits, x, nthreads: int = 1) -> np.ndarray:
    W, x = _u16(W_bits), _f64(x)
    rows, cols = W.shape
    y = np.empty(rows, dtype=np.float64)
    lib().orc_gemv_fp8(W.ctypes.data, rows, cols, x.ctypes.data, y.ctypes.data, nthreads)
    return y


def gemv_fp8_rows(W_bits, x, nthreads: int = 1) -> np.ndarray:
    """FP8 (E4M3) GEMV with one scale per row (the row's largest magnitude / 448)."""
    W, x = _u16(W_bits), _f64(x)
    rows, cols = W.shape
    y = np.empty(rows, dtype=np.float64)
    lib().orc_gemv_fp8_rows(W.ctypes.data, rows, cols, x.ctypes.data, y.ctypes.data, nthreads)
    return y


def rope(v, pos: int, theta: float) -> np.ndarray:
    v = _f64(v).copy()
    lib().orc_rope(v.ctypes.data, v.size, pos, theta)
    return v


def attention(q, K_bits, V_bits) -> np.ndarray:
    q, K, V = _f64(q), _u16(K_bits), _u16(V_bits)
    n, D = K.shape
    out = np.empty(D, dtype=np.float64)
    lib().orc_attention(q.ctypes.data, K.ctypes.data, V.ctypes.data, n, D, out.ctypes.data)
    return out


def silu(z: float) -> float:
    return lib().orc_silu(float(z))


class Oracle:
    """Holds weight pointers (the numpy arrays stay referenced) for repeated steps."""

    def __init__(self, shape, weights: Dict[str, object], batch: int, max_seq: int, fp8=False):
        """fp8: False (bf16 weights), True or "matrix" (FP8, one scale per matrix), "row" (FP8, one
        scale per output row)."""
        self.shape = shape
        mode = 0 if not fp8 else 2 if fp8 == "row" else 1
        self.cfg = OrcConfig(shape.n_layers, shape.hidden, shape.n_q_heads, shape.n_kv_heads,
                             shape.head_dim, shape.ffn, shape.vocab, batch, max_seq,
                             1 if shape.tied else 0, shape.rms_eps, shape.rope_theta, mode)
        self._keep = weights
        L = shape.n_layers
        w = OrcWeights()
        w.embed = _u16(weights["embed"]).ctypes.data
        w.final_norm = _u16(weights["final_norm"]).ctypes.data
        lm = weights.get("lm_head")
        w.lm_head = _u16(lm).ctypes.data if lm is not None else None
        self._ptr_arrays = []
        for kind in ["attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w_gate", "w_up", "w_down"]:
            arr = (_P * L)(*[_u16(weights["layers"][l][kind]).ctypes.data for l in range(L)])
            self._ptr_arrays.append(arr)
            setattr(w, kind, ctypes.cast(arr, ctypes.POINTER(_P)))
        self.w = w

    def kv_cache_bytes(self) -> int:
        return int(lib().orc_kv_cache_bytes(ctypes.byref(self.cfg)))

    def decode_step(self, kv_cache: np.ndarray, tokens, positions, nthreads: int = 1
                    ) -> np.ndarray:
        """Runs one step in place on `kv_cache` (uint16, the bf16 layout
        [L][2][B][Hkv][max_seq][D]); returns logits float64 [B][V]."""
        assert kv_cache.dtype == np.uint16 and kv_cache.flags.c_contiguous
        assert kv_cache.nbytes == self.kv_cache_bytes()
        B, V = self.cfg.batch, self.cfg.vocab
        t = np.ascontiguousarray(tokens, dtype=np.int32).reshape(B)
        p = np.ascontiguousarray(positions, dtype=np.int32).reshape(B)
        logits = np.empty((B, V), dtype=np.float64)
        rc = lib().orc_decode_step(ctypes.byref(self.cfg), ctypes.byref(self.w),
                                   kv_cache.ctypes.data, t.ctypes.data, p.ctypes.data,
                                   logits.ctypes.data, nthreads)
        if rc != 0:
            raise ValueError(f"orc_decode_step failed with code {rc}")
        return logits


def argmax(v) -> int:
    v = _f64(v)
    return int(lib().orc_argmax(v.ctypes.data, v.size))
