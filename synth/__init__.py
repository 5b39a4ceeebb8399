"""Seeded synthetic inputs for the decode path and the CPU oracle.

Holds the model shapes and run workloads (sizes only) and the builders that
turn a seed into bf16 weights, prompt token ids and pre-filled KV caches.
No step of the decode method is computed here; both the GPU library and the
oracle consume the identical bytes this module produces.

Weights are nn.Linear layout ``[out][in]``, bf16 stored as ``numpy.uint16``.
Matrices (embedding included) are N(0, 0.02); RMSNorm gains are 1.0 unless a
test asks for ``gain_std > 0`` (then 1 + N(0, gain_std)).
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Dict, List, Optional

import numpy as np

from . import build as _build

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        L = ctypes.CDLL(_build.LIB)
        u64, i32, u32 = ctypes.c_uint64, ctypes.c_int, ctypes.c_uint32
        L.synth_normal_bf16.argtypes = [u64, u64, u64, u64, ctypes.c_double, ctypes.c_double,
                                        ctypes.c_void_p, i32]
        L.synth_normal_bf16.restype = None
        L.synth_uniform_ids.argtypes = [u64, u64, u64, u64, u32, ctypes.c_void_p, i32]
        L.synth_uniform_ids.restype = None
        L.synth_draw_u64.argtypes = [u64, u64, u64]
        L.synth_draw_u64.restype = u64
        L.synth_normal_at.argtypes = [u64, u64, u64]
        L.synth_normal_at.restype = ctypes.c_double
        _lib = L
    return _lib


def default_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def normal_bf16(seed: int, stream: int, n: int, std: float = 1.0, mean: float = 0.0,
                offset: int = 0, threads: Optional[int] = None,
                out: Optional[np.ndarray] = None) -> np.ndarray:
    if out is None:
        out = np.empty(n, dtype=np.uint16)
    assert out.dtype == np.uint16 and out.flags.c_contiguous and out.size == n
    lib().synth_normal_bf16(seed, stream, offset, n, mean, std, out.ctypes.data,
                            threads or default_threads())
    return out


def uniform_ids(seed: int, stream: int, n: int, modulus: int, offset: int = 0,
                threads: Optional[int] = None) -> np.ndarray:
    out = np.empty(n, dtype=np.int32)
    lib().synth_uniform_ids(seed, stream, offset, n, modulus, out.ctypes.data,
                            threads or 1)
    return out


@dataclasses.dataclass(frozen=True)
class ModelShape:
    name: str
    n_layers: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int
    rms_eps: float
    rope_theta: float
    tied: bool

    def weight_bytes(self) -> int:
        """bf16 bytes of every parameter tensor the model holds."""
        H, D = self.hidden, self.head_dim
        per_layer = (self.n_q_heads * D * H + 2 * self.n_kv_heads * D * H
                     + H * self.n_q_heads * D + 3 * self.ffn * H + 2 * H)
        total = self.n_layers * per_layer + self.vocab * H + H
        if not self.tied:
            total += self.vocab * H
        return 2 * total


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    model: ModelShape
    batch: int
    prompt: int          # tokens already in the KV cache when timed decode starts
    decode: int          # greedy decode steps
    prefill: str         # "real": prefill by decode steps; "synthetic": seeded N(0,1) KV rows

    @property
    def max_seq(self) -> int:
        return self.prompt + self.decode


TINY = ModelShape("tiny", 2, 256, 4, 2, 64, 688, 1024, 1e-5, 10000.0, True)
LLAMA_1B = ModelShape("llama-3.2-1b-shaped", 16, 2048, 32, 8, 64, 8192, 128256, 1e-5,
                      500000.0, True)
LLAMA_8B = ModelShape("llama-3.1-8b-shaped", 32, 4096, 32, 8, 128, 14336, 128256, 1e-5,
                      500000.0, False)
# one GPU's share of the 1B shape under 8-way tensor parallelism with one KV
# group per GPU: 4 query heads, 1 K/V head, F/8 gate/up rows (and down
# columns), V/8 rows of the tied embedding / LM head; the hidden size stays H
LLAMA_1B_TP8_SHARD = ModelShape("llama-3.2-1b-tp8-shard", 16, 2048, 4, 1, 64, 1024, 16032, 1e-5,
                                500000.0, True)

WORKLOADS: Dict[str, Workload] = {w.name: w for w in [
    Workload("tiny_b1_p32", TINY, 1, 32, 16, "real"),
    Workload("llama1b_b1_p1024", LLAMA_1B, 1, 1024, 256, "synthetic"),
    Workload("llama1b_b4_p1024", LLAMA_1B, 4, 1024, 128, "synthetic"),
    Workload("llama1b_b8_p1024", LLAMA_1B, 8, 1024, 128, "synthetic"),
    Workload("llama1b_b1_p8192", LLAMA_1B, 1, 8192, 128, "synthetic"),
    Workload("llama1b_b1_p32768", LLAMA_1B, 1, 32768, 128, "synthetic"),
    Workload("llama8b_b1_p1024", LLAMA_8B, 1, 1024, 128, "synthetic"),
    Workload("llama1b_tp8shard_b1_p1024", LLAMA_1B_TP8_SHARD, 1, 1024, 256, "synthetic"),
]}

WEIGHT_SEED = 1234
PROMPT_SEED = 4321
KV_SEED = 777

# stream ids: one per tensor so that tensors are independent of each other
_EMBED, _FINAL_NORM, _LM_HEAD = 1, 2, 3
_LAYER_KINDS = ["attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w_gate", "w_up", "w_down"]


def _layer_stream(layer: int, kind: str) -> int:
    return 1000 + 16 * layer + _LAYER_KINDS.index(kind)


def layer_shapes(m: ModelShape) -> Dict[str, tuple]:
    H, D = m.hidden, m.head_dim
    return {
        "attn_norm": (H,), "wq": (m.n_q_heads * D, H), "wk": (m.n_kv_heads * D, H),
        "wv": (m.n_kv_heads * D, H), "wo": (H, m.n_q_heads * D), "mlp_norm": (H,),
        "w_gate": (m.ffn, H), "w_up": (m.ffn, H), "w_down": (H, m.ffn),
    }


def _matrix(seed, stream, shape, std, threads):
    n = int(np.prod(shape))
    return normal_bf16(seed, stream, n, std=std, threads=threads).reshape(shape)


def _gain(seed, stream, n, gain_std, threads):
    if gain_std > 0:
        return normal_bf16(seed, stream, n, std=gain_std, mean=1.0, threads=threads)
    return np.full(n, 0x3F80, dtype=np.uint16)  # bf16 1.0


def make_weights(m: ModelShape, seed: int = WEIGHT_SEED, std: float = 0.02,
                 gain_std: float = 0.0, threads: Optional[int] = None,
                 zero_layers: bool = False) -> Dict[str, object]:
    """All parameters of model `m`: {'embed', 'final_norm', 'lm_head' (None if tied),
    'layers': [ {attn_norm, wq, wk, wv, wo, mlp_norm, w_gate, w_up, w_down}, ... ]}.

    ``zero_layers`` makes every layer matrix zero (gains stay), a degenerate model
    whose output has a closed form."""
    th = threads or default_threads()
    w: Dict[str, object] = {
        "embed": _matrix(seed, _EMBED, (m.vocab, m.hidden), std, th),
        "final_norm": _gain(seed, _FINAL_NORM, m.hidden, gain_std, th),
        "lm_head": None if m.tied else _matrix(seed, _LM_HEAD, (m.vocab, m.hidden), std, th),
    }
    layers: List[Dict[str, np.ndarray]] = []
    for l in range(m.n_layers):
        d = {}
        for kind, shape in layer_shapes(m).items():
            s = _layer_stream(l, kind)
            if kind.endswith("norm"):
                d[kind] = _gain(seed, s, shape[0], gain_std, th)
            elif zero_layers:
                d[kind] = np.zeros(shape, dtype=np.uint16)
            else:
                d[kind] = _matrix(seed, s, shape, std, th)
        layers.append(d)
    w["layers"] = layers
    return w


def make_prompts(vocab: int, batch: int, length: int, seed: int = PROMPT_SEED) -> np.ndarray:
    """int32 [batch][length]; row b uses seed + b, ids uniform in [0, vocab)."""
    out = np.empty((batch, length), dtype=np.int32)
    for b in range(batch):
        out[b] = uniform_ids(seed + b, 0, length, vocab)
    return out


def make_first_tokens(vocab: int, batch: int, seed: int = PROMPT_SEED) -> np.ndarray:
    """Seeded first decode input when the cache is pre-filled synthetically."""
    return np.array([uniform_ids(seed + b, 1, 1, vocab)[0] for b in range(batch)],
                    dtype=np.int32)


def kv_cache_shape(m: ModelShape, batch: int, max_seq: int) -> tuple:
    """bf16 cache layout [L][2 (K, V)][B][Hkv][max_seq][D]."""
    return (m.n_layers, 2, batch, m.n_kv_heads, max_seq, m.head_dim)


def make_kv_cache(m: ModelShape, batch: int, max_seq: int, filled: int, seed: int = KV_SEED,
                  threads: Optional[int] = None) -> np.ndarray:
    """Cache with slots [0, filled) of every (layer, K/V, row, group) drawn N(0,1) (bf16)
    and the remaining slots zero."""
    shape = kv_cache_shape(m, batch, max_seq)
    cache = np.zeros(shape, dtype=np.uint16)
    if filled <= 0:
        return cache
    D = m.head_dim
    th = threads or default_threads()
    for l in range(m.n_layers):
        for kv in range(2):
            for b in range(batch):
                for g in range(m.n_kv_heads):
                    stream = ((l * 2 + kv) * 64 + b) * 64 + g
                    blk = normal_bf16(seed, stream, filled * D, threads=th)
                    cache[l, kv, b, g, :filled, :] = blk.reshape(filled, D)
    return cache
