"""Shared test helpers: device copies of synthetic weights, greedy decode loops
through the C ABI, and the teacher-forced oracle comparison."""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np

import synth

# parity bar for logits (bf16 weights, fp32 accumulate), per decode step over all B x V
TOL_ABS = 3e-2
TOL_REL = 2e-2       # max |diff| / max |ref|
GAP_STRICT = 0.05    # greedy tokens must match where the oracle's top-2 gap exceeds this


def to_device_u16(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


def device_weights(w: Dict[str, object]) -> Dict[str, object]:
    out = {"embed": to_device_u16(w["embed"]), "final_norm": to_device_u16(w["final_norm"]),
           "lm_head": to_device_u16(w["lm_head"]) if w.get("lm_head") is not None else None,
           "layers": [{k: to_device_u16(v) for k, v in L.items()} for L in w["layers"]]}
    return out


def logits_error(gpu: np.ndarray, ref: np.ndarray):
    """(max |diff|, max |diff| / max |ref|) over a whole step."""
    d = np.max(np.abs(gpu.astype(np.float64) - ref))
    return float(d), float(d / max(np.max(np.abs(ref)), 1e-30))


def top2_gap(row: np.ndarray) -> float:
    s = np.sort(row)
    return float(s[-1] - s[-2])


@dataclasses.dataclass
class Run:
    tokens: List[np.ndarray]     # input tokens per step [B]
    positions: List[np.ndarray]  # positions per step [B]
    logits: List[np.ndarray]     # GPU logits per step [B][V]


class GpuDecoder:
    """A handle plus its device buffers; steps through mk_decode_step(_multikernel)."""

    def __init__(self, shape: synth.ModelShape, weights, batch: int, max_seq: int, n_cus: int = 0,
                 n_splits: int = 0, n_chunks: int = 0, kv_init: Optional[np.ndarray] = None, flags: int = 0):
        import torch
        from decode_megakernel_02_amd import mk
        self.mk, self.torch = mk, torch
        self.shape, self.B, self.max_seq = shape, batch, max_seq
        self.cfg = mk.make_config(shape, batch, max_seq, n_cus=n_cus, n_splits=n_splits, n_chunks=n_chunks,
                                  flags=flags)
        self.h = mk.mk_create(self.cfg)
        self.dw = device_weights(weights)
        mk.mk_load_weights(self.h, self.dw, mk.current_stream())
        nbytes = mk.mk_kv_cache_bytes(self.cfg)
        if kv_init is not None:
            assert kv_init.nbytes == nbytes
            self.kv = to_device_u16(kv_init.reshape(-1))
        else:
            self.kv = torch.zeros(nbytes // 2, dtype=torch.int16, device="cuda")
        self.tokens = torch.zeros(batch, dtype=torch.int32, device="cuda")
        self.positions = torch.zeros(batch, dtype=torch.int32, device="cuda")
        self.logits = torch.zeros(batch, shape.vocab, dtype=torch.float32, device="cuda")

    def step(self, tokens, positions, multikernel: bool = False) -> np.ndarray:
        torch = self.torch
        self.tokens.copy_(torch.as_tensor(np.asarray(tokens, dtype=np.int32)))
        self.positions.copy_(torch.as_tensor(np.asarray(positions, dtype=np.int32)))
        fn = self.mk.mk_decode_step_multikernel if multikernel else self.mk.mk_decode_step
        fn(self.h, self.tokens, self.positions, self.kv, self.logits, self.mk.current_stream())
        torch.cuda.synchronize()
        err = self.mk.mk_get_device_error(self.h)
        if err is not None:
            raise RuntimeError(f"device error code {err.code} wg {err.workgroup} pc {err.pc} op {err.opcode} "
                               f"wave {err.wave} detail {err.detail:#x}")
        return self.logits.cpu().numpy().copy()

    def kv_host(self) -> np.ndarray:
        return self.kv.cpu().numpy().view(np.uint16).reshape(
            synth.kv_cache_shape(self.shape, self.B, self.max_seq))

    def close(self):
        if self.h is not None:
            self.mk.mk_destroy(self.h)
            self.h = None

    def greedy(self, first_tokens: np.ndarray, start_pos: np.ndarray, n_steps: int,
               multikernel: bool = False) -> Run:
        toks = np.asarray(first_tokens, dtype=np.int32).copy()
        pos = np.asarray(start_pos, dtype=np.int32).copy()
        run = Run([], [], [])
        for _ in range(n_steps):
            lg = self.step(toks, pos, multikernel)
            run.tokens.append(toks.copy())
            run.positions.append(pos.copy())
            run.logits.append(lg)
            toks = np.argmax(lg, axis=1).astype(np.int32)  # lowest index on ties, as torch.argmax
            pos = pos + 1
        return run


def oracle_replay(shape, weights, batch, max_seq, run: Run, kv_init: Optional[np.ndarray] = None,
                  nthreads: int = 8, fp8=False) -> List[np.ndarray]:
    """Teacher-forced oracle logits for the exact inputs the GPU saw (fp8: as oracle.Oracle)."""
    import oracle
    orc = oracle.Oracle(shape, weights, batch, max_seq, fp8=fp8)
    cache = (np.zeros(synth.kv_cache_shape(shape, batch, max_seq), dtype=np.uint16) if kv_init is None
             else kv_init.copy())
    return [orc.decode_step(cache, t, p, nthreads) for t, p in zip(run.tokens, run.positions)]


def compare(run: Run, ref: List[np.ndarray], label: str = "") -> Dict[str, float]:
    """Asserts the parity bar on every step; returns summary statistics."""
    worst_abs = worst_rel = 0.0
    checked = skipped = 0
    for i, (g, r) in enumerate(zip(run.logits, ref)):
        a, rel = logits_error(g, r)
        worst_abs, worst_rel = max(worst_abs, a), max(worst_rel, rel)
        assert a <= TOL_ABS and rel <= TOL_REL, f"{label} step {i}: max|d| {a:.3g}, rel {rel:.3g}"
        for b in range(r.shape[0]):
            if top2_gap(r[b]) > GAP_STRICT:
                checked += 1
                assert int(np.argmax(g[b])) == int(np.argmax(r[b])), \
                    f"{label} step {i} row {b}: token {np.argmax(g[b])} vs oracle {np.argmax(r[b])}"
            else:
                skipped += 1
    return {"max_abs": worst_abs, "max_rel": worst_rel, "tokens_checked": checked, "tokens_close": skipped}
