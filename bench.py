#!/usr/bin/env python3
"""Decode throughput of the single-launch megakernel on one MI355X.

Workload (default): Llama-3.2-1B-shaped decoder with random bf16 weights
N(0, 0.02), batch 1, a 1024-token context pre-filled in the KV cache with
seeded N(0,1) bf16 rows, greedy decode.  One timed step = one
mk_decode_step_greedy launch: the whole forward pass and the argmax into the
next step's tokens (positions + 1) in a single kernel, on one stream with no
host synchronisation inside the timed region.  The two-launch form (the step,
then mk_greedy_advance) is timed beside it.

Prints ONE JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode tokens/s at batch 1 + achieved % of HBM roofline (Llama-1B-shaped)"
KERNEL_NAME = "mk_decode_kernel"  # the single-launch step kernel (the per-op path launches mk_stage_kernel)


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in ["mk_kernels.hip", "mk_internal.h", "mk_plan.cpp", "mk_api.cpp"]:
        with open(os.path.join(ROOT, "decode_megakernel_02_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, only if
    it was taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_{KERNEL_NAME}_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_hash") != kernel_source_hash():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def _pmc_per_dispatch(csv_path, name_part):
    """Counter value per dispatch (summed over the counter's instances) of kernels whose name contains name_part."""
    import csv
    import collections
    agg = collections.OrderedDict()
    with open(csv_path) as fh:
        for r in csv.DictReader(fh):
            if name_part in r["Kernel_Name"]:
                agg[r["Dispatch_Id"]] = agg.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    return list(agg.values())


def write_traffic_summary(fetch_csv, write_csv, workload, copy_bytes, command):
    """HBM bytes per launch of the step kernel from rocprofv3 FETCH_SIZE and WRITE_SIZE passes (KiB per
    dispatch), each scaled by what the same counter reads for a plain copy kernel of copy_bytes read and
    copy_bytes written (the elementwise copy that --calib-copy-mib launches in the same process)."""
    import statistics
    copy_kernel = "vectorized_elementwise_kernel"
    f_copy = [v for v in _pmc_per_dispatch(fetch_csv, copy_kernel) if v > copy_bytes / 1024 / 4]
    w_copy = [v for v in _pmc_per_dispatch(write_csv, copy_kernel) if v > copy_bytes / 1024 / 4]
    f_scale = (copy_bytes / 1024) / statistics.median(f_copy)
    w_scale = (copy_bytes / 1024) / statistics.median(w_copy)
    f_mk = _pmc_per_dispatch(fetch_csv, KERNEL_NAME)
    w_mk = _pmc_per_dispatch(write_csv, KERNEL_NAME)
    fetch = statistics.median(f_mk) * 1024 * f_scale
    write = statistics.median(w_mk) * 1024 * w_scale
    path = os.path.join(ROOT, "profiles", f"traffic_{KERNEL_NAME}_{workload}.txt")
    with open(path, "w") as fh:
        fh.write(f"# HBM traffic of {KERNEL_NAME}, workload {workload}, from rocprofv3 counter passes\n")
        fh.write(f"# command: {command}\n")
        fh.write(f"# {len(f_mk)} / {len(w_mk)} dispatches; copy-kernel calibration: {copy_bytes} B read + written, "
                 f"FETCH_SIZE reads {statistics.median(f_copy):.1f} KiB, WRITE_SIZE reads {statistics.median(w_copy):.1f} KiB\n")
        fh.write(f"fetch_scale: {f_scale:.4f}\n")
        fh.write(f"write_scale: {w_scale:.4f}\n")
        fh.write(f"fetch_bytes_per_launch: {fetch:.0f}\n")
        fh.write(f"write_bytes_per_launch: {write:.0f}\n")
        fh.write(f"hbm_bytes_per_launch: {fetch + write:.0f}\n")
        fh.write(f"kernel_source_hash: {kernel_source_hash()}\n")
    return path


def write_stats_summary(stats_csv, workload, command):
    """Per-kernel duration table from a rocprofv3 --kernel-trace --stats run."""
    import csv
    rows = list(csv.DictReader(open(stats_csv)))
    path = os.path.join(ROOT, "profiles", f"kernel_trace_{KERNEL_NAME}_{workload}.md")
    with open(path, "w") as fh:
        fh.write(f"# Kernel durations, workload {workload} (rocprofv3 --kernel-trace --stats)\n\n")
        fh.write(f"Command: `{command}`\n\n")
        fh.write("| kernel | calls | average us | min us | max us | share % |\n|---|---|---|---|---|---|\n")
        for r in rows:
            name = r["Name"]
            short = name.split("(")[0].replace("void ", "")[:80]
            fh.write(f"| `{short}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                     f"{float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.2f} |\n")
    return path


def cpu_baseline(shape, weights, kv_host, first_toks, prompt, n_steps: int, threads: int = 0):
    """The oracle on the host cores: n_steps greedy steps of every batch row after one warm-up
    step; threads = 0 uses every core (at most 64)."""
    import numpy as np

    import oracle
    threads = threads or max(1, min(64, os.cpu_count() or 1))
    B = kv_host.shape[2]
    orc = oracle.Oracle(shape, weights, B, kv_host.shape[4])
    cache = kv_host.copy()
    tok = np.asarray(first_toks, dtype=np.int32).reshape(B)
    orc.decode_step(cache, tok, np.full(B, prompt, dtype=np.int32), threads)  # warm-up
    t0 = time.perf_counter()
    for i in range(n_steps):
        lg = orc.decode_step(cache, tok, np.full(B, prompt + 1 + i, dtype=np.int32), threads)
        tok = np.argmax(lg, axis=1).astype(np.int32)
    dt = (time.perf_counter() - t0) / n_steps
    return {"value": B / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{n_steps} greedy decode steps of the same workload (batch {B}) after 1 warm-up step "
                      f"(fp64 C oracle, {threads} threads, rows split across threads); "
                      f"{dt * 1e3:.1f} ms/step"}


def write_stage_summary(trace_csv, workload, command):
    """Per-op durations of the per-op-launch path from a rocprofv3 --kernel-trace run: the stage
    launches of a step come in op order (six per layer, then the LM head), so a launch's position
    in its step names its op; also the idle gap between consecutive launches of a step."""
    import csv
    import synth
    shape = synth.WORKLOADS[workload].model
    n = shape.n_layers * 6 + 1
    ops = ["RMS_QKV_ROPE", "ATTENTION", "ATTN_REDUCE", "O_PROJ_RES", "RMS_UP_GATE", "DOWN_RES"]
    rows = [r for r in csv.DictReader(open(trace_csv)) if "mk_stage_kernel" in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    if not rows or len(rows) % n:
        raise SystemExit(f"{len(rows)} stage launches is not a multiple of {n}")
    dur, gap = {}, {}
    for i, r in enumerate(rows):
        j = i % n
        op = "RMS_LM_HEAD" if j == n - 1 else ops[j % 6]
        dur.setdefault(op, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        if j:
            gap.setdefault(op, []).append((int(r["Start_Timestamp"]) - int(rows[i - 1]["End_Timestamp"])) / 1e3)
    steps = len(rows) // n
    total = sum(sum(v) for v in dur.values()) / steps
    path = os.path.join(ROOT, "profiles", f"stage_durations_mk_stage_kernel_{workload}.md")
    with open(path, "w") as fh:
        fh.write(f"# Per-op launches of the decode step, workload {workload} (rocprofv3 --kernel-trace)\n\n")
        fh.write(f"Command: `{command}`\n\n")
        fh.write(f"{steps} steps of {n} launches; kernel time {total:.1f} us per step.\n\n")
        fh.write("| op | launches per step | average us | us per step | share % | average gap before, us |\n"
                 "|---|---|---|---|---|---|\n")
        for op in ops + ["RMS_LM_HEAD"]:
            v = dur[op]
            per_step = sum(v) / steps
            g = gap.get(op, [])
            fh.write(f"| {op} | {len(v) // steps} | {sum(v) / len(v):.2f} | {per_step:.1f} | "
                     f"{100 * per_step / total:.1f} | {sum(g) / len(g) if g else 0:.2f} |\n")
    return path


OPCODES = ["RMS_QKV_ROPE", "ATTENTION", "ATTN_REDUCE", "O_PROJ_RES", "RMS_UP_GATE", "DOWN_RES", "RMS_LM_HEAD"]


def ablation_table(mk, h, tokens, positions, kv, logits, stream, P, K, W, args):
    """Single-launch step time (CUDA-event mean over K launches, median of 5 interleaved rounds)
    with no opcode and with each opcode's arithmetic switched off; Markdown."""
    import torch
    cur = torch.cuda.current_stream()
    rounds = {op: [] for op in range(8)}
    for _ in range(5):
        for op in range(8):
            mk.mk_set_ablation(h, op)
            positions.fill_(P)
            for _ in range(W):
                mk.mk_decode_step(h, tokens, positions, kv, logits, stream)
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
            for a, b in ev:
                a.record(cur)
                mk.mk_decode_step(h, tokens, positions, kv, logits, stream)
                b.record(cur)
            torch.cuda.synchronize()
            err = mk.mk_get_device_error(h)
            if err is not None:
                raise RuntimeError(f"device error with opcode {op} switched off: code {err.code}")
            rounds[op].append(statistics.mean(a.elapsed_time(b) * 1e3 for a, b in ev))
    mk.mk_set_ablation(h, 0)
    base = statistics.median(rounds[0])
    lines = [f"# Single-launch step with one opcode's arithmetic switched off, workload {args.workload}",
             "",
             "The ablation build (mk_set_ablation) keeps every dependency: the switched-off opcode's weight "
             "units still stream through the rings unread, its inputs are still awaited and its tagged "
             "outputs still written. Kernel time per step: CUDA events around each launch, mean over "
             f"{K} launches, median of 5 interleaved rounds.",
             "",
             f"Command: `python bench.py --ablation --workload {args.workload} --steps {K} --warmup {W}`",
             "",
             "| switched off | us per step | shrink us | shrink % |",
             "|---|---|---|---|",
             f"| nothing | {base:.1f} | | |"]
    for op in range(1, 8):
        t = statistics.median(rounds[op])
        lines.append(f"| {OPCODES[op - 1]} | {t:.1f} | {base - t:.1f} | {100 * (base - t) / base:.1f} |")
    return "\n".join(lines)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="llama1b_b1_p1024")
    ap.add_argument("--mk-steps", type=int, default=64, help="timed steps of the per-op-launch path")
    ap.add_argument("--cpu-steps", type=int, default=32, help="timed oracle steps (0: skip the CPU baseline)")
    ap.add_argument("--stats-summary", nargs=2, metavar=("STATS_CSV", "COMMAND"),
                    help="write the profiles/ kernel-duration summary from a rocprofv3 --stats run and exit")
    ap.add_argument("--traffic-summary", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "COMMAND"),
                    help="write the profiles/ traffic summary from two rocprofv3 counter passes and exit")
    ap.add_argument("--stage-summary", nargs=2, metavar=("TRACE_CSV", "COMMAND"),
                    help="write the profiles/ per-op table of the per-op-launch path from a rocprofv3 "
                         "--kernel-trace run and exit")
    ap.add_argument("--cpu-threads", type=int, default=0, help="oracle threads (0: every core, at most 64)")
    ap.add_argument("--fp8", action="store_true",
                    help="FP8 (E4M3, one scale per output row) weights instead of bf16 (a variant, not the headline)")
    ap.add_argument("--cpu-only", action="store_true",
                    help="time only the CPU oracle on the workload and print it as one JSON line")
    ap.add_argument("--prefill", action="store_true",
                    help="time batched prefill (mk_prefill) of the workload's prompt instead of decode; one JSON line")
    ap.add_argument("--ablation", action="store_true",
                    help="print the table of the single-launch step time with each opcode's arithmetic "
                         "switched off (mk_set_ablation) instead of the JSON line")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="first run a plain device copy of this many MiB (3 launches), the reference "
                         "kernel for scaling HBM byte counters")
    args = ap.parse_args()
    if args.stats_summary:
        print(write_stats_summary(args.stats_summary[0], args.workload, args.stats_summary[1]))
        return
    if args.stage_summary:
        print(write_stage_summary(args.stage_summary[0], args.workload, args.stage_summary[1]))
        return
    if args.cpu_only:
        import synth
        wl = synth.WORKLOADS[args.workload]
        t0 = time.perf_counter()
        weights = synth.make_weights(wl.model)
        kv_host = synth.make_kv_cache(wl.model, wl.batch, wl.prompt + args.cpu_steps + 2, wl.prompt)
        log(f"inputs generated in {time.perf_counter() - t0:.1f}s")
        cb = cpu_baseline(wl.model, weights, kv_host, synth.make_first_tokens(wl.model.vocab, wl.batch), wl.prompt,
                          max(1, args.cpu_steps), args.cpu_threads)
        print(json.dumps({"workload": args.workload, "cpu_baseline": cb}), flush=True)
        return
    if args.traffic_summary:
        print(write_traffic_summary(args.traffic_summary[0], args.traffic_summary[1], args.workload,
                                    (args.calib_copy_mib or 1024) << 20, args.traffic_summary[2]))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}): the decode path runs on a "
              "single GPU and has no multi-GPU variant.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    from decode_megakernel_02_amd import mk
    from decode_megakernel_02_amd import roofline as R

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(3)
    if args.calib_copy_mib > 0:
        n = args.calib_copy_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)  # reads n bytes, writes n bytes
        torch.cuda.synchronize()
        log(f"copy calibration: 3 launches, {n} bytes read + {n} bytes written each")
        del src, dst
    wl = synth.WORKLOADS[args.workload]
    shape, B, P = wl.model, wl.batch, wl.prompt
    K, W = args.steps, args.warmup
    max_seq = P + W + max(K, args.mk_steps) + 8

    t0 = time.perf_counter()
    weights = synth.make_weights(shape)
    log(f"weights generated in {time.perf_counter() - t0:.1f}s ({shape.weight_bytes() / 1e9:.2f} GB)")
    kv_host = synth.make_kv_cache(shape, B, max_seq, P)
    first = synth.make_first_tokens(shape.vocab, B)

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()

    dw = {"embed": up(weights["embed"]), "final_norm": up(weights["final_norm"]),
          "lm_head": up(weights["lm_head"]) if weights["lm_head"] is not None else None,
          "layers": [{k: up(v) for k, v in L.items()} for L in weights["layers"]]}
    cfg = mk.make_config(shape, B, max_seq, flags=mk.MK_FLAG_FP8_WEIGHTS if args.fp8 else 0)
    h = mk.mk_create(cfg)
    stream = mk.current_stream()
    mk.mk_load_weights(h, dw, stream)
    if args.prefill:  # whole-prompt pass: W untimed and K timed calls of mk_prefill (each synchronous)
        kvz = torch.zeros(mk.mk_kv_cache_bytes(cfg) // 2, dtype=torch.int16, device="cuda")
        ptoks = torch.as_tensor(synth.make_prompts(shape.vocab, B, P)).cuda()
        lg = torch.empty(B, shape.vocab, dtype=torch.float32, device="cuda")
        for _ in range(max(W, 1)):
            mk.mk_prefill(h, dw, ptoks, P, kvz, lg, stream)
        ts = []
        for _ in range(K):
            torch.cuda.synchronize()
            t1 = time.perf_counter()
            mk.mk_prefill(h, dw, ptoks, P, kvz, lg, stream)
            ts.append(time.perf_counter() - t1)
        med = float(np.median(ts))
        QD, KD = shape.n_q_heads * shape.head_dim, shape.n_kv_heads * shape.head_dim
        # algorithmic flops: the projections of every position, causal attention (q.k and p.v over
        # P (P + 1) / 2 query-key pairs per row and head), the LM head of the last position
        flops = (2.0 * B * P * shape.n_layers * shape.hidden * (QD + 2 * KD + QD + 3 * shape.ffn)
                 + 4.0 * B * shape.n_layers * shape.n_q_heads * shape.head_dim * P * (P + 1) / 2
                 + 2.0 * B * shape.vocab * shape.hidden)
        peak = 2500.0  # dense bf16 matrix cores (each product runs as two bf16 MFMAs: hi and lo terms)
        print(json.dumps({"metric": "prefill_tokens_per_s", "value": B * P / med, "unit": "tokens/s", "n_gpus": 1,
                          "steps": K, "warmup": W, "ms_per_step": med * 1e3, "higher_is_better": True,
                          "dtype": "bf16 MFMA (fp32 activations as hi + lo bf16 terms), fp32 sums",
                          "data": "synthetic",
                          "config": {"workload": args.workload, "batch": B, "prompt": P},
                          "roofline": {"bound": "mfma", "achieved": flops / med / 1e12, "peak": peak,
                                       "unit": "TFLOP/s", "frac": flops / med / 1e12 / peak, "traffic": None}}),
              flush=True)
        mk.mk_destroy(h)
        return
    del dw
    torch.cuda.empty_cache()
    kv = up(kv_host.reshape(-1))
    tokens = torch.tensor(first, dtype=torch.int32, device="cuda")
    positions = torch.full((B,), P, dtype=torch.int32, device="cuda")
    logits = torch.empty(B, shape.vocab, dtype=torch.float32, device="cuda")
    log(f"handle ready; schedule: {mk.mk_schedule_inspect(cfg, torch.cuda.get_device_properties(0).multi_processor_count).total_insts} instructions")

    if args.ablation:
        print(ablation_table(mk, h, tokens, positions, kv, logits, stream, P, K, W, args), flush=True)
        torch.cuda.synchronize()
        mk.mk_destroy(h)
        return

    def greedy(n, fn):
        for _ in range(n):
            fn(h, tokens, positions, kv, logits, stream)
            mk.mk_greedy_advance(h, logits, tokens, positions, stream)  # argmax -> tokens, positions += 1

    def fused(n):  # one launch per step: the step advances tokens and positions itself
        for _ in range(n):
            mk.mk_decode_step_greedy(h, tokens, positions, kv, logits, stream)

    def check_device():
        err = mk.mk_get_device_error(h)
        if err is not None:
            raise RuntimeError(f"device error record: code {err.code} wg {err.workgroup} pc {err.pc} "
                               f"op {err.opcode} detail {err.detail:#x}")

    # ---- megakernel with greedy selection fused in: warm-up, then K timed steps
    fused(W)
    torch.cuda.synchronize()
    check_device()
    t0 = time.perf_counter()
    fused(K)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    check_device()
    log(f"megakernel (fused greedy): {K} steps in {wall * 1e3:.1f} ms")

    # ---- per-launch kernel time (events on the launch stream), same positions
    positions.fill_(P + W)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    cur = torch.cuda.current_stream()  # the stream mk_decode_step launches on
    for i in range(K):
        ev[i][0].record(cur)
        mk.mk_decode_step_greedy(h, tokens, positions, kv, logits, stream)
        ev[i][1].record(cur)
    torch.cuda.synchronize()
    check_device()
    kern_us = [a.elapsed_time(b) * 1e3 for a, b in ev]
    kern_mean = statistics.mean(kern_us)

    # ---- the two-launch form: the step, then the argmax kernel
    positions.fill_(P)
    greedy(3, mk.mk_decode_step)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    greedy(K, mk.mk_decode_step)
    torch.cuda.synchronize()
    wall_two = time.perf_counter() - t0
    check_device()
    log(f"megakernel + argmax launch: {K} steps in {wall_two * 1e3:.1f} ms")

    # ---- per-op launches (same op bodies, 6L+1 launches per step)
    KM = args.mk_steps
    positions.fill_(P)
    greedy(3, mk.mk_decode_step_multikernel)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    greedy(KM, mk.mk_decode_step_multikernel)
    torch.cuda.synchronize()
    wall_mk = time.perf_counter() - t0
    positions.fill_(P + 3)
    evm = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(KM)]
    for i in range(KM):
        evm[i][0].record(cur)
        mk.mk_decode_step_multikernel(h, tokens, positions, kv, logits, stream)
        evm[i][1].record(cur)
        mk.mk_greedy_advance(h, logits, tokens, positions, stream)
    torch.cuda.synchronize()
    check_device()
    kern_mk = statistics.mean(a.elapsed_time(b) * 1e3 for a, b in evm)
    log(f"multikernel: {KM} steps in {wall_mk * 1e3:.1f} ms")

    ncu = torch.cuda.get_device_properties(0).multi_processor_count

    # ---- the same loops captured once as HIP graphs (one replay = step + argmax), and the
    # launch cost alone: as many empty kernels as the per-op step launches, eager and in a graph
    def graph_us(flags, n):
        g = mk.mk_graph_create(h, tokens, positions, kv, logits, 1, flags)
        try:
            positions.fill_(P)
            for _ in range(3):
                mk.mk_graph_launch(g, stream)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(cur)
            for _ in range(n):
                mk.mk_graph_launch(g, stream)
            e1.record(cur)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) * 1e3 / n
        finally:
            mk.mk_graph_destroy(g)

    n_launch = shape.n_layers * 6 + 1
    graph_mk = graph_us(mk.MK_GRAPH_MULTIKERNEL, KM)
    check_device()
    try:
        graph_mega = graph_us(mk.MK_GRAPH_FUSED_GREEDY, KM)
        check_device()
    except mk.MkError as e:  # the runtime may refuse to capture a cooperative launch
        graph_mega = None
        log(f"single-launch step not capturable: {e}")
    graph_empty = graph_us(mk.MK_GRAPH_EMPTY, 20)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    mk.mk_empty_launches(n_launch, ncu, mk.MK_STEP_THREADS, stream)
    e0.record(cur)
    for _ in range(20):
        mk.mk_empty_launches(n_launch, ncu, mk.MK_STEP_THREADS, stream)
    e1.record(cur)
    torch.cuda.synchronize()
    eager_empty = e0.elapsed_time(e1) * 1e3 / 20
    log(f"graphs: per-op step {graph_mk:.1f} us, single-launch step {graph_mega} us; "
        f"{n_launch} empty launches: eager {eager_empty:.1f} us, graph {graph_empty:.1f} us")

    # ---- the device's sustained read rate (4 GiB, past the memory-side cache), best of 5
    probe_buf = torch.empty(4 << 30, dtype=torch.uint8, device="cuda")
    probe_buf.fill_(1)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    probe_gbps = 0.0
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(cur)
        mk.mk_read_probe(probe_buf, sink, ncu, stream)
        e1.record(cur)
        torch.cuda.synchronize()
        probe_gbps = max(probe_gbps, probe_buf.numel() / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    del probe_buf
    torch.cuda.empty_cache()
    log(f"read probe: {probe_gbps:.0f} GB/s")

    # ---- roofline of the dominant (only) kernel
    keys = R.mean_keys(P, W, K)  # the event-timed pass covers steps W .. W+K-1
    bytes_step = R.step_bytes(shape, B, keys, 1 if args.fp8 else 2)
    achieved = bytes_step / (kern_mean * 1e-6) / 1e9
    peak = R.MI355X_HBM_PEAK_GBPS
    traffic = None if args.fp8 else measured_traffic(args.workload)  # counters were taken for bf16
    ms_per_step = wall / K * 1e3

    out = {
        "metric": METRIC,
        "value": B * K / wall,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-e4m3 weights" if args.fp8 else "bf16",
        "data": "synthetic",
        "config": {"workload": f"{shape.name}, batch {B}, {P}-token synthetic KV prefill, greedy decode",
                   "batch": B, "prompt_tokens": P, "decode_steps": K, "kv_prefill": "seeded N(0,1) bf16 rows",
                   "weights": "seeded N(0,0.02) bf16, norm gains 1.0" + (
                       ", projections and LM head quantised to FP8 E4M3 with one scale per output row" if args.fp8 else ""),
                   "accumulate": "fp32",
                   "kernel_launches_per_step": 1},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": peak, "unit": "GB/s", "frac": achieved / peak,
                     "traffic": traffic},
        "hbm_read_probe_GBps": probe_gbps,
        "achieved_frac_of_read_probe": achieved / probe_gbps,
        "kernel_us_per_step": kern_mean,
        "two_launch_ms_per_step": wall_two / K * 1e3,
        "kernel_us_median": statistics.median(kern_us),
        "bytes_per_step": bytes_step,
        "floor_us_per_step": R.floor_us(bytes_step),
        "multikernel": {"ms_per_step": wall_mk / KM * 1e3, "tokens_per_s": B * KM / wall_mk,
                        "kernel_us_per_step": kern_mk, "launches_per_step": shape.n_layers * 6 + 1,
                        "megakernel_speedup": kern_mk / kern_mean,
                        "graph_us_per_step": graph_mk, "megakernel_speedup_vs_graph": graph_mk / (wall / K * 1e6)},
        "graph": {"megakernel_us_per_step": graph_mega, "per_op_us_per_step": graph_mk,
                  "note": "one replay = one step: the per-op launches + the argmax launch, or the single fused "
                          "launch; captured once, replayed back to back"},
        "launch_overhead": {"launches": n_launch, "blocks": ncu, "threads": mk.MK_STEP_THREADS, "eager_empty_us": eager_empty,
                            "graph_empty_us": graph_empty},
        "kernel_source_hash": kernel_source_hash(),
    }
    if args.cpu_steps > 0:
        log("timing the CPU oracle")
        out["cpu_baseline"] = cpu_baseline(shape, weights, kv_host, first, P, args.cpu_steps, args.cpu_threads)
    # release everything device-side before returning (graphs were destroyed above), so that
    # nothing of the library or torch's caching allocator is left for exit-time teardown
    torch.cuda.synchronize()
    mk.mk_destroy(h)
    del kv, tokens, positions, logits
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
