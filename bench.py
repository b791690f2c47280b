#!/usr/bin/env python3
"""Benchmark of the MoE token-routing path on one MI355X.

One step = the whole path over one batch of the chosen workload:
    moe_mask_padding -> moe_create_indices -> moe_dispatch (bf16)
    -> moe_dispatch_mxfp4 -> moe_combine
with inputs resident in HBM.  Prints ONE JSON line on stdout (progress goes
to stderr).  `value` = routed token-slots per second of the whole step.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402

HBM_PEAK_GBPS = 8000.0       # MI355X HBM3E, AMD published peak
METRIC = "routed token-slots/s + achieved HBM GB/s vs peak (index+dispatch+combine)"
STAGES = ("mask", "indices", "dispatch_bf16", "dispatch_mxfp4", "combine")
KERNEL_OF_STAGE = {"dispatch_bf16": "k_dispatch_bf16", "dispatch_mxfp4": "k_dispatch_mxfp4",
                   "combine": "k_combine"}
PROFILES = os.path.join(ROOT, "profiles")


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def stage_bytes(w: workloads.Workload, n_routed: int) -> dict:
    """Algorithmic HBM bytes per stage (what the method must move: x read once
    per real token, only routed rows of the dispatch buffer and of y)."""
    n, r, h, e, k = w.n_rows, w.real_tokens, w.hidden, w.n_experts, w.top_k
    s, v = n * k, n_routed
    return {
        "mask": 4 + (n - r) * k * 4,
        "indices": s * 4 + 2 * s * 4 + (2 * e + 3) * 4,
        "dispatch_bf16": v * 4 + r * h * 2 + v * h * 2,
        "dispatch_mxfp4": v * 4 + r * h * 2 + v * (h // 2 + h // 32),
        "combine": s * 4 + v * 4 + v * h * 2 + n * h * 2,
    }


def source_digest(kernel: str) -> str:
    """Digest of the sources a kernel is built from (to tell stale counters)."""
    csrc = os.path.join(ROOT, "expert_grouping_dispatch_amd", "csrc")
    files = {"k_combine": ["combine.hip", "rows.h", "common.h"],
             "k_dispatch_bf16": ["dispatch.hip", "rows.h", "common.h"],
             "k_dispatch_mxfp4": ["dispatch.hip", "rows.h", "common.h"]}.get(kernel, [])
    hsh = hashlib.sha256()
    for f in files:
        with open(os.path.join(csrc, f), "rb") as fh:
            hsh.update(fh.read())
    return hsh.hexdigest()[:16]


def read_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary of
    this kernel and workload, if it was taken on the current source."""
    path = os.path.join(PROFILES, f"{kernel}_{workload}_pmc.md")
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m_src = re.search(r"source_digest:\s*([0-9a-f]+)", txt)
    m_b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    if not m_src or not m_b or m_src.group(1) != source_digest(kernel):
        return None
    return float(m_b.group(1))


def cpu_baseline(w, cfg, ids, wts, x, y, target_s: float = 20.0):
    """The oracle, as it stands, on a smaller instance of the same workload:
    the first n_s rows (all real), their x rows and the first n_s*k rows of y."""
    import oracle
    import torch

    def run(n_s):
        ids_s = ids[:n_s].copy()
        xb = x[:n_s].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        yb = y[: n_s * w.top_k].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        t0 = time.perf_counter()
        m = oracle.mask_routing_padding(ids_s, n_s)
        r = oracle.create_indices(m, w.n_experts)
        oracle.dispatch(xb, r["token_expert_order"], w.top_k, r["n_routed"])
        oracle.dispatch_mxfp4(xb, r["token_expert_order"], w.top_k, r["n_routed"])
        oracle.combine(yb, wts[:n_s], r["restore_token_order"], w.top_k)
        return time.perf_counter() - t0, r["n_routed"]

    n_s = min(w.real_tokens, 128)   # calibration pass: per-row cost, fixed costs amortised
    dt, v = run(n_s)
    n_s = int(min(w.real_tokens, max(16, n_s * target_s / max(dt, 1e-3))))
    dt, v = run(n_s)
    return {"value": v / dt, "unit": "token-slots/s", "cores": 1, "kind": "oracle",
            "sample": f"first {n_s} real rows of {w.name} (slots {n_s * w.top_k}, H={w.hidden}, "
                      f"E={w.n_experts}, k={w.top_k}), whole path mask+indices+dispatch bf16+MXFP4+combine, "
                      f"{dt:.1f} s, NumPy single-threaded on a {os.cpu_count()}-thread host"}


def time_extensions(torch, moe, w, x, y, d_ids, d_w, idx, n_routed, reps):
    """Event-timed runs of the extension entry points on the same workload,
    outside the step: int64 ids with aligned scale offsets, even-mode and
    packed MXFP4 dispatch, and the combine epilogue with a residual."""
    n, k, h, e = w.n_rows, w.top_k, w.hidden, w.n_experts
    s, v, r = n * k, n_routed, w.real_tokens
    ids64 = d_ids.to(torch.int64)
    ix = moe.alloc_indices(s, e, d_ids.device, scales_offset=True)
    qp, _ = moe.alloc_dispatch_mxfp4(s, h, d_ids.device, packed=True)
    q, sc = moe.alloc_dispatch_mxfp4(s, h, d_ids.device)
    out = torch.empty((n, h), dtype=torch.bfloat16, device=d_ids.device)
    rest = idx["restore_token_order"]
    cases = {
        "indices_i64_scales_offset": (lambda: moe.moe_create_indices(
            ids64, e, ix["token_expert_order"], ix["expert_start_indices"], ix["restore_token_order"],
            ix["expert_ids"], ix["expert_usage_stats"], ix["workspace"], ix["scales_offset"], 128),
            s * 8 + 2 * s * 4 + (3 * e + 4) * 4),
        "dispatch_mxfp4_even": (lambda: moe.moe_dispatch_mxfp4(x, k, rest, q, sc, flags=moe.MXFP4_EVEN_SCALE),
                                v * 4 + r * h * 2 + v * (h // 2 + h // 32)),
        "combine_epilogue_residual": (lambda: moe.moe_combine_epilogue(y, d_w, rest, k, out, 2.5, x),
                                      s * 4 + v * 4 + v * h * 2 + n * h * 2 + n * h * 2),
    }
    if h % 512 == 0:
        cases["dispatch_mxfp4_even_packed"] = (
            lambda: moe.moe_dispatch_mxfp4(x, k, rest, qp, None, flags=moe.MXFP4_EVEN_SCALE | moe.MXFP4_PACKED_ROWS),
            v * 4 + r * h * 2 + v * (h // 2 + h // 32))
    res = {}
    for name, (fn, nbytes) in cases.items():
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / reps
        res[name] = {"ms": round(ms, 4), "bytes": nbytes, "gbps": round(nbytes / (ms * 1e-3) / 1e9, 1)}
    del ix, qp, q, sc, out, ids64
    return res


def copy_ceiling(torch, gib: float = 2.0, reps: int = 10) -> float:
    """Read+write GB/s of a plain device-to-device copy (a measured ceiling)."""
    n = int(gib * (1 << 30))
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        b.copy_(a)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / reps
    del a, b
    return 2 * n / (ms * 1e-3) / 1e9


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="large_prefill_stress", choices=sorted(workloads.BY_NAME))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-copy-ceiling", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="time the step as a HIP graph replay (one launch per step from the host)")
    ap.add_argument("--no-extensions", action="store_true",
                    help="skip timing the extension entry points after the step")
    ap.add_argument("--calib-copy", action="store_true",
                    help="run one 1 GiB device copy before the steps (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this path is measured on one GPU only; --gpus must be 1 "
              "(multi-GPU expert parallelism is not part of this library)", file=sys.stderr)
        sys.exit(2)

    import torch
    import expert_grouping_dispatch_amd as moe

    cfg = [w.name for w in workloads.WORKLOADS].index(args.workload)
    w = workloads.WORKLOADS[cfg]
    n, k, h, e = w.n_rows, w.top_k, w.hidden, w.n_experts
    s = n * k
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    log(f"workload {w.name}: N={n} R={w.real_tokens} H={h} E={e} k={k}")

    ids, wts, real = workloads.make_routing(w, cfg)
    x, y = workloads.make_dense(w, cfg, dev)
    d_src = torch.from_numpy(ids).to(dev)
    d_ids = d_src.clone()
    d_cnt = torch.tensor([real], dtype=torch.int32, device=dev)
    d_w = torch.from_numpy(wts).to(dev)
    idx = moe.alloc_indices(s, e, dev)
    disp = moe.alloc_dispatch(s, h, dev)
    q, sc = moe.alloc_dispatch_mxfp4(s, h, dev)
    comb = torch.empty((n, h), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()
    log("inputs resident")

    def stage_calls():
        return [
            lambda: moe.moe_mask_padding(d_ids, d_cnt, 0),
            lambda: moe.moe_create_indices(d_ids, e, idx["token_expert_order"], idx["expert_start_indices"],
                                           idx["restore_token_order"], idx["expert_ids"],
                                           idx["expert_usage_stats"], idx["workspace"]),
            lambda: moe.moe_dispatch(x, k, idx["restore_token_order"], disp),
            lambda: moe.moe_dispatch_mxfp4(x, k, idx["restore_token_order"], q, sc),
            lambda: moe.moe_combine(y, d_w, idx["restore_token_order"], k, comb),
        ]

    if args.calib_copy:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b
        log("calibration copy of 1073741824 bytes done")

    calls = stage_calls()
    for _ in range(args.warmup):
        for c in calls:
            c()
    torch.cuda.synchronize()
    n_routed = int(idx["expert_start_indices"][idx["expert_usage_stats"][1].to(torch.int64)].item()) \
        if int(idx["expert_usage_stats"][1].item()) > 0 else 0
    log(f"warmup done, routed slots V={n_routed}")

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(STAGES) + 1)] for _ in range(args.steps)]
    graph = None
    if args.graph:
        # stage boundaries are event nodes inside the captured graph
        graph_ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(STAGES) + 1)]
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for c in calls:
                c()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for c in calls:
                c()
        graph.replay()
        torch.cuda.synchronize()
        log("captured the step as one graph")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        if graph is not None:
            ev[i][0].record()
            graph.replay()
            for j in range(1, len(STAGES) + 1):
                ev[i][j].record()
            continue
        for j, c in enumerate(calls):
            ev[i][j].record()
            c()
        ev[i][len(STAGES)].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    stage_ms = {name: float(np.mean([ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(args.steps)]))
                for j, name in enumerate(STAGES)}
    if graph is not None:  # a replay is one unit: per-stage times come from an eager pass of the same step
        eager = [torch.cuda.Event(enable_timing=True) for _ in range(len(STAGES) + 1)]
        for j, c in enumerate(calls):
            eager[j].record()
            c()
        eager[len(STAGES)].record()
        torch.cuda.synchronize()
        stage_ms = {name: eager[j].elapsed_time(eager[j + 1]) for j, name in enumerate(STAGES)}
    step_ms = float(np.mean([ev[i][0].elapsed_time(ev[i][len(STAGES)]) for i in range(args.steps)]))
    span_ms = ev[0][0].elapsed_time(ev[-1][len(STAGES)]) / args.steps
    log(f"timed {args.steps} steps: {step_ms:.3f} ms/step (events), span {span_ms:.3f}, wall {wall / args.steps * 1e3:.3f}")

    bts = stage_bytes(w, n_routed)
    step_bytes = sum(bts.values())
    ms_per_step = span_ms
    value = n_routed / (ms_per_step * 1e-3)
    gbps = step_bytes / (ms_per_step * 1e-3) / 1e9
    stages = {name: {"ms": round(stage_ms[name], 4), "bytes": bts[name],
                     "gbps": round(bts[name] / (stage_ms[name] * 1e-3) / 1e9, 1)} for name in STAGES}
    pipelines = {}
    for pname, disp_stage in (("bf16", "dispatch_bf16"), ("mxfp4", "dispatch_mxfp4")):
        names = ("mask", "indices", disp_stage, "combine")
        t = sum(stage_ms[nm] for nm in names)
        b = sum(bts[nm] for nm in names)
        pipelines[pname] = {"ms": round(t, 4), "slots_per_s": n_routed / (t * 1e-3),
                            "gbps": round(b / (t * 1e-3) / 1e9, 1),
                            "frac_of_peak": round(b / (t * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}

    dom = max(KERNEL_OF_STAGE, key=lambda nm: stage_ms[nm])
    kern = KERNEL_OF_STAGE[dom]
    achieved = bts[dom] / (stage_ms[dom] * 1e-3) / 1e9
    roofline = {"bound": "hbm", "kernel": kern, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": read_traffic(kern, w.name), "algorithmic_bytes_per_launch": bts[dom],
                "avg_launch_ms": round(stage_ms[dom], 4)}

    extensions = None if args.no_extensions else time_extensions(torch, moe, w, x, y, d_ids, d_w, idx, n_routed,
                                                                 args.steps)
    copy_gbps = None if args.no_copy_ceiling else copy_ceiling(torch)
    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        cpu = cpu_baseline(w, cfg, ids, wts, x, y)

    out = {
        "metric": METRIC, "value": value, "unit": "token-slots/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": w.name, "n_rows": n, "real_token_count": real, "hidden": h, "n_experts": e,
                   "top_k": k, "routing": w.routing,
                   "step": "mask+create_indices+dispatch_bf16+dispatch_mxfp4+combine"},
        "gbps": round(gbps, 1), "frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4),
        "copy_ceiling_gbps": None if copy_gbps is None else round(copy_gbps, 1),
        "stages": stages, "pipelines": pipelines, "graph_replay": bool(args.graph),
        "extensions": extensions, "roofline": roofline, "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
