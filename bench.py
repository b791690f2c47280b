#!/usr/bin/env python3
"""Benchmark of the MoE token-routing path on one MI355X.

One step = the whole path over one batch of the chosen workload:
    moe_mask_create_indices (mask + indices, one call) -> moe_dispatch (bf16)
    -> moe_dispatch_mxfp4 -> moe_combine
with inputs resident in HBM.  Stage times also cover moe_mask_padding and
moe_create_indices as separate calls.  Prints ONE JSON line on stdout (progress goes
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
ROW_STAGES = ("dispatch_bf16", "dispatch_mxfp4", "combine")


def kernel_of_stage(stage: str, w) -> str:
    """Name of the kernel the library launches for a row stage on workload w
    (a label for the roofline line and the profile it is checked against).
    top_k <= 8 takes the loop-free bf16 dispatch; combine takes it too when
    the routed rows of y are under 1 GiB, whole-row workgroups otherwise;
    MXFP4 outputs of at least 256 MiB with top_k <= 8 take the
    four-lanes-per-block kernel."""
    if stage == "dispatch_mxfp4":
        out_bytes = w.n_rows * w.top_k * (w.hidden // 32) * 17
        return "k_dispatch_mxfp4_quad" if w.top_k <= 8 and out_bytes >= (256 << 20) else "k_dispatch_mxfp4"
    if w.top_k > 8:
        return "k_dispatch_bf16" if stage == "dispatch_bf16" else "k_combine"
    if stage == "dispatch_bf16":
        return "k_dispatch_bf16_parts"
    return "k_combine_parts" if w.n_rows * w.top_k * w.hidden * 2 < (1 << 30) else "k_combine"
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
    """Digest of the code a kernel is built from (to tell stale counters):
    its sources with comments and whitespace removed, so that only a change
    of code, not of its comments, marks the counters as stale."""
    csrc = os.path.join(ROOT, "expert_grouping_dispatch_amd", "csrc")
    files = (["combine.hip", "rows.h", "common.h"] if kernel.startswith("k_combine") else
             ["dispatch_mxfp4.hip", "rows.h", "common.h"] if kernel.startswith("k_dispatch_mxfp4") else
             ["dispatch.hip", "rows.h", "common.h"] if kernel.startswith("k_dispatch") else [])
    hsh = hashlib.sha256()
    for f in files:
        with open(os.path.join(csrc, f), encoding="utf-8") as fh:
            code = re.sub(r"/\*.*?\*/", " ", fh.read(), flags=re.S)
        code = re.sub(r"//[^\n]*", " ", code)
        hsh.update("".join(code.split()).encode())
    return hsh.hexdigest()[:16]


def library_digest() -> str:
    """Digest of every library source (comments and whitespace removed), so
    that a recorded bench line can be matched with the code it measured."""
    csrc = os.path.join(ROOT, "expert_grouping_dispatch_amd", "csrc")
    hsh = hashlib.sha256()
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".h")):
            with open(os.path.join(csrc, f), encoding="utf-8") as fh:
                code = re.sub(r"/\*.*?\*/", " ", fh.read(), flags=re.S)
            code = re.sub(r"//[^\n]*", " ", code)
            hsh.update(f.encode() + b"\0" + "".join(code.split()).encode())
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


def cpu_baseline(w, cfg, ids, wts, x, y, gpu=None, target_s: float = 20.0):
    """The oracle, as it stands, on a smaller instance of the same workload:
    the first n_s rows (all real), their x rows and the first n_s*k rows of y.
    With `gpu` (this run's device outputs) it also checks them against the
    oracle on the full routing map and on sampled tokens."""
    import oracle
    import torch

    def run(n_s):
        ids_s = ids[:n_s].copy()
        xb = x[:n_s].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        yb = y[: n_s * w.top_k].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        t0, c0 = time.perf_counter(), time.process_time()
        m = oracle.mask_routing_padding(ids_s, n_s)
        r = oracle.create_indices(m, w.n_experts)
        oracle.dispatch(xb, r["token_expert_order"], w.top_k, r["n_routed"])
        oracle.dispatch_mxfp4(xb, r["token_expert_order"], w.top_k, r["n_routed"])
        oracle.combine(yb, wts[:n_s], r["restore_token_order"], w.top_k)
        return time.perf_counter() - t0, r["n_routed"], time.process_time() - c0

    n_s = min(w.real_tokens, 128)   # calibration pass: per-row cost, fixed costs amortised
    dt, v, _ = run(n_s)
    n_s = int(min(w.real_tokens, max(16, n_s * target_s / max(dt, 1e-3))))
    dt, v, cpu_s = run(n_s)
    sw = workloads.scaled(w, n_rows=n_s, real_tokens=n_s)
    nbytes = sum(stage_bytes(sw, v).values())
    # cores actually used: process CPU time over wall time of the timed sample (~1: NumPy's
    # element-wise and sort routines run on one thread)
    res = {"value": v / dt, "unit": "token-slots/s", "cores": max(1, round(cpu_s / dt)), "kind": "oracle",
           "cpu_time_over_wall": round(cpu_s / dt, 3), "gbps": round(nbytes / dt / 1e9, 4),
           "sample": f"first {n_s} real rows of {w.name} (slots {n_s * w.top_k}, H={w.hidden}, "
                     f"E={w.n_experts}, k={w.top_k}), whole path mask+indices+dispatch bf16+MXFP4+combine, "
                     f"{dt:.1f} s, NumPy single-threaded on a {os.cpu_count()}-thread host"}
    if gpu is not None:
        res["parity_of_this_run"] = parity_sample(oracle, torch, w, ids, wts, x, y, gpu)
    return res


def parity_sample(oracle, torch, w, ids, wts, x, y, gpu, n_tok: int = 48):
    """This run's device outputs against the oracle: the masked map and every
    index output in full; dispatch (bf16, MXFP4) and combine rows of seeded
    sampled tokens, real and padding."""
    k, h = w.top_k, w.hidden

    def u16(t):
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)

    def u32(t):
        return t.contiguous().view(torch.int32).cpu().numpy().view(np.uint32)

    m = oracle.mask_routing_padding(ids, w.real_tokens)
    ok = {"mask": bool(np.array_equal(gpu["ids"].cpu().numpy(), m))}
    ref = oracle.create_indices(m, w.n_experts)
    idx = gpu["idx"]
    ok["indices"] = all(
        np.array_equal(u32(idx[key]), ref[key].astype(np.uint32))
        for key in ("token_expert_order", "expert_start_indices", "restore_token_order", "expert_usage_stats")) \
        and np.array_equal(idx["expert_ids"].cpu().numpy(), ref["expert_ids"].astype(np.int32))
    g = np.random.default_rng(12345)
    toks = np.unique(np.concatenate([g.integers(0, w.real_tokens, n_tok),
                                     g.integers(0, w.n_rows, max(1, n_tok // 8))]))
    rest = ref["restore_token_order"].reshape(w.n_rows, k)[toks]
    routed = rest != oracle.SENT
    xs = u16(x[torch.from_numpy(toks).to(x.device)])
    pos = torch.from_numpy(rest[routed].astype(np.int64)).to(x.device)
    src = np.repeat(np.arange(len(toks)), k).reshape(-1, k)[routed]
    ok["dispatch_bf16"] = bool(np.array_equal(u16(gpu["disp"][pos]), xs[src]))
    pq, ps = oracle.mxfp4_quantize(xs)
    ok["dispatch_mxfp4"] = bool(np.array_equal(gpu["q"][pos].cpu().numpy(), pq[src])
                                and np.array_equal(gpu["sc"][pos].cpu().numpy(), ps[src]))
    # combine over the sampled tokens: their y rows, gathered at the oracle's positions
    ys = u16(y[pos]) if pos.numel() else np.zeros((0, h), np.uint16)
    mini = np.full(rest.shape, oracle.SENT, np.uint32)
    mini[routed] = np.arange(int(routed.sum()), dtype=np.uint32)
    want = oracle.combine(ys, wts[toks], mini.reshape(-1), k)
    got = u16(gpu["comb"][torch.from_numpy(toks).to(x.device)])
    ok["combine"] = bool(np.array_equal(got, want))
    ok["index_error_word_clear"] = int(idx["workspace"][:4].view(torch.int32).item()) == 0
    ok["tokens_sampled"] = int(len(toks))
    ok["all"] = all(v for key, v in ok.items() if key != "tokens_sampled")
    return ok


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


def time_pipelines(torch, calls, bts, n_routed, steps, warmup, scrub, fused_front):
    """Each single-format pipeline (the one-call mask + indices -> one
    dispatch -> combine) run as its own loop of `steps` passes, events around
    each pass (and around every stage in a second loop, for the stage times).
    A stage's writes can still be draining from the memory-side cache when
    the next kernel starts, so only a pipeline's own loop charges it what it
    leaves behind.  The *_separate_front lines take the mask and the indices
    as two calls (calls[0], calls[1]) instead."""
    res = {}
    plans = [("bf16", [("mask_indices", fused_front), ("dispatch_bf16", calls[2]), ("combine", calls[4])]),
             ("mxfp4", [("mask_indices", fused_front), ("dispatch_mxfp4", calls[3]), ("combine", calls[4])]),
             ("bf16_separate_front", [(STAGES[j], calls[j]) for j in (0, 1, 2, 4)]),
             ("mxfp4_separate_front", [(STAGES[j], calls[j]) for j in (0, 1, 3, 4)])]
    bts = dict(bts, mask_indices=bts["mask"] + bts["indices"])
    for pname, plan in plans:
        names = [nm for nm, _ in plan]
        fns = [f for _, f in plan]
        for _ in range(warmup):
            for f in fns:
                f()
        torch.cuda.synchronize()
        # totals with events at the ends of each pass only; stage times from a second loop
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
        for i in range(steps):
            if scrub is not None:
                scrub()
            ev[i][0].record()
            for f in fns:
                f()
            ev[i][1].record()
        torch.cuda.synchronize()
        per = [ev[i][0].elapsed_time(ev[i][1]) for i in range(steps)]
        ms = float(np.mean(per)) if scrub is not None else ev[0][0].elapsed_time(ev[-1][1]) / steps
        n_stage = min(steps, 50)
        sev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(fns) + 1)] for _ in range(n_stage)]
        for i in range(n_stage):
            if scrub is not None:
                scrub()
            for j, f in enumerate(fns):
                sev[i][j].record()
                f()
            sev[i][len(fns)].record()
        torch.cuda.synchronize()
        b = sum(bts[nm] for nm in names)
        st = {nm: round(float(np.mean([sev[i][j].elapsed_time(sev[i][j + 1]) for i in range(n_stage)])), 4)
              for j, nm in enumerate(names)}
        res[pname] = {"ms": round(ms, 4), "ms_median": round(float(np.median(per)), 4),
                      "ms_min": round(float(np.min(per)), 4), "slots_per_s": n_routed / (ms * 1e-3), "bytes": b,
                      "gbps": round(b / (ms * 1e-3) / 1e9, 1),
                      "frac_of_peak": round(b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4), "stage_ms": st}
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
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default: 20 on the stress workload, 200 on the mid-size ones, "
                         "1000 on the latency-bound tiny and decode workloads)")
    ap.add_argument("--warmup", type=int, default=None, help="warm-up steps (default: 3, or 10 below stress size)")
    ap.add_argument("--workload", default="large_prefill_stress", choices=sorted(workloads.BY_NAME))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-copy-ceiling", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="time the step as a HIP graph replay (one launch per step from the host)")
    ap.add_argument("--no-extensions", action="store_true",
                    help="skip timing the extension entry points after the step")
    ap.add_argument("--calib-copy", action="store_true",
                    help="run one 1 GiB device copy before the steps (counter calibration)")
    ap.add_argument("--scrub", choices=("auto", "on", "off"), default="auto",
                    help="read a 1 GiB buffer between steps, outside the timed events, so that no step "
                         "finds its inputs in L2 or the 256 MB Infinity Cache (auto: when the working "
                         "set is under 1 GiB)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this path is measured on one GPU only; --gpus must be 1 "
              "(multi-GPU expert parallelism is not part of this library)", file=sys.stderr)
        sys.exit(2)

    import torch
    import expert_grouping_dispatch_amd as moe

    cfg = [w.name for w in workloads.WORKLOADS].index(args.workload)
    w = workloads.WORKLOADS[cfg]
    if args.steps is None:
        args.steps = {"large_prefill_stress": 20, "tiny": 1000, "decode": 1000}.get(w.name, 200)
    if args.warmup is None:
        args.warmup = 3 if w.name == "large_prefill_stress" else 10
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
    work_set = sum(t.numel() * t.element_size() for t in (x, y, d_ids, d_w, disp, q, sc, comb)) + \
        sum(t.numel() * t.element_size() for t in idx.values() if t is not None)
    scrub = None
    if args.scrub == "on" or (args.scrub == "auto" and work_set < (1 << 30)):
        scrub_buf = torch.empty(1 << 28, dtype=torch.int32, device=dev)

        def scrub():  # a read of 1 GiB evicts L2 and Infinity Cache and leaves no dirty lines
            scrub_buf.max()
    torch.cuda.synchronize()
    log(f"inputs resident, working set {work_set / 2 ** 20:.1f} MiB, scrub between steps: {scrub is not None}")

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

    def fused_front():
        moe.moe_mask_create_indices(d_ids, d_cnt, 0, e, idx["token_expert_order"], idx["expert_start_indices"],
                                    idx["restore_token_order"], idx["expert_ids"], idx["expert_usage_stats"],
                                    idx["workspace"])

    calls = stage_calls()                      # the five entry points one by one (stage times)
    step_calls = [fused_front] + calls[2:]     # the step: mask + indices in one call
    for _ in range(args.warmup):
        for c in calls:
            c()
        for c in step_calls:
            c()
    torch.cuda.synchronize()
    n_routed = int(idx["expert_start_indices"][idx["expert_usage_stats"][1].to(torch.int64)].item()) \
        if int(idx["expert_usage_stats"][1].item()) > 0 else 0
    log(f"warmup done, routed slots V={n_routed}")

    graph = None
    if args.graph:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for c in step_calls:
                c()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for c in step_calls:
                c()
        graph.replay()
        torch.cuda.synchronize()
        log("captured the step as one graph")
    torch.cuda.synchronize()
    # the timed steps carry events at their two ends only: an event recorded
    # between two kernels costs a few microseconds of queue processing, which
    # latency-bound steps would otherwise be charged
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        if scrub is not None:
            scrub()
        ev[i][0].record()
        if graph is not None:
            graph.replay()
        else:
            for c in step_calls:
                c()
        ev[i][1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_step = [ev[i][0].elapsed_time(ev[i][1]) for i in range(args.steps)]
    step_ms = float(np.mean(per_step))
    span_ms = ev[0][0].elapsed_time(ev[-1][1]) / args.steps
    log(f"timed {args.steps} steps: {step_ms:.3f} ms/step (events), span {span_ms:.3f}, wall {wall / args.steps * 1e3:.3f}")
    # per-stage times from a separate eager loop with an event before every stage
    n_stage = min(args.steps, 50)
    sev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(STAGES) + 1)] for _ in range(n_stage)]
    for i in range(n_stage):
        if scrub is not None:
            scrub()
        for j, c in enumerate(calls):
            sev[i][j].record()
            c()
        sev[i][len(STAGES)].record()
    torch.cuda.synchronize()
    stage_ms = {name: float(np.mean([sev[i][j].elapsed_time(sev[i][j + 1]) for i in range(n_stage)]))
                for j, name in enumerate(STAGES)}

    bts = stage_bytes(w, n_routed)
    step_bytes = sum(bts.values())
    # back-to-back steps: the span; scrubbed steps: the mean of the per-step times
    ms_per_step = span_ms if scrub is None else step_ms
    value = n_routed / (ms_per_step * 1e-3)
    gbps = step_bytes / (ms_per_step * 1e-3) / 1e9
    stages = {name: {"ms": round(stage_ms[name], 4), "bytes": bts[name],
                     "gbps": round(bts[name] / (stage_ms[name] * 1e-3) / 1e9, 1)} for name in STAGES}
    # HBM bytes the counters measured per launch (committed profiles taken on
    # the current sources), next to the algorithmic figures
    for name in ROW_STAGES:
        counted = read_traffic(kernel_of_stage(name, w), w.name)
        if counted is not None:
            stages[name]["counter_bytes"] = counted
            stages[name]["counter_gbps"] = round(counted / (stage_ms[name] * 1e-3) / 1e9, 1)
    pipelines = time_pipelines(torch, calls, bts, n_routed, args.steps, args.warmup, scrub, fused_front)
    mi = pipelines["bf16"]["stage_ms"]["mask_indices"]  # the one-call front, as the step runs it
    stages["mask_indices"] = {"ms": mi, "bytes": bts["mask"] + bts["indices"],
                              "gbps": round((bts["mask"] + bts["indices"]) / (mi * 1e-3) / 1e9, 1)}
    for pname, pl in pipelines.items():
        log(f"{pname} pipeline: {pl['ms']:.3f} ms/pass, {pl['gbps']} GB/s ({pl['frac_of_peak'] * 100:.1f}% of peak)")

    dom = max(ROW_STAGES, key=lambda nm: stage_ms[nm])
    kern = kernel_of_stage(dom, w)
    achieved = bts[dom] / (stage_ms[dom] * 1e-3) / 1e9
    traffic = read_traffic(kern, w.name)
    roofline = {"bound": "hbm", "kernel": kern, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": traffic, "algorithmic_bytes_per_launch": bts[dom],
                "avg_launch_ms": round(stage_ms[dom], 4),
                "traffic_gbps": None if traffic is None else round(traffic / (stage_ms[dom] * 1e-3) / 1e9, 1)}

    extensions = None if args.no_extensions else time_extensions(torch, moe, w, x, y, d_ids, d_w, idx, n_routed,
                                                                 args.steps)
    copy_gbps = None if args.no_copy_ceiling else copy_ceiling(torch)
    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        cpu = cpu_baseline(w, cfg, ids, wts, x, y,
                           gpu=dict(ids=d_ids, idx=idx, disp=disp, q=q, sc=sc, comb=comb))
        log(f"parity of this run against the oracle: {cpu['parity_of_this_run']}")

    out = {
        "metric": METRIC, "value": value, "unit": "token-slots/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": w.name, "n_rows": n, "real_token_count": real, "hidden": h, "n_experts": e,
                   "top_k": k, "routing": w.routing,
                   "step": "mask_create_indices+dispatch_bf16+dispatch_mxfp4+combine"},
        "gbps": round(gbps, 1), "frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4),
        "step_ms_median": round(float(np.median(per_step)), 4), "step_ms_min": round(float(np.min(per_step)), 4),
        "scrub_between_steps": scrub is not None,
        "copy_ceiling_gbps": None if copy_gbps is None else round(copy_gbps, 1),
        "frac_of_copy_ceiling": None if copy_gbps is None else round(gbps / copy_gbps, 4),
        "stages": stages, "pipelines": pipelines, "graph_replay": bool(args.graph),
        "extensions": extensions, "roofline": roofline, "cpu_baseline": cpu,
        "library_digest": library_digest(),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
