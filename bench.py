#!/usr/bin/env python3
"""Benchmark of the context-parallel decode combine on one MI355X.

One step = the whole hot path over one batch: per-shard split-KV decode
attention, the merge of each shard's chunks and the cross-shard LSE merge.
By default a step is one cpdec_cp_decode call (one kernel launch when the
shape allows it); --two-calls times cpdec_attn_partial followed by
cpdec_lse_merge instead.  The merge-only workload (c5) runs cpdec_lse_merge
alone.  Inputs are synthetic, seeded, and resident in HBM before the timed
region starts.

Prints ONE JSON line:
  value          eager microseconds per call (wall clock of K back-to-back
                 steps launched from Python / K)
  roofline       the dominant kernel (the step's attention kernel, which
                 also merges when the step is one launch; the merge kernel
                 for c5): algorithmic bytes per launch / its mean duration
                 from HIP events recorded around its launches on every 8th
                 step of the timed region, against MI355X's 8 TB/s HBM peak
                 (when the step takes several launches the span covers them
                 all); `traffic` is filled from the committed rocprofv3
                 counter summary when it was taken on the current kernel
                 source, else null
  cpu_baseline   the CPU oracle timed on this host on a bounded sample of the
                 same workload, scaled to microseconds per call

Workloads smaller than the 256 MB Infinity Cache rotate through enough input
copies that a step never finds its inputs cache-resident.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

from synth import configs as sc  # noqa: E402

METRIC = "merge+partial-attn µs/call and achieved HBM GB/s (% of peak) on 1 MI355X"
HBM_PEAK_GBPS = 8000.0
MALL_BYTES = 256 << 20
PROFILE_DIR = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = ["lse_merge_split_amd/csrc/attn_partial.hip", "lse_merge_split_amd/csrc/lse_merge.hip",
                  "lse_merge_split_amd/csrc/device_common.h", "lse_merge_split_amd/csrc/kernels.h"]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# ------------------------------------------------------------------ bytes
def attn_alg_bytes(w: sc.Workload, lens: np.ndarray, o_elem: int = 4) -> int:
    """K and V of every valid token once (shared by the G heads), q once,
    o_part + lse_part written once."""
    e = 2
    kv = int(lens.astype(np.int64).sum()) * w.Hkv * 2 * w.D * e
    q = w.B * w.Hq * w.D * e
    o = w.R * w.B * w.Hq * (w.D * o_elem + 4)
    return kv + q + o


def merge_alg_bytes(R: int, rows: int, D: int, live: int, in_elem: int, out_elem: int) -> int:
    """o_part rows of live (finite-lse) shards, every lse once, out + lse_out."""
    return live * D * in_elem + R * rows * 4 + rows * (D * out_elem + 4)


# ------------------------------------------------------------------ GPU setup
def build_attn_steps(w: sc.Workload, torch, cp, sg, fused: bool = True):
    inp = sg.attn_inputs(w)
    lens = inp["lens_np"]
    per_copy = 2 * inp["k"].numel() * inp["k"].element_size()
    copies = 1
    if per_copy < MALL_BYTES:
        copies = min(16, max(1, math.ceil(3 * MALL_BYTES / per_copy)))
    sets = [inp]
    for _ in range(copies - 1):
        k2, v2, q2 = inp["k"].clone(), inp["v"].clone(), inp["q"].clone()
        sets.append(dict(q=q2, k=k2, v=v2, lens=inp["lens"],
                         k_shards=[k2[r] for r in range(w.R)], v_shards=[v2[r] for r in range(w.R)]))
    o_part = torch.empty((w.R, w.B, w.Hq, w.D), dtype=torch.float32, device="cuda")
    lse_part = torch.empty((w.R, w.B, w.Hq), dtype=torch.float32, device="cuda")
    out = torch.empty((w.B, w.Hq, w.D), dtype=inp["q"].dtype, device="cuda")
    lse_out = torch.empty((w.B, w.Hq), dtype=torch.float32, device="cuda")
    steps = []
    for s in sets:
        if fused:  # cpdec_cp_decode: the whole step as one call
            a = cp.StepCall(s["q"], s["k_shards"], s["v_shards"], s["lens"], o_part, lse_part,
                            out, lse_out)
            m = None
        else:
            a = cp.AttnCall(s["q"], s["k_shards"], s["v_shards"], s["lens"], o_part, lse_part)
            m = cp.MergeCall(o_part, lse_part, out, lse_out)
        steps.append((a, m))
    alg_attn = attn_alg_bytes(w, lens)
    live_rows = int((np.repeat(lens[:, :, None] > 0, w.Hq, axis=2)).sum())
    alg_merge = merge_alg_bytes(w.R, w.B * w.Hq, w.D, live_rows, 4, 2)
    info = dict(copies=copies, chunk=steps[0][0].plan["chunk_tokens"],
                nchunks=steps[0][0].plan["num_chunks"], waves=steps[0][0].plan["waves"],
                workspace_bytes=steps[0][0].workspace_bytes,
                longest_first=steps[0][0].plan["longest_first"],
                attn_launches=steps[0][0].plan["launches"],
                launches=(steps[0][0].launches if fused else steps[0][0].plan["launches"] + 1))
    return steps, alg_attn, alg_merge, info


def build_merge_steps(w: sc.Workload, torch, cp, sg):
    inp = sg.merge_inputs(w)
    out = torch.empty((w.rows, w.D), dtype=torch.bfloat16, device="cuda")
    lse_out = torch.empty(w.rows, dtype=torch.float32, device="cuda")
    steps = [(None, cp.MergeCall(inp["o_part"], inp["lse_part"], out, lse_out))]
    live = int(np.isfinite(inp["lse_np"]).sum())
    alg = merge_alg_bytes(w.R, w.rows, w.D, live, 2, 2)
    return steps, 0, alg, dict(copies=1, _keep=inp)


# ------------------------------------------------------------------ CPU baseline
def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
        return max(n) if n else 1
    except Exception:
        return 1


def cpu_baseline(w: sc.Workload, budget_s: float):
    """Time the CPU oracle on a bounded sample of the workload; inputs are
    generated before the clock starts."""
    from oracle import oracle as orc
    cores = blas_threads()
    if w.merge_only:
        nrows = 2048
        rows = np.random.default_rng(0).choice(w.rows, size=nrows, replace=False)
        lse = sc.merge_lse(w)[:, rows]
        o = np.stack([np.stack([sc.merge_opart_values(w, r, int(n), 1)[0] for n in rows])
                      for r in range(w.R)]).astype(np.float64)
        t0 = time.perf_counter()
        reps = 0
        while True:
            orc.merge_rows(o, lse)
            reps += 1
            if time.perf_counter() - t0 >= budget_s or reps >= 50:
                break
        per = (time.perf_counter() - t0) / reps
        us = per * (w.rows / nrows) * 1e6
        sample = (f"{nrows} random rows of {w.rows} ({w.R} shards, D={w.D}), oracle merge "
                  f"repeated {reps}x, scaled linearly to all rows")
        return dict(value=us, unit="µs/call", cores=cores, kind="oracle", sample=sample)

    lens = sc.lens(w)
    groups = [(b, h) for b in range(w.B) for h in range(w.Hkv)]
    # bounded sample: at most ~40M K/V elements generated for the oracle
    per_group = max(1, int(lens.sum(axis=0).mean()) * w.D * 2)
    ng = max(1, min(len(groups), (40_000_000 // per_group)))
    rng = np.random.default_rng(1)
    pick = [groups[i] for i in sorted(rng.choice(len(groups), size=ng, replace=False))]
    data = []
    for (b, h) in pick:
        qg = sc.q_rows(w, b, h * w.G, w.G).astype(np.float64)
        kv = [(sc.kv_values(w, "k", r, b, h, int(lens[r, b])).astype(np.float64),
               sc.kv_values(w, "v", r, b, h, int(lens[r, b])).astype(np.float64))
              for r in range(w.R)]
        data.append((qg, kv))
    t0 = time.perf_counter()
    reps = 0
    while True:
        for qg, kv in data:
            parts = [orc.attend_shard(qg, k, v, w.sm_scale) for (k, v) in kv]
            o_p = np.stack([p[0] for p in parts])
            l_p = np.stack([p[1] for p in parts])
            for g in range(w.G):
                orc.merge(o_p[:, g], l_p[:, g])
        reps += 1
        if time.perf_counter() - t0 >= budget_s or reps >= 200:
            break
    per = (time.perf_counter() - t0) / reps
    us = per * (len(groups) / ng) * 1e6
    sample = (f"{ng} of {len(groups)} (sequence, kv head) groups, all {w.R} shards each, oracle "
              f"attention + merge repeated {reps}x, scaled linearly to the whole batch; "
              f"host os.cpu_count()={os.cpu_count()}")
    return dict(value=us, unit="µs/call", cores=cores, kind="oracle", sample=sample)


# ------------------------------------------------------------------ traffic
def committed_traffic(workload: str, kernel: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary,
    if it was taken on the current kernel sources; else None."""
    path = os.path.join(PROFILE_DIR, f"{kernel}_{workload}_hbm_counters.json")
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            d = json.load(f)
        if d.get("kernel_source_hash") != kernel_source_hash():
            return None
        return d.get("traffic_bytes_per_launch")
    except Exception:
        return None


# ------------------------------------------------------------------ main
def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="c2", choices=sorted(sc.WORKLOADS))
    ap.add_argument("--cpu-budget-s", type=float, default=12.0,
                    help="seconds of oracle work for cpu_baseline (0 disables it)")
    ap.add_argument("--graph", action="store_true", help="also time HIP-graph replay of a step")
    ap.add_argument("--two-calls", action="store_true",
                    help="time cpdec_attn_partial + cpdec_lse_merge instead of one "
                         "cpdec_cp_decode call per step")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run a plain 1 GiB device copy after the timed region (counter scaling)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported: the path "
              "here is one GPU's share of the work and has no cross-GPU step.", file=sys.stderr)
        sys.exit(2)

    import torch
    import lse_merge_split_amd as cp
    from synth import gpu as sg

    w = sc.WORKLOADS[args.workload]
    torch.cuda.set_device(0)
    if w.merge_only:
        steps, alg_attn, alg_merge, info = build_merge_steps(w, torch, cp, sg)
        K = args.steps or 100
    else:
        steps, alg_attn, alg_merge, info = build_attn_steps(w, torch, cp, sg,
                                                            fused=not args.two_calls)
        K = args.steps or (200 if alg_attn < (1 << 30) else 20)
    W = args.warmup
    torch.cuda.synchronize()
    print(f"[bench] workload {w.name}: {w.note}; copies={info['copies']} steps={K} warmup={W}",
          file=sys.stderr, flush=True)

    stream = torch.cuda.current_stream().cuda_stream  # every call goes on this stream

    def step(i, ev=None):
        a, m = steps[i % len(steps)]
        if a is not None:
            if ev is not None:
                ev[0].record()
            a(stream)
        if ev is not None and (m is not None or a is not None):
            ev[1].record()
        if m is not None:
            m(stream)
            if ev is not None:
                ev[2].record()

    for i in range(W):
        step(i)
    torch.cuda.synchronize()

    # HIP events bracket the kernels of every EVERY-th timed step (each event
    # record costs a few microseconds of device time, so bracketing every step
    # would inflate the per-step time of the small workloads; a one-call step
    # takes two events).
    EVERY = 16
    sampled = list(range(0, K, EVERY))
    evs = {i: [torch.cuda.Event(enable_timing=True) for _ in range(3)] for i in sampled}
    edge = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    edge[0].record()
    for i in range(K):
        step(i, evs.get(i))
    edge[1].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    print(f"[bench] timed {K} steps", file=sys.stderr, flush=True)

    us_per_call = (t1 - t0) / K * 1e6
    attn_us = (float(np.mean([evs[i][0].elapsed_time(evs[i][1]) for i in sampled])) * 1e3
               if not w.merge_only else None)
    fused = not w.merge_only and not args.two_calls
    merge_us = (float(np.mean([evs[i][1].elapsed_time(evs[i][2]) for i in sampled])) * 1e3
                if not fused else None)
    device_us = edge[0].elapsed_time(edge[1]) * 1e3 / K

    if w.merge_only:
        dom_name, dom_us, dom_bytes, kernel = "lse_merge_kernel", merge_us, alg_merge, "lse_merge"
    elif fused:  # the event span covers the whole step
        rows = w.B * w.Hq
        step_bytes = alg_attn + rows * (w.D * 2 + 4)  # + out and lse_out written once
        dom_name = ("attn_partial_kernel (whole step, one launch)" if info["launches"] == 1 else
                    f"cpdec_cp_decode ({info['launches']} launches)")
        dom_us, dom_bytes, kernel = attn_us, step_bytes, "attn_partial"
    else:
        dom_name, dom_us, dom_bytes, kernel = "attn_partial_kernel", attn_us, alg_attn, "attn_partial"
    # A step that is one kernel launch (the merge alone, or the whole step in
    # one launch): its mean duration is the span of the events around all K
    # back-to-back launches divided by K, free of the per-sample event cost.
    single_launch = w.merge_only or (fused and info["launches"] == 1)
    dom_timing = "events around the K timed launches" if single_launch else \
        f"events around the launches of every {EVERY}th step"
    if single_launch:
        dom_us = device_us
    achieved = dom_bytes / (dom_us * 1e-6) / 1e9
    traffic = committed_traffic(w.name, kernel)

    graph_us = graph_device_us = None
    if args.graph:
        # One graph per input copy, replayed in the same rotation as the eager
        # steps, so a replay finds its inputs no more cache-resident than an
        # eager step does.
        graphs = []
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        for a, m in steps:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.stream(side):
                with torch.cuda.graph(g):
                    cs = torch.cuda.current_stream().cuda_stream  # the capture stream
                    if a is not None:
                        a(cs)
                    if m is not None:
                        m(cs)
            graphs.append(g)
        torch.cuda.synchronize()
        for i in range(W):
            graphs[i % len(graphs)].replay()
        torch.cuda.synchronize()
        gedge = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        tg0 = time.perf_counter()
        gedge[0].record()
        for i in range(K):
            graphs[i % len(graphs)].replay()
        gedge[1].record()
        torch.cuda.synchronize()
        graph_us = (time.perf_counter() - tg0) / K * 1e6
        graph_device_us = gedge[0].elapsed_time(gedge[1]) * 1e3 / K
        del graphs

    if args.calibrate_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(1)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print("[bench] calibration copy: 1073741824 bytes read, 1073741824 written",
              file=sys.stderr, flush=True)

    cpu = None
    if args.cpu_budget_s > 0:
        print("[bench] timing the CPU oracle baseline", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w, args.cpu_budget_s)

    # algorithmic bytes of the whole step: the two-call form also writes and
    # re-reads o_part between its calls
    step_bytes = dom_bytes if fused else alg_attn + alg_merge
    line = {
        "metric": METRIC,
        "value": round(us_per_call, 3),
        "unit": "µs/call",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(us_per_call / 1e3, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f16",
        "data": "synthetic (seeded Philox streams; no dataset)",
        "config": {"workload": f"{w.name}: {w.note}",
                   "entry": ("cpdec_lse_merge" if w.merge_only else
                             "cpdec_cp_decode" if fused else "cpdec_attn_partial + cpdec_lse_merge"),
                   "launches_per_step": info.get("launches", 1),
                   "R": w.R, "B": w.B or None,
                   "Hq": w.Hq or None, "Hkv": w.Hkv or None, "D": w.D,
                   "rows": w.rows or None, "input_copies": info["copies"],
                   "chunk_tokens": info.get("chunk"), "chunks_per_shard": info.get("nchunks"),
                   "waves_per_workgroup": info.get("waves"),
                   "longest_first": info.get("longest_first"), "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": dom_name + (" + attn_combine_kernel" if not fused
                                                           and not w.merge_only
                                                           and info.get("nchunks", 1) > 1
                                                           and info.get("attn_launches", 1) >
                                                           1 + int(bool(info.get("longest_first")))
                                                           else "")
                     + (" + order_kernel" if info.get("longest_first") and not fused else ""),
                     "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic, "alg_bytes_per_launch": dom_bytes,
                     "mean_launch_us": round(dom_us, 3), "timing": dom_timing,
                     "event_samples": len(sampled)},
        "cpu_baseline": cpu,
        "attn_us": round(attn_us, 3) if attn_us is not None else None,
        "merge_us": round(merge_us, 3) if merge_us is not None else None,
        "device_us_per_call": round(device_us, 3),
        "graph_us_per_call": round(graph_us, 3) if graph_us is not None else None,
        "graph_device_us_per_call": round(graph_device_us, 3) if graph_device_us is not None else None,
        "step_alg_bytes": step_bytes,
        "effective_GBps": round(step_bytes / (us_per_call * 1e-6) / 1e9, 1),
        "kernel_source_hash": kernel_source_hash(),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
