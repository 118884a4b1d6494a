#!/usr/bin/env python3
"""Benchmark of the context-parallel decode combine on one MI355X.

One step = the whole hot path over one batch: per-shard split-KV decode
attention, the merge of each shard's chunks and the cross-shard LSE merge.
By default a step is one cpdec_cp_decode call (one kernel launch when the
shape allows it); --two-calls times cpdec_attn_partial followed by
cpdec_lse_merge instead.  The merge-only workload (c5) runs cpdec_lse_merge
alone.  Inputs are synthetic, seeded, and resident in HBM before the timed
region starts.

The headline workload (default c4: 8 shards, batch 256, 64/8 heads, D=128,
ragged lengths, the largest one-GPU workload) is timed for exactly --steps
steps after --warmup untimed ones.  The other large workloads (c3, the
merge-only c5) and the small c2 and c1, each with its HIP-graph replay, are
then timed in the same process, each in a block of its own (--extras; "none"
skips them).

Prints ONE JSON line:
  value          eager microseconds per call (wall clock of K back-to-back
                 steps launched from Python / K)
  roofline       the step's kernels (the attention kernel, with the order
                 pre-pass and merge when the step has several launches; the
                 merge kernel for c5): algorithmic bytes per step / their
                 mean duration, the span of HIP events recorded on the launch
                 stream around the K timed steps divided by K, against
                 MI355X's 8 TB/s HBM peak; `traffic` is filled from the
                 committed rocprofv3 counter summary when it was taken on the
                 current kernel source, else null
  cpu_baseline   the CPU oracle timed on this host's cores (one process per
                 core) on a bounded sample of the headline workload,
                 extrapolated to microseconds per call

Workloads smaller than the 256 MB Infinity Cache rotate through enough input
copies that a step never finds its inputs cache-resident; so does the merge
workload (three copies of its 0.6 GB of partials).
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
    a0 = steps[0][0]
    info = dict(copies=copies, chunk=a0.plan["chunk_tokens"], nchunks=a0.plan["num_chunks"],
                waves=a0.plan["waves"], workspace_bytes=a0.workspace_bytes,
                longest_first=a0.plan["longest_first"], attn_launches=a0.plan["launches"],
                launches=(a0.launches if fused else a0.plan["launches"] + 1))
    return steps, alg_attn, alg_merge, info, sets


MERGE_COPIES = 3   # 3 x 0.6 GB of partials: no step finds its inputs in the 256 MB MALL


def build_merge_steps(w: sc.Workload, torch, cp, sg, copies: int = MERGE_COPIES):
    inp = sg.merge_inputs(w)
    sets = [inp] + [dict(o_part=inp["o_part"].clone(), lse_part=inp["lse_part"].clone())
                    for _ in range(copies - 1)]
    out = torch.empty((w.rows, w.D), dtype=torch.bfloat16, device="cuda")
    lse_out = torch.empty(w.rows, dtype=torch.float32, device="cuda")
    steps = [(None, cp.MergeCall(s["o_part"], s["lse_part"], out, lse_out)) for s in sets]
    live = int(np.isfinite(inp["lse_np"]).sum())
    alg = merge_alg_bytes(w.R, w.rows, w.D, live, 2, 2)
    return steps, 0, alg, dict(copies=copies, launches=1), sets


def kernels_of(w: sc.Workload, fused: bool, info: dict) -> str:
    """The kernels one timed step launches, in launch order."""
    if w.merge_only:
        return "lse_merge_wave_row_kernel" if w.D * 2 >= 1024 and w.R <= 8 else "lse_merge_kernel"
    ks = []
    if info.get("longest_first"):
        ks.append("order_kernel")
    ks.append("attn_partial_kernel")
    if fused:
        n = info["launches"] - len(ks)
        if n == 1:
            ks.append("row_merge_kernel" if info.get("nchunks", 1) > 1 else "lse_merge_kernel")
        elif n == 2:
            ks += ["attn_combine_kernel", "lse_merge_kernel"]
    else:
        if info.get("attn_launches", 1) > 1 + int(bool(info.get("longest_first"))):
            ks.append("attn_combine_kernel")
        ks.append("lse_merge_kernel")
    return " + ".join(ks)


def time_workload(name: str, K: int, W: int, torch, cp, sg, fused: bool = True,
                  graph: bool = False, traffic_kernel: str | None = None) -> dict:
    """Build the workload's inputs, run W untimed steps, then time exactly K
    steps back to back on one stream: wall clock (value) and the span of HIP
    events on that stream around all K (the step kernels' mean duration).
    Returns the workload's block of the result line."""
    w = sc.WORKLOADS[name]
    if w.merge_only:
        steps, alg_attn, alg_merge, info, sets = build_merge_steps(w, torch, cp, sg)
        fused = False
    else:
        steps, alg_attn, alg_merge, info, sets = build_attn_steps(w, torch, cp, sg, fused=fused)
    torch.cuda.synchronize()
    print(f"[bench] workload {w.name}: {w.note}; copies={info['copies']} steps={K} warmup={W}",
          file=sys.stderr, flush=True)
    stream = torch.cuda.current_stream().cuda_stream  # every call goes on this stream

    def step(i):
        a, m = steps[i % len(steps)]
        if a is not None:
            a(stream)
        if m is not None:
            m(stream)

    for i in range(W):
        step(i)
    torch.cuda.synchronize()
    # Steps of a millisecond or more also get an event pair each (an event
    # record costs a few microseconds of device time, negligible there), for
    # the spread of the step time; shorter steps are timed by the span alone.
    per_step = alg_attn + alg_merge >= (4 << 30)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)] \
        if per_step else None
    edge = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    edge[0].record()
    for i in range(K):
        if evs:
            evs[i][0].record()
        step(i)
        if evs:
            evs[i][1].record()
    edge[1].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    print(f"[bench] {w.name}: timed {K} steps", file=sys.stderr, flush=True)
    us_per_call = (t1 - t0) / K * 1e6
    device_us = edge[0].elapsed_time(edge[1]) * 1e3 / K
    spread = None
    if evs:
        ts = np.array([a.elapsed_time(b) * 1e3 for a, b in evs])
        spread = {"p10": round(float(np.percentile(ts, 10)), 1),
                  "median": round(float(np.median(ts)), 1),
                  "p90": round(float(np.percentile(ts, 90)), 1)}

    if w.merge_only:
        step_bytes = alg_merge
    elif fused:
        step_bytes = alg_attn + w.B * w.Hq * (w.D * 2 + 4)  # + out and lse_out written once
    else:
        step_bytes = alg_attn + alg_merge   # the two calls also write and re-read o_part
    achieved = step_bytes / (device_us * 1e-6) / 1e9
    kernel = "lse_merge" if w.merge_only else "attn_partial"
    traffic = committed_traffic(w.name, traffic_kernel or kernel)

    block = {
        "value": round(us_per_call, 3), "unit": "µs/call", "steps": K, "warmup": W,
        "config": {"workload": f"{w.name}: {w.note}",
                   "entry": ("cpdec_lse_merge" if w.merge_only else
                             "cpdec_cp_decode" if fused else "cpdec_attn_partial + cpdec_lse_merge"),
                   "launches_per_step": info.get("launches", 1),
                   "R": w.R, "B": w.B or None, "Hq": w.Hq or None, "Hkv": w.Hkv or None, "D": w.D,
                   "rows": w.rows or None, "input_copies": info["copies"],
                   "chunk_tokens": info.get("chunk"), "chunks_per_shard": info.get("nchunks"),
                   "waves_per_workgroup": info.get("waves"),
                   "longest_first": info.get("longest_first"), "seed": w.seed,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": kernels_of(w, fused, info),
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "alg_bytes_per_launch": step_bytes, "mean_launch_us": round(device_us, 3),
                     "timing": f"HIP events on the launch stream around the {K} timed steps / {K}"},
        "device_us_per_call": round(device_us, 3),
        "effective_GBps": round(step_bytes / (us_per_call * 1e-6) / 1e9, 1),
    }
    if spread:
        block["step_us_events"] = spread

    if graph:
        # One graph per input copy, replayed in the same rotation as the eager
        # steps (a replay finds its inputs no more cache-resident than an eager
        # step); and one graph holding every rotated step, replayed K/copies times.
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
        g_all = torch.cuda.CUDAGraph()
        with torch.cuda.stream(side):
            with torch.cuda.graph(g_all):
                cs = torch.cuda.current_stream().cuda_stream
                for a, m in steps:
                    if a is not None:
                        a(cs)
                    if m is not None:
                        m(cs)
        torch.cuda.synchronize()
        for i in range(W):
            graphs[i % len(graphs)].replay()
        g_all.replay()
        torch.cuda.synchronize()
        gedge = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        tg0 = time.perf_counter()
        gedge[0].record()
        for i in range(K):
            graphs[i % len(graphs)].replay()
        gedge[1].record()
        torch.cuda.synchronize()
        tg1 = time.perf_counter()
        reps = max(1, K // len(steps))
        gedge[2].record()
        for _ in range(reps):
            g_all.replay()
        gedge[3].record()
        torch.cuda.synchronize()
        block["graph_us_per_call"] = round((tg1 - tg0) / K * 1e6, 3)
        block["graph_device_us_per_call"] = round(gedge[0].elapsed_time(gedge[1]) * 1e3 / K, 3)
        block["graph_all_steps_device_us_per_call"] = round(
            gedge[2].elapsed_time(gedge[3]) * 1e3 / (reps * len(steps)), 3)
        block["graph_note"] = ("graph_*: one HIP graph per step replayed in the eager rotation; "
                               f"graph_all_steps: the {len(steps)} rotated steps captured in one "
                               f"graph, replayed {reps}x")
        del graphs, g_all
    del steps, sets
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return block


EXTRA_STEPS = {"c3": (20, 5), "c5": (100, 10), "c2": (200, 10), "c1": (200, 10), "c4": (20, 5)}


# ------------------------------------------------------------------ CPU baseline
def host_cpu_model() -> str:
    """The host CPU's model name (what lscpu prints as "Model name")."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.lower().startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_group_inputs(w: sc.Workload, lens, b: int, h: int):
    qg = sc.q_rows(w, b, h * w.G, w.G).astype(np.float64)
    kv = [(sc.kv_values(w, "k", r, b, h, int(lens[r, b])).astype(np.float64),
           sc.kv_values(w, "v", r, b, h, int(lens[r, b])).astype(np.float64))
          for r in range(w.R)]
    return qg, kv


def _cpu_worker(name, units, budget_s, barrier, results):
    """One host process: generate its units' inputs (untimed), wait for every
    process, then run the oracle over its units repeatedly for budget_s and
    report (seconds per pass, work items per pass).  One BLAS thread."""
    from threadpoolctl import threadpool_limits
    from oracle import oracle as orc
    w = sc.WORKLOADS[name]
    with threadpool_limits(1):
        if w.merge_only:
            lse = sc.merge_lse(w)
            data = (np.stack([np.stack([sc.merge_opart_values(w, r, int(n), 1)[0] for n in units])
                              for r in range(w.R)]).astype(np.float64),
                    lse[:, units].astype(np.float64))
            work = len(units)
        else:
            lens = sc.lens(w)
            data = [_oracle_group_inputs(w, lens, b, h) for (b, h) in units]
            work = sum(int(lens[:, b].sum()) for (b, _) in units)
        barrier.wait()
        t0 = time.perf_counter()
        reps = 0
        while True:
            if w.merge_only:
                orc.merge_rows(*data)
            else:
                for qg, kv in data:
                    parts = [orc.attend_shard(qg, k, v, w.sm_scale) for (k, v) in kv]
                    o_p = np.stack([p[0] for p in parts])
                    l_p = np.stack([p[1] for p in parts])
                    for g in range(w.G):
                        orc.merge(o_p[:, g], l_p[:, g])
            reps += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        results.put(((time.perf_counter() - t0) / reps, work, reps))


def cpu_baseline(w: sc.Workload, budget_s: float, procs: int | None = None):
    """The CPU oracle on the host cores: one process per core (one BLAS
    thread each), each over its own random sample of (sequence, kv head)
    groups -- all shards of a group -- or merge rows; inputs generated before
    the clock starts; the oracle math repeated for budget_s in every process
    at once.  The whole workload's time is extrapolated linearly from the
    measured rate: attention by tokens (sum over the group's shards of the
    valid lengths, times its kv heads), the merge by rows.  Must run before
    the GPU is touched (the workers are forked)."""
    import multiprocessing as mp
    cores = os.cpu_count() or 1
    P = max(1, min(procs or cores, cores, 16))
    rng = np.random.default_rng(1)
    if w.merge_only:
        per = 256
        picks = rng.choice(w.rows, size=P * per, replace=False)
        units = [sorted(int(x) for x in picks[i * per:(i + 1) * per]) for i in range(P)]
        total_work = w.rows
        unit_name = f"{per} merge rows (all {w.R} shards, D={w.D})"
    else:
        lens = sc.lens(w)
        groups = [(b, h) for b in range(w.B) for h in range(w.Hkv)]
        # bounded generation: about 32M K/V elements per process
        mean_tokens = max(1.0, float(lens.sum(axis=0).mean()))
        per = int(max(1, min(len(groups) // P, 32_000_000 // (mean_tokens * w.D * 2))))
        picks = rng.choice(len(groups), size=min(len(groups), P * per), replace=False)
        units = [[groups[int(i)] for i in picks[p * per:(p + 1) * per]] for p in range(P)]
        units = [u for u in units if u]
        P = len(units)
        total_work = int(lens.sum()) * w.Hkv
        unit_name = f"{per} (sequence, kv head) groups (all {w.R} shards, G={w.G} query heads)"
    ctx = mp.get_context("fork")
    barrier = ctx.Barrier(P)
    results = ctx.Queue()
    ps = [ctx.Process(target=_cpu_worker, args=(w.name, u, budget_s, barrier, results))
          for u in units]
    t_start = time.perf_counter()
    for p in ps:
        p.start()
    got = [results.get() for _ in ps]
    for p in ps:
        p.join()
    wall = time.perf_counter() - t_start
    rate = sum(work / sec for sec, work, _ in got)        # work items per second, all processes
    us = total_work / rate * 1e6
    reps = min(r for _, _, r in got)
    if w.merge_only:
        sample = (f"{P} processes x {unit_name}, random rows, oracle merge repeated >= {reps}x "
                  f"in every process at once; whole {w.rows}-row merge extrapolated linearly by rows")
    else:
        sampled = sum(work for _, work, _ in got)
        sample = (f"{P} processes x {unit_name}, random groups ({sampled} of {total_work} "
                  f"token-heads), oracle attention + merge repeated >= {reps}x in every process "
                  f"at once; whole workload extrapolated linearly by tokens x kv heads")
    return dict(value=round(us, 1), unit="µs/call", cores=P, kind="oracle", sample=sample,
                processes=P, blas_threads_per_process=1, host_cpu_count=os.cpu_count(),
                host_cpu_model=host_cpu_model(), timed_s_per_process=budget_s,
                wall_s=round(wall, 1))


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
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps of the headline workload (default 20 for c3/c4, "
                         "100 for c5, 200 for c1/c2)")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="c4", choices=sorted(sc.WORKLOADS),
                    help="headline workload (default c4, the largest one-GPU workload)")
    ap.add_argument("--extras", default="c3,c5,c2,c1",
                    help="other workloads timed after the headline, each in a block of its own "
                         "(the c2 and c1 blocks include their HIP-graph replay); 'none' for none")
    ap.add_argument("--cpu-budget-s", type=float, default=8.0,
                    help="seconds of oracle work per host process for cpu_baseline (0 disables it)")
    ap.add_argument("--cpu-procs", type=int, default=None,
                    help="host processes for cpu_baseline (default: one per core, at most 16)")
    ap.add_argument("--graph", action="store_true", help="also time HIP-graph replay of the headline")
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

    w = sc.WORKLOADS[args.workload]
    extras = [] if args.extras in ("", "none") else [e for e in args.extras.split(",")
                                                    if e != args.workload]
    for e in extras:
        if e not in sc.WORKLOADS:
            ap.error(f"unknown extra workload {e}")

    # The oracle's host processes are forked before anything touches the GPU.
    cpu = None
    if args.cpu_budget_s > 0:
        print("[bench] timing the CPU oracle baseline", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w, args.cpu_budget_s, args.cpu_procs)

    import torch
    import lse_merge_split_amd as cp
    from synth import gpu as sg

    torch.cuda.set_device(0)
    K = args.steps or EXTRA_STEPS.get(w.name, (20, 5))[0]
    W = args.warmup
    head = time_workload(w.name, K, W, torch, cp, sg, fused=not args.two_calls, graph=args.graph)

    extra_blocks = {}
    for e in extras:
        ke, we = EXTRA_STEPS.get(e, (20, 5))
        extra_blocks[e] = time_workload(e, ke, we, torch, cp, sg, graph=(e in ("c1", "c2")))

    # Context for the roofline: a plain 1 GiB device-to-device copy on this GPU
    # (read + write bytes over its time), the attainable rate of a simple stream.
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    dst.copy_(src)
    torch.cuda.synchronize()
    ce = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ce[0].record()
    for _ in range(10):
        dst.copy_(src)
    ce[1].record()
    torch.cuda.synchronize()
    copy_gbps = 2 * (1 << 30) * 10 / (ce[0].elapsed_time(ce[1]) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()

    if args.calibrate_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(1)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print("[bench] calibration copy: 1073741824 bytes read, 1073741824 written",
              file=sys.stderr, flush=True)

    line = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "µs/call",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(head["value"] / 1e3, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f16",
        "data": "synthetic (seeded Philox streams; no dataset)",
        "config": head["config"],
        "roofline": head["roofline"],
        "cpu_baseline": cpu,
        "device_us_per_call": head["device_us_per_call"],
        "effective_GBps": head["effective_GBps"],
        "step_us_events": head.get("step_us_events"),
        "d2d_copy_GBps": round(copy_gbps, 1),
        "kernel_source_hash": kernel_source_hash(),
    }
    for k in ("graph_us_per_call", "graph_device_us_per_call", "graph_all_steps_device_us_per_call",
              "graph_note"):
        if k in head:
            line[k] = head[k]
    for e, blk in extra_blocks.items():
        line[e] = blk
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
