"""Shared test helpers: tolerances and the GPU call sequence.

Tolerances (from the acceptance bar of this path):
  output      |gpu - oracle| <= 2^-7 |oracle| + 1e-3   (oracle unrounded, float64)
  merged lse  |gpu - oracle| <= 1e-5 |oracle|;  -inf must match -inf exactly
  per-shard lse (diagnostic)   <= 1e-5 max(1, |oracle|)
"""
from __future__ import annotations

import numpy as np

OUT_REL = 2.0 ** -7
OUT_ABS = 1e-3
LSE_REL = 1e-5


def out_ratio(gpu: np.ndarray, ref: np.ndarray) -> float:
    """max over elements of error / allowed error (<= 1 passes)."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if gpu.size == 0:
        return 0.0
    assert np.isfinite(gpu).all(), "non-finite output"
    return float((np.abs(gpu - ref) / (OUT_REL * np.abs(ref) + OUT_ABS)).max())


def assert_out(gpu, ref, what="out"):
    r = out_ratio(gpu, ref)
    assert r <= 1.0, f"{what}: max error/bound = {r:.3f}"
    return r


def assert_lse(gpu, ref, what="lse", floor: bool = False):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    ninf_g, ninf_r = np.isneginf(gpu), np.isneginf(ref)
    assert np.array_equal(ninf_g, ninf_r), f"{what}: -inf pattern differs"
    fin = ~ninf_r
    assert np.isfinite(gpu[fin]).all(), f"{what}: non-finite where oracle is finite"
    scale = np.maximum(1.0, np.abs(ref[fin])) if floor else np.abs(ref[fin])
    err = np.abs(gpu[fin] - ref[fin])
    bad = err > LSE_REL * scale
    assert not bad.any(), (f"{what}: {int(bad.sum())} values over 1e-5 relative; worst "
                           f"gpu={gpu[fin][bad][0]!r} ref={ref[fin][bad][0]!r}")


def to64(t) -> np.ndarray:
    """Device or host tensor -> float64 numpy (exact for every storage dtype)."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def run_path(inp, o_dtype=None, chunk_tokens=0, workspace=None, lse_out=True):
    """partial attention + merge on the GPU through the binding; returns tensors."""
    import torch
    import lse_merge_split_amd as cp
    q = inp["q"]
    R = len(inp["k_shards"])
    B, Hq, D = q.shape
    o_dtype = o_dtype or torch.float32
    o_part = torch.empty((R, B, Hq, D), dtype=o_dtype, device=q.device)
    lse_part = torch.empty((R, B, Hq), dtype=torch.float32, device=q.device)
    cp.attn_partial(q, inp["k_shards"], inp["v_shards"], inp["lens"], o_part, lse_part,
                    chunk_tokens=chunk_tokens, workspace=workspace)
    out = torch.empty((B, Hq, D), dtype=q.dtype, device=q.device)
    lo = torch.empty((B, Hq), dtype=torch.float32, device=q.device) if lse_out else None
    cp.lse_merge(o_part, lse_part, out, lo)
    torch.cuda.synchronize()
    return dict(o_part=o_part, lse_part=lse_part, out=out, lse_out=lo)
