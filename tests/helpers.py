"""Shared test helpers: tolerances and the GPU call sequence.

Tolerances (from the acceptance bar of this path):
  output      |gpu - oracle| <= 2^-7 |oracle| + 1e-3   (oracle unrounded, float64)
  merged lse  |gpu - oracle| <= 1e-5 |oracle| for the merge of given partials
              (cpdec_lse_merge: exact inputs, FP64 arithmetic); on the whole
              path <= 1e-5 max(1, |oracle|): it inherits the per-shard lse
              values' absolute error (FP32 scores, ~1e-7 of their size), so a
              merged lse that cancels towards 0 cannot meet a purely relative
              bar.  -inf must match -inf exactly.
  per-shard lse (diagnostic)   <= 1e-5 max(1, |oracle|)
  16-bit partials: the output against the storage-aware oracle (exact
              partials rounded to the storage type, merged exactly), plus,
              per element, the weighted storage step of every partial that
              lies within FP32 accuracy (4e-5 of its row's magnitude) of a
              rounding boundary: the GPU's partial may round to either side.
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


FLOOR_ONLY = {"values": 0, "checked": 0}  # lse values that passed only through the floor


def assert_lse(gpu, ref, what="lse", floor: bool = False):
    """-inf must match exactly; finite values within 1e-5 relative (floor:
    relative to max(1, |oracle|)).  Returns how many values passed only
    through the floor (they would fail the strict relative bar); they are
    also counted in FLOOR_ONLY and printed."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    ninf_g, ninf_r = np.isneginf(gpu), np.isneginf(ref)
    assert np.array_equal(ninf_g, ninf_r), f"{what}: -inf pattern differs"
    fin = ~ninf_r
    assert np.isfinite(gpu[fin]).all(), f"{what}: non-finite where oracle is finite"
    strict = np.abs(ref[fin])
    scale = np.maximum(1.0, strict) if floor else strict
    err = np.abs(gpu[fin] - ref[fin])
    bad = err > LSE_REL * scale
    assert not bad.any(), (f"{what}: {int(bad.sum())} values over 1e-5 relative; worst "
                           f"gpu={gpu[fin][bad][0]!r} ref={ref[fin][bad][0]!r}")
    floor_only = int((err > LSE_REL * strict).sum()) if floor else 0
    FLOOR_ONLY["values"] += floor_only
    FLOOR_ONLY["checked"] += int(fin.sum())
    if floor_only:
        print(f"[info] {what}: {floor_only} of {int(fin.sum())} values pass only through the "
              f"max(1, |lse|) floor", flush=True)
    return floor_only


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


PARTIAL_REL = 4e-5  # accuracy of an FP32 partial, relative to its row's magnitude


def assert_out_stored(gpu, o_exact, lse_exact, dtype, what="out"):
    """gpu [G, D] against the merge of the exact partials o_exact [R, G, D]
    (lse_exact [R, G]) stored as `dtype`.  A partial within PARTIAL_REL of its
    row's magnitude from a rounding boundary may be stored on either side of
    it; the merged output may then move by that step times the partial's
    weight, which is added to the bar."""
    from oracle import oracle as orc
    o_exact = np.asarray(o_exact, dtype=np.float64)
    lse_exact = np.asarray(lse_exact, dtype=np.float64)
    G = o_exact.shape[1]
    ref = np.stack([orc.merge_stored(o_exact[:, g], lse_exact[:, g], dtype)[0] for g in range(G)])
    eps = PARTIAL_REL * np.abs(o_exact).max(axis=-1, keepdims=True)
    step = np.abs(orc.round_storage(o_exact + eps, dtype) - orc.round_storage(o_exact - eps, dtype))
    live = np.isfinite(lse_exact)
    M = np.where(live, lse_exact, -np.inf).max(axis=0)
    w = np.where(live, np.exp(np.where(live, lse_exact, 0.0) - np.where(np.isfinite(M), M, 0.0)), 0.0)
    S = w.sum(axis=0)
    allow = np.where(S[:, None] > 0, (w[:, :, None] * step).sum(axis=0) / np.where(S > 0, S, 1.0)[:, None],
                     0.0)
    gpu = np.asarray(gpu, dtype=np.float64)
    assert np.isfinite(gpu).all(), f"{what}: non-finite output"
    r = float((np.abs(gpu - ref) / (OUT_REL * np.abs(ref) + OUT_ABS + allow)).max())
    assert r <= 1.0, f"{what}: max error/bound = {r:.3f}"
    return r
