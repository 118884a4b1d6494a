"""Oracle results for slices of the synthetic workloads.

TEST INFRASTRUCTURE ONLY (see ``oracle/oracle.py``).  Inputs are regenerated
on the CPU from the seeded streams in ``synth``; nothing is read back from
the GPU, so a GPU-side corruption of the inputs cannot hide itself.
"""
from __future__ import annotations

import numpy as np

from synth import configs as sc

from .oracle import attend_shard, merge, NEG_INF


def group(w: sc.Workload, lens: np.ndarray, b: int, h: int, scale: float | None = None):
    """Oracle for the G query heads of kv head h of sequence b, all shards,
    with softmax scale ``scale`` (the workload's 1/sqrt(D) when None).

    Returns dict with o_part [R,G,D], lse_part [R,G], out [G,D], lse_out [G]
    (float64, unrounded)."""
    G, D = w.G, w.D
    qg = sc.q_rows(w, b, h * G, G)
    o_part = np.zeros((w.R, G, D))
    lse_part = np.full((w.R, G), NEG_INF)
    for r in range(w.R):
        L = int(lens[r, b])
        k = sc.kv_values(w, "k", r, b, h, L)
        v = sc.kv_values(w, "v", r, b, h, L)
        o_part[r], lse_part[r] = attend_shard(qg, k, v, w.sm_scale if scale is None else scale)
    out = np.zeros((G, D))
    lse_out = np.full(G, NEG_INF)
    for g in range(G):
        out[g], lse_out[g] = merge(o_part[:, g], lse_part[:, g])
    return dict(o_part=o_part, lse_part=lse_part, out=out, lse_out=lse_out)


def merge_rows(w: sc.Workload, rows: np.ndarray):
    """Oracle for selected rows of the merge-only workload.

    Returns (out [n, D], lse_out [n]) float64 for the row indices given."""
    lse_all = sc.merge_lse(w)
    rows = np.asarray(rows)
    out = np.zeros((len(rows), w.D))
    lse_out = np.full(len(rows), NEG_INF)
    for i, row in enumerate(rows):
        o = np.stack([sc.merge_opart_values(w, r, int(row), 1)[0] for r in range(w.R)])
        out[i], lse_out[i] = merge(o, lse_all[:, row])
    return out, lse_out
