"""CPU oracle for context-parallel decode attention and the LSE merge.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The
product path (``lse_merge_split_amd``) never imports it, and this module
imports nothing from the product path: the two share no code.  Inputs come
from ``synth`` (seeded streams, no method arithmetic).

Everything is plain float64 numpy: the definitions written out, with a
library matrix product as the only borrowed step.  bf16/fp16 inputs convert
to float64 exactly.

Source of the method (cited by page title and section):
  [CP] the page "FlashInfer's Context-Parallel Decode optimisation: Fused
       A2A + LSE Reduce" (analysis of flashinfer PR #4929).
  - section "Introduction": the KV cache of a sequence is split across
    ranks; each rank attends over its local KV shard and produces a partial
    output o_r and a log-sum-exp lse_r used for normalisation; the partials
    are then merged with LSE weights.
  - section "Code analysis, 1. Fused kernel": the legacy merge multiplies the
    partial outputs (read as float) by weights, sums over the shard axis and
    divides by a denominator; the fused kernel computes LSE-based softmax
    weights, accumulates in FP32 and converts to FP16/BF16.

Readings where the page is silent:
  * lse is a natural logarithm; softmax scale 1/sqrt(D) unless given.
  * GQA: query head hq reads kv head hq // (Hq / Hkv).
  * weights = exp(lse_r - max_r lse_r) and denominator = sum of weights.
  * An empty shard (L = 0) yields o_r = 0, lse_r = -inf, and the merge skips
    -inf shards entirely (their o_r is never read, so garbage cannot leak).
  * All shards empty: out = 0, lse_out = -inf.

Pins: every function here is pinned by the CPU tests in
``tests/test_oracle_pins.py`` against closed forms, hand-derived values,
brute force, an independent library routine and the method's invariants;
``tests/test_oracle_mutations.py`` plants plausible mistakes in copies of
these functions and checks that the pins catch each one.  The workload glue
in ``oracle/workloads.py`` is tied to ``cp_decode`` and ``merge_rows`` over
whole materialised workloads by ``tests/test_oracle_workloads.py``.
"""
from __future__ import annotations

import math

import numpy as np

NEG_INF = -np.inf


# ----------------------------------------------------------------- attention
def attend_shard(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float):
    """Decode attention of G query rows over one shard's L tokens.

    [CP] "Introduction": each rank attends over its local KV shard and emits
    the partial output o_r together with lse_r.

    q: [G, D]; k, v: [L, D]  ->  o: [G, D], lse: [G]   (float64)
    For L = 0 the shard is empty: o = 0, lse = -inf.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    G, D = q.shape
    L = k.shape[0]
    if L == 0:
        return np.zeros((G, D)), np.full(G, NEG_INF)
    s = scale * (k @ q.T)                    # [L, G]  scores
    m = s.max(axis=0)                        # [G]     max score
    p = np.exp(s - m)                        # [L, G]  unnormalised probabilities
    l = p.sum(axis=0)                        # [G]     exp-sum relative to m
    o = (p.T @ v) / l[:, None]               # [G, D]  normalised partial output
    lse = m + np.log(l)                      # [G]     natural-log LSE
    return o, lse


# ----------------------------------------------------------------- merge
def merge(o_parts: np.ndarray, lse_parts: np.ndarray):
    """LSE merge of R partials of one row.

    [CP] "Code analysis, 1. Fused kernel": out = sum_r o_r * w_r / denom with
    LSE-based softmax weights, w_r = exp(lse_r - max lse), denom = sum w_r;
    the merged LSE is max lse + ln(denom).

    o_parts: [R, D]; lse_parts: [R]  ->  out: [D], lse_out: scalar (float64)
    Shards with lse = -inf are skipped (never read).
    """
    o_parts = np.asarray(o_parts)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    D = o_parts.shape[-1]
    live = lse_parts > NEG_INF
    if not live.any():
        return np.zeros(D), NEG_INF
    lse_live = lse_parts[live]
    M = lse_live.max()
    w = np.exp(lse_live - M)                         # softmax weights over shards
    denom = w.sum()
    o_live = o_parts[live].astype(np.float64)
    out = (w[:, None] * o_live).sum(axis=0) / denom
    lse_out = M + math.log(denom)
    return out, lse_out


def round_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """Values of x after storing them as fp16 or bf16 (round to nearest even),
    returned as float64.  Used for partials that travel in 16 bits.

    bf16 keeps the top 16 bits of the float32 pattern; rounding adds half an
    ulp plus the tie-to-even bit before truncating.  x is first rounded to
    float32 (exact for every value the merge produces in float32)."""
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    if dtype == "fp16":
        return x32.astype(np.float16).astype(np.float64)
    if dtype != "bf16":
        raise ValueError(dtype)
    u = x32.view(np.uint32).astype(np.uint64)
    r = ((u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)) << np.uint64(16)
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


def merge_stored(o_parts: np.ndarray, lse_parts: np.ndarray, dtype: str):
    """The merge of partials that were stored in 16 bits on their way (what a
    context-parallel exchange carries when its payload is fp16/bf16): the
    exact partials rounded to the storage type, then merged exactly."""
    return merge(round_storage(o_parts, dtype), lse_parts)


def merge_rows(o_parts: np.ndarray, lse_parts: np.ndarray):
    """``merge`` applied row by row.  o_parts [R, N, D], lse_parts [R, N]."""
    R, N, D = o_parts.shape
    out = np.empty((N, D))
    lse = np.empty(N)
    for n in range(N):
        out[n], lse[n] = merge(o_parts[:, n, :], lse_parts[:, n])
    return out, lse


# ----------------------------------------------------------------- the whole path
def cp_decode(q: np.ndarray, k_shards, v_shards, lens: np.ndarray, Hkv: int,
              scale: float | None = None):
    """Per-shard partials and their merge for a whole batch.

    q: [B, Hq, D]; k_shards[r], v_shards[r]: [B, Hkv, >=L, D]; lens: [R, B].
    Returns (o_part [R,B,Hq,D], lse_part [R,B,Hq], out [B,Hq,D], lse_out [B,Hq]).
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, D = q.shape
    R = len(k_shards)
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    o_part = np.zeros((R, B, Hq, D))
    lse_part = np.full((R, B, Hq), NEG_INF)
    for r in range(R):
        for b in range(B):
            L = int(lens[r][b])
            for h in range(Hkv):
                heads = slice(h * G, (h + 1) * G)   # query heads that read kv head h
                o, lse = attend_shard(q[b, heads], k_shards[r][b, h, :L],
                                      v_shards[r][b, h, :L], scale)
                o_part[r, b, heads] = o
                lse_part[r, b, heads] = lse
    out = np.zeros((B, Hq, D))
    lse_out = np.full((B, Hq), NEG_INF)
    for b in range(B):
        for hq in range(Hq):
            out[b, hq], lse_out[b, hq] = merge(o_part[:, b, hq], lse_part[:, b, hq])
    return o_part, lse_part, out, lse_out
