"""The five synthetic workloads and their seeded recipes (CPU side).

No attention or merge arithmetic lives here: only shapes, seeds and the
mapping from logical tensor positions to positions in the counter-based
streams of ``synth.philox``.  The GPU generator (``synth/csrc/synth.hip``)
fills device tensors from the same streams with the same logical indexing.

Logical layouts (the element index into a stream):
  q        [B][Hq][D]                      tag TAG_Q
  k, v     [R][B][Hkv][Lcap][D]            tags TAG_K, TAG_V
  lens     [R][B]   (ragged workload only) tags TAG_LEN, TAG_LEN_EMPTY
  o_part   [R][rows][D] (merge workload)   tag TAG_OPART
  lse_part [R][rows]    (merge workload)   tags TAG_LSE, TAG_LSE_EMPTY
Physical device tensors use exactly these layouts (contiguous), so a
physical offset equals the logical index.
"""
from __future__ import annotations

from dataclasses import dataclass, field
import math

import numpy as np

from . import philox

TAG_Q = 1
TAG_K = 2
TAG_V = 3
TAG_LEN = 4
TAG_LEN_EMPTY = 5
TAG_OPART = 6
TAG_LSE = 7
TAG_LSE_EMPTY = 8

# Unaligned KV lengths forced into fixed (shard, sequence) slots of the
# ragged workload: one either side of every power-of-two tile edge a kernel
# is likely to use, plus the capacity itself.
EDGE_LENGTHS = (1, 2, 15, 16, 17, 63, 64, 65, 127, 128, 129, 16383, 16384)


@dataclass(frozen=True)
class Workload:
    name: str
    R: int
    B: int = 0
    Hq: int = 0
    Hkv: int = 0
    D: int = 0
    dtype: str = "bf16"
    Lcap: int = 0
    L: int = 0                 # constant length; 0 with ragged=True
    ragged: bool = False
    empty_p: float = 0.0       # probability a (shard, seq) or lse entry is empty
    k_scale: float = 1.0       # k = round(k_scale * z)
    merge_only: bool = False
    rows: int = 0              # merge workload: rows = batch * heads
    lse_sigma: float = 0.0     # merge workload: lse = lse_sigma * z
    seed: int = 0
    note: str = ""

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    def scaled(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


WORKLOADS = {
    "c1": Workload("c1", R=2, B=1, Hq=2, Hkv=2, D=64, dtype="fp16", Lcap=512, L=512,
                   seed=1001, note="R=2 x 512 tokens, batch 1, 2 heads MHA, D=64, fp16"),
    "c2": Workload("c2", R=4, B=1, Hq=8, Hkv=8, D=128, dtype="bf16", Lcap=4096, L=4096,
                   seed=1002, note="R=4 x 4096 tokens, batch 1, 8/8 heads, D=128, bf16"),
    "c3": Workload("c3", R=8, B=64, Hq=32, Hkv=8, D=128, dtype="bf16", Lcap=8192, L=8192,
                   seed=1003, note="R=8 x 8192 tokens, batch 64, 32/8 heads (GQA 4), D=128, bf16"),
    "c4": Workload("c4", R=8, B=256, Hq=64, Hkv=8, D=128, dtype="bf16", Lcap=16384,
                   ragged=True, empty_p=0.05, k_scale=3.0, seed=1004,
                   note="R=8, batch 256, 64/8 heads (GQA 8), D=128, bf16, lens U[0,16384], "
                        "5% empty, k x3"),
    "c5": Workload("c5", R=8, D=512, dtype="bf16", merge_only=True, rows=512 * 128,
                   empty_p=0.05, lse_sigma=4.0, seed=1005,
                   note="merge only: R=8, 512 x 128 rows, D=512, bf16 o_part, "
                        "fp32 lse ~ N(0, 16), 5% -inf"),
}


# ---------------------------------------------------------------- lengths
def lens(w: Workload) -> np.ndarray:
    """KV lengths [R][B] (int32)."""
    if not w.ragged:
        return np.full((w.R, w.B), w.L, dtype=np.int32)
    n = w.R * w.B
    L = philox.uniform_int(w.seed, TAG_LEN, 0, n, w.Lcap + 1)
    empty = philox.bernoulli(w.seed, TAG_LEN_EMPTY, 0, n, w.empty_p)
    L = np.where(empty, 0, L).reshape(w.R, w.B)
    for i, e in enumerate(EDGE_LENGTHS):
        if i < w.B:
            L[i % w.R, i] = min(e, w.Lcap)
    return L.astype(np.int32)


# ---------------------------------------------------------------- q / k / v
def q_index(w: Workload, b: int, h: int) -> int:
    return (b * w.Hq + h) * w.D


def kv_index(w: Workload, r: int, b: int, h: int, t: int = 0) -> int:
    return (((r * w.B + b) * w.Hkv + h) * w.Lcap + t) * w.D


def _draw(w: Workload, tag: int, start: int, count: int, scale: float = 1.0):
    z = philox.normal_f32(w.seed, tag, start, count)
    if scale != 1.0:
        z = (z * np.float32(scale)).astype(np.float32)
    return philox.round_to(z, w.dtype)


def q_values(w: Workload) -> np.ndarray:
    """q [B][Hq][D] as float32 holding the exact storage values."""
    _, v = _draw(w, TAG_Q, 0, w.B * w.Hq * w.D)
    return v.reshape(w.B, w.Hq, w.D)


def q_rows(w: Workload, b: int, h0: int, nheads: int) -> np.ndarray:
    """q[b, h0:h0+nheads] as float32 [nheads][D] (exact storage values)."""
    _, v = _draw(w, TAG_Q, q_index(w, b, h0), nheads * w.D)
    return v.reshape(nheads, w.D)


def q_storage(w: Workload) -> np.ndarray:
    bits, _ = _draw(w, TAG_Q, 0, w.B * w.Hq * w.D)
    return bits.reshape(w.B, w.Hq, w.D)


def kv_values(w: Workload, which: str, r: int, b: int, h: int, L: int) -> np.ndarray:
    """Tokens [0, L) of k or v for (shard r, sequence b, kv head h): [L][D] float32."""
    tag = TAG_K if which == "k" else TAG_V
    scale = w.k_scale if which == "k" else 1.0
    _, v = _draw(w, tag, kv_index(w, r, b, h), L * w.D, scale)
    return v.reshape(L, w.D)


def kv_storage(w: Workload, which: str) -> np.ndarray:
    """Whole k or v tensor [R][B][Hkv][Lcap][D] in storage form (small workloads)."""
    tag = TAG_K if which == "k" else TAG_V
    scale = w.k_scale if which == "k" else 1.0
    n = w.R * w.B * w.Hkv * w.Lcap * w.D
    bits, _ = _draw(w, tag, 0, n, scale)
    return bits.reshape(w.R, w.B, w.Hkv, w.Lcap, w.D)


# ---------------------------------------------------------------- merge inputs
def merge_lse(w: Workload, rows: slice | None = None) -> np.ndarray:
    """lse_part [R][rows] float32 with -inf entries (merge workload)."""
    out = np.empty((w.R, w.rows), dtype=np.float32)
    for r in range(w.R):
        z = philox.normal_f32(w.seed, TAG_LSE, r * w.rows, w.rows)
        v = (z * np.float32(w.lse_sigma)).astype(np.float32)
        e = philox.bernoulli(w.seed, TAG_LSE_EMPTY, r * w.rows, w.rows, w.empty_p)
        out[r] = np.where(e, np.float32(-np.inf), v)
    return out if rows is None else out[:, rows]


def merge_opart_values(w: Workload, r: int, row0: int, nrows: int) -> np.ndarray:
    """o_part rows [row0, row0+nrows) of shard r: [nrows][D] float32 (exact)."""
    _, v = philox.round_to(
        philox.normal_f32(w.seed, TAG_OPART, (r * w.rows + row0) * w.D, nrows * w.D), w.dtype)
    return v.reshape(nrows, w.D)


def merge_opart_storage(w: Workload) -> np.ndarray:
    n = w.R * w.rows * w.D
    bits, _ = philox.round_to(philox.normal_f32(w.seed, TAG_OPART, 0, n), w.dtype)
    return bits.reshape(w.R, w.rows, w.D)


def small(name: str, **kw) -> Workload:
    """A reduced copy of a workload (same recipe, smaller shape) for fast tests."""
    return WORKLOADS[name].scaled(name=name + "_small", **kw)
