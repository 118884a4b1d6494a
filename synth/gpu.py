"""Device-side inputs for the synthetic workloads (GPU twin of ``configs``).

Large tensors (K, V, the merge workload's o_part, q) are filled on the GPU by
``libsynth.so`` from the same seeded streams the CPU side uses; small ones
(lens, the merge lse) are drawn on the CPU and copied.  torch provides the
device memory.  No attention or merge arithmetic lives here.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import configs as sc

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsynth.so")
_LIB = None
_DT = {"fp32": 0, "fp16": 1, "bf16": 2}


def lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} missing: run `python -m synth.build`")
        L = ctypes.CDLL(LIB_PATH)
        L.synth_fill_normal.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_uint64,
                                        ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32,
                                        ctypes.c_float, ctypes.c_void_p]
        L.synth_fill_normal.restype = ctypes.c_int
        _LIB = L
    return _LIB


def torch_dtype(name: str):
    import torch
    return {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}[name]


def fill_normal(t, seed: int, tag: int, start: int = 0, scale: float = 1.0):
    """Fill contiguous device tensor ``t`` with stream elements start .. start+numel-1."""
    import torch
    assert t.is_contiguous() and t.is_cuda
    name = {torch.float32: "fp32", torch.float16: "fp16", torch.bfloat16: "bf16"}[t.dtype]
    rc = lib().synth_fill_normal(t.data_ptr(), _DT[name], t.numel(), start, seed & 0xFFFFFFFF,
                                 tag, scale, torch.cuda.current_stream(t.device).cuda_stream)
    if rc != 0:
        raise RuntimeError(f"synth_fill_normal failed with hipError {rc}")
    return t


def attn_inputs(w: sc.Workload, device="cuda", poison_padding: bool = False):
    """q, K, V, lens of an attention workload on the device.

    K and V are single [R][B][Hkv][Lcap][D] tensors (shard r is ``k[r]``).
    With ``poison_padding`` every token position >= lens[r][b] holds NaN."""
    import torch
    dt = torch_dtype(w.dtype)
    q = torch.empty((w.B, w.Hq, w.D), dtype=dt, device=device)
    fill_normal(q, w.seed, sc.TAG_Q)
    k = torch.empty((w.R, w.B, w.Hkv, w.Lcap, w.D), dtype=dt, device=device)
    v = torch.empty_like(k)
    fill_normal(k, w.seed, sc.TAG_K, scale=w.k_scale)
    fill_normal(v, w.seed, sc.TAG_V)
    lens_np = sc.lens(w)
    if poison_padding:
        for r in range(w.R):
            for b in range(w.B):
                L = int(lens_np[r, b])
                k[r, b, :, L:, :] = float("nan")
                v[r, b, :, L:, :] = float("nan")
    lens = torch.from_numpy(lens_np).to(device)
    return dict(q=q, k=k, v=v, lens=lens, lens_np=lens_np,
                k_shards=[k[r] for r in range(w.R)], v_shards=[v[r] for r in range(w.R)])


def merge_inputs(w: sc.Workload, device="cuda"):
    """o_part [R][rows][D] and lse_part [R][rows] of the merge workload."""
    import torch
    o = torch.empty((w.R, w.rows, w.D), dtype=torch_dtype(w.dtype), device=device)
    fill_normal(o, w.seed, sc.TAG_OPART)
    lse_np = sc.merge_lse(w)
    lse = torch.from_numpy(lse_np).to(device)
    return dict(o_part=o, lse_part=lse, lse_np=lse_np)


def as_float64(t) -> np.ndarray:
    """Device tensor -> float64 numpy (exact for every storage dtype)."""
    return t.detach().float().cpu().numpy().astype(np.float64)
