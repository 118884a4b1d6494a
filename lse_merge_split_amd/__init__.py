"""cpdec -- context-parallel decode combine on AMD MI355X (gfx950).

Python binding over the C ABI in ``include/cpdec.h`` (libcpdec.so).  It only
marshals arguments: every step of the computation runs in the library's HIP
kernels.  PyTorch supplies device memory and the current stream.

Method: the page "FlashInfer's Context-Parallel Decode optimisation: Fused
A2A + LSE Reduce" (flashinfer PR #4929) -- per-shard decode attention giving
(o_r, lse_r) (section "Introduction") and their LSE merge (section "Code
analysis, 1. Fused kernel").
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["lib", "AttnDesc", "CpdecError", "AttnCall", "MergeCall", "StepCall",
           "StepCallNoAlloc", "attn_partial",
           "lse_merge", "cp_decode", "attn_workspace_bytes", "step_workspace_bytes", "attn_plan",
           "step_launches", "workspace_clear", "make_attn_desc", "DTYPE_CODES", "STATUS",
           "STEP_COUNTER_BYTES", "NOALLOC_SCRATCH_BYTES"]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcpdec.so")

STATUS = {0: "CPDEC_OK", 1: "CPDEC_ERR_INVALID_ARG", 2: "CPDEC_ERR_UNSUPPORTED",
          3: "CPDEC_ERR_ALIGNMENT", 4: "CPDEC_ERR_WORKSPACE", 5: "CPDEC_ERR_HIP"}
F32, F16, BF16 = 0, 1, 2
STEP_COUNTER_BYTES = 65536  # CPDEC_STEP_COUNTER_BYTES: counter region at the workspace start
NOALLOC_SCRATCH_BYTES = 16 << 20  # CPDEC_NOALLOC_SCRATCH_BYTES: cpdec_cp_decode_noalloc's scratch


class CpdecError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {STATUS.get(code, code)}")
        self.code = code


class AttnDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("num_shards", ctypes.c_int32), ("kv_capacity", ctypes.c_int32),
                ("kv_stride_batch", ctypes.c_int64), ("kv_stride_head", ctypes.c_int64),
                ("kv_stride_token", ctypes.c_int64), ("sm_scale", ctypes.c_float),
                ("qkv_dtype", ctypes.c_int), ("opart_dtype", ctypes.c_int),
                ("chunk_tokens", ctypes.c_int32)]


_LIB = None


def lib() -> ctypes.CDLL:
    """The loaded libcpdec.so; raises if it has not been built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m lse_merge_split_amd.build` (or __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        L.cpdec_attn_workspace_bytes.argtypes = [ctypes.POINTER(AttnDesc)]
        L.cpdec_attn_workspace_bytes.restype = sz
        L.cpdec_step_workspace_bytes.argtypes = [ctypes.POINTER(AttnDesc)]
        L.cpdec_step_workspace_bytes.restype = sz
        pi = ctypes.POINTER(ctypes.c_int32)
        L.cpdec_step_plan.argtypes = [ctypes.POINTER(AttnDesc), pi]
        L.cpdec_step_plan.restype = ctypes.c_int
        L.cpdec_attn_plan.argtypes = [ctypes.POINTER(AttnDesc), pi, pi, pi]
        L.cpdec_attn_plan.restype = ctypes.c_int
        L.cpdec_attn_order.argtypes = [ctypes.POINTER(AttnDesc), pi]
        L.cpdec_attn_order.restype = ctypes.c_int
        L.cpdec_attn_launches.argtypes = [ctypes.POINTER(AttnDesc), pi]
        L.cpdec_attn_launches.restype = ctypes.c_int
        L.cpdec_attn_partial.argtypes = [ctypes.POINTER(AttnDesc), vp, ctypes.POINTER(vp),
                                         ctypes.POINTER(vp), vp, vp, vp, vp, sz, vp]
        L.cpdec_attn_partial.restype = ctypes.c_int
        L.cpdec_cp_decode.argtypes = [ctypes.POINTER(AttnDesc), vp, ctypes.POINTER(vp),
                                      ctypes.POINTER(vp), vp, vp, vp, vp, vp, vp, sz, vp]
        L.cpdec_cp_decode.restype = ctypes.c_int
        L.cpdec_cp_decode_noalloc.argtypes = [ctypes.POINTER(AttnDesc), vp, ctypes.POINTER(vp),
                                              ctypes.POINTER(vp), vp, vp, vp, vp, vp, vp]
        L.cpdec_cp_decode_noalloc.restype = ctypes.c_int
        L.cpdec_lse_merge.argtypes = [vp, vp, i32, i64, i32, ctypes.c_int, ctypes.c_int, vp, vp, vp]
        L.cpdec_lse_merge.restype = ctypes.c_int
        L.cpdec_workspace_clear.argtypes = [vp, sz, vp]
        L.cpdec_workspace_clear.restype = ctypes.c_int
        L.cpdec_status_string.argtypes = [ctypes.c_int]
        L.cpdec_status_string.restype = ctypes.c_char_p
        L.cpdec_version.argtypes = []
        L.cpdec_version.restype = ctypes.c_char_p
        _LIB = L
    return _LIB


# ------------------------------------------------------------------ torch glue
def _torch():
    import torch
    return torch


def dtype_code(dt) -> int:
    torch = _torch()
    codes = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16}
    if dt not in codes:
        raise TypeError(f"unsupported dtype {dt}")
    return codes[dt]


DTYPE_CODES = {"fp32": F32, "fp16": F16, "bf16": BF16}


def make_attn_desc(q, k_shards, *, kv_capacity=None, sm_scale=0.0, opart_dtype=None,
                   chunk_tokens=0) -> AttnDesc:
    """Descriptor from q [B, Hq, D] and K shards [B, Hkv, cap, D] (any strides
    with a contiguous last dimension; every shard must share them)."""
    torch = _torch()
    B, Hq, D = q.shape
    k0 = k_shards[0]
    _, Hkv, cap, Dk = k0.shape
    if Dk != D:
        raise ValueError("head_dim mismatch between q and K")
    for k in k_shards:
        if k.shape != k0.shape or k.stride() != k0.stride() or k.stride(-1) != 1:
            raise ValueError("all K/V shards need one shape and one stride set, D contiguous")
    d = AttnDesc()
    d.batch, d.num_q_heads, d.num_kv_heads, d.head_dim = B, Hq, Hkv, D
    d.num_shards = len(k_shards)
    d.kv_capacity = cap if kv_capacity is None else kv_capacity
    d.kv_stride_batch, d.kv_stride_head, d.kv_stride_token = k0.stride(0), k0.stride(1), k0.stride(2)
    d.sm_scale = float(sm_scale or 0.0)
    d.qkv_dtype = dtype_code(q.dtype)
    d.opart_dtype = dtype_code(opart_dtype if opart_dtype is not None else torch.float32)
    d.chunk_tokens = int(chunk_tokens)
    return d


def attn_plan(desc: AttnDesc) -> dict:
    """The library's launch plan for a descriptor: chunk tokens, chunks, waves,
    whether the units are launched longest first, and cpdec_attn_partial's
    kernel launches."""
    c, n, wv, lf = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    rc = lib().cpdec_attn_plan(ctypes.byref(desc), ctypes.byref(c), ctypes.byref(n), ctypes.byref(wv))
    if rc != 0:
        raise CpdecError(rc, "cpdec_attn_plan")
    rc = lib().cpdec_attn_order(ctypes.byref(desc), ctypes.byref(lf))
    if rc != 0:
        raise CpdecError(rc, "cpdec_attn_order")
    nl = ctypes.c_int32()
    rc = lib().cpdec_attn_launches(ctypes.byref(desc), ctypes.byref(nl))
    if rc != 0:
        raise CpdecError(rc, "cpdec_attn_launches")
    return dict(chunk_tokens=c.value, num_chunks=n.value, waves=wv.value,
                longest_first=bool(lf.value), launches=nl.value)


def attn_workspace_bytes(desc: AttnDesc) -> int:
    """Workspace bytes cpdec_attn_partial needs (0: none)."""
    return int(lib().cpdec_attn_workspace_bytes(ctypes.byref(desc)))


def step_workspace_bytes(desc: AttnDesc) -> int:
    """Workspace bytes cpdec_cp_decode needs (counter region + partials)."""
    return int(lib().cpdec_step_workspace_bytes(ctypes.byref(desc)))


def step_launches(desc: AttnDesc) -> int:
    """Kernel launches cpdec_cp_decode makes for a descriptor (1 normally)."""
    n = ctypes.c_int32()
    rc = lib().cpdec_step_plan(ctypes.byref(desc), ctypes.byref(n))
    if rc != 0:
        raise CpdecError(rc, "cpdec_step_plan")
    return n.value


_WS_CACHE: dict = {}


def _workspace(device, nbytes, stream=None):
    """A workspace of at least nbytes for the stream `stream` (a hipStream_t
    handle; None: the current stream of `device`), reused across calls and
    shapes on that stream.  Calls on different streams may overlap, so each
    stream has its own.  Both attention entry points need the counter region
    to start at zero and leave it zero, so a new workspace is zero-filled --
    on `stream` itself, which also makes it that stream's allocation for
    torch's caching allocator: the fill is ordered before the kernels that
    use it, and a workspace replaced by a larger one is only handed out again
    after the work already enqueued on that stream."""
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(device).cuda_stream
    key = (str(device), int(stream))
    ws = _WS_CACHE.get(key)
    if ws is None or ws.numel() < nbytes:
        current = torch.cuda.current_stream(device)
        default = torch.cuda.default_stream(device)
        target = (current if current.cuda_stream == stream else
                  default if default.cuda_stream == stream else
                  torch.cuda.ExternalStream(stream, device=device))
        with torch.cuda.stream(target):
            ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)
        _WS_CACHE[key] = ws
    return ws


def _check_tensors(named, device=None):
    """Every tensor a GPU tensor on one device (a host pointer handed to a
    kernel would fault the GPU).  `named` maps names to tensors (None
    skipped).  Returns the device."""
    for name, t in named.items():
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor (got device {t.device})")
        if device is None:
            device = t.device
        elif t.device != device:
            raise ValueError(f"{name} is on {t.device}, other tensors on {device}")
    return device


class AttnCall:
    """A cpdec_attn_partial call with its arguments marshalled once.

    Calling it enqueues the kernel(s) on the current stream (or ``stream``).
    A workspace passed in must have its first STEP_COUNTER_BYTES bytes zero
    before the first call (see workspace_clear) and belongs to the caller:
    calls that may overlap need separate ones.  Without one, the binding uses
    its zero-filled workspace of the stream the call is enqueued on, so calls
    on different streams never share one.

    Every argument is checked before anything reaches the library: each
    tensor must be a GPU tensor on q's device, K and V must have q's dtype,
    lens must be int32 and lse_part float32."""

    _workspace_query = staticmethod(attn_workspace_bytes)
    _entry = "cpdec_attn_partial"

    def __init__(self, q, k_shards, v_shards, lens, o_part, lse_part, *, sm_scale=0.0,
                 kv_capacity=None, workspace=None, chunk_tokens=0, stream=None):
        torch = _torch()
        k_shards, v_shards = list(k_shards), list(v_shards)
        if not k_shards or len(k_shards) != len(v_shards):
            raise ValueError("k_shards and v_shards must be non-empty and of one length")
        for v, k in zip(v_shards, k_shards):
            if v.shape != k.shape or v.stride() != k.stride():
                raise ValueError("V shards must match K shards in shape and strides")
        if q.dtype not in (torch.float16, torch.bfloat16):
            raise TypeError(f"q must be float16 or bfloat16, not {q.dtype}")
        for name, t in (("k_shards", k_shards), ("v_shards", v_shards)):
            if any(x.dtype != q.dtype for x in t):
                raise TypeError(f"every tensor of {name} must have q's dtype {q.dtype}")
        if not (q.is_contiguous() and o_part.is_contiguous() and lse_part.is_contiguous()
                and lens.is_contiguous()):
            raise ValueError("q, o_part, lse_part and lens must be contiguous")
        if lens.dtype != torch.int32 or lse_part.dtype != torch.float32:
            raise TypeError("lens must be int32 and lse_part float32")
        if workspace is not None and not workspace.is_contiguous():
            raise ValueError("workspace must be contiguous")
        tensors = {"q": q, "lens": lens, "o_part": o_part, "lse_part": lse_part,
                   "workspace": workspace}
        tensors.update({f"k_shards[{r}]": k for r, k in enumerate(k_shards)})
        tensors.update({f"v_shards[{r}]": v for r, v in enumerate(v_shards)})
        desc = make_attn_desc(q, k_shards, kv_capacity=kv_capacity, sm_scale=sm_scale,
                              opart_dtype=o_part.dtype, chunk_tokens=chunk_tokens)
        R = len(k_shards)
        if tuple(o_part.shape) != (R, desc.batch, desc.num_q_heads, desc.head_dim):
            raise ValueError("o_part must be [R, B, Hq, D]")
        if (tuple(lse_part.shape) != (R, desc.batch, desc.num_q_heads)
                or tuple(lens.shape) != (R, desc.batch)):
            raise ValueError("lse_part must be [R, B, Hq] and lens [R, B]")
        self._tensors = tensors
        self._setup(desc, workspace)
        if stream is not None:
            self._args_for(_stream_handle(stream))   # the stream's workspace, allocated now

    def _setup(self, desc, workspace):
        """Check devices, plan, and marshal the pointers (StepCall adds its
        own tensors and outputs)."""
        t = self._tensors
        self._device = _check_tensors(t)
        R = desc.num_shards
        self.desc = desc
        self.workspace_bytes = self._workspace_query(desc)
        self.plan = attn_plan(desc)
        self._own_ws = workspace
        ks = (ctypes.c_void_p * R)(*[t[f"k_shards[{r}]"].data_ptr() for r in range(R)])
        vs = (ctypes.c_void_p * R)(*[t[f"v_shards[{r}]"].data_ptr() for r in range(R)])
        self._arrays = (ks, vs)
        self._head = [ctypes.byref(desc), t["q"].data_ptr(), ks, vs, t["lens"].data_ptr()]
        self._outs = [t["o_part"].data_ptr(), t["lse_part"].data_ptr()]
        self._fn = getattr(lib(), self._entry)
        self._by_stream = {}

    def _args_for(self, stream: int):
        args = self._by_stream.get(stream)
        if args is None:
            ws = self._own_ws
            if ws is None and self.workspace_bytes > 0:
                ws = _workspace(self._device, self.workspace_bytes, stream)
            ws_ptr = ws.data_ptr() if ws is not None else None
            ws_bytes = ws.numel() * ws.element_size() if ws is not None else 0
            args = (self._head + self._outs + [ws_ptr, ws_bytes], ws)
            self._by_stream[stream] = args
        return args

    def workspace(self, stream=None):
        """The workspace a call on `stream` uses (None when it needs none)."""
        stream = _stream_handle(stream)
        if stream is None:
            stream = _torch().cuda.current_stream(self._device).cuda_stream
        return self._args_for(stream)[1]

    def __call__(self, stream=None):
        """Enqueue on `stream` (a hipStream_t handle), else torch's current stream."""
        stream = _stream_handle(stream)
        if stream is None:
            stream = _torch().cuda.current_stream(self._device).cuda_stream
        rc = self._fn(*self._args_for(stream)[0], stream)
        if rc != 0:
            raise CpdecError(rc, self._entry)


class StepCall(AttnCall):
    """A cpdec_cp_decode call (the whole step: partials and their merge,
    normally one launch) with its arguments marshalled once.  A workspace
    passed in must have its first STEP_COUNTER_BYTES bytes zero before the
    first call (see workspace_clear).  out must be [B, Hq, D] of q's dtype
    and lse_out (optional) [B, Hq] float32, on q's device."""

    _workspace_query = staticmethod(step_workspace_bytes)
    _entry = "cpdec_cp_decode"

    def __init__(self, q, k_shards, v_shards, lens, o_part, lse_part, out, lse_out=None, **kw):
        torch = _torch()
        if out.dtype != q.dtype or tuple(out.shape) != tuple(q.shape) or not out.is_contiguous():
            raise ValueError("out must be a contiguous [B, Hq, D] tensor of q's dtype")
        if lse_out is not None:
            if lse_out.dtype != torch.float32:
                raise TypeError(f"lse_out must be float32, not {lse_out.dtype}")
            if tuple(lse_out.shape) != tuple(q.shape[:2]) or not lse_out.is_contiguous():
                raise ValueError("lse_out must be a contiguous [B, Hq] float32 tensor")
        self._step_outs = (out, lse_out)
        super().__init__(q, k_shards, v_shards, lens, o_part, lse_part, **kw)

    def _setup(self, desc, workspace):
        out, lse_out = self._step_outs
        self._tensors.update({"out": out, "lse_out": lse_out})
        super()._setup(desc, workspace)
        self._outs = self._outs + [out.data_ptr(),
                                   lse_out.data_ptr() if lse_out is not None else None]
        self.launches = step_launches(desc)


class StepCallNoAlloc(StepCall):
    """A cpdec_cp_decode_noalloc call: the whole step with the library's own
    static scratch (one per GPU, shared by every such call on it: calls that
    may overlap on one GPU must be serialised by the caller).  No workspace
    is allocated for it; a step that needs more scratch than
    NOALLOC_SCRATCH_BYTES raises CpdecError (CPDEC_ERR_WORKSPACE)."""

    _entry = "cpdec_cp_decode_noalloc"

    def __init__(self, q, k_shards, v_shards, lens, o_part, lse_part, out, lse_out=None, **kw):
        if kw.get("workspace") is not None:
            raise ValueError("cpdec_cp_decode_noalloc takes no workspace")
        super().__init__(q, k_shards, v_shards, lens, o_part, lse_part, out, lse_out, **kw)

    def _args_for(self, stream: int):
        args = self._by_stream.get(stream)
        if args is None:
            args = (self._head + self._outs, None)
            self._by_stream[stream] = args
        return args


def cp_decode(q, k_shards, v_shards, lens, o_part, lse_part, out, lse_out=None, *, stream=None,
              **kw):
    """Whole step: per-shard partials into o_part/lse_part and their merge into out/lse_out."""
    StepCall(q, k_shards, v_shards, lens, o_part, lse_part, out, lse_out, stream=stream, **kw)(
        _stream_handle(stream))


class MergeCall:
    """A cpdec_lse_merge call with its arguments marshalled once:
    o_part [R, ..., D] and lse_part [R, ...] into out [..., D], lse_out [...].
    lse_part and lse_out must be float32; every tensor a GPU tensor on one
    device."""

    def __init__(self, o_part, lse_part, out, lse_out=None):
        torch = _torch()
        if o_part.dim() < 2:
            raise ValueError("o_part must be [R, ..., D]")
        R = o_part.shape[0]
        D = o_part.shape[-1]
        rows = o_part.numel() // (R * D) if R * D else 0
        if not (o_part.is_contiguous() and lse_part.is_contiguous() and out.is_contiguous()):
            raise ValueError("o_part, lse_part and out must be contiguous")
        if lse_part.dtype != torch.float32:
            raise TypeError(f"lse_part must be float32, not {lse_part.dtype}")
        if lse_out is not None and lse_out.dtype != torch.float32:
            raise TypeError(f"lse_out must be float32, not {lse_out.dtype}")
        in_code, out_code = dtype_code(o_part.dtype), dtype_code(out.dtype)
        if lse_part.numel() != R * rows or out.numel() != rows * D:
            raise ValueError("shape mismatch between o_part, lse_part and out")
        if lse_out is not None and (lse_out.numel() != rows or not lse_out.is_contiguous()):
            raise ValueError("lse_out must hold one value per row")
        self._device = _check_tensors({"o_part": o_part, "lse_part": lse_part, "out": out,
                                       "lse_out": lse_out})
        self._keep = (o_part, lse_part, out, lse_out)
        self.rows, self.R, self.D = rows, R, D
        self._args = [o_part.data_ptr(), lse_part.data_ptr(), R, rows, D, in_code, out_code,
                      out.data_ptr(), lse_out.data_ptr() if lse_out is not None else None]
        self._fn = lib().cpdec_lse_merge

    def __call__(self, stream=None):
        """Enqueue on `stream` (a hipStream_t handle), else torch's current stream."""
        stream = _stream_handle(stream)
        if stream is None:
            stream = _torch().cuda.current_stream(self._device).cuda_stream
        rc = self._fn(*self._args, stream)
        if rc != 0:
            raise CpdecError(rc, "cpdec_lse_merge")


def attn_partial(q, k_shards, v_shards, lens, o_part, lse_part, *, sm_scale=0.0,
                 kv_capacity=None, workspace=None, chunk_tokens=0, stream=None):
    """Per-shard decode attention into o_part [R,B,Hq,D] and lse_part [R,B,Hq].

    lens: int32 device tensor [R, B]."""
    AttnCall(q, k_shards, v_shards, lens, o_part, lse_part, sm_scale=sm_scale,
             kv_capacity=kv_capacity, workspace=workspace, chunk_tokens=chunk_tokens,
             stream=stream)(_stream_handle(stream))


def lse_merge(o_part, lse_part, out, lse_out=None, *, stream=None):
    """Merge o_part [R, ..., D] with lse_part [R, ...] into out [..., D] and lse_out [...]."""
    MergeCall(o_part, lse_part, out, lse_out)(_stream_handle(stream))


def _stream_handle(stream):
    """A hipStream_t handle as an int from a handle or a torch stream (None stays None)."""
    if stream is None:
        return None
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def workspace_clear(ws, *, stream=None):
    """Zero-fill a workspace tensor with the library's clear kernel on `stream`
    (default: the current stream); needed once for a new workspace."""
    torch = _torch()
    _check_tensors({"workspace": ws})
    s = _stream_handle(stream)
    if s is None:
        s = torch.cuda.current_stream(ws.device).cuda_stream
    rc = lib().cpdec_workspace_clear(ws.data_ptr(), ws.numel() * ws.element_size(), s)
    if rc != 0:
        raise CpdecError(rc, "cpdec_workspace_clear")
