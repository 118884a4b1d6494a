"""The C ABI on a CPU host: the library loads, exports every function that
include/cpdec.h declares, and rejects bad arguments before any HIP call."""
import ctypes
import os
import re

import pytest

import lse_merge_split_amd as cp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, INVALID, UNSUPPORTED, ALIGN, WS = 0, 1, 2, 3, 4


def _declared():
    txt = open(os.path.join(ROOT, "include", "cpdec.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(cpdec_[a-z_]+)\s*\(", txt)))


def test_every_declared_symbol_is_exported():
    lib = cp.lib()
    names = _declared()
    assert {"cpdec_attn_partial", "cpdec_lse_merge", "cpdec_attn_workspace_bytes",
            "cpdec_workspace_clear", "cpdec_status_string", "cpdec_version"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings_and_version():
    lib = cp.lib()
    for code, name in cp.STATUS.items():
        assert lib.cpdec_status_string(code).decode() == name
    assert lib.cpdec_status_string(99).decode() == "CPDEC_ERR_UNKNOWN"
    assert b"gfx950" in lib.cpdec_version()


def _desc(**kw):
    d = cp.AttnDesc()
    d.batch, d.num_q_heads, d.num_kv_heads, d.head_dim, d.num_shards = 2, 8, 2, 128, 4
    d.kv_capacity = 1000
    d.kv_stride_token, d.kv_stride_head = 128, 1000 * 128
    d.kv_stride_batch = 2 * 1000 * 128
    d.sm_scale, d.qkv_dtype, d.opart_dtype, d.chunk_tokens = 0.0, cp.BF16, cp.F32, 0
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def test_workspace_bytes():
    lib = cp.lib()
    C = cp.STEP_COUNTER_BYTES
    one = _desc(chunk_tokens=1024)   # a single chunk covers the capacity
    assert lib.cpdec_attn_workspace_bytes(ctypes.byref(one)) == 0
    assert lib.cpdec_step_workspace_bytes(ctypes.byref(one)) == C  # counters only
    split = _desc(chunk_tokens=128)  # 8 chunks -> partials after the counter region
    nb = lib.cpdec_attn_workspace_bytes(ctypes.byref(split))
    units, nch, Gb, D = 4 * 2 * 2, 8, 4, 128
    assert nb >= C + units * nch * Gb * (D + 1) * 4
    assert lib.cpdec_step_workspace_bytes(ctypes.byref(split)) == nb
    for f in (lib.cpdec_attn_workspace_bytes, lib.cpdec_step_workspace_bytes):
        assert f(None) == 0
        assert f(ctypes.byref(_desc(head_dim=96))) == 0


def test_step_plan_launches():
    assert cp.step_launches(_desc(chunk_tokens=1024)) == 1     # shards merged in the launch
    assert cp.step_launches(_desc(chunk_tokens=128)) == 1      # chunks and shards in the launch
    # 16 heads x 256/4 vectors per shard: more than one merging workgroup's threads
    wide = dict(num_q_heads=32, num_kv_heads=2, head_dim=256, kv_stride_token=256,
                kv_stride_head=1000 * 256, kv_stride_batch=2 * 1000 * 256)
    # split, 16 heads x 64 vectors beyond the workgroup: attention, then one kernel that
    # combines the chunks and merges the shards per (sequence, query head)
    assert cp.step_launches(_desc(chunk_tokens=128, **wide)) == 2
    # split, 4 heads x 32 vectors fit, 8 shards do not: two levels in the one launch
    # (chunk combine per unit, shard merge per group)
    assert cp.step_launches(_desc(chunk_tokens=128, num_shards=8)) == 1
    assert cp.step_launches(_desc(chunk_tokens=1024, **wide)) == 2  # attention, merge
    # more than 16 chunks per shard: two levels; more than 64 (shards x chunks beyond one
    # wave): attention, combine, merge
    assert cp.step_launches(_desc(chunk_tokens=32)) == 1
    long = dict(kv_capacity=4096, kv_stride_head=4096 * 128, kv_stride_batch=2 * 4096 * 128)
    assert cp.step_launches(_desc(chunk_tokens=32, **long)) == 3
    # two levels need a counter line per unit and per group (at most 1024 lines); beyond,
    # attention + the per-row combine-and-merge kernel (8 shards x 8 chunks = one wave)
    many8 = dict(num_shards=8, batch=100, kv_stride_batch=2 * 1000 * 128)
    assert cp.step_launches(_desc(chunk_tokens=128, **many8)) == 2
    many8_long = dict(many8, kv_capacity=2000, kv_stride_head=2000 * 128,
                      kv_stride_batch=2 * 2000 * 128)
    assert cp.step_launches(_desc(chunk_tokens=128, **many8_long)) == 3  # 8 x 16 chunks
    # more than 8 whole shards
    assert cp.step_launches(_desc(chunk_tokens=1024, num_shards=9)) == 2
    # more (sequence, kv head) groups than counters
    many = dict(batch=8193, kv_stride_batch=2 * 1000 * 128)
    assert cp.step_launches(_desc(chunk_tokens=1024, **many)) == 2  # attention, merge
    n = ctypes.c_int32(-1)
    assert cp.lib().cpdec_step_plan(ctypes.byref(_desc(head_dim=96)), ctypes.byref(n)) == UNSUPPORTED
    assert n.value == -1
    assert cp.lib().cpdec_step_plan(None, None) == INVALID


def _attn_launches(d):
    n = ctypes.c_int32(-1)
    rc = cp.lib().cpdec_attn_launches(ctypes.byref(d), ctypes.byref(n))
    return rc, n.value


def test_attn_partial_launches():
    """cpdec_attn_partial: one launch, the chunk combine inside it when shards
    are split (at most 64 chunks, 1024 units); a combine launch beyond."""
    assert _attn_launches(_desc(chunk_tokens=1024)) == (OK, 1)   # one chunk
    assert _attn_launches(_desc(chunk_tokens=128)) == (OK, 1)    # 8 chunks, combined in the launch
    long = dict(kv_capacity=4096, kv_stride_head=4096 * 128, kv_stride_batch=2 * 4096 * 128)
    assert _attn_launches(_desc(chunk_tokens=64, **long)) == (OK, 1)   # 64 chunks
    assert _attn_launches(_desc(chunk_tokens=32, **long)) == (OK, 2)   # 128 chunks: combine launch
    many = dict(batch=200, kv_stride_batch=2 * 1000 * 128)              # 4 x 200 x 2 = 1600 units
    assert _attn_launches(_desc(chunk_tokens=128, **many)) == (OK, 2)
    assert cp.attn_plan(_desc(chunk_tokens=128))["launches"] == 1
    assert _attn_launches(_desc(head_dim=96)) == (UNSUPPORTED, -1)
    assert cp.lib().cpdec_attn_launches(None, None) == INVALID


def _order(d):
    lf = ctypes.c_int32(-1)
    rc = cp.lib().cpdec_attn_order(ctypes.byref(d), ctypes.byref(lf))
    return rc, lf.value


def test_longest_first_order_plan():
    """Longest-first launch order: large unsplit grids when the library picks
    the schedule; the order entries (32 bytes per (shard, sequence) pair)
    follow the counter region, and the pre-pass is one more launch."""
    C = cp.STEP_COUNTER_BYTES
    lib = cp.lib()
    # 8 shards x 64 sequences x 8 kv heads = 4096 units, 8192 tokens per shard (unsplit)
    big = dict(batch=64, num_q_heads=32, num_kv_heads=8, num_shards=8, kv_capacity=8192,
               kv_stride_head=8192 * 128, kv_stride_batch=8 * 8192 * 128)
    d = _desc(**big)
    assert _order(d) == (OK, 1)
    assert cp.attn_plan(d)["num_chunks"] == 1 and cp.attn_plan(d)["longest_first"]
    assert lib.cpdec_attn_workspace_bytes(ctypes.byref(d)) == C + 8 * 64 * 32
    assert lib.cpdec_step_workspace_bytes(ctypes.byref(d)) == C + 8 * 64 * 32
    assert cp.step_launches(d) == 3  # order pre-pass, attention, merge
    assert _attn_launches(d) == (OK, 2)  # order pre-pass, attention
    # an explicit chunk length fixes the schedule: index order, no workspace
    fixed = _desc(chunk_tokens=8192, **big)
    assert _order(fixed) == (OK, 0)
    assert lib.cpdec_attn_workspace_bytes(ctypes.byref(fixed)) == 0
    assert cp.step_launches(fixed) == 2
    # fewer than 2048 units (here 1024 = 8 x 16 x 8): index order
    small = dict(big, batch=16, kv_stride_batch=8 * 8192 * 128)
    assert _order(_desc(**small)) == (OK, 0)
    # more than 4096 (shard, sequence) pairs: index order
    many = dict(big, batch=513, num_kv_heads=1, num_q_heads=4, kv_stride_batch=8192 * 128)
    assert _order(_desc(**many)) == (OK, 0)
    ok = dict(many, batch=512)
    assert _order(_desc(**ok)) == (OK, 1)
    # under 4 GiB of K and V at capacity (8 x 64 x 8 x 512 tokens x 512 B = 1 GiB): index order
    short = dict(big, kv_capacity=512, kv_stride_head=512 * 128, kv_stride_batch=8 * 512 * 128)
    assert cp.attn_plan(_desc(**short))["num_chunks"] == 1
    assert _order(_desc(**short)) == (OK, 0)
    # split shards never reorder
    assert _order(_desc()) == (OK, 0)
    # descriptor errors, output untouched
    assert _order(_desc(head_dim=96)) == (UNSUPPORTED, -1)
    assert lib.cpdec_attn_order(None, None) == INVALID


# Fake (never dereferenced) device addresses.  Every call below must fail
# validation, which runs before any HIP call; with a GPU visible a wrong
# acceptance would launch a kernel on these addresses, so the cases run only
# on hosts without a GPU.
def _no_gpu():
    try:
        import torch
        return torch.cuda.device_count() == 0
    except Exception:
        return True


needs_cpu_host = pytest.mark.skipif(not _no_gpu(), reason="fake-pointer cases run on GPU-less hosts")
A = 1 << 20  # aligned fake address


def _attn(d, q=A, k=A, v=A, lens=A, o=A, lse=A, ws=None, wsb=0, R=None):
    if R is None and d is not None:
        R = max(d.num_shards, 1)
    R = 1 if d is None else R
    ks = (ctypes.c_void_p * max(R, 1))(*([k] * max(R, 1)))
    vs = (ctypes.c_void_p * max(R, 1))(*([v] * max(R, 1)))
    return cp.lib().cpdec_attn_partial(ctypes.byref(d) if d is not None else None, q, ks, vs,
                                       lens, o, lse, ws, wsb, None)


@needs_cpu_host
@pytest.mark.parametrize("case,code", [
    (dict(batch=0), INVALID), (dict(num_q_heads=7), INVALID), (dict(num_kv_heads=0), INVALID),
    (dict(num_shards=0), INVALID), (dict(num_shards=65), INVALID), (dict(kv_capacity=-1), INVALID),
    (dict(head_dim=96), UNSUPPORTED), (dict(head_dim=512), UNSUPPORTED),
    (dict(qkv_dtype=cp.F32), UNSUPPORTED), (dict(opart_dtype=7), UNSUPPORTED),
    (dict(kv_stride_token=64), INVALID), (dict(kv_stride_token=132), ALIGN),
    (dict(kv_stride_head=1000 * 128 + 4), ALIGN), (dict(chunk_tokens=100), INVALID),
    (dict(sm_scale=-1.0), INVALID), (dict(sm_scale=float("inf")), INVALID),
])
def test_attn_descriptor_errors(case, code):
    kw = dict(chunk_tokens=1024)
    kw.update(case)
    assert _attn(_desc(**kw)) == code


@needs_cpu_host
def test_attn_pointer_errors():
    d = _desc(chunk_tokens=1024)
    assert _attn(None) == INVALID
    assert _attn(d, q=None) == INVALID
    assert _attn(d, k=None) == INVALID
    assert _attn(d, lens=None) == INVALID
    assert _attn(d, o=None) == INVALID
    assert _attn(d, lse=None) == INVALID
    assert _attn(d, q=A + 8) == ALIGN
    assert _attn(d, k=A + 2) == ALIGN
    assert _attn(d, v=A + 4) == ALIGN
    assert _attn(d, o=A + 4) == ALIGN
    assert _attn(d, lse=A + 2) == ALIGN
    split = _desc(chunk_tokens=128)
    need = cp.lib().cpdec_attn_workspace_bytes(ctypes.byref(split))
    assert _attn(split) == WS
    assert _attn(split, ws=A, wsb=need - 1) == WS
    assert _attn(split, ws=A + 16, wsb=need) == WS


@needs_cpu_host
def test_cp_decode_errors():
    d = _desc(chunk_tokens=1024)
    f = cp.lib().cpdec_cp_decode
    ks = (ctypes.c_void_p * 4)(*([A] * 4))
    assert f(ctypes.byref(d), A, ks, ks, A, A, A, None, A, None, 0, None) == INVALID
    assert f(ctypes.byref(d), A, ks, ks, A, A, A, A + 8, A, None, 0, None) == ALIGN
    assert f(ctypes.byref(d), A, ks, ks, A, A, A, A, A + 2, None, 0, None) == ALIGN
    bad = _desc(chunk_tokens=1024, head_dim=96)
    assert f(ctypes.byref(bad), A, ks, ks, A, A, A, A, A, None, 0, None) == UNSUPPORTED
    split = _desc(chunk_tokens=128)
    assert f(ctypes.byref(split), A, ks, ks, A, A, A, A, A, None, 0, None) == WS
    # the whole step needs the counter region even when nothing is split
    assert f(ctypes.byref(d), A, ks, ks, A, A, A, A, A, None, 0, None) == WS
    assert f(ctypes.byref(d), A, ks, ks, A, A, A, A, A, A, cp.STEP_COUNTER_BYTES - 1, None) == WS
    assert f(ctypes.byref(d), A, ks, ks, A, A, A, A, A, A + 16, cp.STEP_COUNTER_BYTES, None) == WS
    # separate launches whose merge would need offsets past 2 GiB: 65536 x 64 rows x 128 x 4 B
    huge = _desc(batch=65536, num_q_heads=64, num_kv_heads=8, kv_capacity=64, kv_stride_token=128,
                 kv_stride_head=64 * 128, kv_stride_batch=8 * 64 * 128, chunk_tokens=64)
    assert cp.step_launches(huge) == 2
    n = cp.step_workspace_bytes(huge)
    assert f(ctypes.byref(huge), A, ks, ks, A, A, A, A, A, A, n, None) == UNSUPPORTED
    # the same rows in 16 bits fit
    huge16 = _desc(batch=65536, num_q_heads=64, num_kv_heads=8, kv_capacity=64, kv_stride_token=128,
                   kv_stride_head=64 * 128, kv_stride_batch=8 * 64 * 128, chunk_tokens=64)
    huge16.opart_dtype = cp.BF16
    assert cp.attn_plan(huge16)["num_chunks"] == 1


@needs_cpu_host
def test_cp_decode_noalloc_errors():
    """The allocation-free step checks everything before its first HIP call
    (the scratch lookup): argument errors as cpdec_cp_decode, and WORKSPACE
    for a step that needs more than CPDEC_NOALLOC_SCRATCH_BYTES."""
    f = cp.lib().cpdec_cp_decode_noalloc
    d = _desc(chunk_tokens=1024)
    ks = (ctypes.c_void_p * 4)(*([A] * 4))
    assert f(None, A, ks, ks, A, A, A, A, A, None) == INVALID
    assert f(ctypes.byref(d), A, ks, ks, A, A, A, None, A, None) == INVALID
    assert f(ctypes.byref(d), None, ks, ks, A, A, A, A, A, None) == INVALID
    assert f(ctypes.byref(d), A, ks, ks, A, A, A, A + 8, A, None) == ALIGN
    assert f(ctypes.byref(d), A, ks, ks, A, A, A, A, A + 2, None) == ALIGN
    assert f(ctypes.byref(_desc(chunk_tokens=1024, head_dim=96)), A, ks, ks, A, A, A, A, A,
             None) == UNSUPPORTED
    # 8 shards x 16 heads at D = 256 in 256 chunks of 32 tokens: 33.8 MB of chunk partials
    big = _desc(batch=1, num_q_heads=16, num_kv_heads=1, head_dim=256, num_shards=8,
                kv_capacity=8192, kv_stride_token=256, kv_stride_head=8192 * 256,
                kv_stride_batch=8192 * 256, chunk_tokens=32)
    assert cp.step_workspace_bytes(big) > cp.NOALLOC_SCRATCH_BYTES
    ks8 = (ctypes.c_void_p * 8)(*([A] * 8))
    assert f(ctypes.byref(big), A, ks8, ks8, A, A, A, A, A, None) == WS
    # the scratch size the header states is the one the binding assumes
    txt = open(os.path.join(ROOT, "include", "cpdec.h")).read()
    assert "#define CPDEC_NOALLOC_SCRATCH_BYTES (16u << 20)" in txt
    assert cp.NOALLOC_SCRATCH_BYTES == 16 << 20


@needs_cpu_host
def test_merge_errors():
    m = cp.lib().cpdec_lse_merge
    assert m(None, A, 4, 10, 128, cp.BF16, cp.BF16, A, A, None) == INVALID
    assert m(A, None, 4, 10, 128, cp.BF16, cp.BF16, A, A, None) == INVALID
    assert m(A, A, 4, 10, 128, cp.BF16, cp.BF16, None, A, None) == INVALID
    assert m(A, A, 0, 10, 128, cp.BF16, cp.BF16, A, A, None) == INVALID
    assert m(A, A, 65, 10, 128, cp.BF16, cp.BF16, A, A, None) == INVALID
    assert m(A, A, 4, -1, 128, cp.BF16, cp.BF16, A, A, None) == INVALID
    assert m(A, A, 4, 10, 96, cp.BF16, cp.BF16, A, A, None) == UNSUPPORTED
    assert m(A, A, 4, 10, 1024, cp.BF16, cp.BF16, A, A, None) == UNSUPPORTED
    assert m(A, A, 4, 10, 128, 5, cp.BF16, A, A, None) == UNSUPPORTED
    assert m(A, A, 4, 10, 128, cp.BF16, 9, A, A, None) == UNSUPPORTED
    assert m(A + 8, A, 4, 10, 128, cp.BF16, cp.BF16, A, A, None) == ALIGN
    assert m(A, A, 4, 10, 128, cp.BF16, cp.BF16, A + 8, A, None) == ALIGN
    assert m(A, A + 2, 4, 10, 128, cp.BF16, cp.BF16, A, A, None) == ALIGN
    assert m(A, A, 4, 10, 128, cp.BF16, cp.BF16, A, A + 1, None) == ALIGN
    assert m(A, A, 4, 0, 128, cp.BF16, cp.BF16, A, None, None) == OK  # nothing enqueued


@needs_cpu_host
def test_workspace_clear_errors():
    c = cp.lib().cpdec_workspace_clear
    assert c(None, 0, None) == OK
    assert c(None, 256, None) == INVALID
    assert c(A + 16, 256, None) == ALIGN


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(cp, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(cp, "_LIB", None)
    with pytest.raises(RuntimeError, match="missing"):
        cp.lib()
