"""Launch-planner invariants over seeded random descriptors (CPU only: the
plan and workspace queries make no HIP call).

For every descriptor the plan must cover the capacity with whole tiles, the
workspace sizes must hold the counter region plus what the plan writes, the
longest-first order must only go with unsplit shards and count as a launch,
and the launch counts must agree between the two queries.
"""
import ctypes

import numpy as np
import pytest

import lse_merge_split_amd as cp

C = cp.STEP_COUNTER_BYTES


def _desc(rng):
    d = cp.AttnDesc()
    D = int(rng.choice([64, 128, 256]))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.choice([1, 2, 4, 8, 16, 20, 32]))
    B = int(rng.choice([1, 2, 3, 8, 64, 256, 1000]))
    R = int(rng.choice([1, 2, 4, 8, 9, 16, 64]))
    cap = int(rng.choice([1, 31, 32, 100, 512, 4096, 16384, 300000, 1 << 20]))
    d.batch, d.num_q_heads, d.num_kv_heads, d.head_dim, d.num_shards = B, G * Hkv, Hkv, D, R
    d.kv_capacity = cap
    d.kv_stride_token, d.kv_stride_head, d.kv_stride_batch = D, cap * D, Hkv * cap * D
    d.sm_scale = 0.0
    d.qkv_dtype = int(rng.choice([cp.BF16, cp.F16]))
    d.opart_dtype = int(rng.choice([cp.F32, cp.F32, cp.BF16]))
    d.chunk_tokens = int(rng.choice([0, 0, 0, 32, 64, 256, 4096, 1 << 21]))
    return d


def _launches(fn, d):
    n = ctypes.c_int32(-1)
    assert fn(ctypes.byref(d), ctypes.byref(n)) == 0
    return n.value


@pytest.mark.parametrize("seed", range(8))
def test_plan_invariants(seed):
    rng = np.random.default_rng(1000 + seed)
    lib = cp.lib()
    checked = 0
    for _ in range(250):
        d = _desc(rng)
        c, n, wv = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        if lib.cpdec_attn_plan(ctypes.byref(d), ctypes.byref(c), ctypes.byref(n), ctypes.byref(wv)) != 0:
            continue  # a descriptor the ABI rejects (tested elsewhere)
        checked += 1
        chunk, nch, waves = c.value, n.value, wv.value
        cap = d.kv_capacity
        plan = cp.attn_plan(d)
        # whole tiles, the capacity covered exactly by nch chunks
        assert chunk % 32 == 0 and chunk > 0
        assert nch * chunk >= cap and (nch - 1) * chunk < cap
        assert waves in (1, 2, 4, 8)
        assert nch <= 256
        assert chunk <= 1 << 18  # short enough for the FP32 p.V accumulation
        if d.head_dim == 256:
            assert waves <= 4    # the 8-wave kernels at D = 256 spill registers
        if not d.chunk_tokens:
            assert nch <= 64     # more would leave only the three-launch step
        if d.chunk_tokens:  # as given, unless that makes more than 256 chunks
            if -(-cap // d.chunk_tokens) <= 256:
                assert chunk == min(d.chunk_tokens, 1 << 18)
            else:           # then the fewest whole tiles that give at most 256
                assert chunk == -(-(-(-cap // 256)) // 32) * 32
        # workspace: counters first, then what the plan writes
        ws_attn = lib.cpdec_attn_workspace_bytes(ctypes.byref(d))
        ws_step = lib.cpdec_step_workspace_bytes(ctypes.byref(d))
        assert ws_step >= C and ws_step >= ws_attn
        Gb = min(d.num_q_heads // d.num_kv_heads, 16)
        gblocks = -(-(d.num_q_heads // d.num_kv_heads) // 16)
        units = d.num_shards * d.batch * d.num_kv_heads * gblocks
        if nch > 1:
            slots = units * nch * Gb
            assert ws_attn >= C + slots * 4 + slots * d.head_dim * 4
        # the longest-first order only for unsplit shards, as one more launch
        attn_launches = _launches(lib.cpdec_attn_launches, d)
        step_launches = _launches(lib.cpdec_step_plan, d)
        assert plan["launches"] == attn_launches and cp.step_launches(d) == step_launches
        assert attn_launches in (1, 2) and step_launches in (1, 2, 3, 4)
        if plan["longest_first"]:
            assert nch == 1 and d.chunk_tokens == 0
            assert attn_launches == 2 and step_launches == 3
            assert ws_attn >= C + d.num_shards * d.batch * 32
        elif nch == 1:
            assert attn_launches == 1 and step_launches in (1, 2)
        else:
            assert step_launches in (1, 2, 3)
    assert checked > 50
