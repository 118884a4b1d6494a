"""Longest-first launch order (cpdec_attn_order).

Large grids of unsplit shards are launched longest (shard, sequence) pair
first, from an order that a one-workgroup pre-pass writes into the
workspace.  The tests check that order entry by entry against its definition
(lengths non-increasing, ties in index order, every pair once, the shard
pointers of the pair), that every output equals the index-order launch of the
same inputs bit for bit (an explicit chunk length fixes the schedule; a unit's
arithmetic does not depend on when it runs), and that sampled groups meet the
oracle's bar, for both attention entry points.
"""
import sys

import numpy as np
import pytest

from oracle import workloads as ow
from synth import configs as sc
from tests.helpers import assert_lse, assert_out, run_path, to64

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
import lse_merge_split_amd as cp  # noqa: E402
from synth import gpu as sg  # noqa: E402

C = cp.STEP_COUNTER_BYTES

# Ordering applies from 2048 units and 4 GiB of K+V at capacity; the lengths
# are ragged in [0, capacity] with 5% empty pairs (the large ragged workload's
# recipe at a smaller batch), so the oracle checks sample groups.
CASES = {
    # 8 shards x 64 sequences x 8 kv heads = 4096 units, 4.3 GB of K+V
    "ragged GQA 4, 4096 units": sc.small("c4", B=64, Hq=32, Hkv=8, Lcap=2048),
    # 8 x 512 = 4096 (shard, sequence) pairs: the largest one-workgroup sort
    "ragged MHA, 4096 pairs": sc.small("c4", B=512, Hq=1, Hkv=1, D=64, Lcap=4096),
    # 3 x 700 = 2100 pairs, not a power of two (padded sort)
    "ragged 3 shards, 2100 pairs": sc.small("c4", R=3, B=700, Hq=2, Hkv=1, D=64, Lcap=8192),
    # equal lengths: the order is the index order
    "uniform lengths": sc.small("c3", B=32, Hq=32, Hkv=8, Lcap=4096, L=4096),
}


def _say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def _sample_groups(w, lens, n=12):
    """(b, h) groups to check against the oracle: the longest and the
    shortest sequences, one with an empty shard, and a seeded spread."""
    tot = lens.sum(axis=0)
    picks = {int(np.argmax(tot)), int(np.argmin(tot))}
    empty = np.where((lens == 0).any(axis=0))[0]
    if len(empty):
        picks.add(int(empty[0]))
    rng = np.random.default_rng(7)
    picks.update(int(b) for b in rng.choice(w.B, size=min(w.B, n), replace=False))
    return [(b, int(rng.integers(w.Hkv))) for b in sorted(picks)]


def _check_oracle(w, inp, res, what):
    for b, h in _sample_groups(w, inp["lens_np"]):
        ref = ow.group(w, inp["lens_np"], b, h)
        hs = slice(h * w.G, (h + 1) * w.G)
        assert_out(to64(res["o_part"][:, b, hs]), ref["o_part"], f"{what} o_part b={b} h={h}")
        assert_lse(to64(res["lse_part"][:, b, hs]), ref["lse_part"], f"{what} lse_part b={b} h={h}",
                   floor=True)
        assert_out(to64(res["out"][b, hs]), ref["out"], f"{what} out b={b} h={h}")
        assert_lse(to64(res["lse_out"][b, hs]), ref["lse_out"], f"{what} lse_out b={b} h={h}", floor=True)


def _check_entries(w, inp, ws):
    """The order entries against their definition."""
    n = w.R * w.B
    raw = ws[C:C + 32 * n].cpu().numpy().view(np.int32).reshape(n, 8)
    ptrs = ws[C:C + 32 * n].cpu().numpy().view(np.uint64).reshape(n, 4)
    r, b, L = raw[:, 4], raw[:, 5], raw[:, 6]
    lens = inp["lens_np"]
    idx = r.astype(np.int64) * w.B + b
    assert np.array_equal(np.sort(idx), np.arange(n)), "not a permutation of the pairs"
    assert np.array_equal(L, lens[r, b]), "entry lengths differ from lens"
    # longest first; equal lengths in index order
    expect = np.lexsort((np.arange(n), -lens.ravel().astype(np.int64)))
    assert np.array_equal(idx, expect), "order is not longest first with index tie-break"
    kp = np.array([t.data_ptr() for t in inp["k_shards"]], dtype=np.uint64)
    vp = np.array([t.data_ptr() for t in inp["v_shards"]], dtype=np.uint64)
    assert np.array_equal(ptrs[:, 0], kp[r]) and np.array_equal(ptrs[:, 1], vp[r])


@pytest.mark.parametrize("name", list(CASES))
def test_longest_first_attention(name):
    w = CASES[name]
    _say(f"longest first: {name}")
    inp = sg.attn_inputs(w)
    desc = cp.make_attn_desc(inp["q"], inp["k_shards"])
    plan = cp.attn_plan(desc)
    assert plan["longest_first"] and plan["num_chunks"] == 1
    fixed_desc = cp.make_attn_desc(inp["q"], inp["k_shards"], chunk_tokens=plan["chunk_tokens"])
    assert not cp.attn_plan(fixed_desc)["longest_first"]

    ws = torch.zeros(cp.attn_workspace_bytes(desc), dtype=torch.uint8, device="cuda")
    ordered = run_path(inp, workspace=ws)
    _check_entries(w, inp, ws)
    assert int(torch.count_nonzero(ws[:C]).item()) == 0, "counter region written"
    index_order = run_path(inp, chunk_tokens=plan["chunk_tokens"])
    for k in ordered:
        assert torch.equal(ordered[k], index_order[k]), f"{k} differs from the index-order launch"
    again = run_path(inp, workspace=ws)
    for k in ordered:
        assert torch.equal(ordered[k], again[k]), f"repeat: {k} differs"
    _check_oracle(w, inp, ordered, "ordered")


def test_longest_first_whole_step():
    """cpdec_cp_decode on an ordered grid: order pre-pass, attention and merge
    launches; the same bits as the two calls, counters left at zero."""
    w = CASES["ragged GQA 4, 4096 units"]
    _say("longest first: whole step")
    inp = sg.attn_inputs(w)
    desc = cp.make_attn_desc(inp["q"], inp["k_shards"])
    assert cp.step_launches(desc) == 3
    ws = torch.zeros(cp.step_workspace_bytes(desc), dtype=torch.uint8, device="cuda")
    q = inp["q"]
    o_part = torch.empty((w.R, w.B, w.Hq, w.D), dtype=torch.float32, device="cuda")
    lse_part = torch.empty((w.R, w.B, w.Hq), dtype=torch.float32, device="cuda")
    out = torch.empty((w.B, w.Hq, w.D), dtype=q.dtype, device="cuda")
    lo = torch.empty((w.B, w.Hq), dtype=torch.float32, device="cuda")
    cp.cp_decode(q, inp["k_shards"], inp["v_shards"], inp["lens"], o_part, lse_part, out, lo,
                 workspace=ws)
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(ws[:C]).item()) == 0
    _check_entries(w, inp, ws)
    two = run_path(inp)
    step = dict(o_part=o_part, lse_part=lse_part, out=out, lse_out=lo)
    for k in step:
        assert torch.equal(step[k], two[k]), f"{k} differs from the two calls"
    _check_oracle(w, inp, step, "step")
