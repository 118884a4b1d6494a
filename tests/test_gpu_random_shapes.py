"""Seeded random shapes through every form of the path.

Shapes are drawn from a fixed seed over shards, batch, heads (MHA to GQA 24,
one or two head blocks), head dim, capacity, ragged or uniform lengths with
empty shards, element type, partial storage type and an optional chunk
length (a second, wider draw reaches 64 shards, GQA 32, one-token capacities
and fp16 partials), so the planner lands on every form: one launch (whole shards, split
shards, two levels), attention + row merge, attention + chunk combine +
merge, and cpdec_attn_partial with and without its in-launch chunk combine.
Each shape is checked against the oracle on every (sequence, kv head) group
(storage-aware oracle for 16-bit partials), and the whole step against the
two calls.  Sizes stay small so the oracle finishes in seconds.
"""
import sys

import numpy as np
import pytest

from oracle import workloads as ow
from synth import configs as sc
from tests.helpers import assert_lse, assert_out, assert_out_stored, run_path, to64

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
import lse_merge_split_amd as cp  # noqa: E402
from synth import gpu as sg  # noqa: E402

N_SHAPES = 24
N_WIDE = 60


def _shapes():
    rng = np.random.default_rng(20261203)
    out = []
    for i in range(N_SHAPES):
        R = int(rng.choice([1, 2, 3, 4, 5, 8, 11, 16]))
        Hkv = int(rng.choice([1, 2, 4]))
        G = int(rng.choice([1, 2, 3, 4, 8, 16, 24]))
        D = int(rng.choice([64, 128, 256]))
        B = int(rng.integers(1, 5))
        Lcap = int(rng.choice([33, 100, 257, 640, 1500]))
        ragged = bool(rng.integers(0, 2))
        dtype = str(rng.choice(["bf16", "fp16"]))
        opart = str(rng.choice(["fp32", "fp32", "bf16"]))
        chunk = int(rng.choice([0, 0, 0, 32, 64, 256]))
        w = sc.WORKLOADS["c4"].scaled(
            name=f"rand{i}", R=R, B=B, Hq=G * Hkv, Hkv=Hkv, D=D, dtype=dtype, Lcap=Lcap,
            ragged=ragged, L=0 if ragged else Lcap - int(rng.integers(0, 3)),
            empty_p=0.1 if ragged else 0.0, k_scale=float(rng.choice([1.0, 3.0])), seed=5000 + i)
        out.append((w, opart, chunk))
    # a wider draw: up to 64 shards, GQA up to 32 (and odd group sizes), capacities
    # from 1 token, fp16 partials, chunk lengths that are not powers of two
    rng = np.random.default_rng(20261204)
    wide = 0
    while wide < N_WIDE:
        R = int(rng.choice([1, 2, 3, 4, 5, 7, 8, 13, 16, 33, 64]))
        Hkv = int(rng.choice([1, 2, 3, 4, 8]))
        G = int(rng.choice([1, 2, 3, 4, 5, 8, 12, 16, 17, 24, 32]))
        D = int(rng.choice([64, 128, 256]))
        B = int(rng.integers(1, 7))
        Lcap = int(rng.choice([1, 5, 31, 32, 33, 64, 100, 257, 640, 1500, 3000, 5000]))
        ragged = bool(rng.integers(0, 2))
        dtype = str(rng.choice(["bf16", "fp16"]))
        opart = str(rng.choice(["fp32", "fp32", "bf16", "fp16"]))
        chunk = int(rng.choice([0, 0, 32, 32, 64, 96, 256, 1024]))
        L = max(0, Lcap - int(rng.integers(0, 3)))
        k_scale = float(rng.choice([1.0, 3.0]))
        if R * B * Hkv * G * D * Lcap > 60_000_000:   # keeps the oracle to seconds
            continue
        w = sc.WORKLOADS["c4"].scaled(
            name=f"wide{wide}", R=R, B=B, Hq=G * Hkv, Hkv=Hkv, D=D, dtype=dtype, Lcap=Lcap,
            ragged=ragged, L=0 if ragged else L, empty_p=0.15 if ragged else 0.0,
            k_scale=k_scale, seed=6000 + wide)
        out.append((w, opart, chunk))
        wide += 1
    # forms the draws may miss: more than 64 chunks (chunk-combine launch in both
    # entry points), and the two-level one launch with 32- and 16-bit partials
    out.append((sc.small("c4", R=2, B=1, Hq=8, Hkv=2, Lcap=2500, seed=5100), "fp32", 32))
    out.append((sc.small("c4", B=2, Hq=32, Lcap=512, seed=5101), "fp32", 0))
    out.append((sc.small("c4", B=2, Hq=32, Lcap=512, dtype="fp16", seed=5102), "fp16", 0))
    return out


SHAPES = _shapes()
N_SHAPES = len(SHAPES)


def _id(i):
    w, opart, chunk = SHAPES[i]
    return (f"{i}:R{w.R}B{w.B}Hq{w.Hq}Hkv{w.Hkv}D{w.D}cap{w.Lcap}{'r' if w.ragged else 'u'}"
            f"{w.dtype}/{opart}c{chunk}")


def _check(w, inp, res, opart, what):
    for b in range(w.B):
        for h in range(w.Hkv):
            ref = ow.group(w, inp["lens_np"], b, h)
            hs = slice(h * w.G, (h + 1) * w.G)
            if opart == "fp32":
                assert_out(to64(res["out"][b, hs]), ref["out"], f"{what} out b={b} h={h}")
            else:  # the exact partials rounded to the storage type, merged exactly
                assert_out_stored(to64(res["out"][b, hs]), ref["o_part"], ref["lse_part"], opart,
                                  f"{what} out b={b} h={h}")
            assert_out(to64(res["o_part"][:, b, hs]), ref["o_part"], f"{what} o_part b={b} h={h}")
            assert_lse(to64(res["lse_part"][:, b, hs]), ref["lse_part"], f"{what} lse_part b={b} h={h}",
                       floor=True)
            assert_lse(to64(res["lse_out"][b, hs]), ref["lse_out"], f"{what} lse_out b={b} h={h}", floor=True)


@pytest.mark.parametrize("i", range(N_SHAPES), ids=_id)
def test_random_shape(i):
    w, opart, chunk = SHAPES[i]
    print(f"[case] random shape {_id(i)}", flush=True)
    sys.stdout.flush()
    inp = sg.attn_inputs(w)
    q = inp["q"]
    o_dt = sg.torch_dtype(opart)
    desc = cp.make_attn_desc(q, inp["k_shards"], opart_dtype=o_dt, chunk_tokens=chunk)
    plan = cp.attn_plan(desc)
    print(f"[case]   plan {plan}, step launches {cp.step_launches(desc)}", flush=True)
    two = run_path(inp, o_dtype=o_dt, chunk_tokens=chunk)
    _check(w, inp, two, opart, "two calls")
    ws = torch.zeros(cp.step_workspace_bytes(desc), dtype=torch.uint8, device="cuda")
    step = dict(o_part=torch.empty_like(two["o_part"]), lse_part=torch.empty_like(two["lse_part"]),
                out=torch.empty_like(two["out"]), lse_out=torch.empty_like(two["lse_out"]))
    cp.cp_decode(q, inp["k_shards"], inp["v_shards"], inp["lens"], step["o_part"], step["lse_part"],
                 step["out"], step["lse_out"], chunk_tokens=chunk, workspace=ws)
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(ws[:cp.STEP_COUNTER_BYTES]).item()) == 0
    _check(w, inp, step, opart, "step")
    # the two forms compute the same partials up to FP32 summation order
    assert torch.equal(torch.isneginf(step["lse_part"]), torch.isneginf(two["lse_part"]))
    fin = torch.isfinite(two["lse_part"])
    assert torch.allclose(step["lse_part"][fin], two["lse_part"][fin], rtol=1e-6, atol=1e-6)
