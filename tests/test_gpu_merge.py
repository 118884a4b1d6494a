"""GPU parity of cpdec_lse_merge against the oracle, plus the merge's exact pins.

Every case prints its name before it runs (flushed), so a run that dies names
the case it died in."""
import math
import sys

import numpy as np
import pytest

from oracle import oracle
from oracle import workloads as ow
from synth import configs as sc
from tests.helpers import assert_lse, assert_out, to64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import lse_merge_split_amd as cp  # noqa: E402

DEV = "cuda"
TDT = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}


def _say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def make_case(R, rows, D, in_dt, seed, empty_p=0.1, sigma=4.0, all_empty=()):
    rng = np.random.default_rng(seed)
    o_host = torch.from_numpy(rng.normal(size=(R, rows, D)).astype(np.float32)).to(TDT[in_dt])
    lse = (rng.normal(size=(R, rows)) * sigma).astype(np.float32)
    lse[rng.random((R, rows)) < empty_p] = -np.inf
    for n in all_empty:
        lse[:, n] = -np.inf
    return o_host, lse


def run_merge(o_host, lse, out_dt, with_lse=True):
    R, rows, D = o_host.shape
    o = o_host.to(DEV)
    l = torch.from_numpy(lse).to(DEV)
    out = torch.empty((rows, D), dtype=TDT[out_dt], device=DEV)
    lo = torch.empty(rows, dtype=torch.float32, device=DEV) if with_lse else None
    cp.lse_merge(o, l, out, lo)
    torch.cuda.synchronize()
    return out, lo


@pytest.mark.parametrize("in_dt", ["fp32", "fp16", "bf16"])
@pytest.mark.parametrize("out_dt", ["fp32", "fp16", "bf16"])
def test_merge_dtypes(in_dt, out_dt):
    _say(f"merge dtypes {in_dt}->{out_dt}")
    o_host, lse = make_case(5, 37, 128, in_dt, seed=1, all_empty=(3, 20))
    out, lo = run_merge(o_host, lse, out_dt)
    ref, ref_lse = oracle.merge_rows(o_host.double().numpy(), lse)
    assert_out(to64(out), ref)
    assert_lse(to64(lo), ref_lse)


@pytest.mark.parametrize("D", [64, 128, 256, 512])
@pytest.mark.parametrize("in_dt", ["fp32", "bf16"])
def test_merge_head_dims(D, in_dt):
    _say(f"merge D={D} {in_dt}")
    o_host, lse = make_case(8, 133, D, in_dt, seed=D)
    out, lo = run_merge(o_host, lse, "bf16")
    ref, ref_lse = oracle.merge_rows(o_host.double().numpy(), lse)
    assert_out(to64(out), ref)
    assert_lse(to64(lo), ref_lse)


@pytest.mark.parametrize("R", [1, 2, 3, 4, 5, 8, 9, 13, 32, 33, 64])
def test_merge_shard_counts(R):
    """Shard counts on both sides of each load-batch size (2 shards per batch
    up to R = 2, 4 up to R = 32, else 8)."""
    _say(f"merge R={R}")
    o_host, lse = make_case(R, 70, 128, "bf16", seed=100 + R, empty_p=0.2, sigma=16.0)
    out, lo = run_merge(o_host, lse, "bf16")
    ref, ref_lse = oracle.merge_rows(o_host.double().numpy(), lse)
    assert_out(to64(out), ref)
    assert_lse(to64(lo), ref_lse)


@pytest.mark.parametrize("R", [2, 4, 33])
@pytest.mark.parametrize("D,in_dt", [(64, "fp32"), (64, "bf16"), (256, "fp32")])
def test_merge_batch_sizes_across_row_widths(R, D, in_dt):
    """Each load-batch size with rows of 128 B to 1 KB (4 to 16 rows or 1 row
    per wave), 20% empty shards, ragged row count."""
    _say(f"merge R={R} D={D} {in_dt}")
    o_host, lse = make_case(R, 301, D, in_dt, seed=500 + R + D, empty_p=0.2, sigma=8.0)
    out, lo = run_merge(o_host, lse, "fp16")
    ref, ref_lse = oracle.merge_rows(o_host.double().numpy(), lse)
    assert_out(to64(out), ref)
    assert_lse(to64(lo), ref_lse)


def test_merge_single_shard_is_identity_bitwise():
    _say("merge R=1 identity")
    o_host, lse = make_case(1, 64, 512, "bf16", seed=3, empty_p=0.0)
    out, lo = run_merge(o_host, lse, "bf16")
    assert torch.equal(out.cpu(), o_host[0])
    assert np.array_equal(lo.cpu().numpy(), lse[0])
    o32, l32 = make_case(1, 64, 128, "fp32", seed=4, empty_p=0.0)
    out, lo = run_merge(o32, l32, "bf16")
    assert torch.equal(out.cpu(), o32[0].to(torch.bfloat16))  # one RNE rounding


def test_merge_empty_shard_insertion_bitwise_and_no_nan_leak():
    _say("merge empty-shard insertion")
    o_host, lse = make_case(4, 96, 256, "bf16", seed=5, empty_p=0.0)
    base, base_l = run_merge(o_host, lse, "bf16")
    for pos in (0, 2, 4):
        o2 = torch.cat([o_host[:pos], torch.full_like(o_host[:1], float("nan")), o_host[pos:]])
        l2 = np.concatenate([lse[:pos], np.full((1, 96), -np.inf, np.float32), lse[pos:]])
        out, lo = run_merge(o2, l2, "bf16")
        assert torch.isfinite(out.float()).all()
        assert torch.equal(out.cpu(), base.cpu()) and torch.equal(lo.cpu(), base_l.cpu())


def test_merge_all_empty_rows_and_lse_none():
    _say("merge all-empty rows")
    o_host, lse = make_case(3, 10, 64, "fp32", seed=6, empty_p=0.0, all_empty=range(10))
    o_host[:] = float("nan")
    out, lo = run_merge(o_host, lse, "fp16")
    assert torch.equal(out.cpu(), torch.zeros(10, 64, dtype=torch.float16))
    assert torch.isneginf(lo.cpu()).all()
    out2, none = run_merge(o_host, lse, "fp16", with_lse=False)
    assert none is None and torch.equal(out2.cpu(), out.cpu())


def test_merge_equal_lse_and_dominant():
    _say("merge closed forms")
    R, rows, D = 4, 16, 128
    o_host, _ = make_case(R, rows, D, "fp32", seed=7)
    lse = np.full((R, rows), 2.5, np.float32)
    out, lo = run_merge(o_host, lse, "fp32")
    assert np.allclose(to64(out), o_host.double().numpy().mean(0), rtol=1e-6, atol=1e-6)
    assert np.allclose(to64(lo), 2.5 + math.log(R), rtol=1e-7)
    lse = np.full((R, rows), -200.0, np.float32)
    lse[2] = 10.0   # e^-210 underflows even float64 products with o: shard 2 carries all weight
    out, lo = run_merge(o_host, lse, "fp32")
    assert torch.equal(out.cpu(), o_host[2]) and np.all(lo.cpu().numpy() == 10.0)


def test_merge_permutation_and_subnormal_weights():
    _say("merge permutation / subnormal gaps")
    R, rows, D = 6, 40, 128
    o_host, lse = make_case(R, rows, D, "bf16", seed=8, empty_p=0.1)
    # gaps of 87..104 put the small weights in or below the fp32 subnormal range
    lse[1:3] = lse[0] - np.linspace(87, 104, rows, dtype=np.float32)[None, :]
    out, lo = run_merge(o_host, lse, "bf16")
    ref, ref_lse = oracle.merge_rows(o_host.double().numpy(), lse)
    assert_out(to64(out), ref)
    assert_lse(to64(lo), ref_lse)
    perm = np.random.default_rng(0).permutation(R)
    out_p, lo_p = run_merge(o_host[perm], lse[perm], "bf16")
    assert_out(to64(out_p), ref)
    assert_lse(to64(lo_p), ref_lse)


def test_merge_full_workload_c5():
    """Merge-only workload at full size (8 x 65536 rows x 512, bf16): every row
    checked for the merge's bounds, sampled rows against the oracle."""
    from synth import gpu as sg
    w = sc.WORKLOADS["c5"]
    _say("merge full c5")
    inp = sg.merge_inputs(w)
    out = torch.empty((w.rows, w.D), dtype=torch.bfloat16, device=DEV)
    lo = torch.empty(w.rows, dtype=torch.float32, device=DEV)
    cp.lse_merge(inp["o_part"], inp["lse_part"], out, lo)
    torch.cuda.synchronize()
    lse_np = inp["lse_np"]
    lo_np = to64(lo)
    fin = np.isfinite(lse_np).any(axis=0)
    M = np.where(fin, np.max(np.where(np.isfinite(lse_np), lse_np, -np.inf), axis=0), -np.inf)
    assert np.array_equal(np.isneginf(lo_np), ~fin)
    nlive = np.isfinite(lse_np).sum(axis=0)
    assert np.all(lo_np[fin] >= M[fin] - 1e-5 * np.abs(M[fin]))
    assert np.all(lo_np[fin] <= M[fin] + np.log(nlive[fin]) + 1e-5 * np.abs(M[fin]) + 1e-6)
    assert torch.isfinite(out.float()).all()
    rows = np.random.default_rng(55).choice(w.rows, size=1024, replace=False)
    rows = np.unique(np.concatenate([rows, np.where(~fin)[0][:4], [0, w.rows - 1]]))
    ref, ref_lse = ow.merge_rows(w, rows)
    assert_out(to64(out[torch.from_numpy(rows).to(DEV)]), ref)
    assert_lse(lo_np[rows], ref_lse)
