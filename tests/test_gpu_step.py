"""cpdec_cp_decode (the whole step in two launches) against the oracle and
against the two-call path (cpdec_attn_partial + cpdec_lse_merge)."""
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

CASES = {
    "c1 (split)": sc.WORKLOADS["c1"],
    "c2 (split)": sc.WORKLOADS["c2"],
    "ragged GQA 8 (split)": sc.small("c4", B=16, Lcap=512),
    "ragged GQA 8 (unsplit)": sc.small("c4", B=64, Lcap=512),
    "D256 G20 (split)": sc.small("c3", R=3, B=2, Hq=40, Hkv=2, D=256, Lcap=300, L=290),
    "fp16 (split)": sc.small("c4", B=4, Lcap=256, dtype="fp16"),
    "D64 G3 (split)": sc.small("c3", R=5, B=3, Hq=6, Hkv=2, D=64, Lcap=97, L=97),
}


def run_step(inp, chunk_tokens=0):
    q = inp["q"]
    R = len(inp["k_shards"])
    B, Hq, D = q.shape
    o_part = torch.empty((R, B, Hq, D), dtype=torch.float32, device=q.device)
    lse_part = torch.empty((R, B, Hq), dtype=torch.float32, device=q.device)
    out = torch.empty((B, Hq, D), dtype=q.dtype, device=q.device)
    lo = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    cp.cp_decode(q, inp["k_shards"], inp["v_shards"], inp["lens"], o_part, lse_part, out, lo,
                 chunk_tokens=chunk_tokens)
    torch.cuda.synchronize()
    return dict(o_part=o_part, lse_part=lse_part, out=out, lse_out=lo)


@pytest.mark.parametrize("name", list(CASES))
def test_step_matches_oracle_and_two_calls(name):
    w = CASES[name]
    print(f"[case] step {name}", flush=True)
    sys.stdout.flush()
    inp = sg.attn_inputs(w)
    step = run_step(inp)
    two = run_path(inp)
    # same per-shard statistics; the chunk sums may be split over a different
    # number of thread groups, so o_part agrees to FP32 rounding
    assert torch.equal(step["lse_part"], two["lse_part"])
    assert torch.allclose(step["o_part"], two["o_part"], rtol=1e-5, atol=1e-6)
    for b in range(w.B):
        for h in range(w.Hkv):
            ref = ow.group(w, inp["lens_np"], b, h)
            hs = slice(h * w.G, (h + 1) * w.G)
            assert_out(to64(step["o_part"][:, b, hs]), ref["o_part"], f"o_part b={b} h={h}")
            assert_out(to64(step["out"][b, hs]), ref["out"], f"out b={b} h={h}")
            assert_lse(to64(step["lse_out"][b, hs]), ref["lse_out"], f"lse_out b={b} h={h}")


def test_step_empty_shards_and_sequences():
    w = sc.small("c4", B=3, Lcap=200, Hq=16, Hkv=4, R=3)
    print("[case] step empty shards", flush=True)
    inp = sg.attn_inputs(w)
    lens = inp["lens_np"].copy()
    lens[:, 1] = 0
    lens[2, 0] = 0
    lens[0, 2] = 1
    inp["lens_np"] = lens
    inp["lens"] = torch.from_numpy(lens).cuda()
    for chunk in (32, 0):
        step = run_step(inp, chunk_tokens=chunk)
        assert torch.count_nonzero(step["out"][1]).item() == 0
        assert torch.isneginf(step["lse_out"][1]).all()
        for b in range(w.B):
            for h in range(w.Hkv):
                ref = ow.group(w, lens, b, h)
                hs = slice(h * w.G, (h + 1) * w.G)
                assert_out(to64(step["out"][b, hs]), ref["out"])
                assert_lse(to64(step["lse_out"][b, hs]), ref["lse_out"])
