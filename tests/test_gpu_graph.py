"""HIP-graph replay of a whole step (partial attention + merge) gives the
eager result bit for bit on every replay, with eager work and
synchronisations between replays (the path records no memset nodes), and
every replay meets the oracle."""
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


@pytest.mark.parametrize("name,w", [
    ("split shards (chunk merge)", sc.small("c4", B=8, Lcap=700)),
    ("whole shards", sc.small("c3", B=4, Lcap=640, L=600)),
    ("whole shards, longest first (order pre-pass)", sc.small("c4", B=64, Hq=32, Hkv=8, Lcap=2048)),
    ("merge-only rows", None),
    ("one-launch step, split", sc.small("c4", B=2, Hq=8, Lcap=700)),
    ("one-launch step, whole shards", sc.small("c3", B=8, Lcap=640, L=600)),
    ("one-launch step, two levels", sc.small("c4", B=2, Hq=32, Lcap=512)),
    ("step as attention + row merge", sc.small("c4", B=2, Lcap=512)),
])
def test_graph_replay_matches_eager(name, w):
    print(f"[case] graph replay: {name}", flush=True)
    sys.stdout.flush()
    if w is None:
        wm = sc.WORKLOADS["c5"].scaled(rows=4096)
        inp = sg.merge_inputs(wm)
        out = torch.empty((wm.rows, wm.D), dtype=torch.bfloat16, device="cuda")
        lo = torch.empty(wm.rows, dtype=torch.float32, device="cuda")
        calls = [cp.MergeCall(inp["o_part"], inp["lse_part"], out, lo)]
        outs = [out, lo]
        ref_out, ref_lo = torch.empty_like(out), torch.empty_like(lo)
        cp.lse_merge(inp["o_part"], inp["lse_part"], ref_out, ref_lo)
        refs = [ref_out, ref_lo]
        eager_work = lambda: cp.lse_merge(inp["o_part"], inp["lse_part"], ref_out, ref_lo)
    elif "step" in name:
        inp = sg.attn_inputs(w)
        R, B, Hq, D = w.R, w.B, w.Hq, w.D
        mk = lambda: (torch.empty((R, B, Hq, D), dtype=torch.float32, device="cuda"),
                      torch.empty((R, B, Hq), dtype=torch.float32, device="cuda"),
                      torch.empty((B, Hq, D), dtype=inp["q"].dtype, device="cuda"),
                      torch.empty((B, Hq), dtype=torch.float32, device="cuda"))
        desc = cp.make_attn_desc(inp["q"], inp["k_shards"])
        assert cp.step_launches(desc) == (2 if "row merge" in name else 1)
        refs = list(mk())
        cp.cp_decode(inp["q"], inp["k_shards"], inp["v_shards"], inp["lens"], *refs)
        outs = list(mk())
        ws = torch.zeros(cp.step_workspace_bytes(desc), dtype=torch.uint8, device="cuda")
        calls = [cp.StepCall(inp["q"], inp["k_shards"], inp["v_shards"], inp["lens"], *outs,
                             workspace=ws)]
        eager_work = lambda: cp.cp_decode(inp["q"], inp["k_shards"], inp["v_shards"], inp["lens"],
                                          *mk())
    else:
        inp = sg.attn_inputs(w)
        ref = run_path(inp)
        R, B, Hq, D = w.R, w.B, w.Hq, w.D
        o_part = torch.empty((R, B, Hq, D), dtype=torch.float32, device="cuda")
        lse_part = torch.empty((R, B, Hq), dtype=torch.float32, device="cuda")
        out = torch.empty((B, Hq, D), dtype=inp["q"].dtype, device="cuda")
        lo = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
        ws = torch.zeros(max(256, cp.attn_workspace_bytes(cp.make_attn_desc(inp["q"], inp["k_shards"]))),
                         dtype=torch.uint8, device="cuda")  # counter region zero before the first call
        calls = [cp.AttnCall(inp["q"], inp["k_shards"], inp["v_shards"], inp["lens"], o_part, lse_part,
                             workspace=ws),
                 cp.MergeCall(o_part, lse_part, out, lo)]
        outs = [o_part, lse_part, out, lo]
        refs = [ref["o_part"], ref["lse_part"], ref["out"], ref["lse_out"]]
        eager_work = lambda: run_path(inp)
    if w is None:
        rows = np.unique(np.concatenate([np.arange(0, wm.rows, 17),
                                         np.where(np.isneginf(inp["lse_np"]).any(axis=0))[0][:64]]))
        o_ref, lo_ref = ow.merge_rows(wm, rows)

        def check_oracle(rep):
            assert_out(to64(out[rows]), o_ref, f"replay {rep} merge out")
            assert_lse(to64(lo[rows]), lo_ref, f"replay {rep} merge lse_out")
    else:
        groups = [(b, h) for b in range(w.B) for h in range(w.Hkv)]
        if len(groups) > 48:   # larger cases: 48 seeded random groups
            pick = np.random.default_rng(77).choice(len(groups), size=48, replace=False)
            groups = [groups[i] for i in sorted(pick)]
        grefs = {g: ow.group(w, inp["lens_np"], *g) for g in groups}
        o_part_t, _, out_t, lo_t = outs

        def check_oracle(rep):
            for (b, h), ref in grefs.items():
                hs = slice(h * w.G, (h + 1) * w.G)
                assert_out(to64(out_t[b, hs]), ref["out"], f"replay {rep} out b={b} h={h}")
                assert_lse(to64(lo_t[b, hs]), ref["lse_out"], f"replay {rep} lse_out b={b} h={h}",
                           floor=True)
                assert_out(to64(o_part_t[:, b, hs]), ref["o_part"], f"replay {rep} o_part b={b} h={h}")
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g):
            cs = torch.cuda.current_stream().cuda_stream
            for c in calls:
                c(cs)
    torch.cuda.synchronize()
    for rep in range(4):
        for t in outs:
            t.fill_(float("nan") if t.dtype.is_floating_point else 0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for t, r in zip(outs, refs):
            assert torch.equal(t, r), f"replay {rep}: output differs from eager"
        check_oracle(rep)
        eager_work()
        torch.cuda.synchronize()
