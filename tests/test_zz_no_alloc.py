"""cpdec_cp_decode_noalloc -- the whole step with the library's static
scratch instead of a caller workspace -- against cpdec_cp_decode, through
the C ABI: every output bit for bit, on calls in a row whose shapes shrink
(each call finds the previous call's contents in the shared scratch), in
the one-launch split and unsplit forms and in a several-launch form, and
against the oracle."""
import sys

import pytest

from oracle import workloads as ow
from synth import configs as sc
from tests.helpers import assert_lse, assert_out, to64

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
import lse_merge_split_amd as cp  # noqa: E402
from synth import gpu as sg  # noqa: E402


def _say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def _outputs(w, dt):
    return dict(o_part=torch.empty((w.R, w.B, w.Hq, w.D), dtype=torch.float32, device="cuda"),
                lse_part=torch.empty((w.R, w.B, w.Hq), dtype=torch.float32, device="cuda"),
                out=torch.empty((w.B, w.Hq, w.D), dtype=dt, device="cuda"),
                lse_out=torch.empty((w.B, w.Hq), dtype=torch.float32, device="cuda"))


def _run(call_cls, inp, res, **kw):
    c = call_cls(inp["q"], inp["k_shards"], inp["v_shards"], inp["lens"], res["o_part"],
                 res["lse_part"], res["out"], res["lse_out"], **kw)
    c()
    return c


# larger first, then smaller: each call reuses what the previous one left in the scratch
SEQUENCE = [
    ("c2 (split shards, one launch, chunk partials in the scratch)", sc.WORKLOADS["c2"], 1),
    ("c1 (smaller, split, one launch)", sc.WORKLOADS["c1"], 1),
    ("ragged GQA 8, B2 (attention + row merge)", sc.small("c4", B=2, Lcap=512), 2),
    ("ragged GQA 8, B16 (whole shards, one launch)", sc.small("c4", B=16, Lcap=300), 1),
    ("ragged GQA 8, B1, short (smallest)", sc.small("c4", B=1, Lcap=96), 1),
]


def test_noalloc_step_matches_workspace_step_on_shrinking_calls():
    for rep in range(2):
        for name, w, launches in SEQUENCE:
            _say(f"noalloc step, round {rep}: {name}")
            inp = sg.attn_inputs(w)
            dt = inp["q"].dtype
            desc = cp.make_attn_desc(inp["q"], inp["k_shards"])
            assert cp.step_launches(desc) == launches
            assert cp.step_workspace_bytes(desc) <= cp.NOALLOC_SCRATCH_BYTES
            ref = _outputs(w, dt)
            _run(cp.StepCall, inp, ref)
            got = _outputs(w, dt)
            for t in got.values():
                t.fill_(float("nan"))
            _run(cp.StepCallNoAlloc, inp, got)
            torch.cuda.synchronize()
            for k in ref:
                assert torch.equal(got[k], ref[k]), f"{name}: {k} differs from cpdec_cp_decode"
            if rep == 0:
                for b in range(w.B):
                    for h in range(w.Hkv):
                        oref = ow.group(w, inp["lens_np"], b, h)
                        hs = slice(h * w.G, (h + 1) * w.G)
                        assert_out(to64(got["out"][b, hs]), oref["out"], f"{name} out b={b} h={h}")
                        assert_lse(to64(got["lse_out"][b, hs]), oref["lse_out"],
                                   f"{name} lse_out b={b} h={h}", floor=True)


def test_noalloc_step_repeats_bitwise_back_to_back():
    """Back-to-back calls on one stream without synchronisation (every call
    must leave the scratch's counters zero for the next)."""
    w = sc.WORKLOADS["c2"]
    _say("noalloc step, 50 back-to-back calls")
    inp = sg.attn_inputs(w)
    ref = _outputs(w, inp["q"].dtype)
    _run(cp.StepCall, inp, ref)
    got = _outputs(w, inp["q"].dtype)
    call = _run(cp.StepCallNoAlloc, inp, got)
    for _ in range(49):
        call()
    torch.cuda.synchronize()
    for k in ref:
        assert torch.equal(got[k], ref[k]), k


def test_noalloc_step_rejects_a_step_beyond_its_scratch():
    """A step whose scratch need passes CPDEC_NOALLOC_SCRATCH_BYTES returns
    CPDEC_ERR_WORKSPACE and leaves the outputs untouched."""
    w = sc.small("c3", R=8, B=1, Hq=16, Hkv=1, D=256, Lcap=8192, L=8192)
    _say("noalloc step beyond its scratch")
    inp = sg.attn_inputs(w)
    desc = cp.make_attn_desc(inp["q"], inp["k_shards"], chunk_tokens=32)
    assert cp.step_workspace_bytes(desc) > cp.NOALLOC_SCRATCH_BYTES
    got = _outputs(w, inp["q"].dtype)
    for t in got.values():
        t.fill_(7.0)
    with pytest.raises(cp.CpdecError, match="WORKSPACE"):
        _run(cp.StepCallNoAlloc, inp, got, chunk_tokens=32)
    torch.cuda.synchronize()
    for t in got.values():
        assert bool((t == 7.0).all())


def _graph_replays_match(call, outs, refs, eager_work, reps=4):
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g):
            call(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    for rep in range(reps):
        for t in outs.values():
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in refs:
            assert torch.equal(outs[k], refs[k]), f"replay {rep}: {k} differs"
        eager_work()
        torch.cuda.synchronize()


def test_noalloc_step_under_graph_capture():
    """The callers it is for may capture it in a HIP graph: every replay, with
    eager calls on the same scratch in between, gives cpdec_cp_decode's bits."""
    _say("noalloc step, HIP graph replay")
    for w in (sc.WORKLOADS["c2"], sc.small("c4", B=2, Lcap=512)):
        inp = sg.attn_inputs(w)
        ref = _outputs(w, inp["q"].dtype)
        _run(cp.StepCall, inp, ref)
        outs = _outputs(w, inp["q"].dtype)
        call = cp.StepCallNoAlloc(inp["q"], inp["k_shards"], inp["v_shards"], inp["lens"],
                                  outs["o_part"], outs["lse_part"], outs["out"], outs["lse_out"])
        scratch_outs = _outputs(w, inp["q"].dtype)
        _graph_replays_match(call, outs, ref,
                             lambda: _run(cp.StepCallNoAlloc, inp, scratch_outs))
        for k in ref:
            assert torch.equal(scratch_outs[k], ref[k]), k


FIRST_CALL_UNDER_CAPTURE = r"""
import sys
sys.path.insert(0, sys.argv[1])
import torch
import lse_merge_split_amd as cp
from synth import configs as sc, gpu as sg
torch.cuda.set_device(0)
w = sc.WORKLOADS["c2"]
inp = sg.attn_inputs(w)
mk = lambda: [torch.empty((w.R, w.B, w.Hq, w.D), dtype=torch.float32, device="cuda"),
              torch.empty((w.R, w.B, w.Hq), dtype=torch.float32, device="cuda"),
              torch.empty((w.B, w.Hq, w.D), dtype=inp["q"].dtype, device="cuda"),
              torch.empty((w.B, w.Hq), dtype=torch.float32, device="cuda")]
ref = mk()
cp.cp_decode(inp["q"], inp["k_shards"], inp["v_shards"], inp["lens"], *ref)
got = mk()
call = cp.StepCallNoAlloc(inp["q"], inp["k_shards"], inp["v_shards"], inp["lens"], *got)
torch.cuda.synchronize()
g = torch.cuda.CUDAGraph()
side = torch.cuda.Stream()
side.wait_stream(torch.cuda.current_stream())
with torch.cuda.stream(side):
    with torch.cuda.graph(g):
        call(torch.cuda.current_stream().cuda_stream)
for rep in range(3):
    for t in got:
        t.fill_(float("nan"))
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(got, ref)), f"replay {rep} differs"
print("first call under capture ok", flush=True)
"""


def test_noalloc_first_call_of_a_process_under_graph_capture():
    """A fresh process whose very first cpdec_cp_decode_noalloc call is made
    under graph capture (the scratch lookup and its counter clear happen
    then): the replays give cpdec_cp_decode's bits."""
    import os
    import subprocess
    _say("noalloc step, first call of a process under capture")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", FIRST_CALL_UNDER_CAPTURE, root], capture_output=True,
                       text=True, timeout=180)
    assert r.returncode == 0, r.stderr[-3000:]
    assert "first call under capture ok" in r.stdout
