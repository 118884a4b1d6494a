"""cpdec_cp_decode (the whole step, normally one launch) against the oracle
and against the two-call path (cpdec_attn_partial + cpdec_lse_merge).

In the one-launch form the workgroup that arrives last at a (sequence, kv
head) group merges it; the tests check that the result does not depend on
that (repeat calls are bit-identical) and that the arrival counters at the
start of the workspace are zero again after every call, whatever the shape.
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

C = cp.STEP_COUNTER_BYTES

# name -> (workload, chunk_tokens, expected launches)
CASES = {
    "c1": (sc.WORKLOADS["c1"], 0, 1),
    "c1 chunk 32": (sc.WORKLOADS["c1"], 32, 1),
    "c2": (sc.WORKLOADS["c2"], 0, 1),
    "c2 chunk 32 (128 chunks: separate launches)": (sc.WORKLOADS["c2"], 32, 3),
    "ragged GQA 8, B16": (sc.small("c4", B=16, Lcap=512), 0, 1),
    "ragged GQA 8, B2 split (group too big: attention + row merge)": (sc.small("c4", B=2, Lcap=512), 0, 2),
    "ragged GQA 4, B2 split (two levels)": (sc.small("c4", B=2, Hq=32, Lcap=512), 0, 1),
    "ragged GQA 8, B1 split, 64 chunks (two levels)": (sc.small("c4", B=1, Lcap=2048), 32, 1),
    "ragged GQA 8, B1 split, 65 chunks (separate launches)": (sc.small("c4", B=1, Lcap=2080), 32, 3),
    "GQA 8 D64 B1 split, 32 chunks (two levels, two head passes)":
        (sc.small("c3", R=8, B=1, Hq=16, Hkv=2, D=64, Lcap=2048, L=2000), 0, 1),
    "ragged GQA 8, B64 (large unsplit grid)": (sc.small("c4", B=64, Lcap=512), 0, 2),
    "D256 G20 (over the merging workgroup: attention + row merge)":
        (sc.small("c3", R=3, B=2, Hq=40, Hkv=2, D=256, Lcap=300, L=290), 0, 2),
    "ragged GQA 8, B2 split, 8 x 32 chunks (4 waves: two levels)": (sc.small("c4", B=2, Lcap=1024), 32, 1),
    "fp16 GQA 8 split (attention + row merge)": (sc.small("c4", B=3, Lcap=256, dtype="fp16"), 0, 2),
    "fp16 GQA 4 split (two levels)": (sc.small("c4", B=3, Hq=32, Lcap=256, dtype="fp16"), 0, 1),
    "fp16 GQA 2 split": (sc.small("c4", B=2, Hq=16, Lcap=256, dtype="fp16"), 0, 1),
    "GQA 32 D64, two head blocks, chunk 256 (two levels)":
        (sc.small("c3", R=8, B=1, Hq=64, Hkv=2, D=64, Lcap=2048, L=1900), 256, 1),
    "GQA 32 D64, two head blocks (attention + row merge)":
        (sc.small("c3", R=8, B=1, Hq=64, Hkv=2, D=64, Lcap=2048, L=1900), 0, 2),
    "GQA 16 D256, 16 shards (attention, combine, merge)":
        (sc.small("c3", R=16, B=1, Hq=32, Hkv=2, D=256, Lcap=1024, L=1000), 0, 3),
    "64 shards (the most), whole shards (attention + merge)":
        (sc.small("c3", R=64, B=2, Hq=4, Hkv=1, D=64, Lcap=96, L=90), 0, 2),
    "64 shards, ragged with empty shards (attention + merge)":
        (sc.small("c4", R=64, B=2, Hq=4, Hkv=1, D=64, Lcap=96), 0, 2),
    "1 shard, split": (sc.small("c3", R=1, B=3, Hq=8, Hkv=2, D=128, Lcap=700, L=650), 0, 1),
    "1 shard, ragged, 47 chunks of 64 (two levels)":
        (sc.small("c4", R=1, B=1, Hq=8, Hkv=1, D=128, Lcap=3000), 64, 1),
    "1 shard, ragged, 47 chunks (attention + row merge)":
        (sc.small("c4", R=1, B=1, Hq=8, Hkv=1, D=128, Lcap=3000), 0, 2),
    "GQA 24, two head blocks (attention + row merge)":
        (sc.small("c3", R=4, B=2, Hq=48, Hkv=2, D=128, Lcap=1024, L=1000), 0, 2),
    "D64 G3": (sc.small("c3", R=5, B=3, Hq=6, Hkv=2, D=64, Lcap=97, L=97), 0, 1),
    "D64 G3 chunk 32": (sc.small("c3", R=5, B=3, Hq=6, Hkv=2, D=64, Lcap=97, L=97), 32, 1),
    "D256 G2 split": (sc.small("c3", R=2, B=1, Hq=4, Hkv=2, D=256, Lcap=700, L=650), 0, 1),
}


def _say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def step_workspace(inp, chunk_tokens=0):
    desc = cp.make_attn_desc(inp["q"], inp["k_shards"], chunk_tokens=chunk_tokens)
    return torch.zeros(cp.step_workspace_bytes(desc), dtype=torch.uint8, device="cuda"), desc


def run_step(inp, chunk_tokens=0, workspace=None, o_dtype=torch.float32):
    q = inp["q"]
    R = len(inp["k_shards"])
    B, Hq, D = q.shape
    o_part = torch.empty((R, B, Hq, D), dtype=o_dtype, device=q.device)
    lse_part = torch.empty((R, B, Hq), dtype=torch.float32, device=q.device)
    out = torch.empty((B, Hq, D), dtype=q.dtype, device=q.device)
    lo = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    cp.cp_decode(q, inp["k_shards"], inp["v_shards"], inp["lens"], o_part, lse_part, out, lo,
                 chunk_tokens=chunk_tokens, workspace=workspace)
    torch.cuda.synchronize()
    return dict(o_part=o_part, lse_part=lse_part, out=out, lse_out=lo)


def counters_zero(ws):
    return int(torch.count_nonzero(ws[:C]).item()) == 0


def check_against_oracle(w, inp, res, what):
    # the five workloads at full size hold the merged lse to the strict 1e-5
    # relative bar; reduced and random shapes may cancel towards 0 (floor)
    full = w.name in sc.WORKLOADS and w == sc.WORKLOADS[w.name]
    for b in range(w.B):
        for h in range(w.Hkv):
            ref = ow.group(w, inp["lens_np"], b, h)
            hs = slice(h * w.G, (h + 1) * w.G)
            assert_out(to64(res["o_part"][:, b, hs]), ref["o_part"], f"{what} o_part b={b} h={h}")
            assert_lse(to64(res["lse_part"][:, b, hs]), ref["lse_part"], f"{what} lse_part b={b} h={h}",
                       floor=True)
            assert_out(to64(res["out"][b, hs]), ref["out"], f"{what} out b={b} h={h}")
            assert_lse(to64(res["lse_out"][b, hs]), ref["lse_out"], f"{what} lse_out b={b} h={h}",
                       floor=not full)


@pytest.mark.parametrize("name", list(CASES))
def test_step_matches_oracle_and_two_calls(name):
    w, chunk, launches = CASES[name]
    _say(f"step {name}")
    inp = sg.attn_inputs(w)
    ws, desc = step_workspace(inp, chunk)
    assert cp.step_launches(desc) == launches
    step = run_step(inp, chunk, ws)
    assert counters_zero(ws), "arrival counters not reset"
    two = run_path(inp, chunk_tokens=chunk)
    # the same formulas; the step adds the chunk weights in another order, so
    # the partials agree with the two calls to FP32 rounding
    assert torch.equal(torch.isneginf(step["lse_part"]), torch.isneginf(two["lse_part"]))
    fin = torch.isfinite(two["lse_part"])
    assert torch.allclose(step["lse_part"][fin], two["lse_part"][fin], rtol=1e-6, atol=1e-6)
    assert torch.allclose(step["o_part"], two["o_part"], rtol=1e-5, atol=1e-6)
    check_against_oracle(w, inp, step, "step")


def test_step_repeat_and_shape_alternation_on_one_workspace():
    """Repeat calls give identical bits whichever workgroup merges; calls of
    other shapes and cpdec_attn_partial calls in between on the same
    workspace disturb nothing, and the counters end at zero."""
    _say("step repeat / shape alternation")
    a_w = sc.WORKLOADS["c2"]
    b_w = sc.small("c4", B=2, Lcap=512)
    a_in, b_in = sg.attn_inputs(a_w), sg.attn_inputs(b_w)
    da = cp.make_attn_desc(a_in["q"], a_in["k_shards"])
    db = cp.make_attn_desc(b_in["q"], b_in["k_shards"], chunk_tokens=32)
    nb = max(cp.step_workspace_bytes(da), cp.step_workspace_bytes(db))
    ws = torch.zeros(nb, dtype=torch.uint8, device="cuda")
    first = run_step(a_in, 0, ws)
    for rep in range(3):
        again = run_step(a_in, 0, ws)
        for k in first:
            assert torch.equal(first[k], again[k]), f"repeat {rep}: {k} differs"
    other = run_step(b_in, 32, ws)
    check_against_oracle(b_w, b_in, other, "other shape")
    run_path(b_in, chunk_tokens=32, workspace=ws)  # partials only, same workspace
    after = run_step(a_in, 0, ws)
    for k in first:
        assert torch.equal(first[k], after[k]), f"after other shapes: {k} differs"
    assert counters_zero(ws)


def test_step_back_to_back_calls_on_one_stream():
    """Many calls on one stream without host synchronisation (each must see
    the counters its predecessor reset)."""
    _say("step back-to-back")
    w = sc.WORKLOADS["c1"]
    inp = sg.attn_inputs(w)
    ws, _ = step_workspace(inp)
    ref = run_step(inp, 0, ws)
    outs = [torch.empty_like(ref["out"]) for _ in range(16)]
    out_t = torch.empty_like(ref["out"])
    call = cp.StepCall(inp["q"], inp["k_shards"], inp["v_shards"], inp["lens"],
                       torch.empty_like(ref["o_part"]), torch.empty_like(ref["lse_part"]),
                       out_t, torch.empty_like(ref["lse_out"]), workspace=ws)
    for o in outs:
        out_t.fill_(float("nan"))
        call()
        o.copy_(out_t)
    torch.cuda.synchronize()
    for o in outs:
        assert torch.equal(o, ref["out"])
    assert counters_zero(ws)


def test_step_empty_shards_and_sequences():
    w = sc.small("c4", B=3, Lcap=200, Hq=16, Hkv=4, R=3)
    _say("step empty shards")
    inp = sg.attn_inputs(w)
    lens = inp["lens_np"].copy()
    lens[:, 1] = 0
    lens[2, 0] = 0
    lens[0, 2] = 1
    inp["lens_np"] = lens
    inp["lens"] = torch.from_numpy(lens).cuda()
    for chunk in (32, 0):
        ws, _ = step_workspace(inp, chunk)
        step = run_step(inp, chunk, ws)
        assert counters_zero(ws)
        assert torch.count_nonzero(step["out"][1]).item() == 0
        assert torch.isneginf(step["lse_out"][1]).all()
        check_against_oracle(w, inp, step, f"chunk {chunk}")


def test_step_padding_is_never_read():
    """NaN in every token position >= L changes no output bit of the step."""
    w = sc.small("c4", B=4, Lcap=300)
    _say("step NaN padding")
    clean = run_step(sg.attn_inputs(w))
    poisoned = run_step(sg.attn_inputs(w, poison_padding=True))
    for key in clean:
        assert torch.equal(clean[key], poisoned[key]), key


@pytest.mark.parametrize("o_dt", ["bf16", "fp16"])
def test_step_16bit_partials(o_dt):
    """o_part stored in 16 bits: the merged output meets the bar against the
    storage-aware oracle (exact partials rounded to the storage type, then
    merged exactly), in the one-launch split, two-level, single-head and
    unsplit forms and the attention + row-merge form."""
    for name, w, launches in (("split", sc.small("c4", B=2, Hq=16, Lcap=512), 1),
                              ("split, single head", sc.small("c4", B=2, Hq=8, Hkv=8, Lcap=512), 1),
                              ("split, single head, c1 shape", sc.WORKLOADS["c1"], 1),
                              ("split, two levels", sc.small("c4", B=2, Hq=32, Lcap=512), 1),
                              ("split, attention + row merge", sc.small("c4", B=2, Lcap=512), 2),
                              ("unsplit", sc.small("c4", B=16, Lcap=512), 1)):
        _say(f"step 16-bit partials {o_dt} {name}")
        inp = sg.attn_inputs(w)
        ws, desc = step_workspace(inp)
        assert cp.step_launches(desc) == launches
        res = run_step(inp, 0, ws, o_dtype=sg.torch_dtype(o_dt))
        for b in range(w.B):
            for h in range(w.Hkv):
                ref = ow.group(w, inp["lens_np"], b, h)
                hs = slice(h * w.G, (h + 1) * w.G)
                assert_out_stored(to64(res["out"][b, hs]), ref["o_part"], ref["lse_part"], o_dt,
                                  f"out vs storage-aware oracle b={b} h={h}")
                assert_out(to64(res["o_part"][:, b, hs]), ref["o_part"], f"o_part b={b} h={h}")


def test_step_on_two_streams_with_binding_workspaces():
    """Calls made for two streams take the binding's workspace of their own
    stream, so they may overlap: repeated interleaved enqueues on two streams
    give the single-stream results bit for bit, and both counter regions end
    at zero."""
    _say("step on two streams")
    wa, wb = sc.WORKLOADS["c1"], sc.small("c4", B=2, Hq=16, Lcap=512)
    ia, ib = sg.attn_inputs(wa), sg.attn_inputs(wb)
    ref_a, ref_b = run_step(ia), run_step(ib)
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    outs = {}
    calls = {}
    for name, inp, ref, s in (("a", ia, ref_a, sa), ("b", ib, ref_b, sb)):
        res = {k: torch.empty_like(v) for k, v in ref.items()}
        outs[name] = res
        calls[name] = cp.StepCall(inp["q"], inp["k_shards"], inp["v_shards"], inp["lens"],
                                  res["o_part"], res["lse_part"], res["out"], res["lse_out"], stream=s)
    assert calls["a"].workspace(sa).data_ptr() != calls["b"].workspace(sb).data_ptr()
    torch.cuda.synchronize()
    for _ in range(20):
        calls["a"](sa.cuda_stream)
        calls["b"](sb.cuda_stream)
    torch.cuda.synchronize()
    for name, ref in (("a", ref_a), ("b", ref_b)):
        for k in ref:
            assert torch.equal(outs[name][k], ref[k]), f"stream {name}: {k} differs"
        assert counters_zero(calls[name].workspace(sa if name == "a" else sb))


def test_step_on_new_streams_without_synchronisation():
    """The binding's workspace for a stream is allocated and zero-filled on
    that stream, so a call made for a new stream may run at once, with no
    synchronisation between making the call and running it: on fresh
    streams, a small shape first and then a larger one (whose workspace
    replaces the smaller one of the same stream) give the single-stream
    results bit for bit, through the marshalled calls and through the
    one-shot functions alike."""
    _say("step on new streams, no synchronisation")
    small_w, big_w = sc.WORKLOADS["c1"], sc.small("c4", B=2, Hq=16, Lcap=1024)
    si, bi = sg.attn_inputs(small_w), sg.attn_inputs(big_w)
    ref_s, ref_b = run_step(si), run_step(bi)
    for rep in range(3):
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())   # inputs are ready before s runs
        got_s = {k: torch.empty_like(v) for k, v in ref_s.items()}
        got_b = {k: torch.empty_like(v) for k, v in ref_b.items()}
        call = cp.StepCall(si["q"], si["k_shards"], si["v_shards"], si["lens"], got_s["o_part"],
                           got_s["lse_part"], got_s["out"], got_s["lse_out"], stream=s)
        call(s.cuda_stream)
        # the larger shape on the same stream: a larger workspace replaces the first
        cp.cp_decode(bi["q"], bi["k_shards"], bi["v_shards"], bi["lens"], got_b["o_part"],
                     got_b["lse_part"], got_b["out"], got_b["lse_out"], stream=s)
        for t in (*got_s.values(), *got_b.values()):
            t.record_stream(s)
        s.synchronize()
        for k in ref_s:
            assert torch.equal(got_s[k], ref_s[k]), f"rep {rep}: small shape {k} differs"
            assert torch.equal(got_b[k], ref_b[k]), f"rep {rep}: larger shape {k} differs"
