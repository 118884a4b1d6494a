"""Guard canaries: every output buffer sits between sentinel regions that no
kernel may touch, for both entry points and the whole step."""
import sys

import pytest

from synth import configs as sc

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
import lse_merge_split_amd as cp  # noqa: E402
from synth import gpu as sg  # noqa: E402

PAD = 4096  # elements of sentinel before and after each output


def guarded(shape, dtype):
    n = 1
    for s in shape:
        n *= s
    buf = torch.empty(n + 2 * PAD, dtype=dtype, device="cuda")
    if dtype == torch.float32:
        buf.view(torch.int32).fill_(0x7F7F7F7F)
    else:
        buf.view(torch.int16).fill_(0x7F7F)
    return buf, buf[PAD:PAD + n].view(shape)


def untouched(buf, dtype):
    v = buf.view(torch.int32 if dtype == torch.float32 else torch.int16)
    want = 0x7F7F7F7F if dtype == torch.float32 else 0x7F7F
    return bool((v[:PAD] == want).all()) and bool((v[-PAD:] == want).all())


@pytest.mark.parametrize("name,w,chunk", [
    ("split ragged", sc.small("c4", B=8, Lcap=400), 64),
    ("unsplit", sc.small("c3", B=2, Lcap=300, L=290), 0),
    ("D64 fp16", sc.small("c1", B=2), 0),
])
def test_outputs_stay_in_bounds(name, w, chunk):
    print(f"[case] guards {name}", flush=True)
    sys.stdout.flush()
    inp = sg.attn_inputs(w)
    R, B, Hq, D = w.R, w.B, w.Hq, w.D
    dt = inp["q"].dtype
    bufs = {}
    bufs["o_part"], o_part = guarded((R, B, Hq, D), torch.float32)
    bufs["lse_part"], lse_part = guarded((R, B, Hq), torch.float32)
    bufs["out"], out = guarded((B, Hq, D), dt)
    bufs["lse_out"], lse_out = guarded((B, Hq), torch.float32)
    desc = cp.make_attn_desc(inp["q"], inp["k_shards"], chunk_tokens=chunk)
    nws = cp.step_workspace_bytes(desc)
    wsb = torch.empty(nws + 2 * PAD * 4, dtype=torch.uint8, device="cuda")
    wsb.fill_(0x7F)
    ws = wsb[PAD * 4:PAD * 4 + nws]
    ws[:cp.STEP_COUNTER_BYTES].zero_()  # the whole step's counters start at zero
    cp.attn_partial(inp["q"], inp["k_shards"], inp["v_shards"], inp["lens"], o_part, lse_part,
                    workspace=ws, chunk_tokens=chunk)
    cp.lse_merge(o_part, lse_part, out, lse_out)
    cp.cp_decode(inp["q"], inp["k_shards"], inp["v_shards"], inp["lens"], o_part, lse_part, out,
                 lse_out, workspace=ws, chunk_tokens=chunk)
    torch.cuda.synchronize()
    for k, b in bufs.items():
        assert untouched(b, torch.float32 if k != "out" else dt), f"{k} guard overwritten"
    assert bool((wsb[:PAD * 4] == 0x7F).all()) and bool((wsb[-PAD * 4:] == 0x7F).all())
    assert int(torch.count_nonzero(ws[:cp.STEP_COUNTER_BYTES]).item()) == 0


@pytest.mark.parametrize("name,w,chunk", [
    ("split, one launch", sc.small("c4", B=4, Hq=16, Lcap=200), 0),
    ("split, chunk 32 (separate launches)", sc.small("c4", B=4, Hq=16, Lcap=200), 32),
    ("unsplit, one launch", sc.small("c4", B=16, Lcap=300), 0),
])
def test_lengths_outside_capacity_are_clamped(name, w, chunk):
    """lens below 0 act as 0 and above the capacity as the capacity, in every
    form of the call: the results equal those of the clamped lengths bit for
    bit (the kernels never read outside a shard's tokens)."""
    print(f"[case] clamped lengths {name}", flush=True)
    sys.stdout.flush()
    from tests.helpers import run_path
    inp = sg.attn_inputs(w)
    lens = inp["lens_np"].copy()
    wild = lens.copy()
    wild[0, 0] = w.Lcap + 1
    wild[-1, -1] = 2 ** 30
    wild[0, -1] = -5
    wild[-1, 0] = -(2 ** 31)
    lens[0, 0] = w.Lcap
    lens[-1, -1] = w.Lcap
    lens[0, -1] = 0
    lens[-1, 0] = 0
    clean = dict(inp, lens=torch.from_numpy(lens).cuda())
    bad = dict(inp, lens=torch.from_numpy(wild).cuda())

    def step(x):
        R, B, Hq, D = w.R, w.B, w.Hq, w.D
        res = dict(o_part=torch.empty((R, B, Hq, D), dtype=torch.float32, device="cuda"),
                   lse_part=torch.empty((R, B, Hq), dtype=torch.float32, device="cuda"),
                   out=torch.empty((B, Hq, D), dtype=x["q"].dtype, device="cuda"),
                   lse_out=torch.empty((B, Hq), dtype=torch.float32, device="cuda"))
        cp.cp_decode(x["q"], x["k_shards"], x["v_shards"], x["lens"], res["o_part"],
                     res["lse_part"], res["out"], res["lse_out"], chunk_tokens=chunk)
        torch.cuda.synchronize()
        return res

    for form, f in (("two calls", lambda x: run_path(x, chunk_tokens=chunk)), ("step", step)):
        a, b = f(clean), f(bad)
        for k in a:
            assert torch.equal(a[k], b[k]), f"{form}: {k} differs with out-of-range lengths"
