"""GPU parity of cpdec_attn_partial (+ cpdec_lse_merge) against the oracle.

Small workloads are compared element by element on every output; the three
large workloads are run at full size in the launch configuration the
benchmark uses and compared on sampled (sequence, kv head) groups, with
properties checked on every row.  Each case prints its name (flushed) first.
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


def _say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def check_groups(w, inp, res, groups, o_part_check=True):
    """Compare the GPU results of the listed (b, h) groups with the oracle."""
    lens = inp["lens_np"]
    G = w.G
    for (b, h) in groups:
        ref = ow.group(w, lens, b, h)
        heads = slice(h * G, (h + 1) * G)
        assert_out(to64(res["out"][b, heads]), ref["out"], f"out b={b} h={h}")
        if res["lse_out"] is not None:
            assert_lse(to64(res["lse_out"][b, heads]), ref["lse_out"], f"lse_out b={b} h={h}", floor=True)
        if o_part_check:
            assert_out(to64(res["o_part"][:, b, heads]), ref["o_part"], f"o_part b={b} h={h}")
            assert_lse(to64(res["lse_part"][:, b, heads]), ref["lse_part"], f"lse_part b={b} h={h}",
                       floor=True)


def all_groups(w):
    return [(b, h) for b in range(w.B) for h in range(w.Hkv)]


SMALL = {
    "c1": sc.WORKLOADS["c1"],
    "c2": sc.WORKLOADS["c2"],
    "c3_small": sc.small("c3", B=2, Lcap=1024, L=1000),
    "c4_small": sc.small("c4", B=16, Lcap=512),
    "d256_g20": sc.small("c3", R=3, B=2, Hq=40, Hkv=2, D=256, Lcap=300, L=290),
    "fp16_g8": sc.small("c4", B=4, Lcap=256, dtype="fp16"),
    "d64_g3": sc.small("c3", R=5, B=3, Hq=6, Hkv=2, D=64, Lcap=97, L=97),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_attn_small_all_outputs(name):
    w = SMALL[name]
    _say(f"attn small {name}")
    inp = sg.attn_inputs(w)
    res = run_path(inp)
    check_groups(w, inp, res, all_groups(w))


@pytest.mark.parametrize("chunk", [32, 64, 128, 256, 2048])
def test_attn_chunk_sizes(chunk):
    """Forced chunk lengths exercise the intra-workgroup merge with idle waves
    and the last-arrival chunk merge."""
    w = SMALL["c4_small"]
    _say(f"attn chunk {chunk}")
    inp = sg.attn_inputs(w)
    res = run_path(inp, chunk_tokens=chunk)
    check_groups(w, inp, res, all_groups(w))


@pytest.mark.parametrize("o_dt", ["bf16", "fp16"])
def test_attn_low_precision_partials(o_dt):
    """o_part stored in 16 bits: each partial within its own rounding of the
    oracle's partial (2^-8 relative for bf16) -- the merged output is not held
    to the fp32-partial bar here."""
    w = SMALL["c3_small"]
    _say(f"attn o_part {o_dt}")
    inp = sg.attn_inputs(w)
    res = run_path(inp, o_dtype=sg.torch_dtype(o_dt))
    for (b, h) in all_groups(w):
        ref = ow.group(w, inp["lens_np"], b, h)
        heads = slice(h * w.G, (h + 1) * w.G)
        got = to64(res["o_part"][:, b, heads])
        assert np.all(np.abs(got - ref["o_part"]) <= 2.0 ** -8 * np.abs(ref["o_part"]) + 1e-3)


@pytest.mark.parametrize("o_dt", ["bf16", "fp16"])
def test_16bit_wire_partials_against_storage_aware_oracle(o_dt):
    """Partials stored in 16 bits (the payload of a 16-bit exchange): the merged
    output meets the output bar against the storage-aware oracle (exact
    partials rounded to the storage type, then merged exactly).  Against the
    unrounded oracle 16-bit partials are not held to the bar; the number of
    elements over it is printed."""
    w = sc.small("c4", B=16, Lcap=512)     # peaky softmax (k x3), ragged lengths
    _say(f"attn 16-bit wire partials {o_dt}")
    inp = sg.attn_inputs(w)
    res = run_path(inp, o_dtype=sg.torch_dtype(o_dt))
    over_unrounded = 0
    total = 0
    for (b, h) in all_groups(w):
        ref = ow.group(w, inp["lens_np"], b, h)
        heads = slice(h * w.G, (h + 1) * w.G)
        got = to64(res["out"][b, heads])
        assert_out_stored(got, ref["o_part"], ref["lse_part"], o_dt,
                          f"out vs storage-aware oracle b={b} h={h}")
        bound = 2.0 ** -7 * np.abs(ref["out"]) + 1e-3
        over_unrounded += int((np.abs(got - ref["out"]) > bound).sum())
        total += got.size
    print(f"[info] {o_dt} partials: {over_unrounded} of {total} outputs over the bar "
          f"against the unrounded oracle", flush=True)


def test_attn_padding_is_never_read():
    """NaN in every token position >= L changes no output bit."""
    w = SMALL["c4_small"]
    _say("attn NaN padding")
    clean = run_path(sg.attn_inputs(w))
    poisoned = run_path(sg.attn_inputs(w, poison_padding=True))
    for key in ("o_part", "lse_part", "out", "lse_out"):
        assert torch.equal(clean[key], poisoned[key]), key


def test_attn_workspace_reuse_and_determinism():
    """Two calls on one workspace give identical bits."""
    w = SMALL["c3_small"]
    _say("attn workspace reuse")
    inp = sg.attn_inputs(w)
    desc = cp.make_attn_desc(inp["q"], inp["k_shards"], chunk_tokens=128)
    ws = torch.zeros(cp.attn_workspace_bytes(desc), dtype=torch.uint8, device="cuda")
    a = run_path(inp, chunk_tokens=128, workspace=ws)
    b = run_path(inp, chunk_tokens=128, workspace=ws)
    for key in a:
        assert torch.equal(a[key], b[key]), key


def test_attn_workspace_contents_do_not_matter():
    """A workspace full of random bytes past its counter region, or one last
    used by a different shape, gives the same bits as a fresh one, and every
    call leaves the counter region zero."""
    w = SMALL["c4_small"]
    _say("attn garbage / cross-shape workspace")
    inp = sg.attn_inputs(w)
    desc = cp.make_attn_desc(inp["q"], inp["k_shards"], chunk_tokens=64)
    nb = cp.attn_workspace_bytes(desc)
    ws = torch.zeros(nb + (1 << 20), dtype=torch.uint8, device="cuda")
    ref = run_path(inp, chunk_tokens=64, workspace=ws)
    C = cp.STEP_COUNTER_BYTES
    ws[C:].random_(0, 256)
    got = run_path(inp, chunk_tokens=64, workspace=ws)
    assert int(torch.count_nonzero(ws[:C]).item()) == 0
    for key in ref:
        assert torch.equal(ref[key], got[key]), key
    # another shape writes its partials over this shape's slot region, then back
    w2 = sc.small("c3", R=3, B=2, Hq=40, Hkv=2, D=256, Lcap=300, L=290)
    other = sg.attn_inputs(w2)
    run_path(other, chunk_tokens=32, workspace=ws)
    again = run_path(inp, chunk_tokens=64, workspace=ws)
    for key in ref:
        assert torch.equal(ref[key], again[key]), key
    assert int(torch.count_nonzero(ws[:C]).item()) == 0
    check_groups(w, inp, again, all_groups(w))


def test_attn_strided_token_major_layout():
    """K/V stored token-major ([B][cap][Hkv][D]) give the same bits as the
    head-major layout (strides passed through the descriptor)."""
    w = SMALL["c3_small"]
    _say("attn NHD strides")
    inp = sg.attn_inputs(w)
    base = run_path(inp)
    k_nhd = inp["k"].permute(0, 1, 3, 2, 4).contiguous()   # [R][B][cap][Hkv][D]
    v_nhd = inp["v"].permute(0, 1, 3, 2, 4).contiguous()
    inp2 = dict(inp)
    inp2["k_shards"] = [k_nhd[r].permute(0, 2, 1, 3) for r in range(w.R)]
    inp2["v_shards"] = [v_nhd[r].permute(0, 2, 1, 3) for r in range(w.R)]
    assert inp2["k_shards"][0].stride(2) == w.Hkv * w.D
    res = run_path(inp2)
    for key in base:
        assert torch.equal(base[key], res[key]), key
    # the whole step on the same strides
    step = _step(inp2)
    step_base = _step(inp)
    for key in step_base:
        assert torch.equal(step_base[key], step[key]), f"step {key}"


def _step(inp, chunk=0):
    q = inp["q"]
    R, (B, Hq, D) = len(inp["k_shards"]), q.shape
    res = dict(o_part=torch.empty((R, B, Hq, D), dtype=torch.float32, device="cuda"),
               lse_part=torch.empty((R, B, Hq), dtype=torch.float32, device="cuda"),
               out=torch.empty((B, Hq, D), dtype=q.dtype, device="cuda"),
               lse_out=torch.empty((B, Hq), dtype=torch.float32, device="cuda"))
    cp.cp_decode(q, inp["k_shards"], inp["v_shards"], inp["lens"], res["o_part"], res["lse_part"],
                 res["out"], res["lse_out"], chunk_tokens=chunk)
    torch.cuda.synchronize()
    return res


@pytest.mark.parametrize("chunk", [0, 64])
def test_attn_sliced_capacity_strides(chunk):
    """K/V viewed out of a larger cache: each (sequence, kv head) row block
    holds 37 more token rows than the capacity the call is given (head
    stride (cap + 37) D), filled with NaN.  Both entry points give the same
    bits as the contiguous layout, so nothing past the capacity is read; so
    do shards that each live in an allocation of their own."""
    w = sc.small("c4", B=3, Hq=8, Hkv=2, Lcap=200)    # ragged, GQA 4
    _say(f"attn sliced capacity strides, chunk {chunk}")
    inp = sg.attn_inputs(w)
    base, base_step = run_path(inp, chunk_tokens=chunk), _step(inp, chunk)
    pad = 37
    big_k = torch.full((w.R, w.B, w.Hkv, w.Lcap + pad, w.D), float("nan"), dtype=inp["k"].dtype,
                       device="cuda")
    big_v = torch.full_like(big_k, float("nan"))
    big_k[:, :, :, :w.Lcap] = inp["k"]
    big_v[:, :, :, :w.Lcap] = inp["v"]
    inp2 = dict(inp)
    inp2["k_shards"] = [big_k[r, :, :, :w.Lcap] for r in range(w.R)]
    inp2["v_shards"] = [big_v[r, :, :, :w.Lcap] for r in range(w.R)]
    assert inp2["k_shards"][0].stride(1) == (w.Lcap + pad) * w.D
    res, res_step = run_path(inp2, chunk_tokens=chunk), _step(inp2, chunk)
    for key in base:
        assert torch.equal(base[key], res[key]), key
        assert torch.equal(base_step[key], res_step[key]), f"step {key}"
    # every shard in an allocation of its own (unrelated base addresses)
    inp3 = dict(inp)
    inp3["k_shards"] = [inp["k"][r].clone() for r in reversed(range(w.R))][::-1]
    inp3["v_shards"] = [inp["v"][r].clone() for r in range(w.R)]
    res3, res3_step = run_path(inp3, chunk_tokens=chunk), _step(inp3, chunk)
    for key in base:
        assert torch.equal(base[key], res3[key]), f"separate shards {key}"
        assert torch.equal(base_step[key], res3_step[key]), f"separate shards step {key}"


def test_attn_empty_shards_and_all_empty_sequence():
    """An empty shard yields (0, -inf); a sequence whose shards are all empty
    yields out = 0, lse = -inf; inserting an empty shard changes no bit of the
    merged result."""
    w = sc.small("c4", B=3, Lcap=200, Hq=16, Hkv=4, R=3)
    _say("attn empty shards")
    inp = sg.attn_inputs(w)
    lens = inp["lens_np"].copy()
    lens[:, 1] = 0            # sequence 1: every shard empty
    lens[2, 0] = 0            # one empty shard of sequence 0
    lens[0, 2] = 200
    inp["lens_np"] = lens
    inp["lens"] = torch.from_numpy(lens).cuda()
    res = run_path(inp, chunk_tokens=128)
    check_groups(w, inp, res, all_groups(w))
    assert torch.count_nonzero(res["out"][1]).item() == 0
    assert torch.isneginf(res["lse_out"][1]).all()
    assert torch.count_nonzero(res["o_part"][2, 0]).item() == 0
    assert torch.isneginf(res["lse_part"][2, 0]).all()
    # insert an empty 4th shard (length 0): merged outputs unchanged bit for bit
    inp4 = dict(inp)
    inp4["k_shards"] = inp["k_shards"] + [inp["k_shards"][0]]
    inp4["v_shards"] = inp["v_shards"] + [inp["v_shards"][0]]
    lens4 = np.concatenate([lens, np.zeros((1, w.B), np.int32)])
    inp4["lens"] = torch.from_numpy(lens4).cuda()
    res4 = run_path(inp4, chunk_tokens=128)
    assert torch.equal(res4["out"], res["out"]) and torch.equal(res4["lse_out"], res["lse_out"])


def test_attn_split_invariance_on_gpu():
    """One KV sequence cut into shards gives the result of the unsplit
    sequence (R=1, L = sum of lengths), within the output tolerance."""
    w = sc.small("c3", R=1, B=2, Hq=8, Hkv=2, Lcap=1500, L=1500)
    _say("attn split invariance")
    inp = sg.attn_inputs(w)
    whole = run_path(inp)
    cuts = [0, 1, 200, 777, 1500]          # shards of length 1, 199, 577, 723
    ks = [inp["k"][0][:, :, a:b] for a, b in zip(cuts[:-1], cuts[1:])]
    vs = [inp["v"][0][:, :, a:b] for a, b in zip(cuts[:-1], cuts[1:])]
    Lmax = max(b - a for a, b in zip(cuts[:-1], cuts[1:]))
    kpad = torch.zeros((4, w.B, w.Hkv, Lmax, w.D), dtype=inp["k"].dtype, device="cuda")
    vpad = torch.zeros_like(kpad)
    for r in range(4):
        kpad[r, :, :, :ks[r].shape[2]] = ks[r]
        vpad[r, :, :, :vs[r].shape[2]] = vs[r]
    lens = np.array([[b - a] * w.B for a, b in zip(cuts[:-1], cuts[1:])], np.int32)
    split = run_path(dict(q=inp["q"], k_shards=[kpad[r] for r in range(4)],
                          v_shards=[vpad[r] for r in range(4)], lens=torch.from_numpy(lens).cuda()))
    for b in range(w.B):
        for h in range(w.Hkv):
            ref = ow.group(w, inp["lens_np"], b, h)  # oracle of the unsplit sequence
            heads = slice(h * w.G, (h + 1) * w.G)
            assert_out(to64(split["out"][b, heads]), ref["out"])
            assert_lse(to64(split["lse_out"][b, heads]), ref["lse_out"], floor=True)
            assert_out(to64(whole["out"][b, heads]), ref["out"])


# ------------------------------------------------------------------ full sizes
def _compare_full(w, res, refs, what):
    """Sampled groups of a full-size run against the oracle: every output
    element, the merged lse at the strict 1e-5 relative bar (at these sizes
    |lse| is far from 0, so the max(1, |lse|) floor is not needed), the
    per-shard partials as diagnostics."""
    G = w.G
    for (b, h), ref in refs.items():
        hs = slice(h * G, (h + 1) * G)
        assert_out(to64(res["out"][b, hs]), ref["out"], f"{what} out b={b} h={h}")
        assert_lse(to64(res["lse_out"][b, hs]), ref["lse_out"], f"{what} lse_out b={b} h={h}")
        assert_out(to64(res["o_part"][:, b, hs]), ref["o_part"], f"{what} o_part b={b} h={h}")
        assert_lse(to64(res["lse_part"][:, b, hs]), ref["lse_part"], f"{what} lse_part b={b} h={h}",
                   floor=True)


def _full(name, groups_fn):
    w = sc.WORKLOADS[name]
    _say(f"attn full {name}: allocating and filling inputs")
    inp = sg.attn_inputs(w)
    torch.cuda.synchronize()
    _say(f"attn full {name}: running")
    res = run_path(inp)
    lens = inp["lens_np"]
    # properties on every row
    lse_out = to64(res["lse_out"])
    lse_part = to64(res["lse_part"])
    assert torch.isfinite(res["out"].float()).all()
    live = np.repeat(lens[:, :, None] > 0, w.Hq, axis=2)        # [R,B,Hq]
    assert np.array_equal(np.isneginf(lse_part), ~live)
    anylive = live.any(axis=0)
    assert np.array_equal(np.isneginf(lse_out), ~anylive)
    Mx = np.where(live, lse_part, -np.inf).max(axis=0)
    nl = live.sum(axis=0)
    assert np.all(lse_out[anylive] >= Mx[anylive] - 1e-5 * np.abs(Mx[anylive]))
    assert np.all(lse_out[anylive] <= Mx[anylive] + np.log(nl[anylive]) + 1e-5 * np.abs(Mx[anylive]))
    # the whole step on the same inputs, in the launch configuration the benchmark times
    _say(f"attn full {name}: whole step")
    step = {k: torch.empty_like(v) for k, v in res.items()}
    desc = cp.make_attn_desc(inp["q"], inp["k_shards"])
    print(f"[info] whole step: {cp.step_launches(desc)} launch(es)", flush=True)
    ws = torch.zeros(cp.step_workspace_bytes(desc), dtype=torch.uint8, device="cuda")
    cp.cp_decode(inp["q"], inp["k_shards"], inp["v_shards"], inp["lens"], step["o_part"],
                 step["lse_part"], step["out"], step["lse_out"], workspace=ws)
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(ws[:cp.STEP_COUNTER_BYTES]).item()) == 0
    assert torch.equal(torch.isneginf(step["lse_part"]), torch.isneginf(res["lse_part"]))
    fin = torch.isfinite(res["lse_part"])
    assert torch.allclose(step["lse_part"][fin], res["lse_part"][fin], rtol=1e-6, atol=1e-6)
    assert torch.allclose(step["o_part"], res["o_part"], rtol=1e-5, atol=1e-6)
    assert np.array_equal(np.isneginf(to64(step["lse_out"])), ~anylive)
    # against the two calls: one output rounding apart at most
    d = (step["out"].float() - res["out"].float()).abs()
    assert bool((d <= 2.0 ** -7 * res["out"].float().abs() + 1e-6).all())
    res = {k: v.cpu() for k, v in res.items()}
    step = {k: v.cpu() for k, v in step.items()}
    del inp, ws
    torch.cuda.empty_cache()
    groups = groups_fn(w, lens)
    _say(f"attn full {name}: oracle on {len(groups)} sampled groups")
    refs = {(b, h): ow.group(w, lens, b, h) for (b, h) in groups}
    _compare_full(w, res, refs, "two calls")
    _compare_full(w, step, refs, "step")


def _random_groups(w, n, seed):
    rng = np.random.default_rng(seed)
    idx = rng.choice(w.B * w.Hkv, size=n, replace=False)
    return [(int(i) // w.Hkv, int(i) % w.Hkv) for i in sorted(idx)]


def test_attn_full_c1():
    _full("c1", lambda w, lens: all_groups(w))


def test_attn_full_c2():
    _full("c2", lambda w, lens: all_groups(w))


def test_attn_full_c3():
    """32 seeded random (sequence, kv head) groups of 512, plus the corners."""
    _full("c3", lambda w, lens: sorted({(0, 0), (63, 7)} | set(_random_groups(w, 32, 3003))))


def test_attn_full_c4():
    """Every kv head of sequences 0..12 (the 13 forced unaligned lengths
    1 ... 16384, one shard each), the last sequence with an empty shard,
    and 32 seeded random groups of 2048."""
    def groups(w, lens):
        forced = {(b, h) for b in range(len(sc.EDGE_LENGTHS)) for h in range(w.Hkv)}
        for i, e in enumerate(sc.EDGE_LENGTHS):
            assert lens[i % w.R, i] == e
        empty_b = int(np.where((lens == 0).any(axis=0))[0][-1])
        return sorted(forced | {(empty_b, 2)} | set(_random_groups(w, 32, 3004)))
    _full("c4", groups)


# ------------------------------------------------------------ maximum capacity
# The largest capacity the ABI accepts at D = 128, 16-bit K/V: one (shard,
# sequence, kv head) spans just under 2 GiB (capacity * token stride * 2 <
# 2^31, the limit of 32-bit buffer offsets).  The oracle cannot hold such
# shards in float64, so the inputs have a closed-form result: ordinary tokens
# have k = 0 and v = c; token 0 has k = b e_1 and v = vf, the last valid token
# k = b e_0 and v = vl; query head 0 is a e_0 and head 1 a e_1.  With
# E = exp(a b / sqrt(D)), head 0 gets o = (E vl + vf + (L-2) c) / (E + L - 1)
# and head 1 o = (E vf + vl + (L-2) c) / (E + L - 1), both with
# lse = ln(E + L - 1).  E is close to L, so the last token, the first and
# every chunk of ordinary tokens all move the result.
MAX_D = 128
MAX_CAP = (2 ** 31 - 1) // (MAX_D * 2)          # 8,388,607 tokens


def _max_cap_case(dt="bf16"):
    a, bk = 12.0, 15.0                            # exact in bf16 and fp16; a * bk / sqrt(128) = 15.91
    tdt = torch.bfloat16 if dt == "bf16" else torch.float16
    R, cap, D = 2, MAX_CAP, MAX_D
    lens = [cap, cap - 13]                        # full, and a ragged tail before NaN padding
    d = torch.arange(1, D + 1, dtype=torch.float64)
    vl = [d / 128, -d / 128]                      # per shard, bf16-exact
    vf = [-d / 256, -d / 512]
    c = [0.25, -0.125]
    q = torch.zeros(1, 2, D, dtype=tdt, device="cuda")
    q[0, 0, 0], q[0, 1, 1] = a, a
    ks, vs = [], []
    for r in range(R):
        L = lens[r]
        k = torch.zeros(1, 1, cap, D, dtype=tdt, device="cuda")
        v = torch.full((1, 1, cap, D), c[r], dtype=tdt, device="cuda")
        k[0, 0, 0, 1] = bk
        k[0, 0, L - 1, 0] = bk
        v[0, 0, 0] = vf[r].to(tdt).cuda()
        v[0, 0, L - 1] = vl[r].to(tdt).cuda()
        if L < cap:                               # padding past the length: NaN, never read
            k[0, 0, L:] = float("nan")
            v[0, 0, L:] = float("nan")
        ks.append(k)
        vs.append(v)
    E = np.exp(a * bk / np.sqrt(D))
    o_ref = np.zeros((R, 1, 2, D))
    o_mag = np.zeros((R, 1, 2, D))                # the same sums over |terms|
    lse_ref = np.zeros((R, 1, 2))
    for r in range(R):
        L = lens[r]
        den = E + (L - 1)
        first, last = vf[r].numpy(), vl[r].numpy()
        o_ref[r, 0, 0] = (E * last + first + (L - 2) * c[r]) / den
        o_ref[r, 0, 1] = (E * first + last + (L - 2) * c[r]) / den
        o_mag[r, 0, 0] = (E * np.abs(last) + np.abs(first) + (L - 2) * abs(c[r])) / den
        o_mag[r, 0, 1] = (E * np.abs(first) + np.abs(last) + (L - 2) * abs(c[r])) / den
        lse_ref[r, 0, :] = np.log(den)
    lens_t = torch.tensor(lens, dtype=torch.int32, device="cuda").view(R, 1)
    return dict(q=q, k_shards=ks, v_shards=vs, lens=lens_t), o_ref, o_mag, lse_ref


@pytest.mark.parametrize("dt", ["bf16", "fp16"])
@pytest.mark.parametrize("chunk", [0, 2 ** 18, 2 ** 23],
                         ids=["library chunks", "longest chunks", "whole shard asked, 2^18 used"])
def test_attn_max_capacity(chunk, dt):
    """Both attention entry points at the largest capacity.  Per-shard
    results against the magnitude of their terms: the FP32 p.V accumulation
    drifts by ~1e-7 of it per tile a wave adds on this input (~5e-5 at 512
    tiles per wave, ~2e-4 at 2048, the most a chunk of 2^18 tokens gives a
    wave), so 1e-4 is allowed up to 512 tiles per wave and 5e-4 beyond;
    dropping one chunk (at least 1/64 of the shard) would move the results
    by ~8e-3.  A request for whole-shard chunks gets the longest chunk the
    library runs, 2^18 tokens: over the 65536 tiles per wave of a whole shard
    the drift passes the output tolerance on this input."""
    from oracle import oracle as orc
    _say(f"attn max capacity {MAX_CAP} tokens, {dt}, chunk_tokens={chunk}: filling inputs")
    inp, o_ref, o_mag, lse_ref = _max_cap_case(dt)
    desc = cp.make_attn_desc(inp["q"], inp["k_shards"], chunk_tokens=chunk)
    plan = cp.attn_plan(desc)
    assert plan["chunk_tokens"] <= 2 ** 18 and plan["num_chunks"] <= 64
    if chunk:
        assert plan["chunk_tokens"] == min(chunk, 2 ** 18)
    wave_tiles = plan["chunk_tokens"] // (32 * plan["waves"])
    over = cp.make_attn_desc(inp["q"], inp["k_shards"], kv_capacity=MAX_CAP + 1, chunk_tokens=chunk)
    with pytest.raises(cp.CpdecError):            # one token more is past the 32-bit offsets
        cp.attn_plan(over)
    torch.cuda.synchronize()
    _say(f"attn max capacity: plan {plan}, step launches {cp.step_launches(desc)}: two calls")
    two = run_path(inp, chunk_tokens=chunk)
    _say("attn max capacity: whole step")
    ws = torch.zeros(cp.step_workspace_bytes(desc), dtype=torch.uint8, device="cuda")
    step = {k: torch.empty_like(t) for k, t in two.items()}
    cp.cp_decode(inp["q"], inp["k_shards"], inp["v_shards"], inp["lens"], step["o_part"],
                 step["lse_part"], step["out"], step["lse_out"], chunk_tokens=chunk, workspace=ws)
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(ws[:cp.STEP_COUNTER_BYTES]).item()) == 0
    out_ref = np.zeros((1, 2, MAX_D))
    lo_ref = np.zeros((1, 2))
    for h in range(2):
        out_ref[0, h], lo_ref[0, h] = orc.merge(o_ref[:, 0, h], lse_ref[:, 0, h])
    for what, res in (("two calls", two), ("step", step)):
        o = to64(res["o_part"])
        err = np.abs(o - o_ref) / o_mag
        tol = 1e-4 if wave_tiles <= 512 else 5e-4
        assert err.max() <= tol, f"{what} o_part: max error / term magnitude {err.max():.2e}"
        assert_lse(to64(res["lse_part"]), lse_ref, f"{what} lse_part")
        assert_out(to64(res["out"]), out_ref, f"{what} out")
        assert_lse(to64(res["lse_out"]), lo_ref, f"{what} lse_out", floor=True)
    del inp, two, step, ws
    torch.cuda.empty_cache()


def test_attn_attention_sink():
    """Token 0 of every (shard, sequence, kv head) carries about half of the
    softmax weight (its key is the least-norm key that gives every query head
    of the group the score 10.5, against ~N(0,1) for the other tokens): the
    pattern under which FP32 running sums lose a fixed fraction of every
    later term.  Ragged lengths up to 20000 tokens, both entry points, every
    output against the oracle."""
    from oracle import oracle as orc
    R, B, Hq, Hkv, D, cap = 2, 2, 8, 2, 128, 20000
    G = Hq // Hkv
    lens = np.array([[20000, 15000], [17001, 20000]], np.int32)
    _say("attention sink: inputs")
    g = torch.Generator().manual_seed(4242)
    q = torch.randn(B, Hq, D, generator=g).to(torch.bfloat16)
    k = torch.randn(R, B, Hkv, cap, D, generator=g).to(torch.bfloat16)
    v = torch.randn(R, B, Hkv, cap, D, generator=g).to(torch.bfloat16)
    Q = q.double().view(B, Hkv, G, D)
    rhs = torch.full((B, Hkv, G, 1), 10.5 * np.sqrt(D), dtype=torch.float64)
    sink = (Q.transpose(-1, -2) @ torch.linalg.solve(Q @ Q.transpose(-1, -2), rhs)).squeeze(-1)
    k[:, :, :, 0] = sink.to(torch.bfloat16).unsqueeze(0)            # same key in every shard
    q64, k64, v64 = (t.double().numpy() for t in (q, k, v))
    o_ref, lp_ref, out_ref, lo_ref = orc.cp_decode(q64, list(k64), list(v64), lens, Hkv)
    # the sink's share of the weight, from the oracle's own lse
    s0 = np.einsum("bhgd,rbhd->rbhg", q64.reshape(B, Hkv, G, D), k64[:, :, :, 0]) / np.sqrt(D)
    share = np.exp(s0.reshape(R, B, Hq) - lp_ref)
    assert 0.3 < share.min() and share.max() < 0.8, f"sink share {share.min():.2f}..{share.max():.2f}"
    inp = dict(q=q.cuda(), k_shards=[t.cuda() for t in k], v_shards=[t.cuda() for t in v],
               lens=torch.from_numpy(lens).cuda())
    _say("attention sink: two calls")
    two = run_path(inp)
    _say("attention sink: whole step")
    desc = cp.make_attn_desc(inp["q"], inp["k_shards"])
    ws = torch.zeros(cp.step_workspace_bytes(desc), dtype=torch.uint8, device="cuda")
    step = {kk: torch.empty_like(t) for kk, t in two.items()}
    cp.cp_decode(inp["q"], inp["k_shards"], inp["v_shards"], inp["lens"], step["o_part"],
                 step["lse_part"], step["out"], step["lse_out"], workspace=ws)
    torch.cuda.synchronize()
    for what, res in (("two calls", two), ("step", step)):
        assert_out(to64(res["o_part"]), o_ref, f"{what} o_part")
        assert_lse(to64(res["lse_part"]), lp_ref, f"{what} lse_part", floor=True)
        assert_out(to64(res["out"]), out_ref, f"{what} out")
        assert_lse(to64(res["lse_out"]), lo_ref, f"{what} lse_out", floor=True)
        # the per-shard partials well inside the bar: 1e-5 relative to the row's scale
        err = np.abs(to64(res["o_part"]) - o_ref).max(axis=-1)
        assert (err <= 1e-5 * np.abs(o_ref).max(axis=-1) + 1e-6).all(), f"{what} o_part drift"


@pytest.mark.parametrize("scale", [0.02, 0.3, 1.0])
def test_attn_custom_scale(scale):
    """An explicit softmax scale (sm_scale) in both entry points, against the
    oracle with the same scale: a nearly flat softmax (0.02), a sharper one
    (0.3) and a very peaky one (1.0 on k x3 scores, std ~30)."""
    w = sc.small("c4", B=4, Hq=16, Hkv=4, Lcap=300)    # ragged, GQA 4, split shards
    _say(f"attn custom scale {scale}")
    inp = sg.attn_inputs(w)
    q, R = inp["q"], w.R
    o_part = torch.empty((R, w.B, w.Hq, w.D), dtype=torch.float32, device="cuda")
    lse_part = torch.empty((R, w.B, w.Hq), dtype=torch.float32, device="cuda")
    cp.attn_partial(q, inp["k_shards"], inp["v_shards"], inp["lens"], o_part, lse_part, sm_scale=scale)
    out = torch.empty((w.B, w.Hq, w.D), dtype=q.dtype, device="cuda")
    lse_out = torch.empty((w.B, w.Hq), dtype=torch.float32, device="cuda")
    cp.lse_merge(o_part, lse_part, out, lse_out)
    step = dict(o_part=torch.empty_like(o_part), lse_part=torch.empty_like(lse_part),
                out=torch.empty_like(out), lse_out=torch.empty_like(lse_out))
    cp.cp_decode(q, inp["k_shards"], inp["v_shards"], inp["lens"], step["o_part"], step["lse_part"],
                 step["out"], step["lse_out"], sm_scale=scale)
    torch.cuda.synchronize()
    two = dict(o_part=o_part, lse_part=lse_part, out=out, lse_out=lse_out)
    for what, res in (("two calls", two), ("step", step)):
        for (b, h) in all_groups(w):
            ref = ow.group(w, inp["lens_np"], b, h, scale=scale)
            hs = slice(h * w.G, (h + 1) * w.G)
            assert_out(to64(res["out"][b, hs]), ref["out"], f"{what} out b={b} h={h}")
            assert_lse(to64(res["lse_out"][b, hs]), ref["lse_out"], f"{what} lse_out b={b} h={h}",
                       floor=True)
            assert_out(to64(res["o_part"][:, b, hs]), ref["o_part"], f"{what} o_part b={b} h={h}")
            assert_lse(to64(res["lse_part"][:, b, hs]), ref["lse_part"], f"{what} lse_part b={b} h={h}",
                       floor=True)
    # the default scale differs from these: the scale really reaches the kernel
    ref0 = ow.group(w, inp["lens_np"], 0, 0)
    assert not np.allclose(ref0["lse_out"], ow.group(w, inp["lens_np"], 0, 0, scale=scale)["lse_out"])


@pytest.mark.parametrize("chunk", [0, 64])
def test_attn_shard_permutation(chunk):
    """Permuting the shards (K/V pointers and lens rows together) permutes
    the per-shard partials bit for bit (a shard's attention does not depend
    on its index) and leaves the merged output within one output rounding
    and the merged lse within 1e-6 (the merge sums in shard order), in both
    entry points; the permuted run also meets the oracle."""
    w = sc.small("c4", R=5, B=3, Hq=8, Hkv=2, Lcap=300)   # ragged with empty shards
    _say(f"attn shard permutation, chunk {chunk}")
    inp = sg.attn_inputs(w)
    perm = [3, 0, 4, 2, 1]
    inp_p = dict(inp)
    inp_p["k_shards"] = [inp["k_shards"][r] for r in perm]
    inp_p["v_shards"] = [inp["v_shards"][r] for r in perm]
    inp_p["lens"] = inp["lens"][perm].contiguous()
    inp_p["lens_np"] = inp["lens_np"][perm]
    for what, run in (("two calls", lambda i: run_path(i, chunk_tokens=chunk)),
                      ("step", lambda i: _step(i, chunk))):
        base, res = run(inp), run(inp_p)
        assert torch.equal(res["o_part"], base["o_part"][perm]), f"{what} o_part"
        assert torch.equal(res["lse_part"], base["lse_part"][perm]), f"{what} lse_part"
        assert torch.equal(torch.isneginf(res["lse_out"]), torch.isneginf(base["lse_out"]))
        fin = torch.isfinite(base["lse_out"])
        assert torch.allclose(res["lse_out"][fin], base["lse_out"][fin], rtol=1e-6, atol=1e-6)
        d = (res["out"].float() - base["out"].float()).abs()
        assert bool((d <= 2.0 ** -7 * base["out"].float().abs() + 1e-6).all()), f"{what} out"
        for b in range(w.B):
            for h in range(w.Hkv):
                ref = ow.group(w, inp["lens_np"], b, h)
                hs = slice(h * w.G, (h + 1) * w.G)
                assert_out(to64(res["out"][b, hs]), ref["out"], f"{what} out b={b} h={h}")
                assert_lse(to64(res["lse_out"][b, hs]), ref["lse_out"], f"{what} lse_out b={b} h={h}",
                           floor=True)
