"""The workload glue under every GPU parity test, tied to the oracle's own
whole-batch functions (CPU only).

``oracle.workloads.group`` regenerates one (sequence, kv head) group's
slices from the seeded streams and runs the oracle on them; here the same
workloads are materialised whole (``synth.configs.kv_storage``,
``q_storage``, ``merge_opart_storage``: the exact storage values of the
tensors the GPU receives) and run through ``oracle.cp_decode`` /
``oracle.merge_rows``.  Any slip in the glue's indexing (a wrong shard,
sequence, head block or token offset, a wrong length, the k scale not
applied) makes the two disagree.  The cases cover GQA, ragged lengths with
the forced unaligned edge lengths, empty shards, an all-empty sequence and
the merge workload's -inf rows."""
import numpy as np
import pytest

from oracle import oracle, workloads as ow
from synth import configs as sc
from synth import philox


def _values(bits, dtype):
    if dtype == "bf16":
        return philox.bf16_bits_to_f32(bits).astype(np.float64)
    if dtype == "fp16":
        return np.asarray(bits).view(np.float16).astype(np.float64)
    return np.asarray(bits, dtype=np.float64)


def _whole(w):
    q = _values(sc.q_storage(w), w.dtype)
    k = _values(sc.kv_storage(w, "k"), w.dtype)
    v = _values(sc.kv_storage(w, "v"), w.dtype)
    return q, k, v


CASES = {
    "uniform lengths, GQA 4 (c3 recipe)": (sc.small("c3", B=3, Lcap=40, L=37), None),
    "ragged, GQA 8, k x3, edge lengths (c4 recipe)": (sc.small("c4", B=14, Lcap=130), None),
    "ragged, forced empty shard and all-empty sequence": (sc.small("c4", R=3, B=4, Hq=16, Hkv=4,
                                                                   Lcap=70), "empties"),
    "fp16, D64, G3": (sc.small("c3", R=5, B=2, Hq=6, Hkv=2, D=64, dtype="fp16", Lcap=33, L=33), None),
    "MHA, one shard (c2 recipe)": (sc.small("c2", R=1, B=2, Lcap=50, L=50), None),
}


@pytest.mark.parametrize("name", list(CASES))
def test_group_matches_whole_batch_oracle(name):
    w, mod = CASES[name]
    lens = sc.lens(w)
    if mod == "empties":
        lens = lens.copy()
        lens[1, 0] = 0          # one empty shard
        lens[:, 2] = 0          # every shard of sequence 2 empty
    if w.ragged and mod is None:
        # the forced edge lengths land in the first min(B, 13) sequences
        for i in range(min(w.B, len(sc.EDGE_LENGTHS))):
            assert lens[i % w.R, i] == min(sc.EDGE_LENGTHS[i], w.Lcap)
    q, k, v = _whole(w)
    o_part, lse_part, out, lse_out = oracle.cp_decode(q, list(k), list(v), lens, w.Hkv,
                                                      scale=w.sm_scale)
    G = w.G
    for b in range(w.B):
        for h in range(w.Hkv):
            g = ow.group(w, lens, b, h)
            hs = slice(h * G, (h + 1) * G)
            for key, ref in (("o_part", o_part[:, b, hs]), ("lse_part", lse_part[:, b, hs]),
                             ("out", out[b, hs]), ("lse_out", lse_out[b, hs])):
                got = g[key]
                assert got.shape == ref.shape, (key, b, h)
                assert np.array_equal(np.isneginf(got), np.isneginf(ref)), (key, b, h)
                fin = np.isfinite(ref)
                assert np.allclose(got[fin], ref[fin], rtol=1e-13, atol=1e-15), (key, b, h)
    if mod == "empties":
        assert np.all(np.isneginf(lse_out[2])) and np.all(out[2] == 0)
        assert np.all(np.isneginf(lse_part[1, 0]))


def test_group_applies_the_workload_k_scale():
    """c4's keys are 3z: the glue's keys equal the whole tensor's, and differ
    from the unscaled stream."""
    w = sc.small("c4", B=2, Lcap=20)
    L = 20
    kv = sc.kv_values(w, "k", 1, 1, 3, L).astype(np.float64)
    whole = _values(sc.kv_storage(w, "k"), w.dtype)[1, 1, 3, :L]
    assert np.array_equal(kv, whole)
    plain = sc.kv_values(w.scaled(k_scale=1.0), "k", 1, 1, 3, L).astype(np.float64)
    assert not np.allclose(kv, plain)
    assert np.allclose(kv, 3.0 * plain, rtol=2.0 ** -7, atol=0)


def test_merge_rows_matches_whole_oracle():
    """The merge workload's rows through the glue against oracle.merge_rows
    over the whole materialised o_part / lse_part, including rows with -inf
    shards."""
    w = sc.WORKLOADS["c5"].scaled(rows=300)
    lse = sc.merge_lse(w).astype(np.float64)
    o = _values(sc.merge_opart_storage(w), w.dtype)
    assert np.isneginf(lse).any()
    out_all, lse_all = oracle.merge_rows(o, lse)
    rows = np.array([0, 1, 7, 150, 299] + [int(n) for n in np.where(np.isneginf(lse).any(axis=0))[0][:5]])
    out, lo = ow.merge_rows(w, rows)
    assert np.array_equal(out, out_all[rows])
    assert np.array_equal(lo, lse_all[rows])
