"""Pins for the CPU oracle: checks against facts fixed by the page and by
mathematics, not by the oracle itself.

Each ``pin_*`` function takes an implementation namespace ``impl`` with
``attend_shard``, ``merge`` and ``cp_decode`` (the oracle, or a copy with a
planted mistake) and raises AssertionError when the implementation disagrees
with the fact it checks.  ``tests/test_oracle_pins.py`` runs them on the
oracle; ``tests/test_oracle_mutations.py`` runs them on planted mistakes.

The method is the one on the page "FlashInfer's Context-Parallel Decode
optimisation: Fused A2A + LSE Reduce" (flashinfer PR #4929): per-shard
partial attention (section "Introduction") merged with LSE softmax weights
(section "Code analysis, 1. Fused kernel").
"""
from __future__ import annotations

import math

import numpy as np

INF = math.inf


def _rng(seed):
    return np.random.default_rng(seed)


# --------------------------------------------------------------- attention pins
def pin_textbook_bruteforce(impl, seed=0, cases=60):
    """Brute force on tiny inputs: softmax written as the textbook ratio with
    Python floats and no max subtraction, o = sum e^s v / sum e^s, lse =
    ln sum e^s."""
    rng = _rng(seed)
    for _ in range(cases):
        G = int(rng.integers(1, 4))
        D = int(rng.integers(1, 5))
        L = int(rng.integers(1, 5))
        q = rng.normal(size=(G, D))
        k = rng.normal(size=(L, D))
        v = rng.normal(size=(L, D))
        scale = float(rng.uniform(0.2, 2.0))
        o, lse = impl.attend_shard(q, k, v, scale)
        for g in range(G):
            e = []
            for t in range(L):
                dot = 0.0
                for d in range(D):
                    dot += q[g][d] * k[t][d]
                e.append(math.exp(scale * dot))
            tot = sum(e)
            assert abs(lse[g] - math.log(tot)) <= 1e-12 * max(1.0, abs(math.log(tot)))
            for d in range(D):
                ref = sum(e[t] * v[t][d] for t in range(L)) / tot
                assert abs(o[g][d] - ref) <= 1e-12 * max(1.0, abs(ref))


def pin_single_token(impl):
    """L = 1: the only token has probability 1, so o = v_0 and lse = s_0."""
    q = np.array([[0.5, -1.25, 2.0]])
    k = np.array([[1.0, 0.5, -0.25]])
    v = np.array([[3.0, -7.0, 0.125]])
    o, lse = impl.attend_shard(q, k, v, 0.5)
    assert np.array_equal(o[0], v[0])
    s0 = 0.5 * (0.5 * 1.0 + -1.25 * 0.5 + 2.0 * -0.25)
    assert abs(lse[0] - s0) <= 1e-15


def pin_uniform_scores(impl):
    """All scores equal (k = 0): uniform softmax, o = mean of v, lse = ln L."""
    rng = _rng(1)
    L, D = 7, 5
    q = rng.normal(size=(2, D))
    k = np.zeros((L, D))
    v = rng.normal(size=(L, D))
    o, lse = impl.attend_shard(q, k, v, 0.3)
    for g in range(2):
        assert np.allclose(o[g], v.mean(axis=0), rtol=0, atol=1e-14)
        assert abs(lse[g] - math.log(L)) <= 1e-14


def pin_constant_values(impl):
    """v identical for every token: o = v whatever the scores (normalisation)."""
    rng = _rng(2)
    L, D = 9, 4
    q = rng.normal(size=(3, D)) * 3
    k = rng.normal(size=(L, D)) * 3
    row = np.array([1.5, -2.0, 0.25, 8.0])
    v = np.tile(row, (L, 1))
    o, _ = impl.attend_shard(q, k, v, 1.0)
    assert np.allclose(o, np.tile(row, (3, 1)), rtol=1e-14, atol=0)


def pin_two_tokens_by_hand(impl):
    """Two tokens with scores 1 and 0 (q = e_0, k = I, scale 1):
    o = (e*v1 + v2)/(e + 1), lse = ln(e + 1)."""
    q = np.array([[1.0, 0.0]])
    k = np.array([[1.0, 0.0], [0.0, 1.0]])
    v = np.array([[2.0, 4.0], [-1.0, 0.5]])
    o, lse = impl.attend_shard(q, k, v, 1.0)
    e = math.e
    want = [(e * 2.0 + -1.0) / (e + 1.0), (e * 4.0 + 0.5) / (e + 1.0)]
    assert abs(o[0][0] - want[0]) <= 1e-15 and abs(o[0][1] - want[1]) <= 1e-15
    assert abs(lse[0] - math.log(e + 1.0)) <= 1e-15


def pin_scale_is_applied_to_scores(impl):
    """Scaling q by c and the softmax scale by 1/c changes nothing."""
    rng = _rng(3)
    q = rng.normal(size=(2, 6))
    k = rng.normal(size=(11, 6))
    v = rng.normal(size=(11, 6))
    o1, l1 = impl.attend_shard(q, k, v, 0.25)
    o2, l2 = impl.attend_shard(q * 0.25, k, v, 1.0)
    assert np.allclose(o1, o2, rtol=1e-13, atol=1e-14)
    assert np.allclose(l1, l2, rtol=1e-13, atol=1e-14)
    o3, _ = impl.attend_shard(q, k, v, 2.0)
    assert not np.allclose(o1, o3)


def pin_large_scores_stable(impl):
    """Scores near 1000 (e^s overflows float64): result equals the shifted
    case, since softmax is shift invariant and lse shifts by the same amount."""
    q = np.array([[1.0, 0.0]])
    k = np.array([[1000.0, 0.0], [999.0, 0.0], [998.0, 0.0]])
    v = np.array([[1.0, 0.0], [0.0, 1.0], [1.0, 1.0]])
    o, lse = impl.attend_shard(q, k, v, 1.0)
    z = 1.0 + math.exp(-1.0) + math.exp(-2.0)
    assert np.isfinite(o).all()
    assert abs(o[0][0] - (1.0 + math.exp(-2.0)) / z) <= 1e-14
    assert abs(lse[0] - (1000.0 + math.log(z))) <= 1e-12


def pin_empty_shard(impl):
    """L = 0: the shard contributes nothing: o = 0, lse = -inf."""
    o, lse = impl.attend_shard(np.ones((2, 3)), np.zeros((0, 3)), np.zeros((0, 3)), 1.0)
    assert np.array_equal(o, np.zeros((2, 3)))
    assert np.all(np.isneginf(lse))


def pin_library_sdpa(impl):
    """Independent library routine: torch CPU float64 scaled_dot_product_attention
    for o and torch.logsumexp for lse."""
    import torch
    rng = _rng(4)
    G, L, D = 4, 37, 16
    q = rng.normal(size=(G, D))
    k = rng.normal(size=(L, D)) * 2
    v = rng.normal(size=(L, D))
    scale = 1.0 / math.sqrt(D)
    o, lse = impl.attend_shard(q, k, v, scale)
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64) for x in (q, k, v))
    to = torch.nn.functional.scaled_dot_product_attention(
        tq[None, None], tk[None, None], tv[None, None], scale=scale)[0, 0].numpy()
    tl = torch.logsumexp(scale * (tq @ tk.T), dim=-1).numpy()
    assert np.allclose(o, to, rtol=1e-12, atol=1e-13)
    assert np.allclose(lse, tl, rtol=1e-13, atol=1e-13)


# --------------------------------------------------------------- merge pins
def pin_merge_single_shard_identity(impl):
    """R = 1: weight 1, denominator 1, ln 1 = 0: out = o_1 and lse_out = lse_1
    exactly."""
    rng = _rng(5)
    o = rng.normal(size=(1, 8))
    out, lse = impl.merge(o, np.array([3.7]))
    assert np.array_equal(out, o[0]) and lse == 3.7


def pin_merge_equal_lse(impl):
    """Equal lse: equal weights, so out = mean of the o_r (exact up to the
    power-of-two divide) and lse_out = lse + ln R."""
    rng = _rng(6)
    for R in (2, 4, 8, 3):
        o = rng.normal(size=(R, 6))
        out, lse = impl.merge(o, np.full(R, -1.25))
        assert np.allclose(out, o.sum(0) / R, rtol=1e-15, atol=1e-15)
        assert abs(lse - (-1.25 + math.log(R))) <= 1e-15


def pin_merge_dominant(impl):
    """A shard whose lse exceeds every other by > 800 carries all the weight
    in float64 (e^-800 underflows): out = o_dom and lse_out = lse_dom."""
    rng = _rng(7)
    o = rng.normal(size=(4, 5))
    lse = np.array([-900.0, 2.0, -850.0, -1000.0])
    out, l = impl.merge(o, lse)
    assert np.array_equal(out, o[1]) and l == 2.0


def pin_merge_two_by_hand(impl):
    """Two shards with lse 0 and ln 3: weights 1/4 and 3/4; lse_out = ln 4."""
    o = np.array([[4.0, -8.0], [0.0, 4.0]])
    out, lse = impl.merge(o, np.array([0.0, math.log(3.0)]))
    assert np.allclose(out, [1.0, 1.0], rtol=0, atol=1e-15)
    assert abs(lse - math.log(4.0)) <= 1e-15


def pin_merge_shift(impl):
    """Adding c to every lse leaves out unchanged and adds c to lse_out."""
    rng = _rng(8)
    o = rng.normal(size=(5, 7))
    lse = rng.normal(size=5) * 4
    out1, l1 = impl.merge(o, lse)
    out2, l2 = impl.merge(o, lse + 37.5)
    assert np.allclose(out1, out2, rtol=1e-13, atol=1e-15)
    assert abs((l2 - l1) - 37.5) <= 1e-12


def pin_merge_bounds(impl):
    """max lse_r <= lse_out <= max lse_r + ln(#live shards); out lies in the
    convex hull of the live o_r (per element)."""
    rng = _rng(9)
    for _ in range(20):
        R = int(rng.integers(1, 9))
        o = rng.normal(size=(R, 4))
        lse = rng.normal(size=R) * 6
        out, l = impl.merge(o, lse)
        assert lse.max() - 1e-12 <= l <= lse.max() + math.log(R) + 1e-12
        assert np.all(out <= o.max(0) + 1e-12) and np.all(out >= o.min(0) - 1e-12)


def pin_merge_permutation(impl):
    """Permuting the shards changes nothing (to rounding)."""
    rng = _rng(10)
    o = rng.normal(size=(6, 9))
    lse = rng.normal(size=6) * 3
    perm = rng.permutation(6)
    out1, l1 = impl.merge(o, lse)
    out2, l2 = impl.merge(o[perm], lse[perm])
    assert np.allclose(out1, out2, rtol=1e-13, atol=1e-15)
    assert abs(l1 - l2) <= 1e-13


def pin_merge_empty_shard(impl):
    """An empty shard (lse = -inf) contributes nothing, even if its o row
    holds NaN: inserting it anywhere leaves the result unchanged."""
    rng = _rng(11)
    o = rng.normal(size=(3, 4))
    lse = np.array([0.5, -2.0, 1.5])
    out1, l1 = impl.merge(o, lse)
    for pos in range(4):
        o2 = np.insert(o, pos, np.full(4, np.nan), axis=0)
        lse2 = np.insert(lse, pos, -INF)
        out2, l2 = impl.merge(o2, lse2)
        assert np.array_equal(out1, out2) and l1 == l2


def pin_merge_all_empty(impl):
    """Every shard empty: out = 0 and lse_out = -inf (empty sum)."""
    out, l = impl.merge(np.full((3, 4), np.nan), np.full(3, -INF))
    assert np.array_equal(out, np.zeros(4)) and l == -INF


def pin_round_storage(impl):
    """16-bit storage rounding: exact values unchanged, ties to even, the
    fp16 range and the bf16 ulp of 1 (2^-7)."""
    if not hasattr(impl, "round_storage"):
        return
    rs = impl.round_storage
    exact = np.array([1.0, -2.5, 0.15625, 3.0 * 2.0 ** -20])
    assert np.array_equal(rs(exact, "bf16"), exact) and np.array_equal(rs(exact, "fp16"), exact)
    assert rs(np.array([1.0 + 2.0 ** -8]), "bf16")[0] == 1.0            # tie -> even
    assert rs(np.array([1.0 + 3 * 2.0 ** -8]), "bf16")[0] == 1.0 + 2.0 ** -6  # tie -> even (up)
    assert rs(np.array([1.0 + 2.0 ** -8 + 2.0 ** -12]), "bf16")[0] == 1.0 + 2.0 ** -7
    assert rs(np.array([1.0 + 2.0 ** -11]), "fp16")[0] == 1.0            # fp16 tie -> even
    assert rs(np.array([1.0 + 2.0 ** -10]), "fp16")[0] == 1.0 + 2.0 ** -10
    rng = _rng(16)
    x = rng.normal(size=1000)
    for dt, ulp in (("bf16", 2.0 ** -8), ("fp16", 2.0 ** -11)):
        y = rs(x, dt)
        assert np.all(np.abs(y - x) <= ulp * np.abs(x) + 1e-30)
        assert np.array_equal(rs(y, dt), y)                              # idempotent
    o = rng.normal(size=(3, 5))
    out, l = impl.merge_stored(o, np.array([0.0, 1.0, -1.0]), "bf16")
    out2, l2 = impl.merge(rs(o, "bf16"), np.array([0.0, 1.0, -1.0]))
    assert np.array_equal(out, out2) and l == l2


# --------------------------------------------------------------- whole-path pins
def _random_split_problem(rng, B, Hq, Hkv, D, R, Lmax, empty_p=0.2):
    lens = rng.integers(0, Lmax + 1, size=(R, B))
    lens[rng.random((R, B)) < empty_p] = 0
    Lcap = max(int(lens.max()), 1)
    q = rng.normal(size=(B, Hq, D))
    ks = [rng.normal(size=(B, Hkv, Lcap, D)) * 2 for _ in range(R)]
    vs = [rng.normal(size=(B, Hkv, Lcap, D)) for _ in range(R)]
    return q, ks, vs, lens


def pin_split_invariance(impl, seed=12):
    """Merging the partials of any split equals attention over the unsplit
    sequence (the method's defining property), here written as the textbook
    concatenation computed by the same pinned single-shard routine with R=1."""
    rng = _rng(seed)
    for (B, Hq, Hkv, D, R) in ((2, 4, 2, 8, 3), (1, 2, 2, 4, 5), (3, 8, 1, 6, 2)):
        q, ks, vs, lens = _random_split_problem(rng, B, Hq, Hkv, D, R, 9)
        _, _, out, lse = impl.cp_decode(q, ks, vs, lens, Hkv)
        # the same tokens as a single shard: concatenate valid prefixes
        Ltot = lens.sum(axis=0)
        Lc = max(int(Ltot.max()), 1)
        k1 = np.zeros((B, Hkv, Lc, D))
        v1 = np.zeros((B, Hkv, Lc, D))
        for b in range(B):
            pos = 0
            for r in range(R):
                L = int(lens[r, b])
                k1[b, :, pos:pos + L] = ks[r][b, :, :L]
                v1[b, :, pos:pos + L] = vs[r][b, :, :L]
                pos += L
        _, _, out1, lse1 = impl.cp_decode(q, [k1], [v1], Ltot[None, :], Hkv)
        fin = np.isfinite(lse1)
        assert np.array_equal(fin, np.isfinite(lse))
        assert np.allclose(out, out1, rtol=1e-12, atol=1e-13)
        assert np.allclose(lse[fin], lse1[fin], rtol=1e-12, atol=1e-12)


def pin_gqa_mapping(impl):
    """Query head hq reads kv head hq // G: with Hq=4, Hkv=2, only kv head 1
    carries non-zero values, so heads 2 and 3 see them and heads 0, 1 don't."""
    B, Hq, Hkv, D, L = 1, 4, 2, 3, 5
    rng = _rng(13)
    q = rng.normal(size=(B, Hq, D))
    k = rng.normal(size=(B, Hkv, L, D))
    v = np.zeros((B, Hkv, L, D))
    v[0, 1] = rng.normal(size=(L, D)) + 5.0
    lens = np.array([[L]])
    _, _, out, _ = impl.cp_decode(q, [k], [v], lens, Hkv)
    assert np.all(out[0, 0] == 0) and np.all(out[0, 1] == 0)
    assert np.all(out[0, 2] > 0) and np.all(out[0, 3] > 0)


def pin_default_scale(impl):
    """Without an explicit scale the softmax scale is 1/sqrt(D)."""
    rng = _rng(14)
    q, ks, vs, lens = _random_split_problem(rng, 1, 2, 2, 16, 2, 6, empty_p=0.0)
    _, _, o1, l1 = impl.cp_decode(q, ks, vs, lens, 2)
    _, _, o2, l2 = impl.cp_decode(q, ks, vs, lens, 2, scale=0.25)
    assert np.allclose(o1, o2, rtol=1e-14, atol=1e-15) and np.allclose(l1, l2, rtol=1e-14)


def pin_partials_are_per_shard(impl):
    """cp_decode's per-shard partials equal attend_shard on that shard alone,
    and empty shards give (0, -inf)."""
    rng = _rng(15)
    q, ks, vs, lens = _random_split_problem(rng, 2, 2, 1, 4, 3, 6, empty_p=0.3)
    o_part, lse_part, _, _ = impl.cp_decode(q, ks, vs, lens, 1)
    for r in range(3):
        for b in range(2):
            L = int(lens[r, b])
            o, l = impl.attend_shard(q[b], ks[r][b, 0, :L], vs[r][b, 0, :L], 0.5)
            assert np.allclose(o_part[r, b], o, rtol=1e-14, atol=1e-15)
            assert np.array_equal(np.isneginf(lse_part[r, b]), np.isneginf(l))


ATTEND_PINS = [pin_textbook_bruteforce, pin_single_token, pin_uniform_scores,
               pin_constant_values, pin_two_tokens_by_hand, pin_scale_is_applied_to_scores,
               pin_large_scores_stable, pin_empty_shard, pin_library_sdpa]
MERGE_PINS = [pin_merge_single_shard_identity, pin_merge_equal_lse, pin_merge_dominant,
              pin_merge_two_by_hand, pin_merge_shift, pin_merge_bounds,
              pin_merge_permutation, pin_merge_empty_shard, pin_merge_all_empty,
              pin_round_storage]
PATH_PINS = [pin_split_invariance, pin_gqa_mapping, pin_default_scale,
             pin_partials_are_per_shard]
ALL_PINS = ATTEND_PINS + MERGE_PINS + PATH_PINS
