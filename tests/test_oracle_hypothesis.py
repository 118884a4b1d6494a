"""Property-based checks of the oracle (CPU, hypothesis, derandomized so a
run is reproducible).  They complement the seeded pins with generated
shapes and values, shrunk to a minimal case on failure:

* attention equals the textbook softmax ratio written with Python floats and
  no max subtraction (scores kept small enough for exp not to overflow);
* splitting a shard at any point and merging the two partials gives the
  unsplit result ([CP] "Introduction": the shards' partials merged with LSE
  weights are ordinary attention over the whole sequence);
* the merge is invariant under permuting shards, an empty shard (lse = -inf,
  any row content) changes nothing, and max lse <= merged lse <=
  max lse + ln(#live shards).
"""
import math

import numpy as np
from hypothesis import given, settings, strategies as st

from oracle import oracle as orc

SETTINGS = settings(max_examples=200, deadline=None, derandomize=True)
finite = st.floats(min_value=-3.0, max_value=3.0, allow_nan=False, allow_infinity=False)


@st.composite
def shard(draw, min_len=1, max_len=6):
    G = draw(st.integers(1, 3))
    D = draw(st.integers(1, 4))
    L = draw(st.integers(min_len, max_len))
    q = np.array(draw(st.lists(st.lists(finite, min_size=D, max_size=D), min_size=G, max_size=G)))
    k = np.array(draw(st.lists(st.lists(finite, min_size=D, max_size=D), min_size=L, max_size=L)))
    v = np.array(draw(st.lists(st.lists(finite, min_size=D, max_size=D), min_size=L, max_size=L)))
    scale = draw(st.floats(min_value=0.05, max_value=2.0))
    return q.reshape(G, D), k.reshape(L, D), v.reshape(L, D), scale


@SETTINGS
@given(shard())
def test_attention_is_the_textbook_ratio(case):
    q, k, v, scale = case
    o, lse = orc.attend_shard(q, k, v, scale)
    G, D = q.shape
    L = k.shape[0]
    for g in range(G):
        e = [math.exp(scale * sum(q[g][d] * k[t][d] for d in range(D))) for t in range(L)]
        tot = sum(e)
        assert abs(lse[g] - math.log(tot)) <= 1e-12 * max(1.0, abs(math.log(tot)))
        for d in range(D):
            ref = sum(e[t] * v[t][d] for t in range(L)) / tot
            assert abs(o[g][d] - ref) <= 1e-12 * max(1.0, abs(ref))


@SETTINGS
@given(shard(min_len=2, max_len=8), st.data())
def test_any_split_merges_to_the_unsplit_result(case, data):
    q, k, v, scale = case
    L = k.shape[0]
    cut = data.draw(st.integers(0, L))              # either side may be empty
    o_a, l_a = orc.attend_shard(q, k[:cut], v[:cut], scale)
    o_b, l_b = orc.attend_shard(q, k[cut:], v[cut:], scale)
    o, lse = orc.attend_shard(q, k, v, scale)
    for g in range(q.shape[0]):
        out, lo = orc.merge(np.stack([o_a[g], o_b[g]]), np.array([l_a[g], l_b[g]]))
        assert np.allclose(out, o[g], rtol=1e-12, atol=1e-12)
        assert abs(lo - lse[g]) <= 1e-12 * max(1.0, abs(lse[g]))


@st.composite
def partials(draw):
    R = draw(st.integers(1, 6))
    D = draw(st.integers(1, 4))
    o = np.array(draw(st.lists(finite, min_size=R * D, max_size=R * D))).reshape(R, D)
    lse = np.array(draw(st.lists(st.one_of(st.floats(-50.0, 50.0), st.just(-math.inf)),
                                 min_size=R, max_size=R)))
    return o, lse


@SETTINGS
@given(partials(), st.randoms(use_true_random=False))
def test_merge_permutation_empty_shard_and_bounds(case, rnd):
    o, lse = case
    out, lo = orc.merge(o, lse)
    perm = list(range(len(lse)))
    rnd.shuffle(perm)
    out_p, lo_p = orc.merge(o[perm], lse[perm])
    assert np.allclose(out_p, out, rtol=1e-12, atol=1e-12)
    assert (lo_p == lo) or abs(lo_p - lo) <= 1e-12 * max(1.0, abs(lo))
    # an empty shard with garbage in its row changes nothing, bit for bit
    pos = rnd.randrange(len(lse) + 1)
    o_e = np.insert(o, pos, np.full(o.shape[1], np.nan), axis=0)
    lse_e = np.insert(lse, pos, -math.inf)
    out_e, lo_e = orc.merge(o_e, lse_e)
    assert np.array_equal(out_e, out) and (lo_e == lo)
    live = np.isfinite(lse)
    if not live.any():
        assert lo == -math.inf and not out.any()
        return
    M = lse[live].max()
    assert M - 1e-12 <= lo <= M + math.log(int(live.sum())) + 1e-12
    # the output lies in the box spanned by the live partials
    assert (out >= o[live].min(axis=0) - 1e-12).all() and (out <= o[live].max(axis=0) + 1e-12).all()
