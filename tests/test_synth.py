"""The seeded input streams (CPU side): generator known answers, rounding,
distribution sanity and the workload recipes."""
import os

import numpy as np
import pytest

from synth import configs as sc
from synth import philox

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _kat():
    rows = []
    with open(os.path.join(GOLDEN, "philox4x32_10_kat.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                rows.append([int(x, 16) for x in line.split()])
    return rows


@pytest.mark.parametrize("row", _kat())
def test_philox_known_answers(row):
    ctr, key, want = row[0:4], row[4:6], row[6:10]
    got = philox.philox4x32(*[[c] for c in ctr], *key)
    assert [int(g[0]) for g in got] == want


def test_stream_slices_are_consistent():
    full = philox.normal_f32(7, 3, 0, 1000)
    for start in (0, 1, 2, 3, 5, 511, 997):
        part = philox.normal_f32(7, 3, start, 1000 - start)
        assert np.array_equal(part, full[start:])
    w = philox.words(7, 3, 0, 64)
    assert np.array_equal(philox.words(7, 3, 13, 20), w[13:33])


def test_normal_moments():
    z = philox.normal_f32(11, 1, 0, 1 << 20).astype(np.float64)
    assert abs(z.mean()) < 5e-3 and abs(z.std() - 1) < 5e-3
    # tail mass beyond 3 sigma ~ 0.0027
    assert abs((np.abs(z) > 3).mean() - 0.0026998) < 4e-4


def test_bf16_round_nearest_even():
    # 1 + 2^-8 is exactly half-way between bf16 1.0 and 1 + 2^-7: ties to even (1.0)
    x = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 1.0 + 2 ** -8 + 2 ** -20], np.float32)
    bits = philox.f32_to_bf16_bits(x)
    vals = philox.bf16_bits_to_f32(bits)
    assert vals[0] == 1.0
    assert vals[1] == 1.0 + 4 * 2 ** -8      # tie goes to the even mantissa
    assert vals[2] == -2.5
    assert vals[3] == 1.0 + 2 ** -7          # above the tie rounds up


def test_uniform_int_and_bernoulli():
    u = philox.uniform_int(5, 4, 0, 200000, 16385)
    assert u.min() >= 0 and u.max() <= 16384
    assert abs(u.mean() - 8192) < 60
    b = philox.bernoulli(5, 5, 0, 200000, 0.05)
    assert abs(b.mean() - 0.05) < 3e-3


def test_ragged_lengths_recipe():
    w = sc.WORKLOADS["c4"]
    L = sc.lens(w)
    assert L.shape == (8, 256) and L.dtype == np.int32
    assert L.min() == 0 and L.max() == 16384
    for i, e in enumerate(sc.EDGE_LENGTHS):
        assert L[i % 8, i] == e
    assert 0.03 < (L == 0).mean() < 0.08


def test_merge_recipe():
    w = sc.WORKLOADS["c5"].scaled(rows=4096)
    lse = sc.merge_lse(w)
    fin = np.isfinite(lse)
    assert abs((~fin).mean() - 0.05) < 0.01
    assert abs(lse[fin].std() - 4.0) < 0.1
    o = sc.merge_opart_values(w, 3, 100, 2)
    s = sc.merge_opart_storage(w)
    assert np.array_equal(philox.bf16_bits_to_f32(s[3, 100:102]), o)


def test_kv_slice_matches_whole_tensor():
    w = sc.small("c3", B=2, Hq=4, Hkv=2, Lcap=40, L=40, R=2)
    kbits = sc.kv_storage(w, "k")
    part = sc.kv_values(w, "k", 1, 1, 0, 33)
    assert np.array_equal(philox.bf16_bits_to_f32(kbits[1, 1, 0, :33]), part)
    w4 = sc.small("c4", B=2, Lcap=64)
    k4 = sc.kv_values(w4, "k", 0, 0, 0, 8)
    z = philox.normal_f32(w4.seed, sc.TAG_K, 0, 8 * w4.D).reshape(8, w4.D)
    assert np.array_equal(k4, philox.round_to((z * np.float32(3)).astype(np.float32), "bf16")[1])
