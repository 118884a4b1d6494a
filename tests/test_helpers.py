"""The storage-aware output check (CPU): a 16-bit partial that lies within
FP32 accuracy of a rounding boundary may be stored on either side of it, and
that alone must not fail the check; an error beyond the bar still must."""
import numpy as np

from oracle import oracle as orc
from tests.helpers import assert_out_stored

MID = 0.2998046875      # halfway between the bf16 values 0.298828125 and 0.30078125


def _case():
    o = np.array([[[-(MID + 3e-8), 0.1, 0.2, 0.3]], [[0.58098857, 0.1, 0.2, 0.3]]])  # [R, G, D]
    lse = np.array([[7.09919993], [6.381107]])
    return o, lse


def test_flip_at_a_rounding_boundary_is_accepted():
    o, lse = _case()
    flipped = o.copy()
    flipped[0, 0, 0] = -(MID - 3e-8)          # within FP32 accuracy, stored one step away
    gpu = orc.merge_stored(flipped[:, 0], lse[:, 0], "bf16")[0][None]
    ref = orc.merge_stored(o[:, 0], lse[:, 0], "bf16")[0][None]
    assert abs(gpu[0, 0] - ref[0, 0]) > 2.0 ** -7 * abs(ref[0, 0]) + 1e-3  # over the plain bar
    assert assert_out_stored(gpu, o, lse, "bf16") <= 1.0


def test_error_beyond_the_bar_is_rejected():
    o, lse = _case()
    gpu = orc.merge_stored(o[:, 0], lse[:, 0], "bf16")[0][None].copy()
    gpu[0, 1] += 0.01                         # no partial near a boundary there
    try:
        assert_out_stored(gpu, o, lse, "bf16")
    except AssertionError:
        return
    raise AssertionError("an error of 0.01 passed the storage-aware check")


def test_empty_shard_has_no_weight():
    o, lse = _case()
    o[1] = np.nan                             # never read: lse = -inf
    lse[1] = -np.inf
    gpu = orc.merge_stored(np.nan_to_num(o[:1, 0]), lse[:1, 0], "bf16")[0][None]
    assert assert_out_stored(gpu, np.nan_to_num(o), lse, "bf16") <= 1.0
