"""The oracle against the pins in tests/pins.py (CPU only)."""
import pytest

from oracle import oracle
from tests import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(oracle)


def test_merge_rows_matches_merge():
    import numpy as np
    rng = np.random.default_rng(0)
    o = rng.normal(size=(3, 5, 4))
    lse = rng.normal(size=(3, 5))
    lse[1, 2] = -np.inf
    out, l = oracle.merge_rows(o, lse)
    for n in range(5):
        a, b = oracle.merge(o[:, n], lse[:, n])
        assert np.array_equal(out[n], a) and l[n] == b
