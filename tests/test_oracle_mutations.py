"""Plant plausible mistakes in copies of the oracle and check that the pins
catch every one (CPU only).

Each mutant is the oracle's own source with one textual change, executed in
a fresh namespace; the test fails if a planted mistake passes all pins, or if
the text to mutate is no longer in the oracle (so the list stays current).
"""
import inspect
import types

import pytest

from oracle import oracle
from tests import pins

MUTATIONS = [
    ("scale dropped", "s = scale * (k @ q.T)", "s = (k @ q.T)"),
    ("max shift sign", "p = np.exp(s - m)", "p = np.exp(s + m)"),
    ("no normalisation by l", "o = (p.T @ v) / l[:, None]", "o = (p.T @ v)"),
    ("k used as values", "o = (p.T @ v) / l[:, None]", "o = (p.T @ k) / l[:, None]"),
    ("lse drops max", "lse = m + np.log(l)", "lse = np.log(l)"),
    ("lse drops log", "lse = m + np.log(l)", "lse = m + l"),
    ("lse base 2", "lse = m + np.log(l)", "lse = m + np.log2(l)"),
    ("empty shard lse 0", "return np.zeros((G, D)), np.full(G, NEG_INF)",
     "return np.zeros((G, D)), np.zeros(G)"),
    ("off-by-one length", "L = int(lens[r][b])\n            for h",
     "L = max(int(lens[r][b]) - 1, 0)\n            for h"),
    ("GQA interleaved", "heads = slice(h * G, (h + 1) * G)   # query heads",
     "heads = slice(h, Hq, Hkv)   # query heads"),
    ("merge reads -inf shards", "live = lse_parts > NEG_INF", "live = lse_parts >= NEG_INF"),
    ("merge weight sign", "w = np.exp(lse_live - M)", "w = np.exp(M - lse_live)"),
    ("merge no denominator", "out = (w[:, None] * o_live).sum(axis=0) / denom",
     "out = (w[:, None] * o_live).sum(axis=0)"),
    ("merge unweighted", "out = (w[:, None] * o_live).sum(axis=0) / denom",
     "out = o_live.sum(axis=0) / denom"),
    ("merged lse without log", "lse_out = M + math.log(denom)", "lse_out = M + denom"),
    ("merged lse is max", "lse_out = M + math.log(denom)", "lse_out = M"),
    ("merged lse drops max", "lse_out = M + math.log(denom)", "lse_out = math.log(denom)"),
    ("all-empty lse 0", "return np.zeros(D), NEG_INF", "return np.zeros(D), 0.0"),
    ("default scale 1/D", "scale = 1.0 / math.sqrt(D)\n    o_part",
     "scale = 1.0 / D\n    o_part"),
    ("bf16 rounding truncates", "(u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1)))",
     "(u)"),
    ("bf16 rounding without ties-to-even", "(u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1)))",
     "(u + np.uint64(0x8000))"),
]


def _mutant(old, new):
    src = inspect.getsource(oracle)
    assert src.count(old) >= 1, f"mutation target not found: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new, 1), "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.filterwarnings("ignore::RuntimeWarning")
@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_mutation(name, old, new):
    mod = _mutant(old, new)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(mod)
        except Exception:  # AssertionError, or a crash the mistake causes
            caught.append(pin.__name__)
    assert caught, f"planted mistake '{name}' passed every pin"
