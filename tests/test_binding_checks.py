"""The Python binding rejects bad tensors before anything reaches the
library (CPU only: no kernel could run here anyway).

A host tensor handed to a kernel would be a host pointer on the GPU (a
fault), an fp16 lse_out would be written 4 bytes per row past its end, and
K/V of another dtype than q would be read as q's dtype; each must raise in
the binding.  The library itself is replaced by a stub that fails the test
if any of its functions is reached."""
import pytest

torch = pytest.importorskip("torch")
import lse_merge_split_amd as cp  # noqa: E402

R, B, Hq, Hkv, D, CAP = 2, 1, 4, 2, 64, 96


@pytest.fixture(autouse=True)
def no_library(monkeypatch):
    def reached():
        raise AssertionError("the library was reached before the arguments were rejected")
    monkeypatch.setattr(cp, "lib", reached)


def _attn_args(**over):
    a = dict(q=torch.zeros(B, Hq, D, dtype=torch.bfloat16),
             k_shards=[torch.zeros(B, Hkv, CAP, D, dtype=torch.bfloat16) for _ in range(R)],
             v_shards=[torch.zeros(B, Hkv, CAP, D, dtype=torch.bfloat16) for _ in range(R)],
             lens=torch.zeros(R, B, dtype=torch.int32),
             o_part=torch.zeros(R, B, Hq, D, dtype=torch.float32),
             lse_part=torch.zeros(R, B, Hq, dtype=torch.float32))
    a.update(over)
    return a


def _step_args(**over):
    a = _attn_args()
    a.update(out=torch.zeros(B, Hq, D, dtype=torch.bfloat16),
             lse_out=torch.zeros(B, Hq, dtype=torch.float32))
    a.update(over)
    return a


def test_host_tensors_are_rejected():
    with pytest.raises(ValueError, match="GPU tensor"):
        cp.AttnCall(**_attn_args())
    with pytest.raises(ValueError, match="GPU tensor"):
        cp.StepCall(**_step_args())
    with pytest.raises(ValueError, match="GPU tensor"):
        cp.attn_partial(**_attn_args())
    with pytest.raises(ValueError, match="GPU tensor"):
        cp.cp_decode(**_step_args())
    with pytest.raises(ValueError, match="GPU tensor"):
        cp.MergeCall(torch.zeros(R, 3, D), torch.zeros(R, 3), torch.zeros(3, D, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="GPU tensor"):
        cp.workspace_clear(torch.zeros(256, dtype=torch.uint8))


@pytest.mark.parametrize("what,over", [
    ("lse_part fp16", dict(lse_part=torch.zeros(R, B, Hq, dtype=torch.float16))),
    ("lse_part fp64", dict(lse_part=torch.zeros(R, B, Hq, dtype=torch.float64))),
    ("lens int64", dict(lens=torch.zeros(R, B, dtype=torch.int64))),
    ("K fp16 with bf16 q", dict(k_shards=[torch.zeros(B, Hkv, CAP, D, dtype=torch.float16)] * R,
                                v_shards=[torch.zeros(B, Hkv, CAP, D, dtype=torch.float16)] * R)),
    ("one V shard fp16", dict(v_shards=[torch.zeros(B, Hkv, CAP, D, dtype=torch.bfloat16),
                                        torch.zeros(B, Hkv, CAP, D, dtype=torch.float16)])),
    ("q fp32", dict(q=torch.zeros(B, Hq, D, dtype=torch.float32))),
    ("o_part fp64", dict(o_part=torch.zeros(R, B, Hq, D, dtype=torch.float64))),
])
def test_attention_dtypes_are_checked(what, over):
    with pytest.raises((TypeError, ValueError)) as e:
        cp.AttnCall(**_attn_args(**over))
    assert "GPU tensor" not in str(e.value), f"{what}: dtype not checked before the device"


@pytest.mark.parametrize("what,over", [
    ("lse_out fp16", dict(lse_out=torch.zeros(B, Hq, dtype=torch.float16))),
    ("lse_out fp64", dict(lse_out=torch.zeros(B, Hq, dtype=torch.float64))),
    ("out of another dtype", dict(out=torch.zeros(B, Hq, D, dtype=torch.float16))),
])
def test_step_dtypes_are_checked(what, over):
    with pytest.raises((TypeError, ValueError)) as e:
        cp.StepCall(**_step_args(**over))
    assert "GPU tensor" not in str(e.value), what


@pytest.mark.parametrize("what,args", [
    ("lse_part fp16", (torch.zeros(R, 3, D), torch.zeros(R, 3, dtype=torch.float16),
                       torch.zeros(3, D), torch.zeros(3))),
    ("lse_out fp16", (torch.zeros(R, 3, D), torch.zeros(R, 3), torch.zeros(3, D),
                      torch.zeros(3, dtype=torch.float16))),
    ("o_part int32", (torch.zeros(R, 3, D, dtype=torch.int32), torch.zeros(R, 3),
                      torch.zeros(3, D), None)),
    ("out fp64", (torch.zeros(R, 3, D), torch.zeros(R, 3), torch.zeros(3, D, dtype=torch.float64),
                  None)),
])
def test_merge_dtypes_are_checked(what, args):
    with pytest.raises((TypeError, ValueError)) as e:
        cp.MergeCall(*args)
    assert "GPU tensor" not in str(e.value), what


def test_mixed_devices_are_rejected():
    """Stand-ins for GPU tensors on two devices (no GPU here): the device
    check compares every tensor with the first; a host tensor fails it."""
    a = _step_args()
    with pytest.raises(ValueError):
        cp._check_tensors({"q": a["q"], "out": a["out"]})
    class FakeCuda:
        def __init__(self, dev):
            self.is_cuda, self.device = True, dev
    with pytest.raises(ValueError, match="other tensors on"):
        cp._check_tensors({"q": FakeCuda(torch.device("cuda", 0)),
                           "out": FakeCuda(torch.device("cuda", 1))})
    assert cp._check_tensors({"q": FakeCuda(torch.device("cuda", 0)), "lse_out": None,
                              "out": FakeCuda(torch.device("cuda", 0))}) == torch.device("cuda", 0)
