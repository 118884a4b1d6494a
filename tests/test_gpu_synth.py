"""The GPU twin of the input streams reproduces the CPU streams bit for bit."""
import numpy as np
import pytest

from synth import philox

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
from synth import gpu as sg  # noqa: E402


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("start", [0, 5, (1 << 34) + 3])
def test_gpu_stream_matches_cpu(dtype, start):
    print(f"[case] synth {dtype} start={start}", flush=True)
    n = 100003
    scale = 3.0 if dtype == "bf16" else 1.0
    t = torch.empty(n, dtype=sg.torch_dtype(dtype), device="cuda")
    sg.fill_normal(t, 1234, 9, start=start, scale=scale)
    z = philox.normal_f32(1234, 9, start, n)
    if scale != 1.0:
        z = (z * np.float32(scale)).astype(np.float32)
    bits, vals = philox.round_to(z, dtype)
    got = t.cpu()
    if dtype == "bf16":
        assert np.array_equal(got.view(torch.int16).numpy().view(np.uint16), bits)
    else:
        assert np.array_equal(got.numpy(), bits)
