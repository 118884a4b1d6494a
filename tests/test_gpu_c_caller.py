"""A plain C program drives the whole path on the GPU (tests/c_abi/step_c.c):
the C ABI with device buffers from the HIP runtime's C API, no Python
binding and no torch on the GPU side.

The test writes seeded inputs (K/V padding past each length filled with
NaN), the program runs cpdec_cp_decode twice on one workspace, the two
calls cpdec_attn_partial + cpdec_lse_merge and the allocation-free
cpdec_cp_decode_noalloc, and every output is checked against the oracle; the
repeat call and the allocation-free step must reproduce the first call bit
for bit.
"""
import os
import shutil
import subprocess
import sys

import numpy as np
import pytest

from oracle import oracle as orc
from tests.helpers import assert_lse, assert_out

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
import lse_merge_split_amd as cp  # noqa: E402

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

# (R, B, Hq, Hkv, D, capacity, dtype, chunk_tokens, lens rule)
CASES = {
    "split MHA, 16 chunks, one launch": (4, 1, 4, 4, 128, 1000, "bf16", 0, "full"),
    "GQA 4, ragged with an empty shard, fp16, one launch": (3, 3, 8, 2, 64, 300, "fp16", 0, "ragged"),
    "79 chunks of 32: attention, chunk combine, merge": (2, 1, 8, 2, 128, 2500, "bf16", 32, "ragged"),
    "GQA 8 at D=256: attention + row merge": (2, 2, 16, 2, 256, 200, "bf16", 0, "ragged"),
    "whole shards, 512 units, fp16": (2, 64, 8, 4, 64, 100, "fp16", 0, "ragged"),
}
NAN_BITS = {"bf16": 0x7FC0, "fp16": 0x7E00}
TORCH_DT = {"bf16": torch.bfloat16, "fp16": torch.float16}
CPDEC_DT = {"bf16": cp.BF16, "fp16": cp.F16}


@pytest.fixture(scope="module")
def step_c(tmp_path_factory):
    if shutil.which("gcc") is None:
        pytest.fail("gcc is needed to build the C caller")
    lib = cp.LIB_PATH
    assert os.path.exists(lib), f"{lib} is missing: build it first"
    exe = tmp_path_factory.mktemp("c_caller") / "step_c"
    cmd = ["gcc", "-std=c99", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
           os.path.join(ROOT, "tests", "c_abi", "step_c.c"), "-o", str(exe), lib,
           f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{os.path.dirname(lib)}:{ROCM}/lib"]
    subprocess.run(cmd, check=True)
    return exe


def _bits(x, dt):
    """float tensor -> (16-bit storage words, exact float64 values)."""
    t = x.to(TORCH_DT[dt])
    return t.view(torch.int16).numpy().view(np.uint16), t.to(torch.float64).numpy()


def _unpack(buf, R, B, Hq, D, dt, at):
    n_op, n_lp, n_o, n_l = R * B * Hq * D, R * B * Hq, B * Hq * D, B * Hq
    o_part = np.frombuffer(buf, np.float32, n_op, at).reshape(R, B, Hq, D); at += 4 * n_op
    lse_part = np.frombuffer(buf, np.float32, n_lp, at).reshape(R, B, Hq); at += 4 * n_lp
    words = np.frombuffer(buf, np.uint16, n_o, at).copy(); at += 2 * n_o
    out = torch.from_numpy(words.view(np.int16)).view(TORCH_DT[dt]).to(torch.float64).numpy()
    lse_out = np.frombuffer(buf, np.float32, n_l, at).reshape(B, Hq); at += 4 * n_l
    return dict(o_part=o_part, lse_part=lse_part, out=out.reshape(B, Hq, D), lse_out=lse_out), at


@pytest.mark.parametrize("name", list(CASES))
def test_c_caller(name, step_c, tmp_path):
    R, B, Hq, Hkv, D, cap, dt, chunk, rule = CASES[name]
    seed = 7000 + list(CASES).index(name)
    g = torch.Generator().manual_seed(seed)
    rng = np.random.default_rng(seed)
    if rule == "full":
        lens = np.full((R, B), cap, np.int32)
    else:
        lens = rng.integers(0, cap + 1, size=(R, B)).astype(np.int32)
        lens[0, 0] = 0           # an empty shard
        lens[-1, -1] = cap       # and a full one
    q_bits, q64 = _bits(torch.randn(B, Hq, D, generator=g), dt)
    k_bits, k64 = _bits(torch.randn(R, B, Hkv, cap, D, generator=g), dt)
    v_bits, v64 = _bits(torch.randn(R, B, Hkv, cap, D, generator=g), dt)
    for r in range(R):           # padding past each length holds NaN (never read)
        for b in range(B):
            k_bits[r, b, :, lens[r, b]:] = NAN_BITS[dt]
            v_bits[r, b, :, lens[r, b]:] = NAN_BITS[dt]
    inp = tmp_path / "inputs.bin"
    hdr = np.array([R, B, Hq, Hkv, D, cap, CPDEC_DT[dt], chunk], np.int32)
    with open(inp, "wb") as f:
        for a in (hdr, q_bits, k_bits, v_bits, lens):
            f.write(np.ascontiguousarray(a).tobytes())
    outp = tmp_path / "outputs.bin"
    print(f"[case] C caller: {name}", flush=True)
    sys.stdout.flush()
    r = subprocess.run([str(step_c), str(inp), str(outp)], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0, r.stderr
    print(r.stdout.strip(), flush=True)

    buf = outp.read_bytes()
    step1, at = _unpack(buf, R, B, Hq, D, dt, 0)
    step2, at = _unpack(buf, R, B, Hq, D, dt, at)
    two, at = _unpack(buf, R, B, Hq, D, dt, at)
    na, at = _unpack(buf, R, B, Hq, D, dt, at)
    assert at == len(buf)

    o_ref, lp_ref, out_ref, lo_ref = orc.cp_decode(q64, list(k64), list(v64), lens, Hkv)
    for what, res in (("step", step1), ("two calls", two)):
        assert_out(res["out"], out_ref, f"{what} out")
        assert_lse(res["lse_out"], lo_ref, f"{what} lse_out", floor=True)
        assert_out(res["o_part"], o_ref, f"{what} o_part")
        assert_lse(res["lse_part"], lp_ref, f"{what} lse_part", floor=True)
    for k in step1:
        assert np.array_equal(step1[k], step2[k], equal_nan=False), f"repeat call: {k} differs"
        assert np.array_equal(step1[k], na[k], equal_nan=False), f"allocation-free step: {k} differs"
