"""Build libcpdec.so (the HIP kernels and the C ABI) in-tree for gfx950."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
ARCH = "gfx950"
SOURCES = ["attn_partial.hip", "lse_merge.hip", "cpdec_api.hip"]
LIB = os.path.join(HERE, "libcpdec.so")

# Packed FP32 VALU forms are kept out of the generated code (device-side
# target feature; the host pass only warns that it does not know it).
HIP_FLAGS = ["-O3", f"--offload-arch={ARCH}", "-std=c++17", "-fPIC", "-shared",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build(verbose: bool = False) -> str:
    """Compile every source into libcpdec.so (always recompiles)."""
    hipcc = os.path.join(ROCM, "bin", "hipcc")
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [hipcc, *HIP_FLAGS, "-I", os.path.join(ROOT, "include"),
           *[os.path.join(HERE, "csrc", s) for s in SOURCES], "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + res.stderr[-8000:])
    if verbose:
        print(" ".join(cmd))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
