"""Build libcpdec.so (the HIP kernels and the C ABI) in-tree for gfx950."""
from __future__ import annotations

import os
import subprocess
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
ARCH = "gfx950"
# (source, extra flags, object): the attention kernels are compiled once per
# element type, so the heaviest file builds as two objects in parallel.
UNITS = [("attn_partial.hip", ["-DCPDEC_ATTN_TYPE=2"], "attn_bf16.o"),
         ("attn_partial.hip", ["-DCPDEC_ATTN_TYPE=1"], "attn_f16.o"),
         ("lse_merge.hip", [], "lse_merge.o"),
         ("cpdec_api.hip", [], "cpdec_api.o")]
SOURCES = sorted({u[0] for u in UNITS})
LIB = os.path.join(HERE, "libcpdec.so")

# Packed FP32 VALU forms are kept out of the generated code (device-side
# target feature; the host pass only warns that it does not know it).
HIP_FLAGS = ["-O3", f"--offload-arch={ARCH}", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build(verbose: bool = False) -> str:
    """Compile every source into libcpdec.so (always recompiles): the objects
    in parallel, then one shared-library link."""
    hipcc = os.path.join(ROCM, "bin", "hipcc")
    with tempfile.TemporaryDirectory(prefix="cpdec_build_") as tmpdir:
        procs, objs = [], []
        for src, extra, obj in UNITS:
            out = os.path.join(tmpdir, obj)
            cmd = [hipcc, *HIP_FLAGS, *extra, "-I", os.path.join(ROOT, "include"), "-c",
                   os.path.join(HERE, "csrc", src), "-o", out]
            procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                                stderr=subprocess.PIPE, text=True)))
            objs.append(out)
        errors = []
        for cmd, pr in procs:
            _, err = pr.communicate()
            if pr.returncode != 0:
                errors.append(" ".join(cmd) + "\n" + err[-8000:])
            elif verbose:
                print(" ".join(cmd))
        if errors:
            raise RuntimeError("hipcc failed:\n" + "\n".join(errors))
        tmp = LIB + f".tmp{os.getpid()}"
        cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError("link failed:\n" + " ".join(cmd) + "\n" + res.stderr[-8000:])
        if verbose:
            print(" ".join(cmd))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
