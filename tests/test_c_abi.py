"""The header is plain C: a C program compiles against include/cpdec.h, links
libcpdec.so and exercises the argument checks (CPU host, no GPU calls)."""
import os
import shutil
import subprocess

import pytest

import lse_merge_split_amd as cp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_plain_c_program(tmp_path):
    lib = cp.LIB_PATH
    if not os.path.exists(lib):
        pytest.skip("libcpdec.so not built")
    exe = tmp_path / "abi_smoke"
    src = os.path.join(ROOT, "tests", "c_abi", "abi_smoke.c")
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"), src,
                    "-o", str(exe), lib, f"-Wl,-rpath,{os.path.dirname(lib)}"], check=True)
    env = dict(os.environ, HIP_VISIBLE_DEVICES="", ROCR_VISIBLE_DEVICES="")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stderr
    assert "abi_smoke ok" in r.stdout
