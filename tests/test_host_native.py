"""Host-compiled checks of the library's integer and host logic (no GPU).

tests/native/host_checks.cpp is compiled with the host C++ compiler against the same
headers and the same validation source the library is built from, and run:
  - the address arithmetic of the direct global->LDS loads (csrc/k_addr.h, which the
    kernels call) over every tile shape and stage length the kernels use: each load
    inside its stage's rows, each LDS granule written once with the row and swizzled
    granule the fragment reads expect, 32-bit offsets that cannot wrap;
  - the classification of pointer lookups (plain host memory refused, pinned host,
    device, managed memory accepted);
  - the accumulation window's checks of gradient tags (other model version, other prompt
    group, unsealed or edited tags, poisoned window)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "resident_kv_response_amd", "csrc")


def _compiler():
    for c in ("g++", "c++", "clang++"):
        if shutil.which(c):
            return c
    return None


def test_host_checks(tmp_path):
    cxx = _compiler()
    if cxx is None:
        pytest.skip("no host C++ compiler")
    exe = str(tmp_path / "host_checks")
    cmd = [cxx, "-std=c++17", "-O1", "-Wall", "-I", CSRC, "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "native", "host_checks.cpp"), os.path.join(CSRC, "rr_validate.cpp"),
           "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"compile failed:\n{r.stderr}"
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all host checks passed" in r.stdout
