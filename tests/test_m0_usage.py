"""Kernels that issue their global->LDS loads from inline assembly set M0 themselves.

The compiler treats M0 as a reserved register and does not model the asm statements'
clobber of it (hipcc warns "inline asm clobber list contains reserved registers: m0").
That is safe only while the compiler itself neither writes nor reads M0 in those kernels.
This test compiles the sources that hold such loads to gfx950 assembly and checks every
kernel: a kernel with asm LDS loads has no compiler-generated LDS-direct load, no compiler
write of M0 and no instruction that reads M0 implicitly (indexed register moves, messages,
interpolation, addtid LDS forms, GWS).  CPU only: hipcc cross-compiles without a GPU.
"""
from __future__ import annotations

import os
import re
import shutil
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

from resident_kv_response_amd import build

SOURCES = ["k_fwd_bf16.hip", "k_dq_bf16.hip", "k_kv_grads.hip", "k_sparse.hip"]
M0_READERS = re.compile(r"^(v_movrel|s_movrel|s_sendmsg|v_interp|ds_\w*addtid|ds_gws|s_ttracedata)")


def _hipcc():
    try:
        return build.hipcc()
    except RuntimeError:
        return None


def _asm(src: str, out_dir: str) -> str:
    out = os.path.join(out_dir, src + ".s")
    cmd = [build.hipcc()] + build.flags() + build.SOURCE_FLAGS.get(src, []) + [
        "--cuda-device-only", "-S", os.path.join(build.CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"{src}: {r.stderr[-2000:]}"
    return open(out).read()


def _kernels(text: str):
    """(name, body lines) of every kernel in a gfx950 assembly listing: from the kernel's
    label to its .Lfunc_end label (a kernel with early exits has several s_endpgm)."""
    name, body = None, []
    for line in text.split("\n"):
        m = re.match(r"^(_Z\w+):", line)
        if m:
            name, body = m.group(1), []
            continue
        if name is None:
            continue
        if re.match(r"^\.Lfunc_end\d+:", line):
            yield name, body
            name = None
        else:
            body.append(line.strip())


def _check_kernel(name: str, body):
    in_asm = False
    own = comp = m0_writes = 0
    readers = []
    for s in body:
        if s.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if s.startswith(";;#ASMEND"):
            in_asm = False
            continue
        if not s or s.startswith(";") or s.startswith("."):
            continue
        if s.startswith("global_load_lds"):
            if in_asm:
                own += 1
            else:
                comp += 1
        if not in_asm:
            if re.match(r"^s_mov_b(32|64)\s+m0\b", s):
                m0_writes += 1
            elif M0_READERS.match(s) or re.search(r"\bm0\b", s):
                readers.append(s)
    problems = []
    if own:
        if comp:
            problems.append(f"{comp} compiler LDS-direct loads beside {own} asm ones")
        if m0_writes:
            problems.append(f"{m0_writes} compiler writes of m0")
        if readers:
            problems.append(f"instructions reading m0: {readers[:3]}")
    return own, problems


@pytest.mark.skipif(_hipcc() is None, reason="hipcc not found")
def test_asm_lds_loads_own_m0():
    tmp = tempfile.mkdtemp(prefix="rr_m0_")
    try:
        with ThreadPoolExecutor(len(SOURCES)) as ex:
            texts = list(ex.map(lambda s: _asm(s, tmp), SOURCES))
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    with_asm = 0
    bad = []
    for src, text in zip(SOURCES, texts):
        for name, body in _kernels(text):
            own, problems = _check_kernel(name, body)
            with_asm += own > 0
            bad += [f"{src} {name}: {p}" for p in problems]
    assert with_asm >= 9, f"only {with_asm} kernels with asm LDS loads found (listing format changed?)"
    assert not bad, "\n".join(bad)


def test_checker_flags_a_mixed_kernel():
    """The checker itself: a listing that mixes the two kinds of load, writes m0 outside
    the asm and moves registers by index is rejected on all three counts."""
    body = [";;#ASMSTART", "s_mov_b32 m0, s4", "s_nop 0", "global_load_lds_dwordx4 v1, s[2:3]", ";;#ASMEND",
            "s_mov_b32 m0, s5", "global_load_lds_dwordx4 v[2:3], off", "v_movrels_b32_e32 v0, v1"]
    own, problems = _check_kernel("k", body)
    assert own == 1 and len(problems) == 3, problems
    own, problems = _check_kernel("k", body[:5])
    assert own == 1 and not problems
