"""Checks on the gfx950 assembly of every kernel source, built on the CPU.

The kernels issue their direct HBM -> LDS loads (``global_load_lds_*``) from
inline assembly whose address base operand must be a pair of scalar
registers.  If the compiler ever holds the computed base in vector registers
it still fills the operand with them, and the encoded instruction would read
from an unrelated address; so every such load in the built code is checked
to name scalar registers.  A vector instruction that writes a scalar
register must also come at least 5 wait states before a memory instruction
that reads it; the compiler does not count a load inside inline assembly,
so every direct load is checked for a vector write of its base registers
among the instructions just before it.  The sources are also built with the
packed fp32 forms switched off, and none may appear.
"""
from __future__ import annotations

import concurrent.futures
import os
import re
import shutil
import subprocess

import pytest

from tiled_attention_flash_amd import build as fa_build

SOURCES = ["fa_fwd_kernel.hip", "fa_fwd_fp8_kernel.hip", "fa_splitkv_kernel.hip", "fa_bwd_kernel.hip"]

DMA = re.compile(r"^\s*(global_load_lds_\w+)\s+(\S+),\s*(\S+)")
PACKED_F32 = re.compile(r"^\s*v_pk_(fma|mul|add|mov)_f32\b")


def _asm(tmp, src):
    out = os.path.join(tmp, src + ".s")
    cmd = [fa_build.hipcc(), *fa_build.HIP_FLAGS, f"-I{fa_build.INCLUDE}", f"-I{fa_build.CSRC}",
           "--cuda-device-only", "-S", "-o", out, os.path.join(fa_build.CSRC, src)]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout
    return src, open(out).read()


@pytest.fixture(scope="module")
def assembly(tmp_path_factory):
    if shutil.which(fa_build.hipcc()) is None and not os.path.exists(fa_build.hipcc()):
        pytest.skip("hipcc not available")
    tmp = str(tmp_path_factory.mktemp("isa"))
    with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
        return dict(ex.map(lambda s: _asm(tmp, s), SOURCES))


@pytest.mark.parametrize("src", SOURCES)
def test_direct_loads_take_scalar_bases(assembly, src):
    loads = [m for m in (DMA.match(line) for line in assembly[src].splitlines()) if m]
    assert loads, f"{src}: no direct loads found"
    bad = [m.group(0).strip() for m in loads if not m.group(3).startswith("s[")]
    assert not bad, f"{src}: direct loads with a non-scalar base: {bad[:4]}"


SREG = re.compile(r"^s(\d+)$|^s\[(\d+):(\d+)\]$")


def _sregs(op):
    m = SREG.match(op.strip().rstrip(","))
    if not m:
        return set()
    if m.group(1) is not None:
        return {int(m.group(1))}
    return set(range(int(m.group(2)), int(m.group(3)) + 1))


def _instructions(text):
    """Instruction lines of the assembly, with labels kept as markers."""
    out = []
    for line in text.splitlines():
        t = line.split(";")[0].strip()
        if not t or t.startswith(".") or t.startswith("_Z"):
            continue
        out.append(t)
    return out


def vsgpr_hazards(text, need=5):
    """Direct loads whose base registers a vector instruction wrote fewer
    than `need` wait states earlier (s_nop n counts n + 1, any other
    instruction 1); the scan stops at a label."""
    ins = _instructions(text)
    bad = []
    for i, t in enumerate(ins):
        m = DMA.match(t)
        if not m:
            continue
        base = _sregs(m.group(3))
        waits = 0
        for j in range(i - 1, -1, -1):
            prev = ins[j]
            if prev.endswith(":"):
                break
            op = prev.split()[0]
            if op.startswith("v_"):
                dst = prev.split(None, 1)[1].split(",")[0] if " " in prev else ""
                if _sregs(dst) & base:
                    bad.append(f"{prev} ... {t} ({waits} wait states)")
                    break
            if op == "s_nop":
                waits += int(prev.split()[1], 0) + 1
            else:
                waits += 1
            if waits >= need:
                break
    return bad


@pytest.mark.parametrize("src", SOURCES)
def test_direct_load_bases_not_written_just_before_by_valu(assembly, src):
    bad = vsgpr_hazards(assembly[src])
    assert not bad, f"{src}: {bad[:4]}"


def test_hazard_check_sees_a_short_gap():
    """The check is not vacuous: a readfirstlane one wait state ahead of the
    load that reads its result is reported, five are not."""
    bad = "v_readfirstlane_b32 s13, v69\nv_readfirstlane_b32 s12, v68\ns_nop 0\nglobal_load_lds_dword v70, s[12:13]"
    ok = "v_readfirstlane_b32 s13, v69\nv_readfirstlane_b32 s12, v68\ns_nop 4\nglobal_load_lds_dword v70, s[12:13]"
    assert vsgpr_hazards(bad) and not vsgpr_hazards(ok)


@pytest.mark.parametrize("src", SOURCES)
def test_no_packed_fp32(assembly, src):
    bad = [line.strip() for line in assembly[src].splitlines() if PACKED_F32.match(line)]
    assert not bad, f"{src}: {bad[:4]}"
