"""Checks on the gfx950 assembly of the kernel sources (run by the build).

The kernels issue their direct HBM -> LDS loads (``global_load_lds_*``) from
inline assembly whose address base operand is a pair of scalar registers.
Two things about those loads depend on the compiler's register allocation
rather than on the source, and both have made a build fault the GPU:

* the base must be held in scalar registers -- if the compiler keeps the
  computed address in vector registers it still fills the operand with them,
  and the encoded instruction reads from an unrelated address;
* a vector instruction that writes a scalar register (``v_readfirstlane``,
  ``v_readlane`` restoring a spilled scalar, a compare with a scalar
  destination) must come at least 5 wait states before a memory instruction
  that reads that register.  The compiler inserts the wait states for its own
  memory instructions but does not count a load inside inline assembly.

Every kernel source is built to assembly with the library's flags and each
direct load is checked for both; the packed fp32 forms, switched off by the
build flags, must not appear either.
"""
from __future__ import annotations

import concurrent.futures
import os
import re
import subprocess

from . import build as fa_build

SOURCES = ["fa_fwd_kernel.hip", "fa_fwd_fp8_kernel.hip", "fa_splitkv_kernel.hip", "fa_bwd_kernel.hip",
           "fa_bwd_kernel_d64.hip"]

DMA = re.compile(r"^\s*(global_load_lds_\w+)\s+(\S+),\s*(\S+)")
PACKED_F32 = re.compile(r"^\s*v_pk_(fma|mul|add|mov)_f32\b")
SREG = re.compile(r"^s(\d+)$|^s\[(\d+):(\d+)\]$")
VALU_SGPR_TO_VMEM_WAITS = 5


def assemble(src: str, outdir: str) -> str:
    """gfx950 assembly of one kernel source, built with the library's flags for it."""
    out = os.path.join(outdir, src + ".s")
    cmd = [fa_build.hipcc(), *fa_build.HIP_FLAGS, *fa_build.SOURCE_FLAGS.get(src, []), f"-I{fa_build.INCLUDE}",
           f"-I{fa_build.CSRC}", "--cuda-device-only", "-S", "-o", out, os.path.join(fa_build.CSRC, src)]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"assembling {src} failed:\n{r.stdout}")
    with open(out) as f:
        return f.read()


def assemble_all(outdir: str) -> dict:
    with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
        return dict(zip(SOURCES, ex.map(lambda s: assemble(s, outdir), SOURCES)))


def _sregs(op: str) -> set:
    m = SREG.match(op.strip().rstrip(","))
    if not m:
        return set()
    if m.group(1) is not None:
        return {int(m.group(1))}
    return set(range(int(m.group(2)), int(m.group(3)) + 1))


def _instructions(text: str) -> list:
    """Instruction lines of the assembly, without labels and directives."""
    out = []
    for line in text.splitlines():
        t = line.split(";")[0].strip()
        if not t or t.startswith(".") or t.startswith("_Z") or t.endswith(":"):
            continue
        out.append(t)
    return out


def direct_loads(text: str) -> list:
    return [m for m in (DMA.match(line) for line in text.splitlines()) if m]


def non_scalar_bases(text: str) -> list:
    return [m.group(0).strip() for m in direct_loads(text) if not m.group(3).startswith("s[")]


def vsgpr_hazards(text: str, need: int = VALU_SGPR_TO_VMEM_WAITS) -> list:
    """Direct loads whose base registers a vector instruction wrote fewer
    than `need` wait states earlier (s_nop n counts n + 1 wait states, any
    other instruction 1).  The backward scan runs through labels along the
    fall-through path, which is the conservative reading."""
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
            op = prev.split()[0]
            if op.startswith("v_") and " " in prev:
                dst = prev.split(None, 1)[1].split(",")[0]
                if _sregs(dst) & base:
                    bad.append(f"{prev} ... {t} ({waits} wait states)")
                    break
            waits += int(prev.split()[1], 0) + 1 if op == "s_nop" else 1
            if waits >= need:
                break
    return bad


def packed_fp32(text: str) -> list:
    return [line.strip() for line in text.splitlines() if PACKED_F32.match(line)]


def problems(asm: dict) -> list:
    """Every violation in the assembly of the kernel sources, as text."""
    out = []
    for src, text in asm.items():
        if not direct_loads(text):
            out.append(f"{src}: no direct loads found (the check would be vacuous)")
        out += [f"{src}: direct load with a non-scalar base: {x}" for x in non_scalar_bases(text)]
        out += [f"{src}: base written by a vector instruction too close: {x}" for x in vsgpr_hazards(text)]
        out += [f"{src}: packed fp32 instruction: {x}" for x in packed_fp32(text)]
    return out
