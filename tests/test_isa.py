"""The build's assembly checks (tiled_attention_flash_amd.isa_check), on the
CPU: every kernel source is built to gfx950 assembly; each direct HBM -> LDS
load must take a scalar base that no vector instruction wrote fewer than 5
wait states before it, and no packed fp32 instruction may appear.  The
checks themselves are pinned on hand-written sequences, among them the one
that faulted the GPU.
"""
from __future__ import annotations

import os

import pytest

from tiled_attention_flash_amd import build as fa_build
from tiled_attention_flash_amd import isa_check


@pytest.fixture(scope="module")
def assembly(tmp_path_factory):
    if not os.path.exists(fa_build.hipcc()) and os.path.sep in fa_build.hipcc():
        pytest.skip("hipcc not available")
    return isa_check.assemble_all(str(tmp_path_factory.mktemp("isa")))


@pytest.mark.parametrize("src", isa_check.SOURCES)
def test_direct_loads_take_scalar_bases(assembly, src):
    assert isa_check.direct_loads(assembly[src]), f"{src}: no direct loads found"
    assert not isa_check.non_scalar_bases(assembly[src])


@pytest.mark.parametrize("src", isa_check.SOURCES)
def test_direct_load_bases_not_written_just_before_by_valu(assembly, src):
    assert not isa_check.vsgpr_hazards(assembly[src])


@pytest.mark.parametrize("src", isa_check.SOURCES)
def test_no_packed_fp32(assembly, src):
    assert not isa_check.packed_fp32(assembly[src])


def test_problems_is_empty(assembly):
    assert isa_check.problems(assembly) == []


# The sequence that faulted: a readfirstlane pair one wait state ahead of the load.
FAULTED = """v_readfirstlane_b32 s13, v69
v_readfirstlane_b32 s12, v68
s_nop 0
global_load_lds_dword v70, s[12:13]"""


@pytest.mark.parametrize("text,hazard", [
    (FAULTED, True),
    (FAULTED.replace("s_nop 0", "s_nop 4"), False),
    # a scalar spilled to a vector lane and restored just before the load
    ("v_readlane_b32 s7, v167, 44\ns_nop 0\nglobal_load_lds_dwordx4 v1, s[6:7]", True),
    # the write is to other registers
    ("v_readfirstlane_b32 s20, v1\ns_nop 0\nglobal_load_lds_dwordx4 v1, s[6:7]", False),
    # scalar writes are not a hazard
    ("s_add_u32 s6, s6, s2\ns_addc_u32 s7, s7, s3\nglobal_load_lds_dwordx4 v1, s[6:7]", False),
    # five other instructions in between are enough
    ("v_readfirstlane_b32 s6, v1\ns_mov_b32 m0, s2\ns_nop 3\nglobal_load_lds_dwordx4 v1, s[6:7]", False),
    # the scan runs through a label (the fall-through path)
    ("v_readfirstlane_b32 s6, v1\n.LBB0_3:\nglobal_load_lds_dwordx4 v1, s[6:7]", True),
])
def test_hazard_check_pins(text, hazard):
    assert bool(isa_check.vsgpr_hazards(text)) == hazard


def test_non_scalar_base_is_reported():
    assert isa_check.non_scalar_bases("global_load_lds_dword v134, v[132:133]")
    assert not isa_check.non_scalar_bases("global_load_lds_dword v134, s[12:13]")
