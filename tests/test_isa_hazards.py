"""The tile loads are inline assembly, so their register hazards are checked here
on the compiled gfx950 code (no GPU needed): every LDS DMA load must be at least
5 wait states after any VALU write of the SGPRs it reads (its base address)."""

import shutil

import pytest

from isa_scan import device_asm, find_hazards

pytestmark = pytest.mark.skipif(shutil.which("hipcc") is None and not __import__("os").path.exists("/opt/rocm/bin/hipcc"),
                                reason="hipcc not available")


def test_scanner_flags_a_short_gap():
    asm = """
    v_readfirstlane_b32 s7, v11
    v_readfirstlane_b32 s6, v10
    s_nop 0
    global_load_lds_dwordx4 v71, s[6:7]
    """
    assert len(find_hazards(asm)) == 1


def test_scanner_accepts_padding():
    asm = """
    v_readfirstlane_b32 s7, v11
    v_readfirstlane_b32 s6, v10
    s_mov_b32 m0, s17
    s_nop 4
    global_load_lds_dwordx4 v71, s[6:7]
    """
    assert find_hazards(asm) == []


def test_scanner_flags_carry_out_writes():
    asm = """
    v_add_co_u32 v2, s[6:7], v3, v4
    s_nop 2
    global_load_lds_dwordx4 v71, s[6:7]
    """
    assert len(find_hazards(asm)) == 1


@pytest.mark.parametrize("debug", [False, True], ids=["release", "debug"])
@pytest.mark.parametrize("source", ["hstu_fwd.hip", "hstu_bwd.hip"])
def test_kernels_have_no_dma_sgpr_hazard(source, debug):
    """Both builds: the debug build's bounds tests change the code around the loads."""
    asm = device_asm(source, ["-DHSTU_DEBUG"] if debug else [])
    assert "global_load_lds_dwordx4" in asm
    bad = find_hazards(asm)
    assert not bad, "\n".join(t for _, t in bad[:10])
    if debug:
        assert "global_atomic_or" in asm  # the tests record failures with vector atomics
