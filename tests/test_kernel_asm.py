"""CPU checks of the main kernel's gfx950 assembly (hipcc cross-compiles it
here with the library's own flags): hazards around the inline-assembly
MFMAs, no copies of registers that staged loads are filling, and no
register-file moves inside the KV tile loop."""
import os
import shutil
import subprocess

import pytest

from mla_token_decode_amd import build as hipbuild
from tests import asm_scan

HIPCC = hipbuild.HIPCC


@pytest.fixture(scope="module")
def kernels(tmp_path_factory):
    if not os.path.exists(HIPCC) and shutil.which("hipcc") is None:
        pytest.skip("hipcc not available")
    tmp = tmp_path_factory.mktemp("asm")
    procs = []
    for name in ("kernels", "kernels_paged"):  # contiguous and paged KV, compiled in parallel
        out = tmp / f"{name}.s"
        src = os.path.join(hipbuild.CSRC, f"{name}.hip")
        cmd = [HIPCC, *hipbuild.compile_flags(), "-S", "--cuda-device-only", "-o", str(out), src]
        procs.append((out, subprocess.Popen(cmd)))
    ks = {}
    for out, p in procs:
        assert p.wait() == 0
        part = asm_scan.kernels(out.read_text())
        assert len(part) == 6, sorted(part)  # {bf16, fp8} x {16, 32, 48 rows per row group}
        ks.update(part)
    assert len(ks) == 12, sorted(ks)
    return ks


def test_main_kernels_use_no_scratch(kernels):
    """Every main kernel keeps its pipeline in registers: no private segment."""
    for name, lines in kernels.items():
        assert asm_scan.scratch_bytes(lines) == 0, name


def test_no_unpadded_mfma_hazards(kernels):
    for name, lines in kernels.items():
        assert asm_scan.mfma_hazards(lines) == [], name


def test_tile_loop_has_staged_loads_and_never_copies_them(kernels):
    for name, lines in kernels.items():
        assert asm_scan.staged_loads_in_loops(lines) > 0, name  # the scan sees the loads
        assert asm_scan.staged_copies_in_loops(lines) == [], name
        assert asm_scan.staged_copies_in_prologues(lines) == [], name


def test_tile_loop_keeps_register_files(kernels):
    for name, lines in kernels.items():
        assert asm_scan.accvgpr_moves_in_loops(lines) == [], name


def test_scan_detects_a_planted_hazard():
    planted = ["\tv_mov_b64_e32 v[6:7], s[4:5]",
               "\tv_mfma_f32_16x16x32_bf16 a[0:3], v[4:7], v[4:7], 0",
               "\ts_nop 15",
               "\tv_accvgpr_read_b32 v8, a1"]
    found = asm_scan.mfma_hazards(planted)
    assert len(found) == 2, found


def test_scan_detects_a_planted_staged_copy():
    loop = [".LBB0_1:                                ; =>This Inner Loop Header: Depth=1",
            "\tbuffer_load_dwordx2 v[10:11], v1, s[4:7], s8 offen",
            "\tv_mfma_f32_16x16x32_bf16 v[0:3], v[4:7], v[4:7], v[0:3]",
            "\tv_mov_b64_e32 v[20:21], v[10:11]",
            "\ts_cbranch_scc1 .LBB0_1"]
    assert len(asm_scan.staged_copies_in_loops(loop)) == 1
    # the register was redefined (reused for another value) before the copy: no flag
    reused = loop[:3] + ["\tv_add_f32_e32 v10, v2, v3"] + loop[3:]
    assert asm_scan.staged_copies_in_loops(reused) == []
