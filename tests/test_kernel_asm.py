"""CPU checks of the decode kernels' gfx950 assembly (hipcc cross-compiles
them here with the library's own flags): hazards around the inline-assembly
MFMAs and transcendental results, KV tiles moved by LDS DMA in the tile loops
where the kernels use it and no copies of registers that staged loads are
filling elsewhere, no register-file moves inside the bf16 KV tile loop, and
no compiler use of the AGPRs that the fp8 kernel allocates by hand."""
import os
import shutil
import subprocess

import pytest

from mla_token_decode_amd import build as hipbuild
from tests import asm_scan

HIPCC = hipbuild.HIPCC


@pytest.fixture(scope="module")
def assembly(tmp_path_factory):
    """Source name -> its gfx950 assembly text (all four compiled in parallel)."""
    if not os.path.exists(HIPCC) and shutil.which("hipcc") is None:
        pytest.skip("hipcc not available")
    tmp = tmp_path_factory.mktemp("asm")
    procs = []
    for name in ("kernels", "kernels_paged", "fp8_decode", "fp8_decode_paged"):
        out = tmp / f"{name}.s"
        src = os.path.join(hipbuild.CSRC, f"{name}.hip")
        cmd = [HIPCC, *hipbuild.compile_flags(), "-S", "--cuda-device-only", "-o", str(out), src]
        procs.append((name, out, subprocess.Popen(cmd)))
    texts = {}
    for name, out, p in procs:
        assert p.wait() == 0
        texts[name] = out.read_text()
    return texts


@pytest.fixture(scope="module")
def kernels(assembly):
    ks = {}
    for name in ("kernels", "kernels_paged"):  # contiguous and paged KV
        part = asm_scan.kernels(assembly[name])
        # bf16 KV, 16 / 32 / 48 rows per row group, with and without the non-temporal KV hint
        assert len(part) == 6, sorted(part)
        ks.update(part)
    assert len(ks) == 12, sorted(ks)
    return ks


@pytest.fixture(scope="module")
def fp8_kernels(assembly):
    ks = {}
    for name in ("fp8_decode", "fp8_decode_paged"):
        part = asm_scan.kernels(assembly[name], asm_scan.FP8_KERNEL)
        assert len(part) == 6, sorted(part)  # 32, 64, 96 rows per unit; two KV hints
        ks.update(part)
    assert len(ks) == 12, sorted(ks)
    return ks


def test_main_kernels_use_no_scratch(kernels):
    """Every main kernel keeps its pipeline in registers: no private segment."""
    for name, lines in kernels.items():
        assert asm_scan.scratch_bytes(lines) == 0, name


def test_merge_kernels_use_no_scratch(assembly):
    """The reduce and shard-merge kernels, in both the forms that read
    sequence descriptors from the kernel arguments and from a large plan's
    workspace tables, hold nothing in private memory (an argument array
    indexed per lane would copy the whole argument block there)."""
    ks = asm_scan.kernels(assembly["kernels"], asm_scan.MERGE_KERNEL)
    # reduce: 1 row layout + 4 chunk-phase layouts, two descriptor sources; shard merge
    assert len(ks) == 11, sorted(ks)
    for name, lines in ks.items():
        assert asm_scan.scratch_bytes(lines) == 0, name


def test_no_unpadded_mfma_hazards(kernels):
    for name, lines in kernels.items():
        assert asm_scan.mfma_hazards(lines) == [], name


def test_no_unpadded_transcendental_reads(kernels, fp8_kernels):
    for name, lines in {**kernels, **fp8_kernels}.items():
        assert asm_scan.trans_hazards(lines) == [], name


def test_fp8_kernels_use_no_scratch_and_leave_agprs_to_the_asm(fp8_kernels):
    """The fp8 kernel keeps O and part of Q in AGPRs that its inline assembly
    names; anything the compiler put there would be overwritten."""
    for name, lines in fp8_kernels.items():
        assert asm_scan.scratch_bytes(lines) == 0, name
        assert asm_scan.compiler_agprs(lines) == [], name


def test_fp8_kernels_pad_mfma_hazards(fp8_kernels):
    for name, lines in fp8_kernels.items():
        assert asm_scan.mfma_hazards(lines) == [], name


def test_tile_loops_move_kv_by_dma_or_uncopied_staging(kernels, fp8_kernels):
    """The fp8 kernels and the bf16 kernels of 48-row row groups move KV tiles
    with LDS DMA inside their tile loops; the narrower bf16 kernels stage
    them in registers, and no compiler copy reads a staged register while its
    load is in flight."""
    for name, lines in fp8_kernels.items():
        assert asm_scan.dma_loads_in_loops(lines) > 0, name
    assert sum("Li3E" in n for n in kernels) == 4, sorted(kernels)
    for name, lines in kernels.items():
        if "Li3E" in name:  # 3 row tiles per row group: DMA
            assert asm_scan.dma_loads_in_loops(lines) > 0, name
            assert asm_scan.staged_loads_in_loops(lines) == 0, name
        else:
            assert asm_scan.staged_loads_in_loops(lines) > 0, name  # the scan sees the loads
        assert asm_scan.staged_copies_in_loops(lines) == [], name
        assert asm_scan.staged_copies_in_prologues(lines) == [], name


def test_scan_sees_dma_loads():
    loop = [".LBB0_1:                                ; =>This Inner Loop Header: Depth=1",
            "\tbuffer_load_dwordx4 v3, s[4:7], 0 offen nt lds",
            "\tv_mfma_f32_16x16x32_bf16 v[0:3], v[4:7], v[4:7], v[0:3]",
            "\tbuffer_load_dwordx4 v5, s[4:7], 0 offen lds",
            "\ts_cbranch_scc1 .LBB0_1"]
    assert asm_scan.dma_loads_in_loops(loop) == 2
    assert asm_scan.staged_loads_in_loops(loop) == 0


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


def test_scan_detects_a_planted_transcendental_read():
    planted = ["\tv_exp_f32_e32 v59, v59",
               ";;#ASMSTART",
               "\tv_max_f32 v105, v58, v59",
               ";;#ASMEND",
               "\tv_exp_f32_e32 v60, v60",
               "\ts_nop 0",
               "\tv_max_f32 v106, v58, v60"]
    assert len(asm_scan.trans_hazards(planted)) == 1


def test_scan_detects_a_compiler_agpr():
    lines = [";;#ASMSTART", "\tv_accvgpr_write_b32 a3, v1", ";;#ASMEND",
             "\tv_accvgpr_read_b32 v2, a4"]
    assert asm_scan.compiler_agprs(lines) == ["v_accvgpr_read_b32 v2, a4"]
