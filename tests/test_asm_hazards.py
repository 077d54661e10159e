"""Host-side checks of the compiled kernels' gfx950 assembly.

Every kernel source is compiled once, with the library's own flags, to gfx950 assembly.
- Wait states around asm MFMAs.  The many-row decode kernel (splitkv_wide.hip) writes its
  P.V MFMAs as asm with the accumulators in AGPRs, so the compiler's hazard recognizer
  cannot see them; the kernel adds the wait states itself.  The check covers every path
  of every instantiation: no AGPR read too soon after an MFMA writes it, and no asm MFMA
  reading a VGPR right after a VALU write of it.  The synthetic cases pin the checker.
- No kernel spills to scratch, and no buffer load sits in a loop over the distinct
  buffer descriptors of a wave's lanes (what the compiler emits when it cannot prove a
  descriptor uniform: four v_readfirstlane, a 64-bit compare and an exec-mask branch per
  load).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import re
import subprocess

import pytest

from split_kv_merge_amd import build as skv_build
from tests.agpr_hazards import check_assembly, check_function

CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                    "split_kv_merge_amd", "csrc")
KERNEL_SOURCES = [s for s in skv_build.SOURCES if s.endswith(".hip")]

# four readfirstlane of a descriptor's words, then the compare against the lanes' values
_DESCRIPTOR_LOOP = re.compile(r"(?:v_readfirstlane_b32 s\d+, v\d+\n\s+){4}v_cmp_eq_u64")


def test_checker_flags_a_copy_right_after_an_mfma():
    lines = ["\tv_mfma_f32_32x32x16_bf16 a[0:15], v[0:3], v[4:7], a[0:15]",
             "\tv_accvgpr_mov_b32 a16, a0"]
    assert len(check_function(lines)) == 1
    fenced = [lines[0], "\ts_nop 7", "\ts_nop 7", "\ts_nop 7", lines[1]]
    assert check_function(fenced) == []


def test_checker_follows_branches_to_a_join():
    # the MFMA sits on one edge into the join; the fence only on the other one
    lines = ["\ts_cbranch_scc1 .LBB0_2",
             "\tv_mfma_f32_32x32x16_bf16 a[0:15], v[0:3], v[4:7], a[0:15]",
             "\ts_branch .LBB0_3",
             ".LBB0_2:",
             "\ts_nop 7",
             ".LBB0_3:",
             "\tv_accvgpr_read_b32 v8, a3"]
    assert len(check_function(lines)) == 1


def test_checker_flags_a_valu_write_right_before_an_asm_mfma():
    lines = ["\tv_mov_b32_e32 v5, v9",
             "\t;;#ASMSTART",
             "\tv_mfma_f32_32x32x16_bf16 a[0:15], v[0:3], v[4:7], a[0:15]",
             "\t;;#ASMEND"]
    assert len(check_function(lines)) == 1


def test_descriptor_loop_pattern_matches_a_loop():
    text = ("\tv_readfirstlane_b32 s12, v22\n\tv_readfirstlane_b32 s13, v23\n"
            "\tv_readfirstlane_b32 s14, v24\n\tv_readfirstlane_b32 s15, v25\n"
            "\tv_cmp_eq_u64_e64 s[6:7], s[12:13], v[22:23]\n")
    assert len(_DESCRIPTOR_LOOP.findall(text)) == 1
    assert not _DESCRIPTOR_LOOP.findall(text.replace("v_readfirstlane_b32 s14, v24\n\t", ""))


@pytest.fixture(scope="module")
def assembly(tmp_path_factory):
    if not os.path.exists(skv_build.hipcc()):
        pytest.skip("hipcc not installed")
    out_dir = tmp_path_factory.mktemp("asm")

    def compile_one(src):
        out = out_dir / (src + ".s")
        cmd = ([skv_build.hipcc()] + skv_build.common_flags() + skv_build.EXTRA_FLAGS.get(src, []) +
               ["--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", str(out)])
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        return src, out.read_text()

    with cf.ThreadPoolExecutor(max_workers=4) as ex:
        return dict(ex.map(compile_one, KERNEL_SOURCES))


def test_many_row_decode_kernel_waits_after_its_asm_mfmas(assembly):
    found = check_assembly(assembly["splitkv_wide.hip"], "splitkv_wide_kernel")
    assert len(found) == 16, sorted(found)   # 2 dtypes x 2 head dims x 2 row blocks x 2 forms
    bad = {k: v[:3] for k, v in found.items() if v}
    assert not bad, bad


@pytest.mark.parametrize("src", KERNEL_SOURCES)
def test_kernels_do_not_spill(assembly, src):
    sizes = re.findall(r"\.set (\S+)\.private_seg_size, (\d+)", assembly[src])
    assert sizes, "no kernel found"
    spilled = {name: int(n) for name, n in sizes if int(n) != 0}
    assert not spilled, spilled


@pytest.mark.parametrize("src", KERNEL_SOURCES)
def test_buffer_loads_use_uniform_descriptors(assembly, src):
    assert not _DESCRIPTOR_LOOP.findall(assembly[src])
