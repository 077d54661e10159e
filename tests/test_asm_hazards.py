"""Host-side check of the wait states around asm MFMAs in the compiled decode kernel.

The many-row decode kernel (splitkv_wide.hip) writes its P.V MFMAs as asm with the
accumulators in AGPRs, so the compiler's hazard recognizer cannot see them; the kernel
adds the wait states itself.  This test compiles that file to gfx950 assembly with the
library's own flags and checks, on every path of every instantiation, that no AGPR is
read too soon after an MFMA writes it and that no asm MFMA reads a VGPR right after a
VALU write of it.  The synthetic cases pin the checker itself.
"""
from __future__ import annotations

import os
import subprocess

import pytest

from split_kv_merge_amd import build as skv_build
from tests.agpr_hazards import check_assembly, check_function

CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                    "split_kv_merge_amd", "csrc")


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


@pytest.mark.skipif(not os.path.exists("/opt/rocm/bin/hipcc"), reason="hipcc not installed")
def test_many_row_decode_kernel_waits_after_its_asm_mfmas(tmp_path):
    src = "splitkv_wide.hip"
    out = tmp_path / "wide.s"
    cmd = ([skv_build.hipcc()] + skv_build.common_flags() + skv_build.EXTRA_FLAGS.get(src, []) +
           ["--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", str(out)])
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    found = check_assembly(out.read_text(), "splitkv_wide_kernel")
    assert len(found) == 16, sorted(found)   # 2 dtypes x 2 head dims x 2 row blocks x 2 forms
    bad = {k: v[:3] for k, v in found.items() if v}
    assert not bad, bad
