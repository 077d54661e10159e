"""Build libskv.so (gfx950) in-tree with hipcc.

Every translation unit is compiled with -O3 for --offload-arch=gfx950 and with the
packed-fp32 target feature switched off (the compiler then emits no
v_pk_{add,mul,fma}_f32).  Objects go to split_kv_merge_amd/_build/, the library
to split_kv_merge_amd/libskv.so.  Usage: python -m split_kv_merge_amd.build
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libskv.so")
INCLUDE = os.path.join(ROOT, "include")

SOURCES = ["api.cpp", "fmha_fwd.hip", "splitkv.hip", "splitkv_wide.hip", "merge.hip",
           "kmean.hip", "sage_quant.hip", "sage_fwd.hip", "scratch.hip"]
# Per-file flags: the many-row decode kernel keeps its output accumulators in AGPRs
# through asm MFMAs and needs its builtin MFMAs in VGPR form, so that the scores stay
# in VGPRs instead of moving between the register files.
EXTRA_FLAGS = {"splitkv_wide.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (expected /opt/rocm/bin/hipcc)")


def common_flags():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", f"-I{INCLUDE}", f"-I{CSRC}",
            "-Wall", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + common_flags() + EXTRA_FLAGS.get(src, []) + ["-c", os.path.join(CSRC, src),
                                                                 "-o", obj]
    if src.endswith(".cpp"):
        cmd += ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [l for l in (r.stderr or "").splitlines() if "packed-fp32-ops" not in l]
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n" + "\n".join(msgs))
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("linking libskv.so failed:\n" + r.stderr)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
