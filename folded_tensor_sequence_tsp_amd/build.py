"""Build libtsp.so (HIP for gfx950) in-tree with hipcc.

``python -m folded_tensor_sequence_tsp_amd.build`` or :func:`build`.  The
library lands next to this file; the ctypes binding loads it from there.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libtsp.so")
SOURCES = ["tsp_api.cpp", "layout.cpp", "gemm.hip", "attention.hip", "prep.hip", "variants.hip", "backward.hip", "attn_backward.hip", "noalloc.hip"]

ARCH = "gfx950"
# Packed fp32 VALU forms are switched off (they are only a codegen choice here).
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", os.path.join(ROOT, "include"), "-I", CSRC]
# Per-file additions.  The attention backward's dK/dV kernel runs one wave per
# SIMD; by default its MFMA results land in AGPRs and are copied to VGPRs for
# the vector work (112 copies per tile).  Selecting the VGPR form of the MFMAs
# keeps the scores and dK/dV accumulators in VGPRs (47 copies left).
FILE_FLAGS = {"attn_backward.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False) -> str:
    cc = hipcc()
    with tempfile.TemporaryDirectory(prefix="tsp_build_") as tmp:
        objs = []
        cmds = []
        for src in SOURCES:
            obj = os.path.join(tmp, src + ".o")
            lang = ["-x", "hip"]
            cmds.append([cc, *lang, *HIP_FLAGS, *FILE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj])
            objs.append(obj)

        def run(cmd):
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                raise RuntimeError(f"hipcc failed ({r.returncode}):\n{' '.join(cmd)}\n{r.stderr}")
            if verbose:
                sys.stderr.write(r.stderr)

        with ThreadPoolExecutor(max_workers=len(cmds)) as ex:
            list(ex.map(run, cmds))
        tmp_lib = LIB + ".tmp"
        run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp_lib])
        os.replace(tmp_lib, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
