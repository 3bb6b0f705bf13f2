"""Build libkvc.so for gfx950 with hipcc, in-tree (kv_cache_attention_kvc_amd/libkvc.so).

Run as `python -m kv_cache_attention_kvc_amd.csrc.build` or call build(). Every HIP translation
unit is compiled with the packed-fp32 target feature disabled (v_pk_*_f32 are never emitted), and
MFMA accumulators are kept in VGPRs.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
PKG = os.path.dirname(HERE)
ROOT = os.path.dirname(PKG)
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(PKG, "libkvc.so")
BUILD_DIR = os.path.join(PKG, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["kvc_pool.cpp", "kvc_decode.hip", "kvc_write.hip", "kvc_prefill.hip", "kvc_probe.hip"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-I", INCLUDE, "-I", HERE]
# The matrix-core decode accumulates in VGPRs (gfx950 MFMA takes C/D there): its softmax
# rescale is VALU work on the accumulator, and AGPR accumulators would need copies both ways
# plus a second register file's worth of space.
HIP_FLAGS = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang",
             "-packed-fp32-ops", "-mllvm", "-amdgpu-mfma-vgpr-form", "-x", "hip"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON]
    if src.endswith(".hip"):
        cmd += HIP_FLAGS
    cmd += ["-c", os.path.join(HERE, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines()
            if "packed-fp32-ops" not in ln]    # the host pass does not know the feature
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n" + "\n".join(msgs))
    if msgs and os.environ.get("KVC_BUILD_VERBOSE"):
        print("\n".join(msgs), file=sys.stderr)
    return obj


def build() -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}{r.stderr}")
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build())
