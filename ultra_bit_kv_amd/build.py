"""Build liboscar_kv.so in-tree with hipcc for gfx950.

Usage: python -m ultra_bit_kv_amd.build [-v]
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "liboscar_kv.so")
SOURCES = ["api.cpp", "k_rotate.hip", "k_quant.hip", "k_dequant.hip", "k_decode.hip", "k_bf16.hip",
           "k_prefill.hip", "k_probe.hip"]
# The decode kernels keep their MFMA accumulators in VGPRs so the (rare) online
# softmax rescale multiplies them in place instead of copying AGPRs each step.
EXTRA = {"k_decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         "k_bf16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         "k_prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}

# Packed fp32 VALU ops are turned off for all device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
          "-Wno-unused-command-line-argument", "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build liboscar_kv)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "unknown target feature"   # host pass does not know the device-only feature
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l and "packed-fp32" not in l)
    if r.returncode != 0:
        raise RuntimeError("build failed:\n" + " ".join(cmd) + "\n" + err)
    if verbose and err.strip():
        print(err, flush=True)


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"]
        cmds.append([cc] + lang + COMMON + DEVICE_FLAGS + EXTRA.get(src, []) +
                    ["-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    with ThreadPoolExecutor(max_workers=min(8, len(cmds))) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = LIB + ".tmp"
    _run([cc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs, verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
