"""Build libmxmoe.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

Usage: python -m mxfp8_block_scaled_06_amd.build
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
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libmxmoe.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)

SOURCES = ["mx_quant.hip", "mx_gemm.hip", "mx_route.hip", "mx_noalloc.hip", "mx_api.cpp"]

# -packed-fp32-ops: never emit packed fp32 VALU instructions.
HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: install ROCm or put hipcc on PATH")


def _run(cmd):
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in proc.stdout.splitlines() if "packed-fp32-ops" not in l)
    if proc.returncode != 0:
        raise RuntimeError(f"command failed ({proc.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    cc = hipcc()
    with tempfile.TemporaryDirectory(prefix="mxmoe_build_") as tmp:
        objs = []
        cmds = []
        for src in SOURCES:
            obj = os.path.join(tmp, src + ".o")
            lang = ["-x", "hip"] if src.endswith(".hip") else []
            cmds.append([cc, *HIP_FLAGS, "-I", INCLUDE, "-I", CSRC, *lang, "-c", os.path.join(CSRC, src), "-o", obj])
            objs.append(obj)
        with ThreadPoolExecutor(max_workers=len(cmds)) as ex:
            for out in ex.map(_run, cmds):
                if verbose and out.strip():
                    print(out)
        tmp_lib = os.path.join(tmp, LIB_NAME)
        _run([cc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp_lib])
        shutil.move(tmp_lib, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH}")
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
