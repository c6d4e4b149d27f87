"""Build libwbmm.so (HIP for gfx950) in-tree: one hipcc compile per source, in parallel, then link.

Usage: python -m receptive_field_spatial_amd.build  (or call build()).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG_DIR, "csrc")
OBJ_DIR = os.path.join(PKG_DIR, "_build")
LIB_PATH = os.path.join(PKG_DIR, "libwbmm.so")
SOURCES = ["wbmm_api.cpp", "wbmm_aux.hip", "wbmm_fwd.hip", "wbmm_bwd.hip", "wbmm_fast.hip", "wbmm_fastroll.hip",
           "wbmm_fastbf.hip", "wbmm_dw.hip",
           "wbmm_probe.hip", "wbmm_bwdbf.hip", "wbmm_repack.hip", "wbmm_fastcm.hip",
           "wbmm_fast28.hip", "wbmm_fast7.hip", "wbmm_fasttab.hip", "wbmm_hiergen.cpp",
           "wbmm_bwdwide.hip"]

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Packed-fp32 VALU ops (v_pk_fma_f32 and kin) are disabled for every device compile: the code
# keeps to scalar fp32 vector instructions, which the kernels were validated with.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-fPIC", "-std=c++17", "-fvisibility=hidden", f"--offload-arch={ARCH}",
          "-Wall", "-Wno-unused-function", "-Wno-unused-variable", "-Wno-pass-failed"]


def _compile(src: str) -> str:
    out = os.path.join(OBJ_DIR, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"]
    cmd = [HIPCC, *COMMON, *DEVICE_FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    # The host pass does not know the packed-fp32 feature and says so; that line is harmless.
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l).strip()
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{msgs}")
    if msgs:
        print(f"[build] {src}:\n{msgs}", file=sys.stderr)
    return out


def build(verbose: bool = True, jobs: int | None = None) -> str:
    """Compile every source for gfx950 and link libwbmm.so next to this file. Always rebuilds."""
    if shutil.which(HIPCC) is None and not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(OBJ_DIR, exist_ok=True)
    jobs = jobs or min(len(SOURCES), max(1, (os.cpu_count() or 4)))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{res.stdout}{res.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"[build] wrote {LIB_PATH}")
    return LIB_PATH


if __name__ == "__main__":
    build()
