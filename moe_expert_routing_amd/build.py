"""Build libmoe_route.so (HIP, gfx950) in-tree with hipcc.

    python -m moe_expert_routing_amd.build

The library is written to moe_expert_routing_amd/_lib/libmoe_route.so, next
to the binding that loads it. The build keeps the device assembly of every
translation unit (in _build/) and fails if it holds a packed FP32
instruction (v_pk_add_f32, v_pk_mul_f32, v_pk_fma_f32): the kernels are
compiled without them, and this check makes sure the flag that keeps them
out still takes effect.
"""
from __future__ import annotations

import glob
import os
import re
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB_DIR = os.path.join(PKG, "_lib")
LIB_PATH = os.path.join(LIB_DIR, "libmoe_route.so")
TEMPS = os.path.join(ROOT, "_build")
SOURCES = [os.path.join(CSRC, "moe_route.hip"), os.path.join(CSRC, "router_gemm.hip")]
ARCH = "gfx950"

HIP_FLAGS = [
    "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-shared",
    # every floating-point operation is rounded on its own (exact sigmoid,
    # double-double arithmetic); FMAs are written explicitly
    "-ffp-contract=off",
    # no packed FP32 instructions on the device. The feature is a gfx9 device
    # feature: the host pass does not know it and warns that it ignores it
    # (that warning is filtered below); the device pass honours it, and
    # packed_fp32_in_device_asm() checks the result.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]
HOST_FEATURE_WARNING = re.compile(r"'-packed-fp32-ops' is not a recognized feature for this target")
PACKED_FP32 = re.compile(r"\bv_pk_(add|mul|fma)_f32\b")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def packed_fp32_in_device_asm(temps: str = TEMPS) -> list:
    """(file, line) of every packed FP32 instruction in the kept device
    assembly of the last build."""
    hits = []
    for path in sorted(glob.glob(os.path.join(temps, "*-hip-amdgcn-amd-amdhsa-*.s"))):
        with open(path, encoding="utf-8", errors="replace") as fh:
            for n, line in enumerate(fh, 1):
                code = line.split(";", 1)[0]
                if PACKED_FP32.search(code):
                    hits.append((os.path.basename(path), n))
    return hits


def build(verbose: bool = False) -> str:
    os.makedirs(LIB_DIR, exist_ok=True)
    if os.path.isdir(TEMPS):
        shutil.rmtree(TEMPS)
    os.makedirs(TEMPS)
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), *HIP_FLAGS, "-save-temps", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           *[s for s in SOURCES if os.path.exists(s)], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True, cwd=TEMPS)
    log = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                    if not HOST_FEATURE_WARNING.search(l) and "argument unused" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{log}")
    if verbose and log.strip():
        print(log, flush=True)
    if not glob.glob(os.path.join(TEMPS, "*-hip-amdgcn-amd-amdhsa-*.s")):
        raise RuntimeError("no device assembly kept: the packed FP32 check cannot run")
    hits = packed_fp32_in_device_asm()
    if hits:
        raise RuntimeError(f"packed FP32 instructions in the device code: {hits[:5]}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
