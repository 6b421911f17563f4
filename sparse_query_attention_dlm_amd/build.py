"""Compile the gfx950 HIP sources into the in-tree shared library libdlm.so.

Every source is compiled with hipcc for gfx950 only; packed fp32 VALU ops are
disabled on the device pass (the compiler still uses scalar fp32 FMA).  Object
files go to <repo>/_build, the library next to this file so that it travels
with the source tree."""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(HERE, "libdlm.so")
SOURCES = ["select.hip", "gemm.hip", "attn.hip", "colsum.hip", "dv.hip", "prefix.hip", "probe.hip",
           "validate.hip", "dlm_abi.hip"]
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
]
# Per-source additions.  The column-sum pass reads every MFMA result back for
# its exponentials; left to itself the compiler puts those results in AGPRs
# and copies them out (32 v_accvgpr_read plus hazard NOPs per tile), so that
# file asks for MFMA results in VGPRs.
EXTRA_FLAGS = {"colsum.hip": ["-mllvm", "--amdgpu-mfma-vgpr-form"]}


def _hipcc() -> str:
    cand = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(cand):
        raise RuntimeError("hipcc not found; the HIP toolchain is required to build libdlm")
    return cand


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{err}")
    return err


def build(verbose: bool = False) -> str:
    """Compile all sources and link libdlm.so; returns the library path."""
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = [os.path.join(BUILD_DIR, s.replace(".hip", ".o")) for s in SOURCES]
    cmds = [[hipcc, *FLAGS, *EXTRA_FLAGS.get(s, []), "-c", os.path.join(CSRC, s), "-o", o]
            for s, o in zip(SOURCES, objs)]
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(cmds))) as ex:
        for cmd, msg in zip(cmds, ex.map(_run, cmds)):
            if verbose and msg:
                print(msg)
    tmp = LIB_PATH + ".tmp"
    _run([hipcc, "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
