"""Build libdgemm.so (GEMM and attention HIP kernels for gfx950, host planner, C ABI) in-tree
with hipcc.

Usage: python -m dense_gemm_operand_amd.build  (or call build()).
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libdgemm.so")
# Test-only build of the same sources with DGEMM_OVERSYNC=1 (a wait for every load and a
# workgroup barrier after every main-loop phase), compared bit for bit with libdgemm.so.
LIB_OVERSYNC = os.path.join(HERE, "libdgemm_oversync.so")
BUILD_DIR = os.path.join(HERE, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# -packed-fp32-ops: never form packed fp32 VALU ops; -ffp-contract=off: no FMA contraction
# (the int4 dequant must round exactly once, in its binary16 multiply).
COMMON = ["-O3", "-std=c++20", "-fPIC", f"--offload-arch={ARCH}", "-ffp-contract=off",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wno-unused-command-line-argument"]
SOURCES = ["inst_f16.hip", "inst_bf16.hip", "inst_f8.hip", "inst_misc.hip", "inst_attn.hip",
           "noalloc.hip", "host.cpp"]


def _compile(src: str, oversync: bool = False) -> str:
    obj = os.path.join(BUILD_DIR, ("oversync_" if oversync else "") + os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON, *(["-DDGEMM_OVERSYNC=1"] if oversync else []), "-c",
           os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def _link(objs, out: str) -> None:
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = False, oversync: bool = True) -> str:
    """Compile every source and link libdgemm.so next to this file (and, with `oversync`,
    the test-only libdgemm_oversync.so). Always rebuilds."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = [(src, False) for src in SOURCES] + ([(src, True) for src in SOURCES] if oversync else [])
    with ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 8)) as ex:
        objs = list(ex.map(lambda j: _compile(*j), jobs))
    _link(objs[:len(SOURCES)], LIB)
    if oversync:
        _link(objs[len(SOURCES):], LIB_OVERSYNC)
    if verbose:
        print(f"built {LIB}" + (f" and {LIB_OVERSYNC}" if oversync else ""))
    return LIB


if __name__ == "__main__":
    build(verbose=True, oversync="--no-oversync" not in sys.argv)
    sys.exit(0)
