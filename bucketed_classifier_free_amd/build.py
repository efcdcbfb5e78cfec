"""Build libbcg.so for gfx950 in-tree with hipcc.

    python -m bucketed_classifier_free_amd.build

Every call recompiles every source (the objects go to ``_build/`` at the
repository root, the library next to this file).  All device code is built
with contraction off (the kernels' evaluation order is part of their
contract) and without packed fp32 instructions.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libbcg.so")

SOURCES = ["bcg_host.cpp", "bcg_api.hip", "bcg_loop.hip", "bcg_step_f32.hip", "bcg_step_bf16.hip",
           "bcg_step_f32_nt.hip", "bcg_step_bf16_nt.hip", "bcg_step_f32_queue.hip", "bcg_step_bf16_queue.hip",
           "bcg_rows_f32.hip", "bcg_rows_bf16.hip", "bcg_weight.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libbcg)")


def common_flags():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-ffp-contract=off",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-function", f"-I{INCLUDE}", f"-I{CSRC}"]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    path = os.path.join(CSRC, src)
    cmd = [hipcc()] + common_flags()
    if src.endswith(".cpp"):
        cmd += ["-x", "c++"]
    cmd += ["-c", path, "-o", obj]
    t = time.time()
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass of hipcc does not know the packed-fp32 feature; drop that note
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{err}")
    if verbose:
        print(f"  {src}: {time.time() - t:.1f}s" + (f"\n{err}" if err.strip() else ""), flush=True)
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    t = time.time()
    jobs = min(len(SOURCES), max(1, (os.cpu_count() or 2)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} in {time.time() - t:.1f}s", flush=True)
    return LIB


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
