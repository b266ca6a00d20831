"""Build the HIP library ``libpa.so`` in-tree for gfx950.

``python -m paged_kv_cache_165_amd.build`` or ``build_library()``. Every
source is compiled for gfx950 only, with packed fp32 instructions disabled.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG_DIR, "libpa.so")
SOURCES = ["pa_api.hip", "pa_decode.hip", "pa_cache.hip", "pa_blocks.hip", "pa_prefill.hip", "pa_probe.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the ROCm toolchain is required to build libpa.so")
    return path


def compile_flags(extra=()) -> list:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # MFMA results go to ordinary VGPRs: the accumulators are then
        # rescaled in place instead of being copied out of AGPRs every tile
        "-mllvm", "-amdgpu-mfma-vgpr-form=1",
        "-Wall", "-Wno-unused-function",
        f"-I{INCLUDE}", f"-I{CSRC}", *extra,
    ]


def build_library(verbose: bool = False, jobs: int = 4, extra_flags=(), out: str = LIB_PATH,
                  objdir: str = None) -> str:
    """Compile every source to an object in parallel, then link the library
    (default: libpa.so in the package directory). `extra_flags` are passed to
    every compile (e.g. -D tuning macros for a side build)."""
    objdir = objdir or os.path.join(PKG_DIR, "_build")
    os.makedirs(objdir, exist_ok=True)
    cc = hipcc()
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        objs.append(obj)
        cmd = [cc, *compile_flags(extra_flags), "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
        while len([p for _, p in procs if p.poll() is None]) >= jobs:
            procs[0][1].wait()
    failed = []
    for src, p in procs:
        log, _ = p.communicate()
        msg = "\n".join(l for l in log.splitlines() if "packed-fp32-ops" not in l)
        if p.returncode != 0:
            failed.append((src, msg))
        elif verbose and msg.strip():
            print(msg)
    if failed:
        raise RuntimeError("hipcc failed:\n" + "\n".join(f"--- {s}\n{m}" for s, m in failed))
    tmp = out + ".tmp"
    link = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(link, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build_library(verbose="-v" in sys.argv))
