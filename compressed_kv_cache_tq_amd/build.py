"""Build libtq.so (host C++ + HIP kernels for gfx950) in-tree with hipcc.

Usage: python -m compressed_kv_cache_tq_amd.build   (or build() from Python)
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJDIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libtq.so")
SOURCES = ["host.cpp", "plan.cpp", "quantize.hip", "attend.hip", "attend_k22.hip", "attend_k33.hip", "attend_k44.hip",
           "attend_k43.hip", "attend_k32.hip", "attend_k88.hip", "search.hip", "noalloc.hip", "fwht.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libtq.so)")


def common_flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++20", "-fPIC",
        "-I", os.path.join(ROOT, "include"),
        # keep the compiler from emitting packed fp32 VALU ops
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wno-unused-result",
    ]


def build(verbose: bool = False) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    cc = hipcc()
    procs, objs = [], []
    for src in SOURCES:
        obj = os.path.join(OBJDIR, src + ".o")
        objs.append(obj)
        cmd = [cc, *common_flags(), "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        if p.returncode != 0:
            failed.append((src, out.decode(errors="replace")))
        elif verbose and out:
            print(out.decode(errors="replace"))
    if failed:
        msg = "\n".join(f"--- {s} ---\n{o}" for s, o in failed)
        raise RuntimeError(f"hipcc failed:\n{msg}")
    tmp = LIB + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout.decode(errors="replace"))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
