"""Build libqkvnr.so for gfx950 with hipcc (no torch extension machinery).

    python -m qkv_norm_rope_amd.build          # build in-tree
    python -m qkv_norm_rope_amd.build --print  # show the commands only

Each .hip source compiles (hipcc, gfx950) and the host-only C ABI layer
host.cpp compiles (the host C++ compiler) to an object under
qkv_norm_rope_amd/_build/, then one shared library links them:
qkv_norm_rope_amd/lib/libqkvnr.so.
"""

from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libqkvnr.so")
INCLUDE = os.path.join(os.path.dirname(PKG), "include")

SOURCES = ["runtime.hip", "no_alloc.hip", "qkv_rmsnorm_rope_cache.hip",
           "mla_prolog_v2.hip"]
HOST_SOURCES = ["host.cpp"]  # plain C++: no HIP, also built under sanitizers

ARCH = "gfx950"
# Packed-fp32 VALU forms are disabled for every device compile.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
CFLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
          "-Wno-unused-function", f"-I{INCLUDE}"] + DEVICE_FLAGS


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc",
                 shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build)")


HOST_CFLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", f"-I{INCLUDE}"]


def host_cxx() -> str:
    for cand in (os.environ.get("CXX"), shutil.which("g++"), shutil.which("c++")):
        if cand and shutil.which(cand):
            return cand
    raise RuntimeError("no host C++ compiler (g++) found")


def commands():
    cc = hipcc()
    objs, cmds = [], []
    for src in SOURCES:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([cc, *CFLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    cxx = host_cxx()
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD, src.replace(".cpp", ".host.o"))
        objs.append(obj)
        cmds.append([cxx, *HOST_CFLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    link = [cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o",
            LIB + ".tmp"]
    return cmds, link


def build(verbose: bool = False, jobs: int = 4) -> str:
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    cmds, link = commands()

    def run(cmd):
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"build failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
        return r.stderr

    with ThreadPoolExecutor(max_workers=jobs) as ex:
        for err in ex.map(run, cmds):
            # hipcc's host pass warns that it does not know the device-only
            # target feature; that warning is expected.
            lines = [ln for ln in err.splitlines()
                     if "packed-fp32-ops" not in ln and ln.strip()]
            if lines and verbose:
                print("\n".join(lines))
    run(link)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--print", action="store_true")
    ap.add_argument("-v", "--verbose", action="store_true")
    args = ap.parse_args(argv)
    if args.print:
        cmds, link = commands()
        for c in cmds + [link]:
            print(" ".join(c))
        return 0
    print(build(verbose=args.verbose))
    return 0


if __name__ == "__main__":
    sys.exit(main())
