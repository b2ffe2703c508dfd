"""Build libmoe_route.so from csrc/*.hip for gfx950 with hipcc (in-tree), and
libmoe_hbm_ceiling.so, the benchmark's reference kernels (bench.py only).

    python -m combine_top_router_select_amd.build [-D NAME=VALUE ...]

Cross-compiles on a machine without a GPU.  Flags: -O3, no fast-math,
denormals kept, packed-fp32 instructions disabled, hidden visibility except for
the C ABI.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmoe_route.so")
OBJ_DIR = os.path.join(PKG, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["abi.hip", "route_topk.hip", "counts.hip", "dispatch.hip", "combine.hip",
           "combine_route.hip", "coselect.hip", "placement.hip", "shuffle.hip", "noalloc.hip"]
CEILING_SOURCES = ["hbm_ceiling.hip"]
CEILING_LIB = os.path.join(PKG, "libmoe_hbm_ceiling.so")

COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-fno-gpu-flush-denormals-to-zero", "-ffp-contract=on",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wextra", "-Wno-unused-command-line-argument",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def build(defines=(), out=LIB, verbose=False) -> str:
    """Builds the library (and, for the in-tree library, the benchmark's
    reference kernels next to it)."""
    res = build_lib(SOURCES, out, defines, verbose)
    if out == LIB:
        build_lib(CEILING_SOURCES, CEILING_LIB, defines, verbose)
    return res


def build_lib(sources, out, defines=(), verbose=False) -> str:
    os.makedirs(OBJ_DIR, exist_ok=True)
    dflags = [f"-D{d}" for d in defines]

    def compile_one(src):
        obj = os.path.join(OBJ_DIR, os.path.splitext(src)[0] + ".o")
        cmd = [HIPCC, *COMMON_FLAGS, *dflags, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(len(sources), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(compile_one, sources))
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    return out


DEMO_SRC = os.path.join(ROOT, "tests", "abi_demo.c")
DEMO = os.path.join(ROOT, "tests", "abi_demo")


def build_abi_demo(out=DEMO) -> str:
    """The plain-C user of the C ABI (tests/abi_demo.c), compiled with gcc as
    C11 against include/moe_route.h and HIP's C runtime API, linked against the
    in-tree library (found through its rpath)."""
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(HIPCC)))
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           f"-I{rocm}/include", f"-I{INCLUDE}", DEMO_SRC, "-o", out, f"-L{PKG}", "-lmoe_route",
           f"-L{rocm}/lib", "-lamdhip64", "-Wl,-rpath,$ORIGIN/../combine_top_router_select_amd",
           f"-Wl,-rpath,{rocm}/lib"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"abi demo build failed:\n{r.stdout}\n{r.stderr}")
    return out


if __name__ == "__main__":
    defs = []
    args = sys.argv[1:]
    i = 0
    while i < len(args):
        if args[i] == "-D":
            defs.append(args[i + 1])
            i += 2
        elif args[i].startswith("-D"):
            defs.append(args[i][2:])
            i += 1
        else:
            raise SystemExit(f"unknown argument {args[i]}")
    print(build(defs, verbose=True))
