"""Build libmoe.so, the C-ABI library of HIP kernels for gfx950.

Every source compiles with hipcc for --offload-arch=gfx950 only. Packed fp32
instructions are disabled for device code (-packed-fp32-ops)."""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libmoe.so")
LIB_DEBUG = os.path.join(HERE, "libmoe_debug.so")  # the same sources with -DMOE_DEBUG (recorded bounds checks)
SOURCES = ["router.hip", "router_mma.hip", "permute.hip", "gemm_mfma.hip", "gemm_simple.hip", "combine.hip", "moe_abi.cpp", "moe_noalloc.hip", "backward.hip"]
OBJDIR = os.path.join(HERE, "_build")
OBJDIR_DEBUG = os.path.join(HERE, "_build_debug")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", INCLUDE, "-I", CSRC]


def _compile(src: str, verbose: bool, debug: bool = False) -> str:
    obj = os.path.join(OBJDIR_DEBUG if debug else OBJDIR, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [HIPCC, *FLAGS, *(["-DMOE_DEBUG"] if debug else []), *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{out}")
    if verbose and out.strip():
        print(out)
    return obj


def build(verbose: bool = False, jobs: int = 6, debug: bool = False) -> str:
    """Compile and link libmoe.so (or, with debug, libmoe_debug.so)."""
    os.makedirs(OBJDIR_DEBUG if debug else OBJDIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, debug), SOURCES))
    lib = LIB_DEBUG if debug else LIB
    tmp = lib + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, lib)
    return lib


def build_all(verbose: bool = False, jobs: int = 6) -> list:
    """Both libraries: the release build and the debug build."""
    return [build(verbose, jobs), build(verbose, jobs, debug=True)]


if __name__ == "__main__":
    print(build_all(verbose="-v" in sys.argv))
