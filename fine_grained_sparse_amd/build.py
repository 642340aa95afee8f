"""Build libmoe.so (the C-ABI HIP library) for gfx950, in-tree.

Every HIP source is compiled with hipcc for --offload-arch=gfx950; packed
fp32 instructions are disabled (-packed-fp32-ops) so the compiler never
emits v_pk_{add,mul,fma}_f32.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build", "moe")
LIB = os.path.join(HERE, "libmoe.so")
SOURCES = ["api.cpp", "gemm.hip", "router.hip", "dispatch.hip", "pack.hip", "noalloc.hip"]
# measurement aid of bench.py (HBM streaming read, bf16 MFMA loop), a library
# of its own so that libmoe.so exports only the layer's C ABI
YARDSTICK_SOURCES = ["yardstick.hip"]
YARDSTICK_LIB = os.path.join(HERE, "libyardstick.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function", "-I" + os.path.join(ROOT, "include")]


def _compile(src, verbose):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC] + FLAGS + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    if verbose and r.stderr.strip():
        print(r.stderr, file=sys.stderr)
    return obj


def _link(objs, lib, verbose):
    tmp = lib + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + YARDSTICK_SOURCES
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = dict(zip(srcs, ex.map(lambda s: _compile(s, verbose), srcs)))
    _link([objs[s] for s in SOURCES], LIB, verbose)
    _link([objs[s] for s in YARDSTICK_SOURCES], YARDSTICK_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
