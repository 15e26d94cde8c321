"""Build the HIP library ``libnegacyclic_ntt.so`` (gfx950) in-tree with hipcc.

Every source is compiled for gfx950 only; objects go to ``_build/`` and the
shared library next to this file, where the binding loads it.
"""
import concurrent.futures
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libnegacyclic_ntt.so")
SOURCES = ["plan.cpp", "capi.cpp", "ntt.hip", "elementwise.hip", "keyswitch.hip", "noalloc.hip"]
ARCH = "gfx950"
FLAGS = [
    "-O3", f"--offload-arch={ARCH}", "-std=c++17", "-fPIC", "-Wall",
    # Keep the compiler from forming packed fp32 ops (this library does no fp32
    # math, but the flag is part of the supported gfx950 build recipe).
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = ["hipcc", *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = [l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip()]
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n" + "\n".join(noise))
    if noise and verbose:
        print("\n".join(noise), flush=True)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    workers = max(1, min(len(SOURCES), len(os.sched_getaffinity(0))))
    with concurrent.futures.ThreadPoolExecutor(workers) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    cmd = ["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", LIB + ".tmp", *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
