"""Build libpsw.so in-tree for gfx950.

Every ``csrc/*.hip`` file is compiled with hipcc (device code for gfx950 only),
then the objects are linked against the HIP runtime that torch itself loads
(torch/lib/libamdhip64.so, referenced by file name), so that a process holding
both torch and libpsw.so runs a single HIP runtime and torch's streams and
device pointers are valid in the library.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(os.path.dirname(HERE), "_build")
LIB = os.path.join(HERE, "libpsw.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # packed fp32 instructions are kept out of every kernel on purpose
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _torch_lib_dir() -> str:
    import torch  # noqa: F401  (only to locate the runtime torch loads)
    d = os.path.join(os.path.dirname(torch.__file__), "lib")
    if not os.path.exists(os.path.join(d, "libamdhip64.so")):
        raise RuntimeError(f"torch's libamdhip64.so not found in {d}")
    return d


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src).replace(".hip", ".o"))
    cmd = [_hipcc(), *HIPCC_FLAGS, "-I", os.path.join(os.path.dirname(HERE), "include"),
           "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tlib = _torch_lib_dir()
    tmp = LIB + ".tmp"
    cmd = ["g++", "-shared", "-o", tmp, *objs, f"-L{tlib}", "-l:libamdhip64.so",
           f"-Wl,-rpath,{tlib}", "-Wl,--no-undefined", "-Wl,-z,defs"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"[build] {LIB} ({len(objs)} objects, {ARCH})")
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
