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


# Variants of the same library (build_variant):
#   asan:  host code instrumented with AddressSanitizer, device code unchanged;
#          load it into a process that preloads asan_runtime() (the interpreter
#          itself is not instrumented)
#   debug: kernels built with PSW_DEBUG check their internal invariants and
#          record failed checks (psw_debug_take_failures) instead of trapping
VARIANTS = {
    "asan": ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"],
    "debug": ["-DPSW_DEBUG"],
}


def _compile(src: str, out_dir: str = BUILD, extra: tuple = ()) -> str:
    obj = os.path.join(out_dir, os.path.basename(src).replace(".hip", ".o"))
    cmd = [_hipcc(), *HIPCC_FLAGS, *extra, "-I", os.path.join(os.path.dirname(HERE), "include"),
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


def variant_path(kind: str) -> str:
    """Where build_variant(kind) puts its library: the debug build in-tree beside
    libpsw.so (GPU runs load it), others under _build/<kind>/."""
    if kind == "debug":
        return os.path.join(HERE, "libpsw_debug.so")
    return os.path.join(BUILD, kind, f"libpsw_{kind}.so")


def _clang() -> str:
    """The clang++ that hipcc drives (ROCm's llvm)."""
    c = os.path.join(os.path.dirname(os.path.realpath(_hipcc())), "..", "lib", "llvm", "bin",
                     "clang++")
    return os.path.normpath(c) if os.path.exists(c) else (shutil.which("clang++") or "clang++")


def asan_runtime() -> str:
    """The clang AddressSanitizer runtime to preload for the asan variant."""
    r = subprocess.run([_clang(), "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError(f"AddressSanitizer runtime not found ({path!r})")
    return path


def build_variant(kind: str, verbose: bool = True) -> str:
    """Compile every source with the variant's extra flags and link it like the
    release library (the asan variant links the sanitizer runtime shared)."""
    extra = tuple(VARIANTS[kind])
    out_dir = os.path.join(BUILD, kind)
    os.makedirs(out_dir, exist_ok=True)
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, out_dir, extra), srcs))
    tlib = _torch_lib_dir()
    lib = variant_path(kind)
    tmp = lib + ".tmp"
    if kind == "asan":
        linker = [_clang(), "-fsanitize=address", "-shared-libasan"]
    else:
        linker = ["g++", "-Wl,--no-undefined", "-Wl,-z,defs"]
    cmd = [*linker, "-shared", "-o", tmp, *objs, f"-L{tlib}", "-l:libamdhip64.so",
           f"-Wl,-rpath,{tlib}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link of the {kind} variant failed:\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"[build] {lib} ({kind} variant, {len(objs)} objects)")
    return lib


if __name__ == "__main__":
    build()
    sys.exit(0)
