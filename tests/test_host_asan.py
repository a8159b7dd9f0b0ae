"""The host layer of libpsw.so under AddressSanitizer.

The asan variant of the library (build.build_variant("asan"): host code
instrumented, device code unchanged) runs the ABI's host-only tests, which
drive every entry point's argument checks, the workspace sizing and the error
text, in a child interpreter that preloads the sanitizer runtime.  CPU only: no
call reaches a kernel launch, and the made-up device addresses of the
host-only tests are never dereferenced.
"""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_host_layer_clean_under_address_sanitizer():
    from paged_sliding_window_amd import build
    lib = build.build_variant("asan", verbose=False)
    env = dict(os.environ, LD_PRELOAD=build.asan_runtime(), PSW_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1")
    # the child really runs the instrumented library with the runtime active
    probe = ("import ctypes, paged_sliding_window_amd as p\n"
             "from paged_sliding_window_amd import _lib\n"
             "h = p.load()\n"
             f"assert _lib.LIB_PATH == {lib!r} and h._name == {lib!r}, (_lib.LIB_PATH, h._name)\n"
             "assert hasattr(ctypes.CDLL(None), '__asan_init')\n"
             "maps = open('/proc/self/maps').read()\n"
             f"assert {lib!r} in maps and 'libclang_rt.asan' in maps\n")
    r = subprocess.run([sys.executable, "-c", probe], env=env, cwd=ROOT, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m",
                        "not gpu", "tests/test_abi.py"], env=env, cwd=ROOT, capture_output=True,
                       text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out, out[-4000:]
    assert " passed" in r.stdout, out[-2000:]
