"""The PSW_DEBUG variant, checked on the CPU.

For every source with debug checks: the debug build's checks are vector
atomics (global_atomic_or), the release build contains none of them (the
checks compile away), and neither build writes through the scalar data cache.
Also: the debug library links and exports every declared entry point (a child
interpreter loads it through PSW_LIBRARY).
"""
import os
import re
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "paged_sliding_window_amd", "csrc")
SOURCES = ["attention_prefill.hip", "attention_decode.hip", "slot_mapping.hip",
           "kv_cache_write.hip"]
SCALAR_WRITE = re.compile(r"^\s*s_(store|atomic|buffer_store|buffer_atomic|scratch_store|"
                          r"dcache_wb|dcache_discard)\w*", re.M)


def _device_asm(src, extra, out):
    from paged_sliding_window_amd.build import HIPCC_FLAGS, _hipcc
    subprocess.run([_hipcc(), *HIPCC_FLAGS, *extra, "-I", os.path.join(ROOT, "include"),
                    "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", str(out)],
                   check=True, capture_output=True)
    return out.read_text()


@pytest.mark.parametrize("src", SOURCES)
def test_debug_checks_are_vector_atomics_and_compile_away(tmp_path, src):
    dbg = _device_asm(src, ["-DPSW_DEBUG"], tmp_path / "debug.s")
    rel = _device_asm(src, [], tmp_path / "release.s")
    assert "global_atomic_or" in dbg
    assert "global_atomic_or" not in rel
    for name, text in (("debug", dbg), ("release", rel)):
        m = SCALAR_WRITE.search(text)
        assert m is None, f"{src} ({name}): {m.group(0).strip()}"


def test_debug_library_exports_every_entry_point():
    from paged_sliding_window_amd import build
    lib = build.build_variant("debug", verbose=False)
    env = dict(os.environ, PSW_LIBRARY=lib)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        "tests/test_abi.py", "-k", "exports or version or debug_checks"],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, (r.stdout + r.stderr)[-3000:]
