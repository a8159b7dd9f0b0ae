"""Invariants of the generated gfx950 code that the kernels rely on.

No kernel spills registers to scratch beyond a stated budget.

The full-width latent decode kernel keeps its 256 output accumulators in AGPRs
that only its inline assembly touches; this holds only while the compiler
allocates no AGPR of its own in that kernel (its other values must stay below
256 VGPRs).  The check compiles the source to assembly and looks for AGPR
operands outside the inline-assembly regions.
"""
import os
import re
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(ROOT, "paged_sliding_window_amd", "csrc", "attention_decode.hip")


def _hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    return None


def _kernel_bodies(asm: str, prefix: str):
    # a kernel's code runs to its .Lfunc_end label: early returns put further
    # s_endpgm instructions inside the body
    for m in re.finditer(r"^(%s\w*):" % re.escape(prefix), asm, re.M):
        end = asm.index(".Lfunc_end", m.end())
        body = asm[m.end():end]
        yield m.group(1), body


@pytest.mark.skipif(_hipcc() is None, reason="hipcc not available")
def test_full_width_decode_leaves_agprs_to_inline_asm(tmp_path):
    import paged_sliding_window_amd.build as b
    out = tmp_path / "dec.s"
    cmd = [_hipcc(), *b.HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), "-S",
           "--cuda-device-only", SRC, "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    asm = out.read_text()
    bodies = list(_kernel_bodies(asm, "_ZN3psw18decode_full_kernel"))
    assert len(bodies) == 2, [n for n, _ in bodies]  # block-table variants
    for name, body in bodies:
        in_asm = False
        for line in body.split("\n"):
            t = line.strip()
            if t.startswith(";;#ASMSTART"):
                in_asm = True
                continue
            if t.startswith(";;#ASMEND"):
                in_asm = False
                continue
            if in_asm or t.startswith(";") or t.startswith("."):
                continue
            code = t.split(";")[0]
            assert not re.search(r"\ba\d+\b|\ba\[\d+", code), f"{name}: compiler AGPR use: {t}"
        assert "scratch_" not in body, f"{name}: register spills"
        # the whole kernel was searched: its main loop has the output MFMAs
        assert body.count("v_mfma") >= 16 and body.count("s_endpgm") >= 1, name
    # the kernel descriptors reserve all 256 AGPRs (the clobber of a255)
    assert len(re.findall(r"\.agpr_count:\s+256", asm)) >= 2


# VGPR spills allowed per kernel: the prefill with the fused cache write keeps
# two values live across its tile loop in scratch (written once before the loop,
# read once after it); every other kernel spills nothing.  A kernel spilling
# inside its loop pays scratch loads whose waits also drain its tile loads.
SPILL_BUDGET = {"prefill_attention_kernel": 4}


@pytest.mark.skipif(_hipcc() is None, reason="hipcc not available")
@pytest.mark.parametrize("src", ["attention_prefill.hip", "attention_decode.hip",
                                 "slot_mapping.hip", "kv_cache_write.hip", "lse_combine.hip",
                                 "vup_projection.hip", "tile_bounds.hip"])
def test_kernels_do_not_spill_registers(tmp_path, src):
    import paged_sliding_window_amd.build as b
    cmd = [_hipcc(), *b.HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), "-c",
           "--cuda-device-only", os.path.join(ROOT, "paged_sliding_window_amd", "csrc", src),
           "-o", str(tmp_path / "k.o"), "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    name, seen = None, 0
    for line in r.stderr.splitlines():
        m = re.search(r"remark: +(Function Name|VGPRs Spill): (\S+)", line)
        if not m:
            continue
        if m.group(1) == "Function Name":
            name = m.group(2)
            continue
        seen += 1
        budget = next((v for k, v in SPILL_BUDGET.items() if k in name), 0)
        assert int(m.group(2)) <= budget, f"{name}: {m.group(2)} VGPRs spilled"
    assert seen >= 1, "no kernel resource remarks"


def test_bench_refuses_more_than_one_gpu():
    """The bench measures one GPU; asking for more ends with a message and a
    non-zero status before any GPU work."""
    r = subprocess.run([os.environ.get("PYTHON", "python3"), os.path.join(ROOT, "bench.py"),
                        "--gpus", "2"], capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU only" in r.stdout + r.stderr
