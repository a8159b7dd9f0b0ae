"""The PSW_DEBUG build on the GPU.

The debug library (built beside libpsw.so by the build step) is opened as a
second handle and swapped in for the calls under test.  On the workloads and
on random small cases every internal check must hold (an empty failure mask),
and the debug build must compute exactly what the release build computes (the
checks add instructions, not arithmetic).  One planted case shows that a failed
check is recorded: a KV-cache slot one past the cache, which both builds skip
(the cache is a view whose allocation has spare rows, so even a write there
would stay inside memory the test owns; the test checks they are untouched).
"""
import contextlib
import ctypes
import os

import numpy as np
import pytest
import torch

import paged_sliding_window_amd as psw
from paged_sliding_window_amd import _lib, build
from tests.gpu_setup import DecodeStep, GpuWorkload, bits_to_bf16, i32, i64
from workloads import make_config, make_small_case
from workloads.synth import make_slot_batch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def debug_lib():
    path = build.variant_path("debug")
    assert os.path.exists(path), f"{path} is not built (__graft_entry__.build() builds it)"
    lib = _lib.open_library(path)
    m = ctypes.c_uint32(0)
    assert lib.psw_debug_take_failures(ctypes.byref(m)) == _lib.PSW_OK, "not a PSW_DEBUG build"
    return lib


@contextlib.contextmanager
def using(lib):
    release = psw.load()
    _lib._lib = lib
    try:
        yield
    finally:
        torch.cuda.synchronize()
        _lib._lib = release


def failures(lib):
    with using(lib):
        return psw.debug_take_failures()


def same_bits(a, b):
    if a.dtype in (torch.bfloat16, torch.float16):
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    return torch.equal(a.view(torch.int32), b.view(torch.int32))


def _attention_both(lib, w, **kw):
    gw = GpuWorkload(w)
    ref = gw.attention(**kw)
    with using(lib):
        gd = GpuWorkload(w)          # cache filled through the debug slot mapping and write
        got = gd.attention(**kw)
    assert same_bits(gd.k_cache, gw.k_cache)
    return ref, got


@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_debug_prefill_workloads(debug_lib, cfg):
    assert failures(debug_lib) == 0
    (o, l), (od, ld) = _attention_both(debug_lib, make_config(cfg))
    assert failures(debug_lib) == 0
    assert same_bits(o, od) and same_bits(l, ld)


@pytest.mark.parametrize("seed", range(6))
def test_debug_prefill_random_splits(debug_lib, seed):
    """Random small cases, unsplit, as segmented splits and as key ranges."""
    rng = np.random.default_rng(700 + seed)
    d = int(rng.choice([64, 128, 256]))
    hkv = int(rng.choice([1, 2]))
    qpk = int(rng.choice([1, 2, 3, 8]))
    w = make_small_case(700 + seed, num_seqs=int(rng.integers(1, 5)), max_len=700,
                        hq=hkv * qpk, hkv=hkv, d=d, block_size=int(rng.choice([1, 16, 64])))
    assert failures(debug_lib) == 0
    for kw in (dict(), dict(num_splits=3, out_dtype=torch.float32)):
        (o, l), (od, ld) = _attention_both(debug_lib, w, **kw)
        assert failures(debug_lib) == 0, kw
        assert same_bits(o, od) and same_bits(l, ld), kw
    L = np.asarray(w.seq_lens)
    kr = np.stack([np.stack([np.zeros_like(L), L // 2], 1),
                   np.stack([L // 2, L], 1)]).astype(np.int32)
    (o, l), (od, ld) = _attention_both(debug_lib, w, key_ranges=kr, out_dtype=torch.float32)
    assert failures(debug_lib) == 0
    assert same_bits(o, od) and same_bits(l, ld)


@pytest.mark.parametrize("splits", [1, 8])
def test_debug_latent_decode(debug_lib, splits):
    """The 64-request latent decode step (history splits + current key, the
    combine and the projection) through both builds."""
    w = make_config(5, decode_splits=splits)
    ds = DecodeStep(w)
    ds.run()
    torch.cuda.synchronize()
    assert failures(debug_lib) == 0
    with using(debug_lib):
        dd = DecodeStep(w)
        dd.run()
    assert failures(debug_lib) == 0
    for a, b in ((ds.part_o, dd.part_o), (ds.part_l, dd.part_l), (ds.out, dd.out),
                 (ds.out_lse, dd.out_lse), (ds.vup_out, dd.vup_out)):
        assert same_bits(a, b)


def test_debug_slot_mapping(debug_lib):
    """Many requests (with empty ones and invalid positions mixed in)."""
    qsl, pos, bt = make_slot_batch(3000, 0, 700, 16, 11)
    pos = pos.copy()
    pos[::97] = -5
    args = (i32(qsl), i64(pos), i32(bt), 16, int(qsl[-1]) + 64)
    ref = psw.slot_mapping(*args)
    assert failures(debug_lib) == 0
    with using(debug_lib):
        got = psw.slot_mapping(*args)
    assert failures(debug_lib) == 0
    assert torch.equal(ref, got)


@pytest.mark.parametrize("which", ["release", "debug"])
def test_kv_write_skips_a_slot_past_the_cache(debug_lib, which):
    """Slots 0 and 1 are written; slot num_slots (one past the cache) is skipped
    by both builds, and the debug build records check 17 once."""
    B, hkv, d, nb = 16, 2, 64, 4
    store = torch.zeros((nb + 2, B, hkv, d), dtype=torch.bfloat16, device="cuda")
    cache = store[:nb]                      # the cache the call sees: nb * B slots
    rows = torch.arange(3 * hkv * d, device="cuda", dtype=torch.float32).reshape(3, hkv, d)
    k_new = (rows + 1).to(torch.bfloat16)
    slots = torch.tensor([0, 1, nb * B], dtype=torch.int32, device="cuda")
    lib = debug_lib if which == "debug" else psw.load()
    assert failures(debug_lib) == 0
    with using(lib):
        psw.kv_cache_write(k_new, None, slots, cache, None)
    flat = store.view(-1, hkv, d)
    assert torch.equal(flat[0], k_new[0]) and torch.equal(flat[1], k_new[1])
    assert not flat[2:].any(), "a slot outside the cache was written"
    mask = failures(debug_lib)
    assert mask == ((1 << 17) if which == "debug" else 0)
    assert failures(debug_lib) == 0     # taking the mask cleared it


def test_debug_random_prefill_sweep(debug_lib):
    """60 random small prefill cases (head dims 64-256, 1-4 KV heads, 1-16
    queries per KV head, cache blocks of 1-128 keys, unsplit or segmented):
    every check holds, the two builds agree bit for bit, and the unsplit
    outputs match the oracle."""
    from tests.gpu_setup import assert_close, assert_lse_close, oracle_rows
    assert failures(debug_lib) == 0
    for i in range(60):
        rng = np.random.default_rng(5000 + i)
        d = int(rng.choice([64, 128, 256]))
        hkv = int(rng.choice([1, 2, 4]))
        qpk = int(rng.choice([1, 2, 3, 4, 6, 8, 16]))
        bs = int(rng.choice([1, 2, 8, 16, 32, 64, 128]))
        w = make_small_case(5000 + i, num_seqs=int(rng.integers(1, 6)),
                            max_len=int(rng.choice([64, 300, 900])), hq=hkv * qpk, hkv=hkv, d=d,
                            block_size=bs)
        splits = int(rng.choice([1, 1, 2, 3]))
        kw = dict(num_splits=splits, out_dtype=torch.float32) if splits > 1 else {}
        (o, l), (od, ld) = _attention_both(debug_lib, w, **kw)
        assert failures(debug_lib) == 0, f"case {i}"
        assert same_bits(o, od) and same_bits(l, ld), f"case {i}"
        if splits == 1:
            out, lse = o.float().cpu().numpy(), l.cpu().numpy()
            for r in range(w.num_seqs):
                s0, ql = int(w.query_start_loc[r]), int(w.query_lens[r])
                ref_o, ref_l = oracle_rows(w, r)
                assert_close(out[s0:s0 + ql], ref_o, f"case {i} seq {r}")
                assert_lse_close(lse[s0:s0 + ql], ref_l, f"case {i} seq {r} lse")


@pytest.mark.parametrize("cfg", [2, 3])
def test_debug_fused_cache_write(debug_lib, cfg):
    """The prefill with the fused cache write through both builds (workload 2
    as the bench times it, workload 3 with cached context); then one slot past
    the cache, which both skip and the debug build records as check 4."""
    from tests.test_gpu_fused_kv_write import FusedCase
    case = FusedCase(make_config(cfg), spare_blocks=1)
    ref = case.fused()
    assert failures(debug_lib) == 0
    with using(debug_lib):
        got = case.fused()
    assert failures(debug_lib) == 0
    for a, b in zip(ref, got):
        assert same_bits(a, b)
    slots = case.slots.clone()
    slots[0] = case.nb * case.w.block_size
    with using(debug_lib):
        k, v, _, _ = case.fused(slots=slots)
    assert failures(debug_lib) == 1 << 4
    assert not k[case.nb:].any() and not v[case.nb:].any()
