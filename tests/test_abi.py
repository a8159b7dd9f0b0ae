"""C-ABI checks that need no GPU: the library is built, loads, exports every
function include/psw.h declares, and rejects bad arguments on the host before
touching the device."""
import ctypes
import os
import re

import pytest

import paged_sliding_window_amd as psw
from paged_sliding_window_amd._lib import (EXPORTS, PSW_ERR_INVALID, PSW_ERR_UNSUPPORTED, PSW_OK,
                                            PswAttnArgs)
from paged_sliding_window_amd.ops import (check_attention_shapes, check_combine_shapes,
                                          check_kv_write_shapes)


def _gpu_visible():
    import torch
    return torch.cuda.is_available()


# Cases that hand the library made-up device addresses rely on its host-side
# checks failing first.  Where a GPU is visible a regression in those checks
# would launch a kernel on such an address, so they run only without one.
no_gpu_only = pytest.mark.skipif(_gpu_visible(), reason="made-up device addresses: host-only "
                                 "check, skipped where a GPU is visible")

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "psw.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(psw_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = psw.load()
    names = declared_functions()
    assert names, "no declarations found"
    for n in names:
        assert hasattr(lib, n), n
        assert n in EXPORTS, f"{n} has no ctypes declaration"
    assert sorted(EXPORTS) == names


def test_version_and_status_strings():
    lib = psw.load()
    assert lib.psw_abi_version() == 8
    assert lib.psw_status_string(PSW_OK) == b"ok"
    assert lib.psw_status_string(PSW_ERR_INVALID) == b"invalid argument"


def test_debug_checks_need_a_debug_build():
    """psw_debug_take_failures: NULL is rejected; a build without PSW_DEBUG
    answers PSW_ERR_UNSUPPORTED with a zero mask, before touching the device."""
    from paged_sliding_window_amd import _lib
    lib = psw.load()
    assert lib.psw_debug_take_failures(None) == PSW_ERR_INVALID
    if "debug" not in os.path.basename(_lib.LIB_PATH):
        m = ctypes.c_uint32(7)
        assert lib.psw_debug_take_failures(ctypes.byref(m)) == PSW_ERR_UNSUPPORTED
        assert m.value == 0
        with pytest.raises(psw.PswError):
            psw.debug_take_failures()


def _args(**kw):
    a = PswAttnArgs()
    a.struct_size = ctypes.sizeof(PswAttnArgs)
    a.num_seqs, a.num_tokens, a.num_q_heads, a.num_kv_heads = 0, 0, 8, 2
    a.head_dim_qk = a.head_dim_v = 128
    a.block_size, a.block_table_stride, a.num_splits, a.scale = 16, 1, 1, 0.1
    a.chunk_lookback = -1
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def test_struct_size_matches_the_c_struct():
    lib = psw.load()
    assert lib.psw_swa_mm_attention(ctypes.byref(_args()), None) == PSW_OK   # nothing to launch
    bad = _args(struct_size=ctypes.sizeof(PswAttnArgs) - 4)
    assert lib.psw_swa_mm_attention(ctypes.byref(bad), None) == PSW_ERR_INVALID
    assert b"struct_size" in lib.psw_last_error()


@pytest.mark.parametrize("field,value", [
    ("num_q_heads", 7), ("block_size", 12), ("scale", 0.0), ("num_splits", 0),
    ("out_dtype", 9), ("num_tokens", -1), ("chunk_size", 0),
])
def test_attention_rejects_bad_scalars(field, value):
    kw = {field: value}
    if field == "chunk_size":
        kw["chunk_lookback"] = 1
    lib = psw.load()
    assert lib.psw_swa_mm_attention(ctypes.byref(_args(**kw)), None) == PSW_ERR_INVALID


def test_segmented_splits_need_a_prefill_shape():
    # v_cache NULL is the latent decode, which takes splits only as key ranges
    lib = psw.load()
    assert lib.psw_swa_mm_attention(ctypes.byref(_args(num_splits=2)), None) == PSW_ERR_UNSUPPORTED


def test_other_entry_points_reject_bad_scalars():
    lib = psw.load()
    assert lib.psw_slot_mapping(None, -1, None, 0, None, 1, 16, None, 0, None) == PSW_ERR_INVALID
    assert lib.psw_slot_mapping(None, 0, None, 5, None, 1, 16, None, 4, None) == PSW_ERR_INVALID
    assert lib.psw_slot_mapping(None, 0, None, 0, None, 1, 16, None, 0, None) == PSW_OK
    assert lib.psw_kv_cache_write(None, None, None, 0, 1, 12, 0, None, None, 0, None) == PSW_ERR_INVALID
    po = (ctypes.c_void_p * 1)()
    assert lib.psw_lse_combine(po, po, 0, 0, 1, 64, None, 0, None, None) == PSW_ERR_INVALID
    assert lib.psw_lse_combine(po, po, 65, 0, 1, 64, None, 0, None, None) == PSW_ERR_INVALID
    assert lib.psw_lse_combine(po, po, 1, 0, 1, 12, None, 0, None, None) == PSW_ERR_INVALID
    assert lib.psw_tile_bounds(ctypes.byref(_args()), 0, 16, 8, None, None, 0, None, None) == PSW_ERR_INVALID


def test_combine_vup_host_checks():
    # every case fails (or has no work) on the host: no pointer is dereferenced
    lib = psw.load()
    po = (ctypes.c_void_p * 17)()
    f = lib.psw_lse_combine_vup
    assert f(po, po, 0, 0, None, None, None, None, 1, 1, 512, 128, None) == PSW_ERR_INVALID
    assert f(po, po, 17, 0, None, None, None, None, 1, 1, 512, 128, None) == PSW_ERR_INVALID
    assert f(po, po, 2, 3, None, None, None, None, 1, 1, 512, 128, None) == PSW_ERR_INVALID
    assert f(po, po, 2, 0, None, None, None, None, -1, 1, 512, 128, None) == PSW_ERR_INVALID
    assert f(po, po, 2, 0, None, None, None, None, 1, 1, 96, 128, None) == PSW_ERR_UNSUPPORTED
    assert f(po, po, 2, 0, None, None, None, None, 1, 1, 512, 96, None) == PSW_ERR_UNSUPPORTED
    # NULL partials with work to do
    assert f(po, po, 2, 0, None, None, None, None, 1, 1, 512, 128, None) == PSW_ERR_INVALID
    # no tokens: nothing to do, nothing launched
    assert f(po, po, 2, 0, None, None, None, None, 0, 1, 512, 128, None) == PSW_OK


def _latent_decode_args(**kw):
    base = dict(num_seqs=4, num_tokens=4, num_q_heads=128, num_kv_heads=1, head_dim_qk=576,
                head_dim_v=512, block_size=64)
    return _args(**{**base, **kw})


def test_workspace_size_query():
    lib = psw.load()
    n = ctypes.c_int64(-1)
    # separate K and V caches (prefill kernels): no workspace
    assert lib.psw_attention_workspace_size(ctypes.byref(_args(num_seqs=1, num_tokens=8)),
                                            ctypes.byref(n)) == PSW_OK
    assert n.value == 0
    # latent decode: prefix + pieces, growing with the number of (token, split) items
    assert lib.psw_attention_workspace_size(ctypes.byref(_latent_decode_args()),
                                            ctypes.byref(n)) == PSW_OK
    one = n.value
    assert one > 0 and one % 4 == 0
    assert lib.psw_attention_workspace_size(
        ctypes.byref(_latent_decode_args(num_splits=8, key_ranges=1)), ctypes.byref(n)) == PSW_OK
    assert n.value >= one
    assert lib.psw_attention_workspace_size(ctypes.byref(_args()), None) == PSW_ERR_INVALID


@no_gpu_only
def test_latent_decode_rejects_missing_or_small_workspace():
    lib = psw.load()
    fake = 0x100000  # never dereferenced: the call fails on the host
    ptrs = dict(q=fake, k_cache=fake, block_table=fake, query_start_loc=fake, seq_lens=fake,
                out=fake)
    a = _latent_decode_args(**ptrs)
    assert lib.psw_swa_mm_attention(ctypes.byref(a), None) == PSW_ERR_INVALID
    assert b"workspace" in lib.psw_last_error()
    n = ctypes.c_int64()
    assert lib.psw_attention_workspace_size(ctypes.byref(a), ctypes.byref(n)) == PSW_OK
    small = _latent_decode_args(workspace=fake, workspace_bytes=n.value - 1, **ptrs)
    assert lib.psw_swa_mm_attention(ctypes.byref(small), None) == PSW_ERR_INVALID
    misaligned = _latent_decode_args(workspace=fake + 16, workspace_bytes=n.value, **ptrs)
    assert lib.psw_swa_mm_attention(ctypes.byref(misaligned), None) == PSW_ERR_INVALID


@no_gpu_only
def test_two_stream_decode_checks_both_calls_before_enqueuing():
    # every failure below is found on the host; no pointer is dereferenced
    lib = psw.load()
    fake = 0x100000
    ptrs = dict(q=fake, k_cache=fake, block_table=fake, query_start_loc=fake, seq_lens=fake,
                out=fake, lse=fake, key_ranges=fake)
    n = ctypes.c_int64()
    probe = _latent_decode_args(num_splits=2, **ptrs)
    assert lib.psw_attention_workspace_size(ctypes.byref(probe), ctypes.byref(n)) == PSW_OK
    ws = dict(workspace=fake, workspace_bytes=n.value)
    hist = _latent_decode_args(num_splits=2, **ptrs, **ws)
    cur = _latent_decode_args(num_splits=1, **ptrs, **ws)

    def call(h, c, out=fake, out_dtype=0):
        return lib.psw_decode_two_streams(ctypes.byref(h), ctypes.byref(c), out, out_dtype, None,
                                          None, None)
    other = dict(ptrs, lse=None)
    assert call(hist, _latent_decode_args(num_splits=1, **other, **ws)) == PSW_ERR_INVALID
    assert b"LSE" in lib.psw_last_error()
    assert call(hist, _latent_decode_args(num_splits=1, num_q_heads=64, **ptrs, **ws)) \
        == PSW_ERR_INVALID
    assert b"disagree" in lib.psw_last_error()
    assert call(hist, _latent_decode_args(num_splits=1, out_dtype=1, **ptrs, **ws)) \
        == PSW_ERR_INVALID
    assert call(hist, cur, out=None) == PSW_ERR_INVALID
    assert call(hist, cur, out_dtype=7) == PSW_ERR_INVALID
    big = dict(workspace=fake, workspace_bytes=1 << 40)
    assert call(_latent_decode_args(num_splits=40, **ptrs, **big),
                _latent_decode_args(num_splits=30, **ptrs, **big)) == PSW_ERR_INVALID
    assert b"partials" in lib.psw_last_error()
    no_ws = _latent_decode_args(num_splits=1, **ptrs)
    assert call(hist, no_ws) == PSW_ERR_INVALID
    assert b"workspace" in lib.psw_last_error()
    assert call(hist, _latent_decode_args(num_splits=1, num_seqs=0, **ptrs, **ws)) == PSW_ERR_INVALID
    assert b"no sequences" in lib.psw_last_error()
    # an empty batch has nothing to enqueue
    empty = _args()
    assert call(empty, empty) == PSW_OK


def test_fp16_is_a_known_dtype():
    lib = psw.load()
    assert lib.psw_swa_mm_attention(ctypes.byref(_args(out_dtype=2)), None) == PSW_OK
    assert lib.psw_swa_mm_attention(ctypes.byref(_args(out_dtype=3)), None) == PSW_ERR_INVALID
    po = (ctypes.c_void_p * 1)()
    # no rows: accepted for every partial / output type pair, nothing launched
    for pd in (0, 1, 2):
        for od in (0, 1, 2):
            assert lib.psw_lse_combine(po, po, 1, pd, 0, 64, None, od, None, None) == PSW_OK
    assert lib.psw_lse_combine(po, po, 1, 3, 0, 64, None, 0, None, None) == PSW_ERR_INVALID


# ---- wrapper shape checks (host logic of ops.py; shapes only) ---------------

ATTN_OK = dict(q=(10, 8, 128), k_cache=(20, 16, 2, 128), v_cache=(20, 16, 2, 128),
               block_table=(3, 7), qsl_numel=4, seq_lens_numel=3, mm_ranges=(3, 2, 2),
               key_ranges=None, head_dim_v=None)


def test_attention_shapes_accepted():
    check_attention_shapes(**ATTN_OK)
    check_attention_shapes(**dict(ATTN_OK, key_ranges=(2, 3, 2), mm_ranges=None))
    # latent cache: V is the first head_dim_v columns of K
    check_attention_shapes(**dict(ATTN_OK, q=(4, 128, 576), k_cache=(9, 64, 1, 576),
                                  v_cache=None, head_dim_v=512))


@pytest.mark.parametrize("change", [
    dict(q=(10, 8, 64)),                       # q head dim != cache head dim
    dict(q=(10, 7, 128)),                      # query heads not a multiple of KV heads
    dict(v_cache=(20, 16, 1, 128)),            # V heads differ from K heads
    dict(v_cache=(21, 16, 2, 128)),            # V blocks differ from K blocks
    dict(seq_lens_numel=2),                    # seq_lens shorter than num_seqs
    dict(block_table=(2, 7)),                  # fewer table rows than sequences
    dict(mm_ranges=(2, 2, 2)),                 # ranges for the wrong number of sequences
    dict(mm_ranges=(3, 2, 3)),                 # ranges not (start, end) pairs
    dict(key_ranges=(2, 4, 2)),                # key ranges for the wrong number of sequences
    dict(key_ranges=(2, 3)),                   # key ranges not 3-D
    dict(v_cache=None, head_dim_v=None),       # latent cache without head_dim_v
    dict(v_cache=None, head_dim_v=129),        # latent V wider than the row
    dict(qsl_numel=0),                         # no query_start_loc entries
], ids=lambda d: ",".join(d))
def test_attention_shape_mismatches_raise(change):
    with pytest.raises(ValueError):
        check_attention_shapes(**dict(ATTN_OK, **change))


def test_kv_write_shapes():
    check_kv_write_shapes((5, 2, 64), (5, 2, 32), 5, (9, 16, 2, 64), (9, 16, 2, 32))
    check_kv_write_shapes((5, 1, 576), None, 8, (9, 64, 1, 576), None)
    bad = [
        ((5, 2, 64), (5, 2, 32), 5, (9, 16, 1, 64), (9, 16, 2, 32)),   # K heads
        ((5, 2, 64), (5, 2, 32), 5, (9, 16, 2, 32), (9, 16, 2, 32)),   # K dim
        ((5, 2, 64), (4, 2, 32), 5, (9, 16, 2, 64), (9, 16, 2, 32)),   # V rows
        ((5, 2, 64), (5, 1, 32), 5, (9, 16, 2, 64), (9, 16, 2, 32)),   # V heads
        ((5, 2, 64), (5, 2, 32), 5, (9, 16, 2, 64), (9, 16, 2, 16)),   # V dim
        ((5, 2, 64), (5, 2, 32), 5, (9, 16, 2, 64), (8, 16, 2, 32)),   # V blocks
        ((5, 2, 64), (5, 2, 32), 4, (9, 16, 2, 64), (9, 16, 2, 32)),   # slots too short
        ((5, 2, 64), None, 5, (9, 16, 2, 64), (9, 16, 2, 32)),         # V cache without V
    ]
    for args in bad:
        with pytest.raises(ValueError):
            check_kv_write_shapes(*args)


def test_combine_shapes():
    check_combine_shapes(10, 64, 640, 10)
    check_combine_shapes(10, 64, 640, None)
    with pytest.raises(ValueError):
        check_combine_shapes(10, 64, 639, None)
    with pytest.raises(ValueError):
        check_combine_shapes(10, 64, 640, 9)


@no_gpu_only
def test_noalloc_rejects_calls_beyond_its_scratch():
    """The allocation-free entry point checks its workspace need against the
    66 MiB scratch on the host: a latent decode of 4 tokens x 120,000 splits
    (480,000 items) is refused before anything is launched, 4 x 100,000 fits;
    a prefill call needs no scratch."""
    lib = psw.load()
    fake = 0x100000
    ptrs = dict(q=fake, k_cache=fake, block_table=fake, query_start_loc=fake, seq_lens=fake,
                out=fake, lse=fake, key_ranges=fake)
    big = _latent_decode_args(num_splits=120000, **ptrs)
    assert lib.psw_swa_mm_attention_noalloc(ctypes.byref(big), None) == PSW_ERR_INVALID
    assert b"scratch" in lib.psw_last_error()
    n = ctypes.c_int64()
    ok = _latent_decode_args(num_splits=100000, **ptrs)
    assert lib.psw_attention_workspace_size(ctypes.byref(ok), ctypes.byref(n)) == PSW_OK
    assert 0 < n.value <= 66 << 20
    assert lib.psw_attention_workspace_size(ctypes.byref(big), ctypes.byref(n)) == PSW_OK
    assert n.value > 66 << 20
    # the empty call is accepted with nothing to do
    assert lib.psw_swa_mm_attention_noalloc(ctypes.byref(_args()), None) == PSW_OK
