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
    assert lib.psw_abi_version() == 4
    assert lib.psw_status_string(PSW_OK) == b"ok"
    assert lib.psw_status_string(PSW_ERR_INVALID) == b"invalid argument"


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
