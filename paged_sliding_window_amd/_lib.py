"""ctypes declarations of libpsw.so (the C ABI in include/psw.h).

The library is loaded after torch so that it binds to the HIP runtime torch has
already loaded.  A missing library is an error: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (loads the HIP runtime libpsw.so links against)

# PSW_LIBRARY selects another build of the same library (the address-sanitizer
# and PSW_DEBUG variants that build.build_variant makes); unset, the in-tree one.
LIB_PATH = os.environ.get("PSW_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                         "libpsw.so")

PSW_OK = 0
PSW_ERR_INVALID = -1
PSW_ERR_UNSUPPORTED = -2
PSW_ERR_HIP = -3
PSW_BF16 = 0
PSW_F32 = 1
PSW_F16 = 2

_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_vp = ctypes.c_void_p


class PswAttnArgs(ctypes.Structure):
    """Mirror of ``psw_attn_args`` (same field order; C alignment rules)."""

    _fields_ = [
        ("struct_size", _i32),
        ("q", _vp), ("k_cache", _vp), ("v_cache", _vp),
        ("block_table", _vp), ("query_start_loc", _vp), ("seq_lens", _vp),
        ("mm_ranges", _vp), ("key_ranges", _vp),
        ("out", _vp), ("lse", _vp),
        ("num_seqs", _i32), ("num_tokens", _i32), ("num_q_heads", _i32),
        ("num_kv_heads", _i32), ("head_dim_qk", _i32), ("head_dim_v", _i32),
        ("block_size", _i32), ("block_table_stride", _i32), ("max_mm_ranges", _i32),
        ("window", _i32), ("causal", _i32), ("chunk_size", _i32), ("chunk_lookback", _i32),
        ("num_splits", _i32), ("out_dtype", _i32),
        ("scale", ctypes.c_float),
        ("workspace", _vp), ("workspace_bytes", _i64),
    ]


EXPORTS = {
    "psw_abi_version": (_i32, []),
    "psw_status_string": (ctypes.c_char_p, [_i32]),
    "psw_last_error": (ctypes.c_char_p, []),
    "psw_slot_mapping": (_i32, [_vp, _i32, _vp, _i32, _vp, _i32, _i32, _vp, _i32, _vp]),
    "psw_slot_mapping_cp": (_i32, [_vp, _i32, _vp, _i32, _vp, _i32, _i32, _i32, _i32, _i32, _i32,
                                   _i32, _vp, _i32, _vp]),
    "psw_kv_cache_write": (_i32, [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _vp, _vp, _i64, _vp]),
    "psw_swa_mm_attention": (_i32, [ctypes.POINTER(PswAttnArgs), _vp]),
    "psw_swa_mm_attention_noalloc": (_i32, [ctypes.POINTER(PswAttnArgs), _vp]),
    "psw_swa_mm_attention_kv_write": (_i32, [ctypes.POINTER(PswAttnArgs), _vp, _vp, _vp, _i64,
                                             _vp]),
    "psw_attention_workspace_size": (_i32, [ctypes.POINTER(PswAttnArgs), ctypes.POINTER(_i64)]),
    "psw_lse_combine": (_i32, [ctypes.POINTER(_vp), ctypes.POINTER(_vp), _i32, _i32, _i64, _i32,
                               _vp, _i32, _vp, _vp]),
    "psw_decode_two_streams": (_i32, [ctypes.POINTER(PswAttnArgs), ctypes.POINTER(PswAttnArgs), _vp,
                                      _i32, _vp, _vp, _vp]),
    "psw_vup_projection": (_i32, [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _vp]),
    "psw_lse_combine_vup": (_i32, [ctypes.POINTER(_vp), ctypes.POINTER(_vp), _i32, _i32, _vp, _vp,
                                   _vp, _vp, _i32, _i32, _i32, _i32, _vp]),
    "psw_tile_bounds": (_i32, [ctypes.POINTER(PswAttnArgs), _i32, _i32, _i32, _vp, _vp, _i32,
                               _vp, _vp]),
    "psw_debug_take_failures": (_i32, [ctypes.POINTER(ctypes.c_uint32)]),
}

_lib = None


class PswError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"psw status {status}: {detail}")
        self.status = status


def open_library(path: str) -> ctypes.CDLL:
    """A handle on the library file at `path` with every export's signature set
    (load() keeps the process's one handle; this opens another build beside it)."""
    lib = ctypes.CDLL(path)
    for name, (res, args) in EXPORTS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


def load() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run paged_sliding_window_amd/build.py "
                              "(or __graft_entry__.build()) first")
        _lib = open_library(LIB_PATH)
    return _lib


def check(status: int) -> None:
    if status != PSW_OK:
        lib = load()
        detail = lib.psw_last_error().decode() or lib.psw_status_string(status).decode()
        raise PswError(status, detail)
