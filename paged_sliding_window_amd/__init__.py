"""Paged sliding-window attention with window-clamped image ranges for MI355X.

Thin torch-facing marshalling over the C ABI of libpsw.so (include/psw.h):
every step of the path runs in the library's HIP kernels; this module only
checks tensor metadata and passes device pointers and the current stream.
"""
from .ops import (  # noqa: F401
    attention_workspace_size,
    debug_take_failures,
    decode_two_streams,
    kv_cache_write,
    lse_combine,
    lse_combine_vup,
    slot_mapping,
    slot_mapping_cp,
    swa_mm_attention,
    swa_mm_attention_kv_write,
    swa_mm_attention_noalloc,
    tile_bounds,
    vup_projection,
)
from ._lib import LIB_PATH, PswError, load  # noqa: F401
