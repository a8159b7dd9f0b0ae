"""Torch-tensor wrappers with the C ABI's names (argument marshalling only)."""
from __future__ import annotations

import ctypes
from typing import Optional, Sequence

import torch

from . import _lib
from ._lib import PSW_BF16, PSW_F16, PSW_F32, PswAttnArgs, check, load

# torch element types of outputs and partials -> psw_dtype codes
_DTYPES = {torch.bfloat16: PSW_BF16, torch.float32: PSW_F32, torch.float16: PSW_F16}


def _dtype_code(dt: torch.dtype, what: str) -> int:
    if dt not in _DTYPES:
        raise TypeError(f"{what} must be bfloat16, float16 or float32, got {dt}")
    return _DTYPES[dt]


# ---- shape consistency (host only; raise before anything is enqueued) -------

def check_kv_write_shapes(k_new, v_new, slots_numel, k_cache, v_cache) -> None:
    """k_new [N, Hkv, Dk] and v_new [N, Hkv, Dv] (or None) against the caches
    [num_blocks, B, Hkv, Dk] / [num_blocks, B, Hkv, Dv]; arguments are shapes."""
    k_new, k_cache = tuple(k_new), tuple(k_cache)
    if len(k_new) != 3 or len(k_cache) != 4:
        raise ValueError(f"k_new {k_new} must be 3-D and k_cache {k_cache} 4-D")
    if k_cache[2:] != k_new[1:]:
        raise ValueError(f"k_cache heads/dim {k_cache[2:]} differ from k_new's {k_new[1:]}")
    if (v_new is None) != (v_cache is None):
        raise ValueError("v_new and v_cache must both be given or both be None")
    if v_new is not None:
        v_new, v_cache = tuple(v_new), tuple(v_cache)
        if len(v_new) != 3 or len(v_cache) != 4:
            raise ValueError(f"v_new {v_new} must be 3-D and v_cache {v_cache} 4-D")
        if v_new[:2] != k_new[:2]:
            raise ValueError(f"v_new rows/heads {v_new[:2]} differ from k_new's {k_new[:2]}")
        if v_cache[2:] != v_new[1:]:
            raise ValueError(f"v_cache heads/dim {v_cache[2:]} differ from v_new's {v_new[1:]}")
        if v_cache[:2] != k_cache[:2]:
            raise ValueError(f"v_cache blocks {v_cache[:2]} differ from k_cache's {k_cache[:2]}")
    if slots_numel < k_new[0]:
        raise ValueError("slot_mapping shorter than the new rows")


def check_attention_shapes(q, k_cache, v_cache, block_table, qsl_numel, seq_lens_numel,
                           mm_ranges, key_ranges, head_dim_v) -> None:
    """Shapes of one attention call (tuples; v_cache, mm_ranges, key_ranges may
    be None): every extent the kernels index with must agree."""
    q, k_cache, block_table = tuple(q), tuple(k_cache), tuple(block_table)
    num_seqs = qsl_numel - 1
    if num_seqs < 0:
        raise ValueError("query_start_loc needs num_seqs + 1 >= 1 entries")
    if len(q) != 3 or len(k_cache) != 4 or len(block_table) != 2:
        raise ValueError("q must be 3-D, k_cache 4-D and block_table 2-D")
    if k_cache[3] != q[2]:
        raise ValueError(f"k_cache head dim {k_cache[3]} differs from q's {q[2]}")
    if k_cache[2] < 1 or q[1] % k_cache[2] != 0:
        raise ValueError(f"{q[1]} query heads are not a multiple of {k_cache[2]} KV heads")
    if v_cache is not None:
        v_cache = tuple(v_cache)
        if len(v_cache) != 4 or v_cache[:3] != k_cache[:3]:
            raise ValueError(f"v_cache {v_cache} does not match k_cache {k_cache} in blocks, "
                             "block size and heads")
    elif head_dim_v is None or not (0 < head_dim_v <= k_cache[3]):
        raise ValueError("a latent cache (v_cache None) needs 0 < head_dim_v <= its row width")
    if seq_lens_numel != num_seqs:
        raise ValueError(f"seq_lens has {seq_lens_numel} entries for {num_seqs} sequences")
    if block_table[0] < num_seqs:
        raise ValueError(f"block_table has {block_table[0]} rows for {num_seqs} sequences")
    if mm_ranges is not None:
        mm_ranges = tuple(mm_ranges)
        if len(mm_ranges) != 3 or mm_ranges[0] != num_seqs or mm_ranges[2] != 2:
            raise ValueError(f"mm_ranges {mm_ranges} must be [num_seqs={num_seqs}, max, 2]")
    if key_ranges is not None:
        key_ranges = tuple(key_ranges)
        if len(key_ranges) != 3 or key_ranges[1:] != (num_seqs, 2):
            raise ValueError(f"key_ranges {key_ranges} must be [splits, num_seqs={num_seqs}, 2]")


def check_combine_shapes(rows, dv, out_numel, out_lse_numel) -> None:
    if out_numel != rows * dv:
        raise ValueError(f"out holds {out_numel} elements, the merge writes {rows} x {dv}")
    if out_lse_numel is not None and out_lse_numel != rows:
        raise ValueError(f"out_lse holds {out_lse_numel} elements for {rows} rows")


def _stream(stream=None) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, ndim: Optional[int] = None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must live on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {t.dim()}")


def slot_mapping(query_start_loc: torch.Tensor, positions: torch.Tensor, block_table: torch.Tensor,
                 block_size: int, max_num_tokens: int, out: Optional[torch.Tensor] = None,
                 stream=None) -> torch.Tensor:
    _need(query_start_loc, "query_start_loc", torch.int32, 1)
    _need(positions, "positions", torch.int64, 1)
    _need(block_table, "block_table", torch.int32, 2)
    if block_table.shape[0] < query_start_loc.numel() - 1:
        raise ValueError("block_table has fewer rows than requests")
    if out is None:
        out = torch.empty(max_num_tokens, dtype=torch.int32, device=positions.device)
    _need(out, "out", torch.int32, 1)
    if out.numel() < max_num_tokens:
        raise ValueError("out is smaller than max_num_tokens")
    check(load().psw_slot_mapping(_ptr(query_start_loc), query_start_loc.numel() - 1,
                                  _ptr(positions), positions.numel(), _ptr(block_table),
                                  block_table.shape[1], int(block_size), _ptr(out),
                                  int(max_num_tokens), _stream(stream)))
    return out


def slot_mapping_cp(query_start_loc: torch.Tensor, positions: torch.Tensor,
                    block_table: torch.Tensor, block_size: int, max_num_tokens: int, *,
                    kv_cache_block_size: Optional[int] = None, cp_world_size: int = 1,
                    cp_rank: int = 0, cp_interleave: int = 1, circular: bool = False,
                    out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Slot mapping of one context-parallel rank, or of a circular cache
    (psw_slot_mapping_cp); kv_cache_block_size defaults to block_size."""
    _need(query_start_loc, "query_start_loc", torch.int32, 1)
    _need(positions, "positions", torch.int64, 1)
    _need(block_table, "block_table", torch.int32, 2)
    if block_table.shape[0] < query_start_loc.numel() - 1:
        raise ValueError("block_table has fewer rows than requests")
    if out is None:
        out = torch.empty(max_num_tokens, dtype=torch.int32, device=positions.device)
    _need(out, "out", torch.int32, 1)
    if out.numel() < max_num_tokens:
        raise ValueError("out is smaller than max_num_tokens")
    kvb = block_size if kv_cache_block_size is None else kv_cache_block_size
    check(load().psw_slot_mapping_cp(_ptr(query_start_loc), query_start_loc.numel() - 1,
                                     _ptr(positions), positions.numel(), _ptr(block_table),
                                     block_table.shape[1], int(block_size), int(kvb),
                                     int(cp_world_size), int(cp_rank), int(cp_interleave),
                                     int(bool(circular)), _ptr(out), int(max_num_tokens),
                                     _stream(stream)))
    return out


def kv_cache_write(k_new: torch.Tensor, v_new: Optional[torch.Tensor], slots: torch.Tensor,
                   k_cache: torch.Tensor, v_cache: Optional[torch.Tensor], stream=None) -> None:
    """k_new [N, Hkv, Dk] bf16 -> k_cache [num_blocks, block_size, Hkv, Dk] (V likewise)."""
    _need(k_new, "k_new", torch.bfloat16, 3)
    _need(slots, "slot_mapping", torch.int32, 1)
    _need(k_cache, "k_cache", torch.bfloat16, 4)
    n, hkv, dk = k_new.shape
    dv = 0
    if v_new is not None:
        _need(v_new, "v_new", torch.bfloat16, 3)
        dv = v_new.shape[2]
    if v_cache is not None:
        _need(v_cache, "v_cache", torch.bfloat16, 4)
    check_kv_write_shapes(k_new.shape, None if v_new is None else v_new.shape, slots.numel(),
                          k_cache.shape, None if v_cache is None else v_cache.shape)
    num_slots = k_cache.shape[0] * k_cache.shape[1]
    check(load().psw_kv_cache_write(_ptr(k_new), _ptr(v_new), _ptr(slots), n, hkv, dk, dv,
                                    _ptr(k_cache), _ptr(v_cache), num_slots, _stream(stream)))


def _attn_args(q, k_cache, v_cache, block_table, query_start_loc, seq_lens, *, scale, window,
               causal, chunk_size, chunk_lookback, mm_ranges, key_ranges, out, lse, head_dim_v,
               out_dtype, num_splits) -> PswAttnArgs:
    a = PswAttnArgs()
    a.struct_size = ctypes.sizeof(PswAttnArgs)
    a.q, a.k_cache, a.v_cache = _ptr(q), _ptr(k_cache), _ptr(v_cache)
    a.block_table, a.query_start_loc, a.seq_lens = _ptr(block_table), _ptr(query_start_loc), _ptr(seq_lens)
    a.mm_ranges, a.key_ranges = _ptr(mm_ranges), _ptr(key_ranges)
    a.out, a.lse = _ptr(out), _ptr(lse)
    a.num_seqs = query_start_loc.numel() - 1
    a.num_tokens = q.shape[0] if q is not None else 0
    a.num_q_heads = q.shape[1] if q is not None else 1
    a.num_kv_heads = k_cache.shape[2] if k_cache is not None else 1
    a.head_dim_qk = q.shape[2] if q is not None else 0
    a.head_dim_v = head_dim_v
    a.block_size = k_cache.shape[1] if k_cache is not None else 1
    a.block_table_stride = block_table.shape[1] if block_table is not None else 1
    a.max_mm_ranges = mm_ranges.shape[1] if mm_ranges is not None else 0
    a.window, a.causal = int(window), int(bool(causal))
    a.chunk_size, a.chunk_lookback = int(chunk_size), int(chunk_lookback)
    a.num_splits = int(num_splits)
    a.out_dtype = out_dtype
    a.scale = float(scale)
    return a


def _prepare_attention(q, k_cache, v_cache, block_table, query_start_loc, seq_lens, *, scale,
                       window, causal, chunk_size, chunk_lookback, mm_ranges, key_ranges,
                       head_dim_v, out, lse, out_dtype, return_lse, num_splits, workspace,
                       alloc_workspace=True):
    """Checks and allocations of one attention call; returns its argument struct,
    out, lse and workspace (tensors the caller keeps alive).  With
    alloc_workspace False and no workspace given, the struct's workspace_bytes
    holds the size the call needs and the caller attaches one."""
    _need(q, "q", torch.bfloat16, 3)
    _need(k_cache, "k_cache", torch.bfloat16, 4)
    if v_cache is not None:
        _need(v_cache, "v_cache", torch.bfloat16, 4)
        head_dim_v = v_cache.shape[3]
    elif head_dim_v is None:
        raise ValueError("head_dim_v is required for a latent cache (v_cache=None)")
    _need(block_table, "block_table", torch.int32, 2)
    _need(query_start_loc, "query_start_loc", torch.int32, 1)
    _need(seq_lens, "seq_lens", torch.int32, 1)
    if mm_ranges is not None:
        _need(mm_ranges, "mm_ranges", torch.int32, 3)
    if key_ranges is not None:
        _need(key_ranges, "key_ranges", torch.int32, 3)
        if num_splits is not None and num_splits != key_ranges.shape[0]:
            raise ValueError("num_splits differs from the number of key ranges")
        num_splits = key_ranges.shape[0]
    elif num_splits is None:
        num_splits = 1
    check_attention_shapes(q.shape, k_cache.shape, None if v_cache is None else v_cache.shape,
                           block_table.shape, query_start_loc.numel(), seq_lens.numel(),
                           None if mm_ranges is None else mm_ranges.shape,
                           None if key_ranges is None else key_ranges.shape, head_dim_v)
    n, hq = q.shape[0], q.shape[1]
    odt = _dtype_code(out_dtype, "out_dtype")
    if out is None:
        out = torch.empty((num_splits, n, hq, head_dim_v), dtype=out_dtype, device=q.device)
    _need(out, "out", out_dtype)
    if out.numel() != num_splits * n * hq * head_dim_v:
        raise ValueError("out has the wrong size")
    if lse is None and (return_lse or num_splits > 1):
        lse = torch.empty((num_splits, n, hq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _need(lse, "lse", torch.float32)
        if lse.numel() != num_splits * n * hq:
            raise ValueError("lse has the wrong size")
    a = _attn_args(q, k_cache, v_cache, block_table, query_start_loc, seq_lens, scale=scale,
                   window=window, causal=causal, chunk_size=chunk_size,
                   chunk_lookback=chunk_lookback, mm_ranges=mm_ranges, key_ranges=key_ranges,
                   out=out, lse=lse, head_dim_v=head_dim_v, out_dtype=odt,
                   num_splits=num_splits)
    need = attention_workspace_size(a)
    if need > 0:
        if workspace is None and not alloc_workspace:
            a.workspace_bytes = need
            return a, out, lse, None
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        _need(workspace, "workspace", torch.uint8)
        a.workspace, a.workspace_bytes = workspace.data_ptr(), workspace.numel()
    return a, out, lse, workspace


def swa_mm_attention(q: torch.Tensor, k_cache: torch.Tensor, v_cache: Optional[torch.Tensor],
                     block_table: torch.Tensor, query_start_loc: torch.Tensor,
                     seq_lens: torch.Tensor, *, scale: float, window: int, causal: bool,
                     chunk_size: int = 0, chunk_lookback: int = -1,
                     mm_ranges: Optional[torch.Tensor] = None,
                     key_ranges: Optional[torch.Tensor] = None, head_dim_v: Optional[int] = None,
                     out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                     out_dtype: torch.dtype = torch.bfloat16, return_lse: bool = False,
                     num_splits: Optional[int] = None,
                     workspace: Optional[torch.Tensor] = None, stream=None):
    """Paged attention; with key_ranges [S, num_seqs, 2] it writes S fp32/bf16
    partials out[S, N, Hq, Dv] and lse[S, N, Hq]; without key_ranges,
    num_splits = S > 1 asks for S segmented splits of every query block's tile
    loop (partials of the same shape).  ``workspace`` (uint8, device) is
    allocated here when the call needs one and none is given."""
    a, out, lse, workspace = _prepare_attention(
        q, k_cache, v_cache, block_table, query_start_loc, seq_lens, scale=scale, window=window,
        causal=causal, chunk_size=chunk_size, chunk_lookback=chunk_lookback, mm_ranges=mm_ranges,
        key_ranges=key_ranges, head_dim_v=head_dim_v, out=out, lse=lse, out_dtype=out_dtype,
        return_lse=return_lse, num_splits=num_splits, workspace=workspace)
    check(load().psw_swa_mm_attention(ctypes.byref(a), _stream(stream)))
    n, hq, dv, num_splits = q.shape[0], q.shape[1], a.head_dim_v, a.num_splits
    if key_ranges is None and num_splits == 1:
        out = out.view(n, hq, dv)
        if lse is not None:
            lse = lse.view(n, hq)
    return (out, lse) if (return_lse or num_splits > 1) else out


def swa_mm_attention_noalloc(q: torch.Tensor, k_cache: torch.Tensor,
                             v_cache: Optional[torch.Tensor], block_table: torch.Tensor,
                             query_start_loc: torch.Tensor, seq_lens: torch.Tensor, *,
                             out: torch.Tensor, scale: float, window: int, causal: bool,
                             lse: Optional[torch.Tensor] = None, chunk_size: int = 0,
                             chunk_lookback: int = -1, mm_ranges: Optional[torch.Tensor] = None,
                             key_ranges: Optional[torch.Tensor] = None,
                             head_dim_v: Optional[int] = None, num_splits: Optional[int] = None,
                             stream=None) -> None:
    """psw_swa_mm_attention_noalloc: the attention of swa_mm_attention with the
    workspace taken from the library's own device scratch.  Nothing is
    allocated here or in the library: ``out`` (and ``lse`` where partials need
    it) are the caller's; out's dtype is the output type.  Calls that overlap
    in time on one device share the scratch and must be ordered by the caller."""
    if out is None:
        raise ValueError("out is required (this entry point allocates nothing)")
    if lse is None and (key_ranges is not None or (num_splits or 1) > 1):
        raise ValueError("partials need lse (this entry point allocates nothing)")
    a, _, _, _ = _prepare_attention(
        q, k_cache, v_cache, block_table, query_start_loc, seq_lens, scale=scale, window=window,
        causal=causal, chunk_size=chunk_size, chunk_lookback=chunk_lookback, mm_ranges=mm_ranges,
        key_ranges=key_ranges, head_dim_v=head_dim_v, out=out, lse=lse, out_dtype=out.dtype,
        return_lse=False, num_splits=num_splits, workspace=None, alloc_workspace=False)
    a.workspace, a.workspace_bytes = None, 0
    check(load().psw_swa_mm_attention_noalloc(ctypes.byref(a), _stream(stream)))


def swa_mm_attention_kv_write(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                              slots: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                              block_table: torch.Tensor, query_start_loc: torch.Tensor,
                              seq_lens: torch.Tensor, *, scale: float, window: int, causal: bool,
                              chunk_size: int = 0, chunk_lookback: int = -1,
                              mm_ranges: Optional[torch.Tensor] = None,
                              key_ranges: Optional[torch.Tensor] = None,
                              out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                              out_dtype: torch.dtype = torch.bfloat16, return_lse: bool = False,
                              num_splits: Optional[int] = None, stream=None):
    """psw_swa_mm_attention_kv_write: kv_cache_write(k_new, v_new, slots, k_cache,
    v_cache) and swa_mm_attention(...) in one launch (prefill shapes; the new
    tokens' keys are read from k_new / v_new).  Returns what swa_mm_attention
    returns."""
    _need(k_new, "k_new", torch.bfloat16, 3)
    _need(v_new, "v_new", torch.bfloat16, 3)
    _need(slots, "slot_mapping", torch.int32, 1)
    if v_cache is None:
        raise ValueError("the fused cache write needs separate K and V caches")
    if k_new.shape[0] != q.shape[0]:
        raise ValueError(f"k_new has {k_new.shape[0]} rows for {q.shape[0]} query tokens")
    check_kv_write_shapes(k_new.shape, v_new.shape, slots.numel(), k_cache.shape, v_cache.shape)
    a, out, lse, _ = _prepare_attention(
        q, k_cache, v_cache, block_table, query_start_loc, seq_lens, scale=scale, window=window,
        causal=causal, chunk_size=chunk_size, chunk_lookback=chunk_lookback, mm_ranges=mm_ranges,
        key_ranges=key_ranges, head_dim_v=None, out=out, lse=lse, out_dtype=out_dtype,
        return_lse=return_lse, num_splits=num_splits, workspace=None)
    num_slots = k_cache.shape[0] * k_cache.shape[1]
    check(load().psw_swa_mm_attention_kv_write(ctypes.byref(a), _ptr(k_new), _ptr(v_new),
                                               _ptr(slots), num_slots, _stream(stream)))
    n, hq, dv, num_splits = q.shape[0], q.shape[1], a.head_dim_v, a.num_splits
    if key_ranges is None and num_splits == 1:
        out = out.view(n, hq, dv)
        if lse is not None:
            lse = lse.view(n, hq)
    return (out, lse) if (return_lse or num_splits > 1) else out


def decode_two_streams(q: torch.Tensor, k_cache: torch.Tensor, v_cache: Optional[torch.Tensor],
                       block_table: torch.Tensor, query_start_loc: torch.Tensor,
                       seq_lens: torch.Tensor, *, history_ranges: torch.Tensor,
                       current_ranges: torch.Tensor, side_stream: torch.cuda.Stream,
                       scale: float, window: int = 0, causal: bool = True,
                       head_dim_v: Optional[int] = None,
                       partial_dtype: torch.dtype = torch.bfloat16,
                       out_dtype: torch.dtype = torch.bfloat16,
                       history_workspace: Optional[torch.Tensor] = None,
                       current_workspace: Optional[torch.Tensor] = None,
                       shared_workspace: bool = False,
                       out: Optional[torch.Tensor] = None, out_lse: Optional[torch.Tensor] = None,
                       stream=None):
    """History partials over ``history_ranges`` on the main stream, the current
    partial over ``current_ranges`` on ``side_stream``, joined and merged by the
    LSE combine on the main stream (psw_decode_two_streams).  One workspace for
    both calls (``shared_workspace``, or one tensor passed as both) orders the
    current call after the history call; separate ones let them overlap.
    Returns (out [N * Hq, Dv], out_lse [N * Hq], (history out, lse), (current out, lse))."""
    main = torch.cuda.current_stream() if stream is None else stream
    if side_stream is None:
        raise ValueError("side_stream is required")
    common = dict(scale=scale, window=window, causal=causal, chunk_size=0, chunk_lookback=-1,
                  mm_ranges=None, head_dim_v=head_dim_v, out=None, lse=None,
                  out_dtype=partial_dtype, return_lse=True, num_splits=None)
    alloc = not shared_workspace
    if shared_workspace and (history_workspace is not None or current_workspace is not None):
        raise ValueError("shared_workspace allocates the one workspace itself")
    ah, ho, hl, hw = _prepare_attention(q, k_cache, v_cache, block_table, query_start_loc,
                                        seq_lens, key_ranges=history_ranges,
                                        workspace=history_workspace, alloc_workspace=alloc,
                                        **common)
    ac, co, cl, cw = _prepare_attention(q, k_cache, v_cache, block_table, query_start_loc,
                                        seq_lens, key_ranges=current_ranges,
                                        workspace=current_workspace, alloc_workspace=alloc,
                                        **common)
    if shared_workspace:
        need = max(ah.workspace_bytes, ac.workspace_bytes)
        if need > 0:
            hw = cw = torch.empty(need, dtype=torch.uint8, device=q.device)
            for a in (ah, ac):
                a.workspace, a.workspace_bytes = hw.data_ptr(), hw.numel()
    rows, dv = q.shape[0] * q.shape[1], ah.head_dim_v
    if out is None:
        out = torch.empty((rows, dv), dtype=out_dtype, device=q.device)
    _need(out, "out", out_dtype)
    if out.numel() != rows * dv:
        raise ValueError("out has the wrong size")
    if out_lse is None:
        out_lse = torch.empty(rows, dtype=torch.float32, device=q.device)
    _need(out_lse, "out_lse", torch.float32)
    if out_lse.numel() != rows:
        raise ValueError("out_lse has the wrong size")
    # tensors the side stream reads or writes stay allocated until it has passed them
    for t in (q, k_cache, v_cache, block_table, query_start_loc, seq_lens, current_ranges, co, cl,
              cw):
        if t is not None:
            t.record_stream(side_stream)
    odt = _dtype_code(out_dtype, "out_dtype")
    check(load().psw_decode_two_streams(ctypes.byref(ah), ctypes.byref(ac), _ptr(out), odt,
                                        _ptr(out_lse), main.cuda_stream, side_stream.cuda_stream))
    return out, out_lse, (ho, hl), (co, cl)


def attention_workspace_size(args: PswAttnArgs) -> int:
    """Bytes of workspace psw_swa_mm_attention needs for ``args`` (0: none)."""
    n = ctypes.c_int64(0)
    check(load().psw_attention_workspace_size(ctypes.byref(args), ctypes.byref(n)))
    return n.value


def lse_combine(partial_outs: Sequence[torch.Tensor], partial_lses: Sequence[torch.Tensor],
                out: Optional[torch.Tensor] = None, out_lse: Optional[torch.Tensor] = None,
                out_dtype: torch.dtype = torch.bfloat16, stream=None):
    """Merge P partials [rows, Dv] (bf16, fp16 or fp32) with lse [rows] fp32, read in place."""
    P = len(partial_outs)
    if P != len(partial_lses) or P == 0:
        raise ValueError("need as many LSE tensors as partial outputs, at least one")
    pdt = partial_outs[0].dtype
    for i, (o, l) in enumerate(zip(partial_outs, partial_lses)):
        _need(o, f"partial_outs[{i}]", pdt)
        _need(l, f"partial_lses[{i}]", torch.float32)
    dv = partial_outs[0].shape[-1]
    rows = partial_outs[0].numel() // dv
    for o, l in zip(partial_outs, partial_lses):
        if o.numel() != rows * dv or l.numel() != rows:
            raise ValueError("partials disagree in size")
    if out is None:
        out = torch.empty((rows, dv), dtype=out_dtype, device=partial_outs[0].device)
    _need(out, "out", out_dtype)
    if out_lse is not None:
        _need(out_lse, "out_lse", torch.float32)
    check_combine_shapes(rows, dv, out.numel(), None if out_lse is None else out_lse.numel())
    po = (ctypes.c_void_p * P)(*[o.data_ptr() for o in partial_outs])
    pl = (ctypes.c_void_p * P)(*[l.data_ptr() for l in partial_lses])
    check(load().psw_lse_combine(po, pl, P, _dtype_code(pdt, "partial dtype"), rows, dv,
                                 _ptr(out), _dtype_code(out_dtype, "out_dtype"), _ptr(out_lse),
                                 _stream(stream)))
    return out if out_lse is None else (out, out_lse)


def vup_projection(x: torch.Tensor, w_uv: torch.Tensor, out: Optional[torch.Tensor] = None,
                   stream=None) -> torch.Tensor:
    """x bf16 [T, H, R] (or [T * H, R]) @ w_uv bf16 [H, R, Dv] per head -> [T, H, Dv]."""
    _need(w_uv, "w_uv", torch.bfloat16, 3)
    H, R, Dv = w_uv.shape
    _need(x, "x", torch.bfloat16)
    if x.dim() == 2:
        if x.shape[0] % H != 0:
            raise ValueError("x rows must be a multiple of the head count")
        x = x.view(x.shape[0] // H, H, x.shape[1])
    if x.dim() != 3 or x.shape[1] != H or x.shape[2] != R:
        raise ValueError(f"x {tuple(x.shape)} does not match w_uv {tuple(w_uv.shape)}")
    T = x.shape[0]
    if out is None:
        out = torch.empty((T, H, Dv), dtype=torch.bfloat16, device=x.device)
    _need(out, "out", torch.bfloat16)
    if out.numel() != T * H * Dv:
        raise ValueError("out must hold num_tokens * num_heads * v_head_dim elements")
    check(load().psw_vup_projection(_ptr(x), _ptr(w_uv), _ptr(out), T, H, R, Dv, _stream(stream)))
    return out


def lse_combine_vup(partial_outs: Sequence[torch.Tensor], partial_lses: Sequence[torch.Tensor],
                    w_uv: torch.Tensor, out: Optional[torch.Tensor] = None,
                    out_lse: Optional[torch.Tensor] = None, merged: Optional[torch.Tensor] = None,
                    stream=None) -> torch.Tensor:
    """psw_lse_combine_vup: merge P partials [T, H, R] (or [T * H, R]; bf16, fp16 or
    fp32, with lse [T, H] fp32) by LSE and project the merged rows with w_uv bf16
    [H, R, Dv] in one launch -> out bf16 [T, H, Dv]; out_lse [T * H] fp32 and the
    merged rows bf16 [T * H, R] are written when given."""
    _need(w_uv, "w_uv", torch.bfloat16, 3)
    H, R, Dv = w_uv.shape
    P = len(partial_outs)
    if P != len(partial_lses) or P == 0:
        raise ValueError("need as many LSE tensors as partial outputs, at least one")
    pdt = partial_outs[0].dtype
    for i, (o, l) in enumerate(zip(partial_outs, partial_lses)):
        _need(o, f"partial_outs[{i}]", pdt)
        _need(l, f"partial_lses[{i}]", torch.float32)
    rows = partial_outs[0].numel() // R if R > 0 else 0
    if rows * R != partial_outs[0].numel() or rows % H != 0 or partial_outs[0].shape[-1] != R:
        raise ValueError(f"partials {tuple(partial_outs[0].shape)} do not match w_uv "
                         f"{tuple(w_uv.shape)}")
    for o, l in zip(partial_outs, partial_lses):
        if o.numel() != rows * R or l.numel() != rows:
            raise ValueError("partials disagree in size")
    T = rows // H
    if out is None:
        out = torch.empty((T, H, Dv), dtype=torch.bfloat16, device=w_uv.device)
    _need(out, "out", torch.bfloat16)
    if out.numel() != T * H * Dv:
        raise ValueError("out must hold num_tokens * num_heads * v_head_dim elements")
    if out_lse is not None:
        _need(out_lse, "out_lse", torch.float32)
        if out_lse.numel() != rows:
            raise ValueError("out_lse must hold num_tokens * num_heads elements")
    if merged is not None:
        _need(merged, "merged", torch.bfloat16)
        if merged.numel() != rows * R:
            raise ValueError("merged must hold num_tokens * num_heads * kv_lora_rank elements")
    po = (ctypes.c_void_p * P)(*[o.data_ptr() for o in partial_outs])
    pl = (ctypes.c_void_p * P)(*[l.data_ptr() for l in partial_lses])
    check(load().psw_lse_combine_vup(po, pl, P, _dtype_code(pdt, "partial dtype"), _ptr(w_uv),
                                     _ptr(out), _ptr(out_lse), _ptr(merged), T, H, R, Dv,
                                     _stream(stream)))
    return out


def tile_bounds(query_start_loc: torch.Tensor, seq_lens: torch.Tensor,
                mm_ranges: Optional[torch.Tensor], *, num_q_heads: int, num_kv_heads: int,
                window: int, causal: bool, chunk_size: int, chunk_lookback: int, tile_size: int,
                block_m: int, block_q: int, seq_idx: torch.Tensor, q_block_idx: torch.Tensor,
                stream=None) -> torch.Tensor:
    """(loop_lo, loop_hi, max_seq_prefix_len) per (seq_idx[n], q_block_idx[n])."""
    _need(query_start_loc, "query_start_loc", torch.int32, 1)
    _need(seq_lens, "seq_lens", torch.int32, 1)
    _need(seq_idx, "seq_idx", torch.int32, 1)
    _need(q_block_idx, "q_block_idx", torch.int32, 1)
    if mm_ranges is not None:
        _need(mm_ranges, "mm_ranges", torch.int32, 3)
    a = PswAttnArgs()
    a.struct_size = ctypes.sizeof(PswAttnArgs)
    a.query_start_loc, a.seq_lens, a.mm_ranges = _ptr(query_start_loc), _ptr(seq_lens), _ptr(mm_ranges)
    a.num_seqs = query_start_loc.numel() - 1
    a.num_q_heads, a.num_kv_heads = int(num_q_heads), int(num_kv_heads)
    a.max_mm_ranges = mm_ranges.shape[1] if mm_ranges is not None else 0
    a.window, a.causal = int(window), int(bool(causal))
    a.chunk_size, a.chunk_lookback = int(chunk_size), int(chunk_lookback)
    n = seq_idx.numel()
    if q_block_idx.numel() != n:
        raise ValueError("seq_idx and q_block_idx must have the same length")
    out = torch.empty((n, 3), dtype=torch.int32, device=seq_idx.device)
    check(load().psw_tile_bounds(ctypes.byref(a), int(tile_size), int(block_m), int(block_q),
                                 _ptr(seq_idx), _ptr(q_block_idx), n, _ptr(out), _stream(stream)))
    return out


def debug_take_failures() -> int:
    """psw_debug_take_failures: the debug checks that failed on the current
    device since the previous call (a bit mask, 0 = every check held), then
    cleared.  Raises PswError (PSW_ERR_UNSUPPORTED) unless the loaded library
    is a PSW_DEBUG build."""
    mask = ctypes.c_uint32(0)
    check(load().psw_debug_take_failures(ctypes.byref(mask)))
    return int(mask.value)
