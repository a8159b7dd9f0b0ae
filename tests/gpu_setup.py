"""Helpers for the GPU parity tests: put a synthetic workload on the GPU through
the library's own slot mapping and cache write, run the path, and compare with
the oracle.  Imported only by tests marked ``gpu``."""
from __future__ import annotations

import numpy as np
import torch

import paged_sliding_window_amd as psw

ATOL = RTOL = 2e-2   # bf16 inputs, fp32 accumulation (parity bar of the path)


def bits_to_bf16(bits: np.ndarray, device="cuda") -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.to(device).view(torch.bfloat16)


def i32(a, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)


def i64(a, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int64)).to(device)


class GpuWorkload:
    """Device copies of a workload with the paged caches filled for every
    position of every request (context and new tokens alike)."""

    def __init__(self, w, fill_cache=True):
        self.w = w
        B = w.block_size
        self.q = bits_to_bf16(w.q_bits)
        self.qsl = i32(w.query_start_loc)
        self.seq_lens = i32(w.seq_lens)
        self.positions = i64(w.positions)
        self.block_table = i32(w.block_table)
        self.mm_ranges = i32(w.mm_ranges) if w.max_mm_ranges > 0 and (w.mm_ranges != 0).any() else None
        hkv = w.num_kv_heads
        self.k_cache = torch.zeros((w.num_blocks, B, hkv, w.head_dim_qk), dtype=torch.bfloat16,
                                   device="cuda")
        self.v_cache = None if w.v_bits is None else torch.zeros(
            (w.num_blocks, B, hkv, w.head_dim_v), dtype=torch.bfloat16, device="cuda")
        if fill_cache:
            self.fill()

    def fill(self):
        w = self.w
        qsl_all = np.concatenate([[0], np.cumsum(w.seq_lens)]).astype(np.int32)
        pos_all = np.concatenate([np.arange(int(L)) for L in w.seq_lens]).astype(np.int64)
        slots = psw.slot_mapping(i32(qsl_all), i64(pos_all), self.block_table, w.block_size,
                                 int(qsl_all[-1]))
        k_all = bits_to_bf16(np.concatenate(w.k_bits))
        v_all = None if w.v_bits is None else bits_to_bf16(np.concatenate(w.v_bits))
        psw.kv_cache_write(k_all, v_all, slots, self.k_cache, self.v_cache)
        torch.cuda.synchronize()

    def attention(self, key_ranges=None, out_dtype=torch.bfloat16, mm=True, **over):
        w = self.w
        kw = dict(scale=w.scale, window=w.window, causal=w.causal, chunk_size=w.chunk_size,
                  chunk_lookback=w.chunk_lookback)
        kw.update(over)
        return psw.swa_mm_attention(
            self.q, self.k_cache, self.v_cache, self.block_table, self.qsl, self.seq_lens,
            mm_ranges=self.mm_ranges if mm else None,
            key_ranges=None if key_ranges is None else i32(key_ranges),
            head_dim_v=w.head_dim_v, out_dtype=out_dtype, return_lse=True, **kw)


def oracle_rows(w, r, rows=None, key_range=None, ranges=True):
    """oracle.attention_ref for request r (rows = new-token indices)."""
    from oracle import attention_ref
    q = w.q_f32()[w.query_start_loc[r]:w.query_start_loc[r + 1]]
    return attention_ref(q, w.k_f32(r), w.v_f32(r), context_len=int(w.context_lens[r]),
                         seq_len=int(w.seq_lens[r]), scale=w.scale, window=w.window,
                         causal=w.causal, chunk_size=w.chunk_size,
                         chunk_lookback=w.chunk_lookback,
                         ranges=w.ranges_of(r) if ranges else [], key_range=key_range, rows=rows)


def assert_close(got, ref, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    err = np.abs(got - ref)
    bad = ~(err <= ATOL + RTOL * np.abs(ref))   # NaN / inf anywhere is a failure
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} elements out of tolerance; "
                             f"max err {err.max():.4g}; first {idx.tolist()} "
                             f"got {got[tuple(idx[0])]:.5g} ref {ref[tuple(idx[0])]:.5g}")


def assert_lse_close(got, ref, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert np.array_equal(np.isneginf(got), np.isneginf(ref)), f"{what}: -inf pattern differs"
    fin = np.isfinite(ref)
    assert_close(got[fin], ref[fin], what)
