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


class DecodeStep:
    """The latent decode step as bench.py times it, on the GPU: context rows
    [0, L-1) are written to the paged latent cache beforehand through the
    library's slot mapping and KV write; one step is then
      slot mapping of the new token -> latent KV write -> ONE attention call
      whose key ranges are the history splits followed by the current key
      (S + 1 partials, each with its LSE) -> LSE combine and V-up projection
      (one launch by default, or the two launches).
    """

    def __init__(self, w, partial_dtype=torch.bfloat16, dv_up=128, wuv_seed=55):
        from workloads.synth import f32_to_bf16_bits
        self.w = w
        B = w.block_size
        R, H, DV = w.num_seqs, w.num_q_heads, w.head_dim_v
        self.q = bits_to_bf16(w.q_bits)
        self.bt = i32(w.block_table)
        self.qsl = i32(w.query_start_loc)
        self.seq_lens = i32(w.seq_lens)
        self.positions = i64(w.positions)
        self.cache = torch.empty((w.num_blocks, B, 1, w.head_dim_qk), dtype=torch.bfloat16,
                                 device="cuda")
        qsl_ctx = np.concatenate([[0], np.cumsum(w.seq_lens - 1)]).astype(np.int32)
        pos_ctx = np.concatenate([np.arange(int(L) - 1) for L in w.seq_lens]).astype(np.int64)
        slots_ctx = psw.slot_mapping(i32(qsl_ctx), i64(pos_ctx), self.bt, B, int(qsl_ctx[-1]))
        psw.kv_cache_write(bits_to_bf16(np.concatenate([k[:-1] for k in w.k_bits])), None,
                           slots_ctx, self.cache, None)
        del slots_ctx
        self.new_rows = bits_to_bf16(np.stack([k[-1] for k in w.k_bits]))
        self.S = w.key_ranges.shape[0]
        self.P = self.S + 1
        self.kr_all = i32(np.concatenate([w.key_ranges, w.current_ranges], axis=0))
        self.pdt = partial_dtype
        self.part_o = torch.empty((self.P, R, H, DV), dtype=partial_dtype, device="cuda")
        self.part_l = torch.empty((self.P, R, H), dtype=torch.float32, device="cuda")
        self.out = torch.empty((R * H, DV), dtype=torch.bfloat16, device="cuda")
        self.out_lse = torch.empty(R * H, dtype=torch.float32, device="cuda")
        self.slots = torch.empty(R, dtype=torch.int32, device="cuda")
        self.outs = [self.part_o[j].view(R * H, DV) for j in range(self.P)]
        self.lses = [self.part_l[j].view(R * H) for j in range(self.P)]
        args = psw.ops._attn_args(self.q, self.cache, None, self.bt, self.qsl, self.seq_lens,
                                  scale=w.scale, window=0, causal=True, chunk_size=0,
                                  chunk_lookback=-1, mm_ranges=None, key_ranges=self.kr_all,
                                  out=self.part_o, lse=self.part_l, head_dim_v=DV, out_dtype=0,
                                  num_splits=self.P)
        self.ws = torch.empty(max(1, psw.ops.attention_workspace_size(args)), dtype=torch.uint8,
                              device="cuda")
        self.dv_up = dv_up
        self.wuv_f32 = (np.random.default_rng(wuv_seed).standard_normal((H, DV, dv_up))
                        .astype(np.float32) / DV ** 0.5)
        wuv_bits = f32_to_bf16_bits(self.wuv_f32)
        self.w_uv = bits_to_bf16(wuv_bits)
        from workloads.synth import bf16_bits_to_f32
        self.wuv_f32 = bf16_bits_to_f32(wuv_bits)   # the values the kernel reads
        self.vup_out = torch.empty((R, H * dv_up), dtype=torch.bfloat16, device="cuda")

    def attention(self):
        w = self.w
        psw.swa_mm_attention(self.q, self.cache, None, self.bt, self.qsl, self.seq_lens,
                             scale=w.scale, window=0, causal=True, key_ranges=self.kr_all,
                             head_dim_v=w.head_dim_v, out=self.part_o, lse=self.part_l,
                             out_dtype=self.pdt, workspace=self.ws)

    def combine(self):
        psw.lse_combine(self.outs, self.lses, out=self.out, out_lse=self.out_lse)

    def combine_vup(self):
        """The combine and the V-up projection in one launch (merged rows and
        their LSEs written too)."""
        psw.lse_combine_vup([self.part_o[j] for j in range(self.P)],
                            [self.part_l[j] for j in range(self.P)], self.w_uv, out=self.vup_out,
                            out_lse=self.out_lse, merged=self.out)

    def run(self, ev=None, fused_tail=True):
        """One step; ev = 4 events recorded before the attention, after it, after
        the combine and after the projection (or None).  fused_tail: the combine
        and the projection as one launch (the last two events then coincide)."""
        w = self.w
        psw.slot_mapping(self.qsl, self.positions, self.bt, w.block_size, w.num_seqs,
                         out=self.slots)
        psw.kv_cache_write(self.new_rows, None, self.slots, self.cache, None)
        if ev is not None:
            ev[0].record()
        self.attention()
        if ev is not None:
            ev[1].record()
        if fused_tail and self.P <= 16:   # the one-launch tail takes up to 16 partials
            self.combine_vup()
            if ev is not None:
                ev[2].record()
                ev[3].record()
            return
        self.combine()
        if ev is not None:
            ev[2].record()
        psw.vup_projection(self.out, self.w_uv, out=self.vup_out)
        if ev is not None:
            ev[3].record()
