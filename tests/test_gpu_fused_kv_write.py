"""psw_swa_mm_attention_kv_write on the GPU: the cache write fused into the
prefill attention.

Each case starts from caches holding only the context rows (positions below
each request's context length, written through the library's slot mapping and
cache write).  The two calls the entry point replaces (psw_kv_cache_write of
the new rows, then psw_swa_mm_attention) and the fused call run on copies of
those caches with the same slot mapping.  The caches afterwards and the
outputs must agree bit for bit (the fused call reads the new keys from the new
rows instead of the cache, the same bf16 values in the same tile order), and
the outputs must match the oracle.
"""
import numpy as np
import pytest
import torch

import paged_sliding_window_amd as psw
from tests.gpu_setup import assert_close, assert_lse_close, bits_to_bf16, i32, i64, oracle_rows
from workloads import make_config, make_small_case

pytestmark = pytest.mark.gpu


def same_bits(a, b):
    if a.dtype in (torch.bfloat16, torch.float16):
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    return torch.equal(a.view(torch.int32), b.view(torch.int32))


class FusedCase:
    def __init__(self, w, spare_blocks=0):
        self.w = w
        B, hkv = w.block_size, w.num_kv_heads
        ctx = np.asarray(w.context_lens)
        self.q = bits_to_bf16(w.q_bits)
        self.qsl = i32(w.query_start_loc)
        self.seq_lens = i32(w.seq_lens)
        self.bt = i32(w.block_table)
        self.mm = i32(w.mm_ranges) if w.max_mm_ranges > 0 and (w.mm_ranges != 0).any() else None
        shape_k = (w.num_blocks + spare_blocks, B, hkv, w.head_dim_qk)
        shape_v = (w.num_blocks + spare_blocks, B, hkv, w.head_dim_v)
        self.k0 = torch.zeros(shape_k, dtype=torch.bfloat16, device="cuda")
        self.v0 = torch.zeros(shape_v, dtype=torch.bfloat16, device="cuda")
        self.nb = w.num_blocks
        if ctx.sum() > 0:
            qsl_ctx = np.concatenate([[0], np.cumsum(ctx)]).astype(np.int32)
            pos_ctx = np.concatenate([np.arange(int(c)) for c in ctx]).astype(np.int64)
            slots = psw.slot_mapping(i32(qsl_ctx), i64(pos_ctx), self.bt, B, int(qsl_ctx[-1]))
            psw.kv_cache_write(bits_to_bf16(np.concatenate([k[:c] for k, c in zip(w.k_bits, ctx)])),
                               bits_to_bf16(np.concatenate([v[:c] for v, c in zip(w.v_bits, ctx)])),
                               slots, self.k0[:self.nb], self.v0[:self.nb])
        self.k_new = bits_to_bf16(np.concatenate([k[c:] for k, c in zip(w.k_bits, ctx)]))
        self.v_new = bits_to_bf16(np.concatenate([v[c:] for v, c in zip(w.v_bits, ctx)]))
        assert self.k_new.shape[0] == w.num_tokens
        self.slots = psw.slot_mapping(self.qsl, i64(w.positions[:w.num_tokens]), self.bt, B,
                                      w.num_tokens)
        torch.cuda.synchronize()

    def _kw(self, key_ranges, out_dtype, num_splits):
        w = self.w
        return dict(scale=w.scale, window=w.window, causal=w.causal, chunk_size=w.chunk_size,
                    chunk_lookback=w.chunk_lookback, mm_ranges=self.mm,
                    key_ranges=None if key_ranges is None else i32(key_ranges),
                    out_dtype=out_dtype, return_lse=True, num_splits=num_splits)

    def two_calls(self, key_ranges=None, out_dtype=torch.bfloat16, num_splits=None, slots=None):
        kc, vc = self.k0.clone(), self.v0.clone()
        psw.kv_cache_write(self.k_new, self.v_new, self.slots if slots is None else slots,
                           kc[:self.nb], vc[:self.nb])
        o, l = psw.swa_mm_attention(self.q, kc[:self.nb], vc[:self.nb], self.bt, self.qsl,
                                    self.seq_lens, **self._kw(key_ranges, out_dtype, num_splits))
        return kc, vc, o, l

    def fused(self, key_ranges=None, out_dtype=torch.bfloat16, num_splits=None, slots=None):
        kc, vc = self.k0.clone(), self.v0.clone()
        o, l = psw.swa_mm_attention_kv_write(
            self.q, self.k_new, self.v_new, self.slots if slots is None else slots,
            kc[:self.nb], vc[:self.nb], self.bt, self.qsl, self.seq_lens,
            **self._kw(key_ranges, out_dtype, num_splits))
        return kc, vc, o, l

    def check_same(self, **kw):
        ref = self.two_calls(**kw)
        got = self.fused(**kw)
        torch.cuda.synchronize()
        for name, a, b in zip(("k_cache", "v_cache", "out", "lse"), ref, got):
            assert same_bits(a, b), f"{name} differs from the two-call result ({kw})"
        return got

    def check_oracle(self, out, lse, what=""):
        w = self.w
        out = out.float().cpu().numpy().reshape(w.num_tokens, w.num_q_heads, w.head_dim_v)
        lse = lse.cpu().numpy().reshape(w.num_tokens, w.num_q_heads)
        for r in range(w.num_seqs):
            s0, ql = int(w.query_start_loc[r]), int(w.query_lens[r])
            ref_o, ref_l = oracle_rows(w, r)
            assert_close(out[s0:s0 + ql], ref_o, f"{what} request {r}")
            assert_lse_close(lse[s0:s0 + ql], ref_l, f"{what} request {r} lse")


@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_fused_matches_two_calls_on_workloads(cfg):
    """The four prefill workloads (head dims 64-256, GQA 1-8, one long
    multimodal request, batched chunked prefill with cached context,
    non-causal chunk lookback)."""
    case = FusedCase(make_config(cfg))
    _, _, o, l = case.check_same()
    case.check_oracle(o, l, f"workload {cfg}")


def test_fused_bench_step_padded_slot_mapping():
    """The headline step as the bench times it: the slot mapping padded with -1
    up to max_num_tokens, then the fused call (workload 2, full size)."""
    w = make_config(2)
    case = FusedCase(w)
    slots = torch.empty(w.max_num_tokens, dtype=torch.int32, device="cuda")
    psw.slot_mapping(case.qsl, i64(w.positions), case.bt, w.block_size, w.max_num_tokens,
                     out=slots)
    assert torch.equal(slots[:w.num_tokens], case.slots)
    ref = case.two_calls(slots=slots)
    got = case.fused(slots=slots)
    torch.cuda.synchronize()
    for name, a, b in zip(("k_cache", "v_cache", "out", "lse"), ref, got):
        assert same_bits(a, b), name


def test_fused_segmented_splits_and_key_ranges():
    """Split-0 workgroups write the cache; every split reads the new rows."""
    w = make_config(4)
    case = FusedCase(w)
    case.check_same(num_splits=3, out_dtype=torch.float32)
    L = np.asarray(w.seq_lens)
    kr = np.stack([np.stack([np.zeros_like(L), L // 3], 1),
                   np.stack([L // 3, L], 1)]).astype(np.int32)
    case.check_same(key_ranges=kr, out_dtype=torch.float32)


@pytest.mark.parametrize("seed", range(40))
def test_fused_random_cases(seed):
    """Random requests with cached context (tiles that hold old and new keys),
    cache blocks of 1-128 keys, head dims 64-256, 1-16 query heads per KV head,
    unsplit or segmented, bf16 / fp16 / fp32 output."""
    rng = np.random.default_rng(9100 + seed)
    d = int(rng.choice([64, 128, 256]))
    hkv = int(rng.choice([1, 2, 4]))
    qpk = int(rng.choice([1, 2, 3, 8, 16]))
    bs = int(rng.choice([1, 2, 8, 16, 32, 64, 128]))
    w = make_small_case(9100 + seed, num_seqs=int(rng.integers(1, 6)),
                        max_len=int(rng.choice([64, 300, 900])), hq=hkv * qpk, hkv=hkv, d=d,
                        block_size=bs)
    case = FusedCase(w)
    splits = int(rng.choice([1, 1, 2, 3]))
    odt = [torch.bfloat16, torch.float16, torch.float32][int(rng.integers(0, 3))]
    _, _, o, l = case.check_same(num_splits=splits, out_dtype=odt)
    if splits == 1:
        case.check_oracle(o, l, f"seed {seed}")


def test_fused_skips_padding_and_slots_past_the_cache():
    """Slots of -1 and one past the cache are skipped exactly as
    psw_kv_cache_write skips them (the spare rows beyond the cache view stay
    zero), while the attention still reads every new key from the new rows."""
    w = make_small_case(77, num_seqs=3, max_len=400, hq=4, hkv=2, d=128, block_size=16)
    case = FusedCase(w, spare_blocks=2)
    slots = case.slots.clone()
    slots[::7] = -1
    slots[3] = case.nb * w.block_size          # one past the cache
    ref_k, ref_v, _, _ = case.two_calls(slots=slots)
    k, v, o, l = case.fused(slots=slots)
    torch.cuda.synchronize()
    assert same_bits(k, ref_k) and same_bits(v, ref_v)
    assert not k[case.nb:].any() and not v[case.nb:].any()
    case.check_oracle(o, l, "padded slots")


def test_fused_rejects_latent_and_missing_rows():
    """Host-side rejections through the C ABI (nothing is launched): the
    latent shape is unsupported, missing new rows are invalid; the binding
    refuses a latent cache before calling the library."""
    import ctypes
    from paged_sliding_window_amd import _lib
    w = make_small_case(5, num_seqs=2, max_len=100, hq=4, hkv=2, d=64, block_size=16)
    case = FusedCase(w)
    with pytest.raises(ValueError, match="separate K and V"):
        psw.swa_mm_attention_kv_write(case.q, case.k_new, case.v_new, case.slots, case.k0,
                                      None, case.bt, case.qsl, case.seq_lens, scale=1.0,
                                      window=0, causal=True)
    lib = psw.load()
    out = torch.empty((w.num_tokens, w.num_q_heads, w.head_dim_v), dtype=torch.bfloat16,
                      device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    num_slots = case.k0.shape[0] * case.k0.shape[1]

    def args(v_cache):
        return psw.ops._attn_args(case.q, case.k0, v_cache, case.bt, case.qsl, case.seq_lens,
                                  scale=1.0, window=0, causal=True, chunk_size=0,
                                  chunk_lookback=-1, mm_ranges=None, key_ranges=None, out=out,
                                  lse=None, head_dim_v=w.head_dim_v, out_dtype=_lib.PSW_BF16,
                                  num_splits=1)
    a = args(None)
    assert lib.psw_swa_mm_attention_kv_write(ctypes.byref(a), case.k_new.data_ptr(),
                                             case.v_new.data_ptr(), case.slots.data_ptr(),
                                             num_slots, stream) == _lib.PSW_ERR_UNSUPPORTED
    a = args(case.v0)
    assert lib.psw_swa_mm_attention_kv_write(ctypes.byref(a), None, case.v_new.data_ptr(),
                                             case.slots.data_ptr(), num_slots,
                                             stream) == _lib.PSW_ERR_INVALID
    assert lib.psw_swa_mm_attention_kv_write(ctypes.byref(a), case.k_new.data_ptr(),
                                             case.v_new.data_ptr(), case.slots.data_ptr(), -1,
                                             stream) == _lib.PSW_ERR_INVALID
    torch.cuda.synchronize()
    assert not out.isnan().any()
