"""The allocation-free attention entry point (psw_swa_mm_attention_noalloc),
called through the C ABI, against psw_swa_mm_attention with a caller-provided
workspace on the same inputs: two calls in a row, the second with a smaller
input (the scratch keeps the first call's contents), both element for element
identical.  Also a prefill call (no scratch needed).  The host-side size limit
is checked without a GPU in tests/test_abi.py."""
import numpy as np
import pytest
import torch

import paged_sliding_window_amd as psw
from tests.gpu_setup import DecodeStep, GpuWorkload, assert_close, oracle_rows
from workloads import make_config, make_small_case

pytestmark = pytest.mark.gpu


def _small_decode(seed):
    from workloads.synth import decode_split_ranges
    w = make_small_case(seed, num_seqs=5, max_len=3000, hq=128, hkv=1, d=576, dv=512,
                        window=0, causal=True, chunk=(0, -1), max_ranges=0, latent=True,
                        block_size=64)
    last = w.query_start_loc[1:] - 1
    w.q_bits = w.q_bits[last]
    w.positions = (w.seq_lens - 1).astype(np.int64)
    w.context_lens = w.seq_lens - 1
    w.query_lens = np.ones(w.num_seqs, dtype=np.int64)
    w.query_start_loc = np.arange(w.num_seqs + 1, dtype=np.int32)
    w.key_ranges = decode_split_ranges(w.seq_lens, 3)
    w.current_ranges = np.stack([np.stack([w.seq_lens - 1, w.seq_lens], 1)]).astype(np.int32)
    return w


def _noalloc_like(ds, out, lse):
    """The same call as ds.attention() through the allocation-free entry point."""
    w = ds.w
    psw.swa_mm_attention_noalloc(ds.q, ds.cache, None, ds.bt, ds.qsl, ds.seq_lens, out=out,
                                 lse=lse, scale=w.scale, window=0, causal=True,
                                 key_ranges=ds.kr_all, head_dim_v=w.head_dim_v)


def test_noalloc_decode_matches_two_calls_in_a_row():
    big = DecodeStep(make_config(5, decode_splits=1), partial_dtype=torch.bfloat16)
    small = DecodeStep(_small_decode(31), partial_dtype=torch.bfloat16)
    for ds in (big, small):   # the second call is the smaller input
        ds.run()              # the reference: caller-provided workspace
        torch.cuda.synchronize()
        out = torch.full_like(ds.part_o, 7.0)
        lse = torch.full_like(ds.part_l, 7.0)
        _noalloc_like(ds, out, lse)
        torch.cuda.synchronize()
        assert torch.equal(out, ds.part_o), ds.w.name
        assert torch.equal(lse, ds.part_l), ds.w.name
        # and to the parity bar against the oracle on a few rows
        got = out.float().cpu().numpy()
        for r in (0, ds.w.num_seqs - 1):
            ref_o, _ = oracle_rows(ds.w, r, key_range=tuple(ds.w.key_ranges[0, r]))
            assert_close(got[0, r], ref_o[0], f"{ds.w.name} history partial of {r}")


def test_noalloc_prefill_matches():
    w = make_config(1)
    gw = GpuWorkload(w)
    ref, ref_lse = gw.attention()
    out = torch.empty_like(ref)
    lse = torch.empty_like(ref_lse)
    psw.swa_mm_attention_noalloc(gw.q, gw.k_cache, gw.v_cache, gw.block_table, gw.qsl,
                                 gw.seq_lens, out=out, lse=lse, scale=w.scale, window=w.window,
                                 causal=w.causal, mm_ranges=gw.mm_ranges)
    torch.cuda.synchronize()
    assert torch.equal(out, ref) and torch.equal(lse, ref_lse)
