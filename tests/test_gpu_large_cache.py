"""GPU parity with paged caches larger than 2 GiB.  Every other table entry of
a request moves to the far end of the cache, so the two 16-key blocks of a
32-key prefill tile lie more than 2^31 bytes apart (the tile loads then take
per-lane 64-bit addresses instead of a base plus 32-bit lane offsets) and slot
byte offsets pass 2^31 in the KV write and in the decode's tile bases.  The
oracle reads the logical (un-paged) K/V, so it does not see the move."""
import numpy as np
import pytest
import torch

from tests.gpu_setup import GpuWorkload, assert_close, assert_lse_close, i32, oracle_rows
from tests.test_gpu_decode import _small_decode_case
from workloads import make_small_case

pytestmark = pytest.mark.gpu


def _spread(w, far_blocks):
    """Move odd table columns far_blocks blocks up; the cache grows to match."""
    bt = w.block_table.copy()
    cols = np.arange(bt.shape[1])[None, :]
    far = (bt >= 0) & (cols % 2 == 1)
    bt[far] += far_blocks
    w.block_table = bt.astype(np.int32)
    w.num_blocks = int(w.num_blocks) + far_blocks


def test_prefill_tiles_with_blocks_over_2gib_apart():
    w = make_small_case(960, num_seqs=2, max_len=700, hq=16, hkv=8, d=256, block_size=16)
    row_bytes = w.num_kv_heads * w.head_dim_qk * 2
    far = (1 << 31) // (w.block_size * row_bytes) + 4000        # blocks: > 2 GiB of K rows
    _spread(w, far)
    assert far * w.block_size * row_bytes > (1 << 31)
    gw = GpuWorkload(w)
    assert gw.k_cache.numel() * 2 > (1 << 31) and gw.v_cache.numel() * 2 > (1 << 31)
    out, lse = gw.attention()
    torch.cuda.synchronize()
    out = out.float().cpu().numpy()
    lse = lse.cpu().numpy()
    for r in range(w.num_seqs):
        s0, s1 = int(w.query_start_loc[r]), int(w.query_start_loc[r + 1])
        ref_o, ref_l = oracle_rows(w, r)
        assert_close(out[s0:s1], ref_o, f"request {r}")
        assert_lse_close(lse[s0:s1], ref_l, f"request {r} lse")


def test_latent_decode_with_cache_over_2gib():
    w = _small_decode_case(961, num_seqs=4, splits=3)
    row_bytes = w.head_dim_qk * 2
    far = (1 << 31) // (w.block_size * row_bytes) + 2000
    _spread(w, far)
    gw = GpuWorkload(w)
    assert gw.k_cache.numel() * 2 > (1 << 31)
    from tests.test_gpu_decode import _decode
    out, lse, *_ = _decode(gw, w, partial_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    out = out.float().cpu().numpy().reshape(w.num_tokens, w.num_q_heads, w.head_dim_v)
    lse = lse.cpu().numpy().reshape(w.num_tokens, w.num_q_heads)
    for r in range(w.num_seqs):
        ref_o, ref_l = oracle_rows(w, r)
        assert_close(out[r], ref_o[0], f"token {r}")
        assert_lse_close(lse[r], ref_l[0], f"token {r} lse")
