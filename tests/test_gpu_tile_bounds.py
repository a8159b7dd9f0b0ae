"""GPU parity: the device tile-interval routine the attention kernels call,
bit-exact against oracle.tile_bounds_ref (printed geometries, every query block
of the workloads at the kernel's own tiling, random small cases)."""
import numpy as np
import pytest
import torch

import paged_sliding_window_amd as psw
from oracle import tile_bounds_ref
from tests.gpu_setup import i32
from workloads import make_config, make_small_case

pytestmark = pytest.mark.gpu


def _gpu(qsl, seq_lens, ranges, hq, hkv, W, causal, C, lb, T, bm, bq, seq_idx, qb_idx):
    out = psw.tile_bounds(i32(qsl), i32(seq_lens), None if ranges is None else i32(ranges),
                          num_q_heads=hq, num_kv_heads=hkv, window=W, causal=causal,
                          chunk_size=C, chunk_lookback=lb, tile_size=T, block_m=bm, block_q=bq,
                          seq_idx=i32(seq_idx), q_block_idx=i32(qb_idx))
    return out.cpu().numpy()


@pytest.mark.parametrize("causal,ranges,C,lb,expect", [
    (True, [[1024, 2303], [0, 0]], -1, -1, [3, 72, 4096]),
    (False, [[1024, 1535], [0, 0]], -1, -1, [3, 68, 4096]),
    (True, [[256, 1535], [0, 0]], 512, 1, [8, 48, 4096]),
])
def test_printed_geometries(causal, ranges, C, lb, expect):
    got = _gpu([0, 4096], [4096], np.array([ranges]), 2, 1, 1024, causal, C, lb, 32, 16, 8,
               [0], [140])
    assert got[0].tolist() == expect


def _check_workload(w, T, block_q, qpk):
    seq_idx, qb_idx, refs = [], [], []
    for r in range(w.num_seqs):
        ql = int(w.query_lens[r])
        for qb in range(-(-ql // block_q)):
            seq_idx.append(r)
            qb_idx.append(qb)
            refs.append(tile_bounds_ref(int(w.context_lens[r]), int(w.seq_lens[r]), ql, qb, T,
                                        block_q * qpk, block_q, qpk, w.window,
                                        w.max_mm_ranges > 0 and (w.mm_ranges != 0).any(),
                                        w.causal, w.chunk_lookback, w.chunk_size,
                                        w.ranges_of(r)))
    use = w.max_mm_ranges > 0 and (w.mm_ranges != 0).any()
    got = _gpu(w.query_start_loc, w.seq_lens, w.mm_ranges if use else None, w.num_q_heads,
               w.num_kv_heads, w.window, w.causal, w.chunk_size, w.chunk_lookback, T,
               block_q * qpk, block_q, seq_idx, qb_idx)
    assert np.array_equal(got, np.array(refs, dtype=np.int32))


@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_every_query_block_of_the_workloads(cfg):
    w = make_config(cfg)
    qpk = w.num_q_heads // w.num_kv_heads
    for block_m in (128, 256):                # the prefill kernel's tilings (32-key tiles)
        _check_workload(w, 32, block_m // qpk, qpk)
    _check_workload(w, 64, 128 // qpk, qpk)
    _check_workload(w, 32, 8, qpk)            # the pages' test tiling


@pytest.mark.parametrize("seed", range(10))
def test_random_small(seed):
    w = make_small_case(300 + seed, num_seqs=3, max_len=400, hq=4, hkv=2)
    _check_workload(w, int(np.random.default_rng(seed).choice([4, 16, 64])), 4, 2)
