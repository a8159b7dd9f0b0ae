"""GPU parity: paged prefill attention against the float64 oracle, element by
element within |g - r| <= 2e-2 + 2e-2 |r| (bf16 inputs, fp32 accumulation)."""
import numpy as np
import pytest
import torch

from tests.gpu_setup import GpuWorkload, assert_close, assert_lse_close, oracle_rows
from workloads import make_config, make_small_case

pytestmark = pytest.mark.gpu


def _check(gw, out, lse, rows_per_seq=None, seed=0):
    w = gw.w
    out = out.float().cpu().numpy()
    lse = lse.cpu().numpy()
    rng = np.random.default_rng(seed)
    for r in range(w.num_seqs):
        ql = int(w.query_lens[r])
        rows = None
        if rows_per_seq is not None and ql > rows_per_seq:
            rows = np.unique(np.concatenate([np.arange(8), ql - 1 - np.arange(8),
                                             rng.choice(ql, rows_per_seq, replace=False)]))
        ref_o, ref_l = oracle_rows(w, r, rows)
        s0 = int(w.query_start_loc[r])
        sel = np.arange(ql) if rows is None else rows
        assert_close(out[s0 + sel], ref_o, f"{w.name} seq {r} out")
        assert_lse_close(lse[s0 + sel], ref_l, f"{w.name} seq {r} lse")


def test_tiny_prefill_full_and_image_sensitivity():
    w = make_config(1)
    gw = GpuWorkload(w)
    out, lse = gw.attention()
    _check(gw, out, lse)
    # the image range matters: the no-image oracle must fail the same tolerance
    ref_no_mm, _ = oracle_rows(w, 0, ranges=False)
    got = out.float().cpu().numpy()
    err = np.abs(got - ref_no_mm)
    assert (err > 2e-2 + 2e-2 * np.abs(ref_no_mm)).any()
    out_no_mm, _ = gw.attention(mm=False)
    assert_close(out_no_mm.float().cpu().numpy(), ref_no_mm, "no-image run")


def test_batched_chunked_prefill_full():
    gw = GpuWorkload(make_config(3))
    out, lse = gw.attention()
    _check(gw, out, lse)


def test_noncausal_chunk_lookback_full():
    """The non-causal chunk-lookback workload, every row of both requests."""
    gw = GpuWorkload(make_config(4))
    out, lse = gw.attention()
    _check(gw, out, lse)


def test_gemma_multimodal_prefill_full_size():
    """The 16,550-token multimodal workload: every row, every head, out and LSE."""
    w = make_config(2)
    gw = GpuWorkload(w)
    out, lse = gw.attention()
    _check(gw, out, lse)


@pytest.mark.parametrize("seed", range(16))
def test_random_small_cases(seed):
    rng = np.random.default_rng(seed)
    d = int(rng.choice([64, 128, 256]))
    hkv = int(rng.choice([1, 2]))
    qpk = int(rng.choice([1, 2, 3, 8]))
    w = make_small_case(500 + seed, num_seqs=int(rng.integers(1, 5)), max_len=700, hq=hkv * qpk,
                        hkv=hkv, d=d, block_size=int(rng.choice([1, 16, 64])))
    gw = GpuWorkload(w)
    out, lse = gw.attention()
    _check(gw, out, lse)


@pytest.mark.parametrize("seed,d,qpk,bs", [
    (0, 64, 128, 16),    # the largest GQA ratio: one position per 128-row query block
    (1, 128, 64, 2),     # two positions per block, two-key cache blocks (per-lane gathers)
    (2, 256, 5, 32),     # a ratio that does not divide 128: rows 125-127 of a block are idle
    (3, 64, 16, 128),    # blocks of 128 keys: four tiles per block on the fast path
    (4, 128, 3, 256),    # blocks of 256 keys
    (5, 256, 1, 4),      # MHA on four-key blocks
])
def test_extreme_gqa_ratios_and_block_sizes(seed, d, qpk, bs):
    """Parity at the edges of the supported shapes: queries per KV head up to
    128 (the query block shrinks to 128 / ratio positions, rounded down) and
    cache blocks from 2 to 256 keys (fast and per-lane tile gathers)."""
    w = make_small_case(800 + seed, num_seqs=3, max_len=600, hq=qpk, hkv=1, d=d, block_size=bs)
    gw = GpuWorkload(w)
    out, lse = gw.attention()
    _check(gw, out, lse)


@pytest.mark.parametrize("seed,pdt", [(0, torch.float32), (1, torch.float32), (2, torch.float16),
                                      (3, torch.bfloat16)])
def test_key_split_partials(seed, pdt):
    w = make_small_case(700 + seed, num_seqs=3, max_len=500, hq=4, hkv=2, d=128)
    gw = GpuWorkload(w)
    rng = np.random.default_rng(seed)
    S = 3
    kr = np.zeros((S, w.num_seqs, 2), dtype=np.int32)
    for r in range(w.num_seqs):
        L = int(w.seq_lens[r])
        cuts = np.sort(rng.integers(0, L + 1, size=S - 1))
        edges = np.concatenate([[0], cuts, [L]])
        kr[:, r, 0], kr[:, r, 1] = edges[:-1], edges[1:]
    out, lse = gw.attention(key_ranges=kr, out_dtype=pdt)
    out, lse = out.float().cpu().numpy(), lse.cpu().numpy()
    for j in range(S):
        for r in range(w.num_seqs):
            s0, s1 = int(w.query_start_loc[r]), int(w.query_start_loc[r + 1])
            ref_o, ref_l = oracle_rows(w, r, key_range=tuple(kr[j, r]))
            assert_close(out[j, s0:s1], ref_o, f"split {j} seq {r}")
            assert_lse_close(lse[j, s0:s1], ref_l, f"split {j} seq {r} lse")


def test_empty_batch_is_a_no_op():
    w = make_small_case(1, num_seqs=1, max_len=40)
    gw = GpuWorkload(w)
    import paged_sliding_window_amd as psw
    q0 = gw.q[:0]
    qsl = torch.zeros(2, dtype=torch.int32, device="cuda")
    out = psw.swa_mm_attention(q0, gw.k_cache, gw.v_cache, gw.block_table, qsl, gw.seq_lens,
                               scale=1.0, window=0, causal=True)
    torch.cuda.synchronize()
    assert out.numel() == 0


@pytest.mark.parametrize("seed", range(6))
def test_segmented_splits_partials_and_combine(seed):
    """Segmented splits: each query block's tile loop cut into S pieces.  Every
    piece must equal the oracle over exactly its keys (the block's tile
    interval from the oracle's tile bounds at the kernel's tiling: 128-row
    blocks, 32- or 64-key tiles), and the LSE combine of the S pieces the
    unsplit attention."""
    import paged_sliding_window_amd as psw
    from oracle import tile_bounds_ref
    rng = np.random.default_rng(900 + seed)
    d = int(rng.choice([64, 128, 256]))
    hkv = int(rng.choice([1, 2]))
    qpk = int(rng.choice([1, 2, 8]))
    w = make_small_case(900 + seed, num_seqs=int(rng.integers(1, 4)), max_len=700, hq=hkv * qpk,
                        hkv=hkv, d=d, block_size=16)
    gw = GpuWorkload(w)
    S = int(rng.choice([2, 3, 5]))
    parts, lses = gw.attention(num_splits=S, out_dtype=torch.float32)
    N, Hq = w.num_tokens, w.num_q_heads
    merged, merged_lse = psw.lse_combine([parts[j].reshape(N * Hq, d) for j in range(S)],
                                         [lses[j].reshape(N * Hq) for j in range(S)],
                                         out_dtype=torch.float32, out_lse=torch.empty(
                                             N * Hq, dtype=torch.float32, device="cuda"))
    parts, lses = parts.cpu().numpy(), lses.cpu().numpy()
    merged = merged.cpu().numpy().reshape(N, Hq, d)
    merged_lse = merged_lse.cpu().numpy().reshape(N, Hq)
    # the kernel's tiling (include/psw.h, segmented splits): 64-key tiles at head
    # dim 128 when a row spans more than 1,536 keys
    span = (1 << 30) if w.window <= 0 else (w.window if w.causal else 2 * w.window - 1)
    block_q, T = 128 // qpk, 64 if d == 128 and span > 1536 else 32
    use_mm = w.max_mm_ranges > 0 and (w.mm_ranges != 0).any()
    for r in range(w.num_seqs):
        s0, ql = int(w.query_start_loc[r]), int(w.query_lens[r])
        ref_o, ref_l = oracle_rows(w, r)
        assert_close(merged[s0:s0 + ql], ref_o, f"seq {r} combined")
        assert_lse_close(merged_lse[s0:s0 + ql], ref_l, f"seq {r} combined lse")
        for qb in range(-(-ql // block_q)):
            lo, hi, _ = tile_bounds_ref(int(w.context_lens[r]), int(w.seq_lens[r]), ql, qb, T,
                                        block_q * qpk, block_q, qpk, w.window, use_mm, w.causal,
                                        w.chunk_lookback, w.chunk_size, w.ranges_of(r))
            seg = -(-(hi - lo) // S) if hi > lo else 0
            rows = np.arange(qb * block_q, min(ql, (qb + 1) * block_q))
            for j in range(S):
                a = min(lo + j * seg, hi)
                b = min(hi, a + seg)
                o_j, l_j = oracle_rows(w, r, rows=rows, key_range=(a * T, b * T))
                assert_close(parts[j, s0 + rows], o_j, f"seq {r} block {qb} piece {j}")
                assert_lse_close(lses[j, s0 + rows], l_j, f"seq {r} block {qb} piece {j} lse")


def test_segmented_splits_rejected_for_the_latent_decode():
    import paged_sliding_window_amd as psw
    w = make_small_case(4, num_seqs=2, max_len=200, hq=32, hkv=1, d=576, dv=512, window=0,
                        causal=True, chunk=(0, -1), max_ranges=0, latent=True, block_size=64)
    gw = GpuWorkload(w)
    with pytest.raises(psw.PswError):
        gw.attention(num_splits=2, out_dtype=torch.float32)
