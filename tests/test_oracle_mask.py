"""Pins for oracle.mask (no GPU)."""
import numpy as np
import pytest

from oracle import allowed_ref, allowed_rows
from workloads import make_config, make_small_case


def _rand_geom(rng):
    seq_len = int(rng.integers(1, 48))
    window = int(rng.choice([0, 1, 2, 5, 9, 16, 64]))
    causal = bool(rng.integers(0, 2))
    if rng.integers(0, 2):
        chunk, lb = int(rng.choice([2, 4, 8])), int(rng.integers(0, 3))
    else:
        chunk, lb = 0, -1
    ranges = []
    for _ in range(int(rng.integers(0, 4))):
        s = int(rng.integers(0, seq_len))
        e = int(rng.integers(s, min(seq_len, s + 20)))
        ranges.append((s, e))
    if rng.integers(0, 3) == 0:
        ranges.append((0, 0))
    return seq_len, window, causal, chunk, lb, ranges


def test_vectorised_equals_scalar_definition():
    rng = np.random.default_rng(11)
    for _ in range(400):
        seq_len, W, causal, C, lb, ranges = _rand_geom(rng)
        q_abs = np.arange(seq_len)
        M = allowed_rows(q_abs, seq_len, W, causal, C, lb, ranges)
        for q in range(seq_len):
            for k in range(seq_len):
                assert M[q, k] == allowed_ref(q, k, seq_len, W, causal, C, lb, ranges)


def test_textbook_special_cases():
    n = 37
    full_causal = allowed_rows(np.arange(n), n, 0, True, 0, -1, [])
    assert (full_causal == (np.tri(n, n, 0) > 0)).all()
    assert allowed_rows(np.arange(n), n, 0, False, 0, -1, []).all()
    for W in (1, 4, 9):
        band = (np.tri(n, n, 0) > 0) & ~(np.tri(n, n, -W) > 0)
        assert (allowed_rows(np.arange(n), n, W, True, 0, -1, []) == band).all()
        sym = (np.tri(n, n, W - 1) > 0) & ~(np.tri(n, n, -W) > 0)
        assert (allowed_rows(np.arange(n), n, W, False, 0, -1, []) == sym).all()


def test_image_range_is_bidirectional_and_left_clamped():
    # range [10, 29], W = 8: row 12 sees keys 5..12 from the window and, from
    # the image, max(10, 12-8+1)=10 .. 29 (no right clamp)
    m = allowed_rows([12], 40, 8, True, 0, -1, [(10, 29)])[0]
    assert np.nonzero(m)[0].tolist() == list(range(5, 30))
    # row 25: window keys 18..25, image keys max(10, 18)=18 .. 29
    m = allowed_rows([25], 40, 8, True, 0, -1, [(10, 29)])[0]
    assert np.nonzero(m)[0].tolist() == list(range(18, 30))
    # a row outside the image gains nothing
    m = allowed_rows([31], 40, 8, True, 0, -1, [(10, 29)])[0]
    assert np.nonzero(m)[0].tolist() == list(range(24, 32))
    # (s, s) and (0, 0) are not valid ranges
    assert (allowed_rows([3], 10, 2, True, 0, -1, [(3, 3), (0, 0)])
            == allowed_rows([3], 10, 2, True, 0, -1, [])).all()


def test_every_row_is_one_interval_containing_q():
    rng = np.random.default_rng(12)
    for _ in range(300):
        seq_len, W, causal, C, lb, ranges = _rand_geom(rng)
        M = allowed_rows(np.arange(seq_len), seq_len, W, causal, C, lb, ranges)
        for q in range(seq_len):
            idx = np.nonzero(M[q])[0]
            assert M[q, q]
            assert idx[-1] - idx[0] + 1 == len(idx)


def _pairs_per_head(w, r=0, row_block=2048):
    total = 0
    ql = int(w.query_lens[r])
    for b0 in range(0, ql, row_block):
        rows = w.context_lens[r] + np.arange(b0, min(ql, b0 + row_block))
        total += int(allowed_rows(rows, int(w.seq_lens[r]), w.window, w.causal, w.chunk_size,
                                  w.chunk_lookback, w.ranges_of(r)).sum())
    return total


def test_gemma_workload_pair_count_closed_form():
    """16,550 causal rows with W = 1024: sum_q min(q + 1, 1024) base pairs; each
    256-token image adds 255 + 254 + ... + 0 look-ahead pairs, wherever it sits."""
    w = make_config(2)
    base = sum(min(q + 1, 1024) for q in range(16550))
    assert base == 16_423_424
    assert _pairs_per_head(w) == base + 60 * (255 * 256 // 2) == 18_381_824


def test_tiny_workload_pair_count_closed_form():
    """256 causal rows, W 64, one image [64, 127] (64 tokens, as wide as W):
    row q in the image sees keys max(64, q-63) .. 127, the rest sees the window."""
    w = make_config(1)
    expect = 0
    for q in range(256):
        if 64 <= q <= 127:
            expect += 127 - max(64, q - 63) + 1 + (max(64, q - 63) - max(0, q - 63))
        else:
            expect += min(q + 1, 64)
    assert _pairs_per_head(w) == expect


def test_chunk_lookback_restricts_base_only():
    # C = 4, lookback 1, W = 100, non-causal: row 9 (chunk 2) sees keys >= 4
    m = allowed_rows([9], 20, 100, False, 4, 1, [])[0]
    assert np.nonzero(m)[0].tolist() == list(range(4, 20))
    # an image [0, 12] re-enables keys 0..3 for row 9, clamped by W = 100 only
    m = allowed_rows([9], 20, 100, False, 4, 1, [(0, 12)])[0]
    assert np.nonzero(m)[0].tolist() == list(range(0, 20))


def test_key_range_intersection():
    w = make_small_case(3, num_seqs=1, max_len=60)
    L = int(w.seq_lens[0])
    full = allowed_rows(np.arange(L), L, w.window, w.causal, w.chunk_size, w.chunk_lookback,
                        w.ranges_of(0))
    part = allowed_rows(np.arange(L), L, w.window, w.causal, w.chunk_size, w.chunk_lookback,
                        w.ranges_of(0), 5, 17)
    expect = full.copy()
    expect[:, :5] = False
    expect[:, 17:] = False
    assert (part == expect).all()
