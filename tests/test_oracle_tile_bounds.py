"""Pins for oracle.tile_bounds_ref (no GPU).

Printed geometries come from [SWA-MM] (vLLM PR #53147 summary): the test kernel
of "Key source snippet" (4096 tokens, W 1024, T 32, BLOCK_M 16, BLOCK_Q 8,
2 queries per KV head, query block 140 = rows 1120..1127, two image-range slots)
and "Implementation breakdown" item 4 (non-causal right window unioned with a
range gives [3, 68)).  The mutation tests plant the mistakes that the page's
review found (and the last-row lower bound) in a copy of the oracle and check
that these pins catch each one.
"""
import inspect
import types

import numpy as np
import pytest

import oracle.tile_bounds as tb
from oracle import allowed_rows, tile_bounds_ref

GEOM = dict(context_len=0, seq_len=4096, query_len=4096, q_block_idx=140, tile_size=32,
            block_m=16, block_q=8, queries_per_kv=2, window=1024, use_mm=True)


def _printed_causal(fn):
    return fn(**GEOM, causal=True, chunk_lookback=-1, chunk_size=-1,
              ranges=[(1024, 2303), (0, 0)])


def _printed_noncausal(fn):
    return fn(**GEOM, causal=False, chunk_lookback=-1, chunk_size=-1,
              ranges=[(1024, 1535), (0, 0)])


def _chunk_case(fn):
    return fn(**GEOM, causal=True, chunk_lookback=1, chunk_size=512,
              ranges=[(256, 1535), (0, 0)])


def _first_row_case(fn):
    g = dict(GEOM, q_block_idx=131, use_mm=False)
    return fn(**g, causal=True, chunk_lookback=-1, chunk_size=-1, ranges=[])


def test_printed_causal_geometry():
    assert list(_printed_causal(tile_bounds_ref)) == [3, 72, 4096]


def test_printed_noncausal_right_window():
    lo, hi, msp = _printed_noncausal(tile_bounds_ref)
    assert (lo, hi) == (3, 68) and msp == 4096


def test_chunk_lookback_lower_bound_reopened_by_image():
    # chunk edge of row 1120 = (2 - 1) * 512 = 512 (tile 16); the image
    # [256, 1535] reopens keys from max(256, 97) = 256 (tile 8)
    assert _chunk_case(tile_bounds_ref)[:2] == (8, 48)


def test_first_row_lower_bound():
    # rows 1048..1055: row 1048 admits key 25, which lies in tile 0
    assert _first_row_case(tile_bounds_ref)[:2] == (0, 33)


def _allowed_tile_hull(ctx, seq_len, ql, qb, T, block_q, W, causal, C, lb, ranges):
    rows = np.arange(qb * block_q, min((qb + 1) * block_q, ql))
    m = allowed_rows(ctx + rows, seq_len, W, causal, C, lb, ranges)
    cols = np.nonzero(m.any(axis=0))[0]
    return int(cols[0]) // T, int(cols[-1]) // T + 1


def _random_cases(seed, n):
    rng = np.random.default_rng(seed)
    for _ in range(n):
        seq_len = int(rng.integers(1, 80))
        ql = int(rng.integers(1, seq_len + 1))
        ctx = seq_len - ql
        T = int(rng.choice([2, 4, 8]))
        qpk = int(rng.choice([1, 2, 4]))
        block_q = int(rng.choice([1, 2, 4, 8]))
        W = int(rng.integers(1, 40))
        causal = bool(rng.integers(0, 2))
        if rng.integers(0, 2):
            C, lb = int(rng.choice([2, 4, 8, 16])), int(rng.integers(0, 3))
        else:
            C, lb = -1, -1
        ranges = []
        for _ in range(int(rng.integers(0, 4))):
            s = int(rng.integers(0, seq_len))
            ranges.append((s, int(rng.integers(s, seq_len))))
        use_mm = bool(ranges) or bool(rng.integers(0, 2))
        yield ctx, seq_len, ql, T, qpk, block_q, W, causal, C, lb, ranges, use_mm


def _brute_force_violations(fn, seed=5, n=1500):
    """Count blocks whose interval misses an allowed key, or is looser than the
    allowed hull where the formula is meant to be tight."""
    unsafe = loose = 0
    for ctx, seq_len, ql, T, qpk, block_q, W, causal, C, lb, ranges, use_mm in _random_cases(seed, n):
        for qb in range(-(-ql // block_q)):
            lo, hi, _ = fn(ctx, seq_len, ql, qb, T, block_q * qpk, block_q, qpk, W, use_mm,
                           causal, lb, C, ranges)
            a_lo, a_hi = _allowed_tile_hull(ctx, seq_len, ql, qb, T, block_q, W, causal, C, lb,
                                            ranges if use_mm else [])
            if lo > a_lo or hi < a_hi:
                unsafe += 1
            tight_expected = lb < 0 or (lb + 1) * C <= W
            if tight_expected and (lo, hi) != (a_lo, a_hi):
                loose += 1
    return unsafe, loose


def test_brute_force_safe_and_tight():
    unsafe, loose = _brute_force_violations(tile_bounds_ref)
    assert unsafe == 0 and loose == 0


def test_without_window_the_interval_is_the_prefix():
    # causal, no window, no ranges: [0, ceil((q_hi + 1) / T))
    assert tile_bounds_ref(0, 100, 100, 3, 8, 4, 4, 1, 0, False, True, -1, 0, []) == (0, 2, 16)
    # non-causal, no window: every tile
    assert tile_bounds_ref(0, 100, 100, 3, 8, 4, 4, 1, 0, False, False, -1, 0, []) == (0, 13, 100)


# --- mutation checks: each planted mistake must fail at least one pin ---------

MUTATIONS = {
    "last_row_lower_bound": ("first = q_lo - window + 1", "first = q_hi - window + 1"),
    "drop_right_window": ("last = q_hi if causal else q_hi + window - 1", "last = q_hi"),
    "chunk_edge_only": ("first = min(first, max(s, q_lo - window + 1))", "first = first"),
    "image_end_not_unioned": ("last = max(last, e)", "last = last"),
    "first_version_upper_bound": ("last = max(last, e)", "last = max(q_hi, e)"),
    "exclusive_end_off_by_one": ("hi = min(last // tile_size + 1, num_tiles)",
                                 "hi = min(last // tile_size, num_tiles)"),
    "intersect_test_uses_first_row_only": ("s <= q_hi and e >= q_lo", "s <= q_lo and e >= q_lo"),
}


def _mutant(name):
    src = inspect.getsource(tb)
    old, new = MUTATIONS[name]
    assert src.count(old) == 1, name
    mod = types.ModuleType("mutant_" + name)
    exec(compile(src.replace(old, new), "<mutant>", "exec"), mod.__dict__)
    return mod.tile_bounds_ref


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name):
    fn = _mutant(name)
    caught = []
    if list(_printed_causal(fn)) != [3, 72, 4096]:
        caught.append("printed causal")
    if _printed_noncausal(fn)[:2] != (3, 68):
        caught.append("printed non-causal")
    if _chunk_case(fn)[:2] != (8, 48):
        caught.append("chunk")
    if _first_row_case(fn)[:2] != (0, 33):
        caught.append("first row")
    if not caught:
        unsafe, loose = _brute_force_violations(fn, n=400)
        if unsafe or loose:
            caught.append("brute force")
    assert caught, f"mutation {name} escaped every pin"
