"""Per-query-block KV tile interval that can hold any allowed key.

[SWA-MM] "Implementation breakdown" items 1-2: with image ranges in the mask,
the tile loop of a query block must still skip tiles outside the window, so
its bounds become the union of the window interval of the block's rows and
the keys that any image range holding one of those rows opens up, each range
clamped on the left by the window of the row it reaches from.  Stated here
in terms of the block's rows:

  rows of the block: positions qpos_lo = q_block * BLOCK_Q up to
    qpos_hi = qpos_lo + (BLOCK_M - 1) // queries_per_kv, clamped to the
    request's last new token; absolute q = context_len + qpos.
  window part: consecutive rows slide the same window, so their union runs
    from the lower edge of the first row (q_lo - W + 1, or with chunk
    lookback the chunk edge of the first row, the page's choice; it ignores
    the window there) to the upper edge of the last row (q_hi causal,
    q_hi + W - 1 with the non-causal right window).
  image part: a valid range [s, e] that holds a row of the block lets that
    row see keys up to e and down to max(s, q - W + 1), so it widens the
    union to [max(s, q_lo - W + 1), e]; with image ranges the upper end is
    kept below seq_len.
  tiles = [max(0, first // T), min(last // T + 1, num_tiles)),
  num_tiles = ceil(max_seq_prefix_len / T); without a window nothing is
  pruned: [0, num_tiles).

tests/test_oracle_tile_bounds.py checks this against the mask's definition
directly (1,500 random geometries: every allowed key of every row lies inside
the interval, and the interval is exactly the tile hull of the allowed keys
wherever the chunk-edge choice does not widen it) and against the printed
geometries.

Readings where the page is silent or unsafe as printed:
  * The page computes the base lower bound from the block's LAST row.  That
    drops keys that earlier rows of the block may see (rows 1048-1055, W 1024,
    T 32: row 1048 admits key 25 in tile 0, the last-row form starts at tile 1).
    The block's FIRST row is used; both give the printed [3, 72).
  * max_seq_prefix_len = seq_len when image ranges are in use or the base is
    non-causal, else min(last row + 1, seq_len); only 4096 is printed.
  * A block with no rows (first position past the request's new tokens)
    visits no tile: (0, 0).
"""


def tile_bounds_ref(context_len, seq_len, query_len, q_block_idx, tile_size, block_m, block_q,
                    queries_per_kv, window, use_mm, causal, chunk_lookback, chunk_size, ranges):
    qpos_lo = q_block_idx * block_q
    qpos_hi = min(qpos_lo + (block_m - 1) // queries_per_kv, query_len - 1)
    q_lo = context_len + qpos_lo
    q_hi = context_len + qpos_hi
    if use_mm or not causal:
        max_seq_prefix_len = seq_len
    else:
        max_seq_prefix_len = min(q_hi + 1, seq_len)
    num_tiles = -(-max_seq_prefix_len // tile_size)
    if qpos_lo >= query_len:
        return 0, 0, max_seq_prefix_len
    if window > 0:
        if chunk_lookback >= 0:
            first = ((q_lo // chunk_size) - chunk_lookback) * chunk_size
        else:
            first = q_lo - window + 1
        last = q_hi if causal else q_hi + window - 1
        if use_mm:
            for s, e in ranges:
                if s < e and s <= q_hi and e >= q_lo:
                    first = min(first, max(s, q_lo - window + 1))
                    last = max(last, e)
            last = min(last, seq_len - 1)
        lo = max(0, first // tile_size)
        hi = min(last // tile_size + 1, num_tiles)
    else:
        lo, hi = 0, num_tiles
    return lo, hi, max_seq_prefix_len
