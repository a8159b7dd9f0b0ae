"""Per-query-block KV tile interval that can hold any allowed key.

Follows [SWA-MM] "Implementation breakdown" items 1-2 and "Key source snippet"
(the union bounds of ``compute_tile_loop_bounds``):

  rows of the block: positions qpos_lo = q_block * BLOCK_Q up to
    qpos_hi = qpos_lo + (BLOCK_M - 1) // queries_per_kv, clamped to the
    request's last new token; absolute q = context_len + qpos.
  pruning applies only with a sliding window (the image ranges here are always
    window-clamped, and the reverse-window variant is not supported):
    first key = chunk-lookback edge of the block's first row when lookback >= 0,
                else first row - W + 1;
    last key  = last row (causal) or last row + W - 1 (non-causal right window);
    every valid image range that intersects the block's rows lowers first to
      max(range start, first row - W + 1) and raises last to the range end;
    last is clamped to seq_len - 1 when image ranges are in use;
    tiles = [max(0, first // T), min(last // T + 1, num_tiles)).
  without a window the interval is [0, num_tiles).
  num_tiles = ceil(max_seq_prefix_len / T).

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
