"""Scalar slot mapping: logical token position -> physical KV-cache slot.

Follows [SLOT] section 1 (one program per request walks the request's tokens
between consecutive ``query_start_loc`` entries), section 2 (non-context-parallel
formula: logical block = position // block size, offset = the remainder,
physical block read from the request's block-table row, slot = physical block
* block size + offset) and section 4.3 / 5.1 (positions from ``num_tokens`` up
to ``max_num_tokens`` are filled with the pad id, -1).

Readings where the page is silent: a position that is negative, whose logical
block lies outside the table row, or whose table entry is negative (an unused
entry) also gets the pad id.
"""
import numpy as np

PAD_SLOT_ID = -1


def slot_mapping_ref(query_start_loc, positions, block_table, block_size, max_num_tokens,
                     pad_id=PAD_SLOT_ID):
    qsl = np.asarray(query_start_loc, dtype=np.int64)
    pos = np.asarray(positions, dtype=np.int64)
    bt = np.asarray(block_table, dtype=np.int64)
    num_reqs = len(qsl) - 1
    stride = bt.shape[1]
    out = np.full(int(max_num_tokens), pad_id, dtype=np.int32)
    for r in range(num_reqs):
        for t in range(int(qsl[r]), int(qsl[r + 1])):
            p = int(pos[t])
            if p < 0:
                continue
            logical_block = p // block_size
            offset = p % block_size
            if logical_block >= stride:
                continue
            physical_block = int(bt[r, logical_block])
            if physical_block < 0:
                continue
            out[t] = physical_block * block_size + offset
    return out
