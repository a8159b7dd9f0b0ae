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


def slot_mapping_cp_ref(query_start_loc, positions, block_table, block_size, max_num_tokens,
                        kv_cache_block_size, cp_world_size, cp_rank, cp_interleave,
                        circular=False, pad_id=PAD_SLOT_ID):
    """Slot mapping of one context-parallel rank, and of a circular cache.

    Context parallel ([SLOT] section 3.1, steps 1-5, in that order): the
    cp_world_size ranks' physical blocks of kv_cache_block_size tokens form one
    virtual block; a position belongs to this rank when its interleave segment
    inside the virtual block does (step 2); the rank's segments of a virtual
    block are laid end to end as local offsets (step 3); the logical block is
    the virtual block times the logical blocks per physical block
    (kv_cache_block_size / block_size, section 4.2) plus the local offset's
    block (step 4); the slot is read through the block table (step 5), and a
    position owned by another rank gets the pad id.

    Circular cache ([SLOT] section 2.2): the logical block is always 0 and the
    offset is the position modulo block_size; a negative position gets the pad
    id.  The page states that a circular cache is not allowed together with
    context parallelism; that combination raises.

    Readings: the interleave must divide kv_cache_block_size (otherwise the
    local offsets of one virtual block would run into the next one's logical
    blocks) and kv_cache_block_size must be a multiple of block_size; a
    negative position, a logical block past the table row or a negative table
    entry gets the pad id, as in slot_mapping_ref.
    """
    world, rank, inter = int(cp_world_size), int(cp_rank), int(cp_interleave)
    kvb = int(kv_cache_block_size)
    if world < 1 or not 0 <= rank < world or inter < 1 or block_size < 1:
        raise ValueError("invalid context-parallel geometry")
    if kvb % block_size != 0 or kvb % inter != 0:
        raise ValueError("kv_cache_block_size must be a multiple of block_size and interleave")
    if circular and world != 1:
        raise ValueError("a circular cache is not allowed with context parallelism")
    blocks_per_kv_block = kvb // block_size
    qsl = np.asarray(query_start_loc, dtype=np.int64)
    pos = np.asarray(positions, dtype=np.int64)
    bt = np.asarray(block_table, dtype=np.int64)
    stride = bt.shape[1]
    out = np.full(int(max_num_tokens), pad_id, dtype=np.int32)
    for r in range(len(qsl) - 1):
        for t in range(int(qsl[r]), int(qsl[r + 1])):
            p = int(pos[t])
            if p < 0:
                continue
            if circular:
                logical_block = 0
                offset = p % block_size
            else:
                # step 1: virtual block of the world's physical blocks
                virtual_block_size = kvb * world
                virtual_block = p // virtual_block_size
                virtual_offset = p % virtual_block_size
                # step 2: is this rank the owner of the position's segment?
                if (virtual_offset // inter) % world != rank:
                    continue
                # step 3: the rank's segments of the virtual block, end to end
                local_offset = (virtual_offset // (world * inter)) * inter + virtual_offset % inter
                # step 4: logical block and offset in it
                logical_block = virtual_block * blocks_per_kv_block + local_offset // block_size
                offset = local_offset % block_size
            # step 5: physical block through the table
            if logical_block >= stride:
                continue
            physical_block = int(bt[r, logical_block])
            if physical_block < 0:
                continue
            out[t] = physical_block * block_size + offset
    return out
