"""Write new K/V rows into the paged cache through the slot mapping.

[SLOT] section 1: the slot id is what attention and cache-write operators use
to read and write a token's K/V vector; a pad slot (-1) is never written.
The cache is viewed as rows indexed by slot (block * block size + offset).
"""
import numpy as np


def kv_cache_write_ref(cache_rows, slot_mapping, new_rows):
    """cache_rows: [num_slots, ...]; new_rows: [num_tokens, ...]; returns a copy."""
    out = np.array(cache_rows, copy=True)
    for t in range(new_rows.shape[0]):
        s = int(slot_mapping[t])
        if s >= 0:
            out[s] = new_rows[t]
    return out
