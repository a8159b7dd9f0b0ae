"""Pin for oracle.kv_cache_write_ref (no GPU): writing every position of each
request through the slot mapping and reading the cache back block by block in
table order gives the logical K rows again; pad slots are never written."""
import numpy as np

from oracle import kv_cache_write_ref, slot_mapping_ref
from workloads import make_small_case


def test_write_then_read_back_by_table_walk():
    w = make_small_case(41, num_seqs=3, max_len=200, block_size=16)
    B = w.block_size
    qsl = np.concatenate([[0], np.cumsum(w.seq_lens)]).astype(np.int32)
    pos = np.concatenate([np.arange(int(L)) for L in w.seq_lens])
    M = int(qsl[-1]) + 5
    slots = slot_mapping_ref(qsl, pos, w.block_table, B, M)
    new = np.concatenate([w.k_bits[r] for r in range(w.num_seqs)])
    new = np.concatenate([new, np.full((5,) + new.shape[1:], 7, dtype=new.dtype)])
    cache = np.zeros((w.num_blocks * B,) + new.shape[1:], dtype=new.dtype)
    cache = kv_cache_write_ref(cache, slots, new)
    for r in range(w.num_seqs):
        L = int(w.seq_lens[r])
        blocks = [cache[b * B:(b + 1) * B] for b in w.block_table[r] if b >= 0]
        assert np.array_equal(np.concatenate(blocks)[:L], w.k_bits[r])
    assert not (cache == 7).all(axis=tuple(range(1, cache.ndim))).any()
