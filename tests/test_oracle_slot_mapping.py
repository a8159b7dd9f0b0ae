"""Pins for oracle.slot_mapping_ref (no GPU)."""
import json
import os

import numpy as np

from oracle import slot_mapping_ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "slot_mapping_worked_example.json")


def test_worked_example_from_the_page():
    g = json.load(open(GOLDEN))
    rng = np.random.default_rng(53)
    lo, hi = g["block_table_entry_range"]
    bt = rng.integers(lo, hi, size=tuple(g["block_table_shape"]), dtype=np.int32)
    out = slot_mapping_ref(g["query_start_loc"], g["positions"], bt, g["block_size"],
                           g["max_num_tokens"])
    assert out.dtype == np.int32 and out.shape == (8192,)
    # every position is below 128, so each token sits in logical block 0 of its row
    for t in range(5):
        assert out[t] == bt[0, 0] * 128 + t
        assert out[5 + t] == bt[1, 0] * 128 + t
    assert (out[10:] == g["pad_id"]).all()


def _concatenated_slots(row, n, block_size):
    """Independent construction: the physical slots of a request, in logical
    order, are the slot ranges of its table's blocks laid end to end."""
    slots = []
    for b in row:
        slots.extend(range(int(b) * block_size, int(b) * block_size + block_size))
        if len(slots) >= n:
            break
    return np.array(slots[:n], dtype=np.int64)


def test_matches_block_concatenation_on_long_requests():
    rng = np.random.default_rng(7)
    for block_size in (1, 16, 64, 128):
        R = 4
        lens = rng.integers(1, 5000, size=R)
        need = [-(-int(L) // block_size) for L in lens]
        perm = rng.permutation(sum(need)).astype(np.int32)
        stride = max(need) + 3
        bt = np.full((R, stride), -1, dtype=np.int32)
        off = 0
        for r, n in enumerate(need):
            bt[r, :n] = perm[off:off + n]
            off += n
        # a chunk of new tokens per request at an arbitrary offset
        starts = [int(rng.integers(0, L)) for L in lens]
        qls = [int(L) - s for L, s in zip(lens, starts)]
        qsl = np.concatenate([[0], np.cumsum(qls)]).astype(np.int32)
        pos = np.concatenate([np.arange(s, int(L)) for s, L in zip(starts, lens)])
        M = int(qsl[-1]) + 37
        out = slot_mapping_ref(qsl, pos, bt, block_size, M)
        for r in range(R):
            full = _concatenated_slots(bt[r], int(lens[r]), block_size)
            assert (out[qsl[r]:qsl[r + 1]] == full[starts[r]:]).all()
        assert (out[qsl[-1]:] == -1).all()
        # distinct requests own disjoint physical blocks, so slots are unique
        assert len(np.unique(out[:qsl[-1]])) == qsl[-1]


def test_invalid_positions_and_empty_requests_pad():
    bt = np.array([[3, 1, -1], [0, 2, 4]], dtype=np.int32)
    qsl = [0, 0, 4]          # request 0 empty
    pos = [-1, 47, 15, 16]   # negative; block 47 // 16 = 2 -> entry 4; 15 -> 0*16+15; 16 -> 2*16+0
    out = slot_mapping_ref(qsl, pos, bt, 16, 6)
    assert out.tolist() == [-1, 4 * 16 + 15, 15, 32, -1, -1]
    # logical block past the row and an unused (-1) entry both pad
    out = slot_mapping_ref([0, 2], [48, 40], bt[:1], 16, 2)
    assert out.tolist() == [-1, -1]
