"""Pins for oracle.slot_mapping_ref (no GPU)."""
import json
import os

import numpy as np
import pytest

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


# ---- context-parallel interleave and circular cache ------------------------
# Each pin is a function of the mapping under test, so that the mutation test
# at the end can run it on copies of the oracle with a planted mistake.

import inspect  # noqa: E402
import types  # noqa: E402

import oracle.slot_mapping as sm  # noqa: E402
from oracle import slot_mapping_cp_ref  # noqa: E402

GOLDEN_CP = os.path.join(os.path.dirname(__file__), "golden", "slot_mapping_cp_example.json")


def _pin_worked_example(fn):
    g = json.load(open(GOLDEN_CP))
    bs = g["block_size"]
    pos = np.arange(384, dtype=np.int64)
    qsl = [0, 384]
    for bt_row in ([4, 5, 6, 7], [9, 2, 30, 1]):
        bt = np.array([bt_row], dtype=np.int32)
        outs = [fn(qsl, pos, bt, bs, 400, g["kv_cache_block_size"], g["cp_world_size"], rank,
                   g["cp_interleave"]) for rank in range(2)]
        for lo, hi, owner in g["owner_segments"]:
            for rank in range(2):
                seg = outs[rank][lo:hi + 1]
                ok = (seg != -1).all() if rank == owner else (seg == -1).all()
                if not ok:
                    return False
        # rank 0: positions 0..127 and 256..383 are local offsets 0..255 in order
        for lo, hi, first_local in g["rank0_local_offsets_of"]:
            local = first_local + np.arange(hi - lo + 1)
            expect = bt[0, local // bs].astype(np.int64) * bs + local % bs
            if not (outs[0][lo:hi + 1] == expect).all():
                return False
        if not ((outs[0][384:] == g["pad_id"]).all() and (outs[1][384:] == g["pad_id"]).all()):
            return False
    # with consecutive physical blocks the rank's slots are one contiguous range
    out0 = fn(qsl, pos, np.array([[4, 5, 6, 7]], np.int32), bs, 384, 128, 2, 0, 128)
    mine = out0[out0 != -1]
    return len(mine) == 256 and (mine == np.arange(4 * 128, 6 * 128)).all()


def _random_table(rng, R, stride, pool):
    return rng.permutation(pool)[:R * stride].reshape(R, stride).astype(np.int32)


def _pin_world_one_is_the_plain_mapping(fn):
    rng = np.random.default_rng(11)
    for _ in range(30):
        bs = int(rng.choice([1, 4, 16, 64]))
        kvb = bs * int(rng.choice([1, 2, 4]))
        inter = int(rng.choice([d for d in (1, 2, 4, 8, 16) if kvb % d == 0]))
        R, stride = 3, 40
        bt = _random_table(rng, R, stride, 4 * R * stride)
        qls = rng.integers(0, 30, size=R)
        qsl = np.concatenate([[0], np.cumsum(qls)]).astype(np.int32)
        pos = rng.integers(-2, stride * bs + 5, size=int(qsl[-1]))
        M = int(qsl[-1]) + 7
        if not (fn(qsl, pos, bt, bs, M, kvb, 1, 0, inter) == slot_mapping_ref(qsl, pos, bt, bs, M)).all():
            return False
    return True


def _owner_ordinal_slots(positions, bt_row, bs, world, inter, rank):
    """Independent construction from [SLOT] section 3's placement rule alone:
    position i lives on rank (i // interleave) % world, and a rank stores its
    positions in increasing order, so a position's local index is the number
    of smaller positions the same rank owns (counted one by one)."""
    top = int(max(positions)) + 1 if len(positions) else 0
    owner = [(i // inter) % world for i in range(top)]
    ordinal, seen = [0] * top, [0] * world
    for i in range(top):
        ordinal[i] = seen[owner[i]]
        seen[owner[i]] += 1
    out = []
    for p in positions:
        if p < 0 or owner[p] != rank:
            out.append(-1)
            continue
        li = ordinal[p]
        blk = li // bs
        out.append(-1 if blk >= len(bt_row) else int(bt_row[blk]) * bs + li % bs)
    return np.array(out, dtype=np.int64)


def _pin_owner_ordinal_construction(fn, cases=40):
    rng = np.random.default_rng(12)
    for _ in range(cases):
        world = int(rng.choice([2, 3, 4, 8]))
        bs = int(rng.choice([1, 2, 8, 16]))
        kvb = bs * int(rng.choice([1, 2, 4]))
        inter = int(rng.choice([d for d in (1, 2, 4, 8, 16) if kvb % d == 0]))
        bt = _random_table(rng, 1, 24, 200)
        n = int(rng.integers(1, 300))
        pos = rng.permutation(n).astype(np.int64)      # any order inside the request
        pos[rng.integers(0, n)] = -1                    # one invalid position
        for rank in range(world):
            got = fn([0, n], pos, bt, bs, n + 3, kvb, world, rank, inter)
            if not ((got[:n] == _owner_ordinal_slots(pos, bt[0], bs, world, inter, rank)).all()
                    and (got[n:] == -1).all()):
                return False
    return True


def _pin_circular(fn):
    bt = np.array([[6, 99, 98], [3, 97, 96]], dtype=np.int32)
    out = fn([0, 4, 7], [-3, 0, 17, 300, 15, -1, 16], bt, 16, 9, 16, 1, 0, 1, circular=True)
    # logical block 0 of the request's row, offset pos % 16; negative -> pad
    return out.tolist() == [-1, 96, 97, 96 + 300 % 16, 48 + 15, -1, 48, -1, -1]


CP_PINS = [_pin_worked_example, _pin_world_one_is_the_plain_mapping,
           _pin_owner_ordinal_construction, _pin_circular]


def test_cp_worked_example_from_the_page():
    assert _pin_worked_example(slot_mapping_cp_ref)


def test_cp_world_one_is_the_plain_mapping():
    assert _pin_world_one_is_the_plain_mapping(slot_mapping_cp_ref)


def test_cp_matches_the_owner_ordinal_construction():
    assert _pin_owner_ordinal_construction(slot_mapping_cp_ref)


def test_circular_cache():
    assert _pin_circular(slot_mapping_cp_ref)


def test_cp_every_position_has_exactly_one_owner():
    bt = np.arange(1024, dtype=np.int32)[None, :]   # long enough for every local block
    pos = np.arange(700, dtype=np.int64)
    for world, inter, bs, kvb in ((2, 16, 16, 32), (4, 1, 4, 8), (8, 8, 8, 64), (3, 2, 2, 4)):
        outs = np.stack([slot_mapping_cp_ref([0, 700], pos, bt, bs, 700, kvb, world, r, inter)
                         for r in range(world)])
        assert ((outs != -1).sum(axis=0) == 1).all()
        # each rank's slots are distinct (its table row maps blocks one to one)
        for r in range(world):
            mine = outs[r][outs[r] != -1]
            assert len(np.unique(mine)) == len(mine)


def test_invalid_geometry_raises():
    bt = np.array([[6, 99, 98]], dtype=np.int32)
    with pytest.raises(ValueError):   # circular with context parallelism (the page forbids it)
        slot_mapping_cp_ref([0, 1], [0], bt, 16, 1, 16, 2, 0, 1, circular=True)
    for bad in (dict(kv_cache_block_size=24), dict(cp_interleave=3), dict(cp_rank=2),
                dict(cp_world_size=0)):
        kw = dict(kv_cache_block_size=32, cp_world_size=2, cp_rank=0, cp_interleave=8)
        kw.update(bad)
        with pytest.raises(ValueError):
            slot_mapping_cp_ref([0, 1], [0], bt, 16, 1, **kw)


CP_MUTATIONS = {
    "owner_ignores_world": ("if (virtual_offset // inter) % world != rank:",
                            "if (virtual_offset // inter) != rank:"),
    "virtual_block_without_world": ("virtual_block_size = kvb * world", "virtual_block_size = kvb"),
    "local_offset_segment_not_scaled": (
        "local_offset = (virtual_offset // (world * inter)) * inter + virtual_offset % inter",
        "local_offset = (virtual_offset // (world * inter)) + virtual_offset % inter"),
    "local_offset_keeps_virtual_offset": (
        "local_offset = (virtual_offset // (world * inter)) * inter + virtual_offset % inter",
        "local_offset = virtual_offset"),
    "blocks_per_kv_block_ignored": (
        "logical_block = virtual_block * blocks_per_kv_block + local_offset // block_size",
        "logical_block = virtual_block + local_offset // block_size"),
    "circular_walks_the_table": ("logical_block = 0", "logical_block = p // block_size"),
}


@pytest.mark.parametrize("name", sorted(CP_MUTATIONS))
def test_cp_pins_catch_planted_mistake(name):
    src = inspect.getsource(sm)
    old, new = CP_MUTATIONS[name]
    assert src.count(old) == 1, name
    mod = types.ModuleType("mutant_" + name)
    exec(compile(src.replace(old, new), "<mutant>", "exec"), mod.__dict__)
    fn = mod.slot_mapping_cp_ref
    caught = [pin.__name__ for pin in CP_PINS if not pin(fn)]
    assert caught, f"mutation {name} escaped every pin"
