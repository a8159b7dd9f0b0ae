"""GPU parity: slot mapping and KV-cache write, bit-exact against the oracle."""
import json
import os

import numpy as np
import pytest
import torch

import paged_sliding_window_amd as psw
from oracle import kv_cache_write_ref, slot_mapping_ref
from tests.gpu_setup import bits_to_bf16, i32, i64
from workloads import make_config, make_small_case

pytestmark = pytest.mark.gpu


def _gpu_slots(qsl, pos, bt, B, M):
    return psw.slot_mapping(i32(qsl), i64(pos), i32(bt), B, M).cpu().numpy()


def test_worked_example_from_the_page():
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                    "slot_mapping_worked_example.json")))
    rng = np.random.default_rng(53)
    bt = rng.integers(*g["block_table_entry_range"], size=tuple(g["block_table_shape"]),
                      dtype=np.int32)
    got = _gpu_slots(g["query_start_loc"], g["positions"], bt, g["block_size"], g["max_num_tokens"])
    ref = slot_mapping_ref(g["query_start_loc"], g["positions"], bt, g["block_size"],
                           g["max_num_tokens"])
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_workload_new_tokens(cfg):
    w = make_config(cfg)
    got = _gpu_slots(w.query_start_loc, w.positions, w.block_table, w.block_size, w.max_num_tokens)
    ref = slot_mapping_ref(w.query_start_loc, w.positions, w.block_table, w.block_size,
                           w.max_num_tokens)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("seed", range(8))
def test_random_with_empty_requests_and_invalid_positions(seed):
    rng = np.random.default_rng(seed)
    R = int(rng.integers(0, 40))
    B = int(rng.choice([1, 3, 16, 64, 128]))
    stride = int(rng.integers(1, 50))
    bt = rng.integers(-1, 1000, size=(max(R, 1), stride)).astype(np.int32)
    qls = rng.integers(0, 60, size=R) * (rng.random(R) > 0.2)
    qsl = np.concatenate([[0], np.cumsum(qls)]).astype(np.int32)
    N = int(qsl[-1])
    pos = rng.integers(-3, stride * B + 5, size=N).astype(np.int64)
    M = N + int(rng.integers(0, 70))
    got = _gpu_slots(qsl, pos, bt, B, M)
    ref = slot_mapping_ref(qsl, pos, bt, B, M)
    assert np.array_equal(got, ref)


def test_scaled_batch_million_tokens():
    rng = np.random.default_rng(77)
    R, B = 512, 16
    lens = rng.integers(512, 4096, size=R)
    need = -(-lens // B)
    bt = np.full((R, int(need.max())), -1, dtype=np.int32)
    perm = rng.permutation(int(need.sum())).astype(np.int32)
    off = 0
    for r in range(R):
        bt[r, :need[r]] = perm[off:off + need[r]]
        off += need[r]
    qsl = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    pos = np.concatenate([np.arange(L) for L in lens]).astype(np.int64)
    M = int(qsl[-1]) + 1000
    got = _gpu_slots(qsl, pos, bt, B, M)
    # oracle on a sample of requests (the scalar loop is slow at this size)
    for r in rng.choice(R, 24, replace=False):
        sub_qsl = np.array([0, lens[r]], dtype=np.int32)
        ref = slot_mapping_ref(sub_qsl, pos[qsl[r]:qsl[r + 1]], bt[r:r + 1], B, int(lens[r]))
        assert np.array_equal(got[qsl[r]:qsl[r + 1]], ref)
    assert (got[qsl[-1]:] == -1).all()


def test_bench_scaled_batch_41m_tokens():
    """The 41 M-token batch the bench times (20,000 requests, block 16):
    sampled requests bit-exact against the oracle, every pad slot -1, and every
    slot of the batch inside the pool and distinct (the tables partition it)."""
    from workloads.synth import make_slot_batch
    qsl, pos, bt = make_slot_batch(20000, 1024, 3072, 16, 7)
    n = int(qsl[-1])
    M = n + 65536
    got_t = psw.slot_mapping(i32(qsl), i64(pos), i32(bt), 16, M)
    pool = int((bt >= 0).sum()) * 16
    valid = got_t[:n]
    assert int(valid.min().item()) >= 0 and int(valid.max().item()) < pool
    assert torch.unique(valid).numel() == n
    assert bool((got_t[n:] == -1).all())
    got = got_t.cpu().numpy()
    rng = np.random.default_rng(41)
    for r in rng.choice(len(qsl) - 1, 16, replace=False):
        L = int(qsl[r + 1] - qsl[r])
        ref = slot_mapping_ref(np.array([0, L], dtype=np.int32), pos[qsl[r]:qsl[r + 1]],
                               bt[r:r + 1], 16, L)
        assert np.array_equal(got[qsl[r]:qsl[r + 1]], ref), f"request {r}"


@pytest.mark.parametrize("latent", [False, True])
def test_kv_cache_write_bit_exact(latent):
    w = make_small_case(5, num_seqs=4, max_len=300, hq=8, hkv=2, d=64, block_size=16,
                        latent=latent)
    B = w.block_size
    slots = slot_mapping_ref(w.query_start_loc, w.positions, w.block_table, B, w.max_num_tokens)
    k_new = np.concatenate([w.k_bits[r][w.context_lens[r]:] for r in range(w.num_seqs)])
    v_new = None if latent else np.concatenate([w.v_bits[r][w.context_lens[r]:]
                                                for r in range(w.num_seqs)])
    rng = np.random.default_rng(9)
    k0 = rng.integers(0, 65535, size=(w.num_blocks * B,) + k_new.shape[1:], dtype=np.uint16)
    kc = bits_to_bf16(k0).view(w.num_blocks, B, *k_new.shape[1:]).contiguous()
    vc = None
    if not latent:
        v0 = rng.integers(0, 65535, size=(w.num_blocks * B,) + v_new.shape[1:], dtype=np.uint16)
        vc = bits_to_bf16(v0).view(w.num_blocks, B, *v_new.shape[1:]).contiguous()
    psw.kv_cache_write(bits_to_bf16(k_new), None if latent else bits_to_bf16(v_new),
                       i32(slots), kc, vc)
    got_k = kc.view(torch.int16).cpu().numpy().view(np.uint16).reshape(k0.shape)
    assert np.array_equal(got_k, kv_cache_write_ref(k0, slots, k_new))
    if not latent:
        got_v = vc.view(torch.int16).cpu().numpy().view(np.uint16).reshape(v0.shape)
        assert np.array_equal(got_v, kv_cache_write_ref(v0, slots, v_new))


@pytest.mark.parametrize("R", [1, 2, 63, 64, 65, 4095, 4096, 4097, 20000])
def test_request_search_across_counts(R):
    """Many short and empty requests: the request of each token is found by a
    64-way search per wave (one to three rounds over these counts), then per
    lane a galloping search to the lane's first token and the read-ahead
    boundaries across the lane's own tokens."""
    rng = np.random.default_rng(1000 + R)
    B = 16
    lens = rng.integers(0, 9, size=R) * (rng.random(R) > 0.3)
    stride = 2
    bt = rng.integers(0, 5000, size=(R, stride)).astype(np.int32)
    qsl = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    N = int(qsl[-1])
    pos = rng.integers(0, stride * B, size=N).astype(np.int64)
    M = N + 37
    got = _gpu_slots(qsl, pos, bt, B, M)
    ref = slot_mapping_ref(qsl, pos, bt, B, M)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("R", [17, 64, 65])
def test_runs_of_empty_requests(R):
    """Most requests empty: a lane's few tokens cross dozens of boundaries,
    past the eight it reads ahead (with at most 64 requests the boundaries
    come from one load of the starts and lane shuffles, beyond 64 from the
    request search)."""
    rng = np.random.default_rng(500 + R)
    B = 16
    lens = np.zeros(R, dtype=np.int64)
    lens[rng.choice(R, size=max(1, R // 8), replace=False)] = rng.integers(1, 20, size=max(1, R // 8))
    lens[-1] = 0                      # trailing empty requests
    stride = 4
    bt = rng.integers(0, 9000, size=(R, stride)).astype(np.int32)
    qsl = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    N = int(qsl[-1])
    pos = rng.integers(0, stride * B, size=N).astype(np.int64)
    M = N + 11
    got = _gpu_slots(qsl, pos, bt, B, M)
    ref = slot_mapping_ref(qsl, pos, bt, B, M)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("R", [64, 511, 4096])
@pytest.mark.parametrize("B", [16, 64])
def test_decode_shaped_batches(R, B):
    """Decode batches: one new token per request at a late position (some
    requests empty), so a lane's first token lies up to several hundred
    requests past its wave's first one."""
    rng = np.random.default_rng(77 + R + B)
    lens = (rng.random(R) > 0.1).astype(np.int64)
    stride = 32768 // B + 1
    bt = rng.permutation(R * stride).reshape(R, stride).astype(np.int32)
    qsl = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    N = int(qsl[-1])
    pos = rng.integers(0, 32768, size=N).astype(np.int64)
    M = N + 5
    got = _gpu_slots(qsl, pos, bt, B, M)
    ref = slot_mapping_ref(qsl, pos, bt, B, M)
    assert np.array_equal(got, ref)


# ---- one context-parallel rank and the circular cache ----------------------

from oracle import slot_mapping_cp_ref  # noqa: E402


def _gpu_cp(qsl, pos, bt, B, M, kvb, world, rank, inter, circular=False):
    return psw.slot_mapping_cp(i32(qsl), i64(pos), i32(bt), B, M, kv_cache_block_size=kvb,
                               cp_world_size=world, cp_rank=rank, cp_interleave=inter,
                               circular=circular).cpu().numpy()


def test_cp_worked_example_from_the_page():
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                    "slot_mapping_cp_example.json")))
    pos = np.arange(384, dtype=np.int64)
    bt = np.array([[9, 2, 30, 1]], dtype=np.int32)
    for rank in range(g["cp_world_size"]):
        args = ([0, 384], pos, bt, g["block_size"], 400, g["kv_cache_block_size"],
                g["cp_world_size"], rank, g["cp_interleave"])
        assert np.array_equal(_gpu_cp(*args), slot_mapping_cp_ref(*args))


# (world, interleave, block size, kv-cache block size): powers of two take the
# shift path, the others the division path; world 1 is the plain mapping
CP_GEOMS = [(2, 128, 128, 128), (8, 16, 16, 64), (4, 1, 16, 16), (8, 64, 16, 128),
            (3, 16, 16, 64), (6, 4, 8, 24), (5, 3, 3, 9), (1, 4, 16, 64), (2, 8, 16, 32)]


@pytest.mark.parametrize("geom", CP_GEOMS)
def test_cp_random_batches_every_rank(geom):
    world, inter, B, kvb = geom
    rng = np.random.default_rng(sum(v * 31 ** i for i, v in enumerate(geom)))
    R = int(rng.integers(1, 12))
    stride = 40
    bt = rng.integers(-1, 3000, size=(R, stride)).astype(np.int32)
    qls = rng.integers(0, 200, size=R) * (rng.random(R) > 0.2)
    qsl = np.concatenate([[0], np.cumsum(qls)]).astype(np.int32)
    N = int(qsl[-1])
    span = stride * kvb * world // max(1, kvb // B) + 5
    pos = rng.integers(-3, span, size=N).astype(np.int64)
    M = N + int(rng.integers(0, 70))
    for rank in range(world):
        got = _gpu_cp(qsl, pos, bt, B, M, kvb, world, rank, inter)
        ref = slot_mapping_cp_ref(qsl, pos, bt, B, M, kvb, world, rank, inter)
        assert np.array_equal(got, ref), (geom, rank)


@pytest.mark.parametrize("B", [16, 12])
def test_circular_cache(B):
    rng = np.random.default_rng(B)
    R = 9
    bt = rng.integers(0, 500, size=(R, 3)).astype(np.int32)
    qls = rng.integers(0, 50, size=R)
    qsl = np.concatenate([[0], np.cumsum(qls)]).astype(np.int32)
    N = int(qsl[-1])
    pos = rng.integers(-5, 100000, size=N).astype(np.int64)
    got = _gpu_cp(qsl, pos, bt, B, N + 11, B, 1, 0, 1, circular=True)
    ref = slot_mapping_cp_ref(qsl, pos, bt, B, N + 11, B, 1, 0, 1, circular=True)
    assert np.array_equal(got, ref)


def test_cp_scaled_batch_sampled():
    """A large batch (about 1.1 M tokens) on ranks 0 and 5 of 8; the oracle
    checks a sample of requests, and over the 8 ranks every position of a
    sampled request is mapped by exactly one."""
    rng = np.random.default_rng(88)
    R, B, kvb, world, inter = 512, 16, 64, 8, 16
    lens = rng.integers(512, 4096, size=R)
    need = -(-lens // (kvb * world)) * (kvb // B)   # logical blocks one rank needs
    bt = np.full((R, int(need.max())), -1, dtype=np.int32)
    perm = rng.permutation(int(need.sum())).astype(np.int32)
    off = 0
    for r in range(R):
        bt[r, :need[r]] = perm[off:off + need[r]]
        off += need[r]
    qsl = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    pos = np.concatenate([np.arange(L) for L in lens]).astype(np.int64)
    M = int(qsl[-1]) + 1000
    outs = {rank: _gpu_cp(qsl, pos, bt, B, M, kvb, world, rank, inter) for rank in range(world)}
    owners = np.stack([outs[r][:qsl[-1]] != -1 for r in range(world)]).sum(axis=0)
    assert (owners == 1).all()
    for rank in (0, 5):
        for r in rng.choice(R, 12, replace=False):
            sub = np.array([0, lens[r]], dtype=np.int32)
            ref = slot_mapping_cp_ref(sub, pos[qsl[r]:qsl[r + 1]], bt[r:r + 1], B, int(lens[r]),
                                      kvb, world, rank, inter)
            assert np.array_equal(outs[rank][qsl[r]:qsl[r + 1]], ref)
        assert (outs[rank][qsl[-1]:] == -1).all()


def test_cp_invalid_geometry_is_rejected():
    qsl, pos, bt = i32([0, 2]), i64([0, 1]), i32(np.zeros((1, 4)))
    for kw in (dict(kv_cache_block_size=24), dict(cp_interleave=3), dict(cp_rank=2),
               dict(cp_world_size=0), dict(circular=True)):
        args = dict(kv_cache_block_size=32, cp_world_size=2, cp_rank=0, cp_interleave=8)
        args.update(kw)
        with pytest.raises(psw.PswError):
            psw.slot_mapping_cp(qsl, pos, bt, 16, 2, **args)
