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
    64-way search per wave (one to three rounds over these counts) and then a
    per-lane walk across the request boundaries inside the lane's tokens."""
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
