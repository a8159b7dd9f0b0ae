"""Pins for oracle.attention_ref / attention_pruned_ref / lse_merge_ref (no GPU).

Special cases reduce to torch's CPU scaled_dot_product_attention in float64
(causal, full, banded masks built with torch.tril/triu, i.e. a construction
independent of oracle.mask); the pruned method must equal the dense reference;
removing the image ranges must move the output past the 2e-2 parity tolerance
([SWA-MM] "Implementation breakdown" item 4 and "Review highlights").
"""
import numpy as np
import pytest
import torch
from scipy.special import logsumexp

from oracle import allowed_rows, attention_pruned_ref, attention_ref, lse_merge_ref
from workloads import make_config, make_small_case


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _sdpa(q, k, v, scale, mask=None, causal=False):
    """torch SDPA, float64, CPU; q [n, Hq, D], k/v [m, Hkv, D] (GQA expanded)."""
    hq, hkv = q.shape[1], k.shape[1]
    K = np.repeat(k, hq // hkv, axis=1)
    V = np.repeat(v, hq // hkv, axis=1)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a.transpose(1, 0, 2)))
    m = None if mask is None else torch.from_numpy(mask)
    o = torch.nn.functional.scaled_dot_product_attention(t(q), t(K), t(V), attn_mask=m,
                                                         is_causal=causal, scale=scale)
    return o.numpy().transpose(1, 0, 2)


@pytest.mark.parametrize("hq,hkv", [(4, 2), (8, 1), (3, 3)])
def test_causal_full_window_is_textbook_causal(hq, hkv):
    n, d = 70, 16
    q, k, v = _rand((n, hq, d), 1), _rand((n, hkv, d), 2), _rand((n, hkv, d), 3)
    out, _ = attention_ref(q, k, v, context_len=0, seq_len=n, scale=0.3, window=0, causal=True)
    assert np.allclose(out, _sdpa(q, k, v, 0.3, causal=True), atol=1e-12, rtol=1e-12)
    out2, _ = attention_ref(q, k, v, context_len=0, seq_len=n, scale=0.3, window=n + 5,
                            causal=True)
    assert np.allclose(out2, out, atol=1e-14)


def test_noncausal_no_window_is_full_attention():
    n, d = 50, 8
    q, k, v = _rand((n, 2, d), 4), _rand((n, 1, d), 5), _rand((n, 1, d), 6)
    out, _ = attention_ref(q, k, v, context_len=0, seq_len=n, scale=0.5, window=0, causal=False)
    assert np.allclose(out, _sdpa(q, k, v, 0.5), atol=1e-12, rtol=1e-12)


@pytest.mark.parametrize("W,causal,ctx", [(5, True, 0), (9, False, 0), (7, True, 13)])
def test_banded_window_matches_torch_band_mask(W, causal, ctx):
    ql, d = 40, 8
    L = ctx + ql
    q, k, v = _rand((ql, 2, d), 7), _rand((L, 2, d), 8), _rand((L, 2, d), 9)
    ones = torch.ones(ql, L, dtype=torch.bool)
    upper = 0 if causal else W - 1
    band = torch.tril(ones, diagonal=ctx + upper) & torch.triu(ones, diagonal=ctx - W + 1)
    ref = _sdpa(q, k, v, 0.4, mask=band.numpy())
    out, _ = attention_ref(q, k, v, context_len=ctx, seq_len=L, scale=0.4, window=W, causal=causal)
    assert np.allclose(out, ref, atol=1e-12, rtol=1e-12)


def test_lse_is_logsumexp_of_allowed_scaled_scores():
    w = make_small_case(21, num_seqs=1, max_len=90, window=10, causal=True)
    q, k, v = w.q_f32().astype(np.float64), w.k_f32(0), w.v_f32(0)
    ctx, L = int(w.context_lens[0]), int(w.seq_lens[0])
    _, lse = attention_ref(q, k, v, context_len=ctx, seq_len=L, scale=w.scale, window=w.window,
                           causal=True, ranges=w.ranges_of(0))
    m = allowed_rows(ctx + np.arange(q.shape[0]), L, w.window, True, 0, -1, w.ranges_of(0))
    qpk = w.num_q_heads // w.num_kv_heads
    for h in range(w.num_q_heads):
        S = w.scale * q[:, h] @ k[:, h // qpk].astype(np.float64).T
        S[~m] = -np.inf
        assert np.allclose(lse[:, h], logsumexp(S, axis=1), atol=1e-12)


@pytest.mark.parametrize("seed", range(12))
def test_pruned_equals_dense_small(seed):
    w = make_small_case(100 + seed, num_seqs=1, max_len=200)
    ctx, L = int(w.context_lens[0]), int(w.seq_lens[0])
    kw = dict(context_len=ctx, seq_len=L, scale=w.scale, window=w.window, causal=w.causal,
              chunk_size=w.chunk_size, chunk_lookback=w.chunk_lookback, ranges=w.ranges_of(0))
    q, k, v = w.q_f32(), w.k_f32(0), w.v_f32(0)
    dense, lse_d = attention_ref(q, k, v, **kw)
    for T, bq in ((4, 2), (16, 8), (32, 1)):
        pruned, lse_p = attention_pruned_ref(q, k, v, tile_size=T, block_q=bq, **kw)
        assert np.allclose(pruned, dense, atol=1e-12, rtol=0)
        assert np.array_equal(np.isinf(lse_p), np.isinf(lse_d))
        fin = np.isfinite(lse_d)
        assert np.allclose(lse_p[fin], lse_d[fin], atol=1e-12)


@pytest.mark.parametrize("cfg", [1, 4])
def test_pruned_equals_dense_on_workloads(cfg):
    w = make_config(cfg)
    r = 0
    kw = dict(context_len=int(w.context_lens[r]), seq_len=int(w.seq_lens[r]), scale=w.scale,
              window=w.window, causal=w.causal, chunk_size=w.chunk_size,
              chunk_lookback=w.chunk_lookback, ranges=w.ranges_of(r))
    q = w.q_f32()[w.query_start_loc[r]:w.query_start_loc[r + 1]]
    if cfg == 4:
        q = q[:, :2]   # two query heads on two KV heads keeps the run short
        k, v = w.k_f32(r)[:, :2], w.v_f32(r)[:, :2]
    else:
        k, v = w.k_f32(r), w.v_f32(r)
    dense, _ = attention_ref(q, k, v, **kw)
    pruned, _ = attention_pruned_ref(q, k, v, tile_size=32, block_q=8, **kw)
    assert np.allclose(pruned, dense, atol=1e-12, rtol=0)


def test_image_ranges_change_the_output_past_tolerance():
    w = make_config(1)
    kw = dict(context_len=0, seq_len=256, scale=w.scale, window=w.window, causal=True)
    q, k, v = w.q_f32(), w.k_f32(0), w.v_f32(0)
    with_mm, _ = attention_ref(q, k, v, ranges=w.ranges_of(0), **kw)
    no_mm, _ = attention_ref(q, k, v, ranges=[], **kw)
    assert not np.allclose(with_mm, no_mm, atol=2e-2, rtol=2e-2)
    # rows outside the image are unchanged
    assert np.array_equal(with_mm[:64], no_mm[:64]) and np.array_equal(with_mm[128:], no_mm[128:])


def test_fully_masked_rows_are_zero_with_minus_inf_lse():
    q, k, v = _rand((4, 1, 4), 1), _rand((10, 1, 4), 2), _rand((10, 1, 4), 3)
    out, lse = attention_ref(q, k, v, context_len=6, seq_len=10, scale=1.0, window=2,
                             causal=True, key_range=(0, 3))
    assert (out == 0).all() and np.isneginf(lse).all()


# --- LSE merge ---------------------------------------------------------------

@pytest.mark.parametrize("seed", range(6))
def test_merge_of_key_splits_equals_single_softmax(seed):
    w = make_small_case(200 + seed, num_seqs=1, max_len=150)
    ctx, L = int(w.context_lens[0]), int(w.seq_lens[0])
    kw = dict(context_len=ctx, seq_len=L, scale=w.scale, window=w.window, causal=w.causal,
              chunk_size=w.chunk_size, chunk_lookback=w.chunk_lookback, ranges=w.ranges_of(0))
    q, k, v = w.q_f32(), w.k_f32(0), w.v_f32(0)
    full, lse_full = attention_ref(q, k, v, **kw)
    rng = np.random.default_rng(seed)
    cuts = sorted(set([0, L] + [int(c) for c in rng.integers(0, L + 1, size=3)]))
    parts = [attention_ref(q, k, v, key_range=(a, b), **kw) for a, b in zip(cuts[:-1], cuts[1:])]
    n, hq, dv = full.shape
    outs = [p[0].reshape(n * hq, dv) for p in parts]
    lses = [p[1].reshape(n * hq) for p in parts]
    merged, lse = lse_merge_ref(outs, lses)
    assert np.allclose(merged, full.reshape(n * hq, dv), atol=1e-12)
    fin = np.isfinite(lse_full.reshape(-1))
    assert np.array_equal(fin, np.isfinite(lse))
    assert np.allclose(lse[fin], lse_full.reshape(-1)[fin], atol=1e-12)
    # order of partials does not matter
    perm = rng.permutation(len(outs))
    merged2, _ = lse_merge_ref([outs[i] for i in perm], [lses[i] for i in perm])
    assert np.allclose(merged2, merged, atol=1e-13)


def test_merge_special_cases():
    rng = np.random.default_rng(3)
    o = rng.standard_normal((5, 7))
    l = rng.standard_normal(5)
    out, lse = lse_merge_ref([o], [l])
    assert np.allclose(out, o) and np.allclose(lse, l)
    # equal LSEs: plain average, lse + log 2
    o2 = rng.standard_normal((5, 7))
    out, lse = lse_merge_ref([o, o2], [l, l])
    assert np.allclose(out, (o + o2) / 2) and np.allclose(lse, l + np.log(2))
    # an empty partial carries no weight; all-empty rows are 0 / -inf
    ninf = np.full(5, -np.inf)
    out, lse = lse_merge_ref([o, np.full((5, 7), 123.0)], [l, ninf])
    assert np.allclose(out, o) and np.allclose(lse, l)
    out, lse = lse_merge_ref([o, o2], [ninf, ninf])
    assert (out == 0).all() and np.isneginf(lse).all()


def test_latent_decode_split_equals_unsplit_mqa():
    """MLA-shaped decode: K = latent row, V = its first Dv columns; history
    splits plus the current key, merged, equal one un-split softmax."""
    w = make_small_case(31, num_seqs=3, max_len=300, hq=16, hkv=1, d=72, dv=64, window=0,
                        causal=True, chunk=(0, -1), max_ranges=0, latent=True)
    for r in range(w.num_seqs):
        ctx, L = int(w.context_lens[r]), int(w.seq_lens[r])
        q = w.q_f32()[w.query_start_loc[r]:w.query_start_loc[r + 1]][-1:]
        k = w.k_f32(r)
        v = k[..., :64]
        kw = dict(context_len=L - 1, seq_len=L, scale=w.scale, window=0, causal=True)
        full, _ = attention_ref(q, k, v, **kw)
        ref = _sdpa(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64), w.scale)
        assert np.allclose(full, ref, atol=1e-12)
        cut = [0, (L - 1) // 3, L - 1, L]
        parts = [attention_ref(q, k, v, key_range=(a, b), **kw) for a, b in zip(cut[:-1], cut[1:])]
        merged, _ = lse_merge_ref([p[0][0] for p in parts], [p[1][0] for p in parts])
        assert np.allclose(merged, full[0], atol=1e-12)
