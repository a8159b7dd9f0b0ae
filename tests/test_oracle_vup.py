"""Pins for oracle.vup_projection_ref (no GPU).

Closed forms (identity projection, one-hot rows) and the reason the step can
follow the merge at all: with the latent cache shared by every head, the
attention output projected by W_UV equals attention whose values are the
latent rows already projected by that head's W_UV (softmax(s) (C W) =
(softmax(s) C) W), computed here by the attention oracle with per-head values.
"""
import numpy as np

from oracle import attention_ref, vup_projection_ref


def test_identity_projection_returns_the_input():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 3, 8))
    w = np.stack([np.eye(8)] * 3)
    assert np.array_equal(vup_projection_ref(x, w), x)


def test_one_hot_rows_select_rows_of_each_heads_matrix():
    rng = np.random.default_rng(2)
    T, H, R, Dv = 6, 4, 16, 5
    w = rng.standard_normal((H, R, Dv))
    r = rng.integers(0, R, size=(T, H))
    x = np.zeros((T, H, R))
    for t in range(T):
        for h in range(H):
            x[t, h, r[t, h]] = 1.0
    out = vup_projection_ref(x, w)
    for t in range(T):
        for h in range(H):
            assert np.array_equal(out[t, h], w[h, r[t, h]])


def test_projection_commutes_with_latent_attention():
    rng = np.random.default_rng(3)
    L, H, D, R, Dv = 40, 4, 24, 16, 6
    q = rng.standard_normal((1, H, D))
    c = rng.standard_normal((L, 1, D))             # one latent row per key, shared by all heads
    w = rng.standard_normal((H, R, Dv))
    o, _ = attention_ref(q, c, c[:, :, :R], context_len=L - 1, seq_len=L, scale=0.2, window=0,
                         causal=True)
    lhs = vup_projection_ref(o, w)                 # project after attention
    # per-head values c[:, :R] @ W_h, keys repeated per head (one KV head per query head)
    v_h = np.stack([c[:, 0, :R] @ w[h] for h in range(H)], axis=1)
    k_h = np.repeat(c, H, axis=1)
    rhs, _ = attention_ref(q, k_h, v_h, context_len=L - 1, seq_len=L, scale=0.2, window=0,
                           causal=True)
    assert np.allclose(lhs, rhs, atol=1e-12, rtol=1e-12)
