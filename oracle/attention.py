"""Masked softmax attention over the logical (un-paged) keys, in float64.

Dense reference: for every new token i of a request (absolute position
q = context_len + i) and query head h (KV head h // (Hq / Hkv), the contiguous
GQA grouping of [SWA-MM] "Key source snippet", ``num_queries_per_kv``), the
scores are scale * q_h . k_j over the keys j allowed by ``oracle.mask`` (and,
for a split-KV partial, inside the partial's key range), followed by a plain
softmax and the weighted sum of the values.  The output also carries the
natural-log log-sum-exp of the scaled scores, the per-partial statistic that
[DCP] "Terms" and section 1.1 merge partials with.

Conventions (readings): a row with no allowed key has output 0 and LSE -inf.
The softmax scale is an argument (the pages do not fix it).
"""
import numpy as np

from .mask import allowed_rows
from .tile_bounds import tile_bounds_ref


def _softmax_rows(S, V):
    """S [n, m] with -inf for excluded keys, V [m, Dv] -> out [n, Dv], lse [n]."""
    n = S.shape[0]
    out = np.zeros((n, V.shape[1]), dtype=np.float64)
    lse = np.full(n, -np.inf, dtype=np.float64)
    if S.shape[1] == 0:
        return out, lse
    m = S.max(axis=1)
    ok = np.isfinite(m)
    if ok.any():
        P = np.exp(S[ok] - m[ok, None])
        l = P.sum(axis=1)
        out[ok] = (P @ V) / l[:, None]
        lse[ok] = m[ok] + np.log(l)
    return out, lse


def attention_ref(q, k, v, *, context_len, seq_len, scale, window, causal, chunk_size=0,
                  chunk_lookback=-1, ranges=(), key_range=None, rows=None, row_block=256):
    """q [query_len, Hq, D]; k [seq_len, Hkv, D]; v [seq_len, Hkv, Dv].

    Returns (out [n, Hq, Dv], lse [n, Hq]) float64 for the selected new-token
    indices ``rows`` (default: all).  ``key_range`` = (begin, end) restricts the
    keys to [begin, end) for a split-KV partial.
    """
    q = np.asarray(q)
    hq, hkv = q.shape[1], k.shape[1]
    qpk = hq // hkv
    rows = np.arange(q.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    kb, ke = (0, seq_len) if key_range is None else (int(key_range[0]), int(key_range[1]))
    out = np.zeros((len(rows), hq, v.shape[2]), dtype=np.float64)
    lse = np.full((len(rows), hq), -np.inf, dtype=np.float64)
    for b0 in range(0, len(rows), row_block):
        blk = rows[b0: b0 + row_block]
        mask = allowed_rows(context_len + blk, seq_len, window, causal, chunk_size,
                            chunk_lookback, ranges, kb, ke)
        cols = np.nonzero(mask.any(axis=0))[0]
        if len(cols) == 0:
            continue
        # rows of the score matrix: (new token, query head of the group), all
        # query heads of one KV head stacked so one matmul serves the group
        mask = np.repeat(mask[:, cols], qpk, axis=0)
        for g in range(hkv):
            K = np.asarray(k[cols, g], dtype=np.float64)
            V = np.asarray(v[cols, g], dtype=np.float64)
            Q = np.asarray(q[blk, g * qpk:(g + 1) * qpk], dtype=np.float64).reshape(-1, q.shape[2])
            S = scale * (Q @ K.T)
            S[~mask] = -np.inf
            o, l = _softmax_rows(S, V)
            out[b0: b0 + len(blk), g * qpk:(g + 1) * qpk] = o.reshape(len(blk), qpk, -1)
            lse[b0: b0 + len(blk), g * qpk:(g + 1) * qpk] = l.reshape(len(blk), qpk)
    return out, lse


def attention_pruned_ref(q, k, v, *, context_len, seq_len, scale, window, causal, chunk_size=0,
                         chunk_lookback=-1, ranges=(), tile_size=32, block_q=8):
    """The method on the CPU: each query block (block_q positions x all query
    heads of one KV head) only looks at keys inside its tile interval from
    ``tile_bounds_ref``, with the mask applied inside those tiles.  Must equal
    ``attention_ref`` exactly up to summation order."""
    q = np.asarray(q)
    query_len, hq = q.shape[0], q.shape[1]
    hkv = k.shape[1]
    qpk = hq // hkv
    block_m = block_q * qpk
    use_mm = len(ranges) > 0
    out = np.zeros((query_len, hq, v.shape[2]), dtype=np.float64)
    lse = np.full((query_len, hq), -np.inf, dtype=np.float64)
    for qb in range(-(-query_len // block_q)):
        lo, hi, _ = tile_bounds_ref(context_len, seq_len, query_len, qb, tile_size, block_m,
                                    block_q, qpk, window, use_mm, causal, chunk_lookback,
                                    chunk_size, ranges)
        i0, i1 = qb * block_q, min((qb + 1) * block_q, query_len)
        keys = np.arange(lo * tile_size, min(hi * tile_size, seq_len))
        if len(keys) == 0:
            continue
        mask = allowed_rows(context_len + np.arange(i0, i1), seq_len, window, causal,
                            chunk_size, chunk_lookback, ranges)[:, keys]
        for g in range(hkv):
            K = np.asarray(k[keys, g], dtype=np.float64)
            V = np.asarray(v[keys, g], dtype=np.float64)
            for h in range(g * qpk, (g + 1) * qpk):
                S = scale * (np.asarray(q[i0:i1, h], dtype=np.float64) @ K.T)
                S[~mask] = -np.inf
                o, l = _softmax_rows(S, V)
                out[i0:i1, h] = o
                lse[i0:i1, h] = l
    return out, lse
