"""Merge split-KV partial attention results by their log-sum-exp.

[DCP] "Terms" (LSE), section 1.1 (the history and current partials each emit an
output and an LSE; merging them is mathematically one softmax over the
concatenated keys) and section 3.2 / code block D (the merge reads every
received history shard plus the local current partial).

With M = max_p lse_p, w_p = exp(lse_p - M):
  out = sum_p w_p * out_p / sum_p w_p,   lse = M + log(sum_p w_p).
Readings: a partial with lse = -inf has weight 0; when every partial is -inf
the row's output is 0 and its lse -inf.  Natural log, float64 here.
"""
import numpy as np


def lse_merge_ref(outs, lses):
    """outs: list of [rows, Dv]; lses: list of [rows] -> (out [rows, Dv], lse [rows])."""
    O = np.stack([np.asarray(o, dtype=np.float64) for o in outs])    # [P, rows, Dv]
    L = np.stack([np.asarray(l, dtype=np.float64) for l in lses])    # [P, rows]
    M = L.max(axis=0)
    rows, dv = O.shape[1], O.shape[2]
    out = np.zeros((rows, dv), dtype=np.float64)
    lse = np.full(rows, -np.inf, dtype=np.float64)
    ok = np.isfinite(M)
    if ok.any():
        W = np.exp(L[:, ok] - M[None, ok])               # exp(-inf) = 0
        den = W.sum(axis=0)
        out[ok] = np.einsum("pr,prd->rd", W, O[:, ok]) / den[:, None]
        lse[ok] = M[ok] + np.log(den)
    return out, lse
