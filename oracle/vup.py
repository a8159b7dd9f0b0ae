"""V-up projection of the merged latent attention output.

[DCP] "Terms" (MLA: after attention over the latent vectors, the output goes
through one V-up projection back to each head's V dimension), section 1.1 (the
merged output is batch-major and is V-up projected before the next layer) and
code block A (the batch-major input [tokens, heads, kv_lora_rank] is
multiplied per head by W_UV [heads, kv_lora_rank, v_head_dim], with no
transposes of the data):

    out[t, h, :] = x[t, h, :] @ W_UV[h]            out: [tokens, heads, v_head_dim]

float64, one matrix product per head.
"""
import numpy as np


def vup_projection_ref(x, w_uv):
    """x [T, H, R], w_uv [H, R, Dv] -> [T, H, Dv] (float64)."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w_uv, dtype=np.float64)
    T, H, R = x.shape
    if w.shape[:2] != (H, R):
        raise ValueError(f"w_uv {w.shape} does not match x {x.shape}")
    out = np.empty((T, H, w.shape[2]), dtype=np.float64)
    for h in range(H):
        out[:, h, :] = x[:, h, :] @ w[h]
    return out
