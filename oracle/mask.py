"""Which keys an absolute query position may attend to.

Definition ([SWA-MM] "Implementation breakdown" items 1-2, "Key source
snippet", "Review highlights"): the image (multimodal-prefix) mask is OR-ed onto
the base mask.

  base, causal:      q - W + 1 <= k <= q            (W <= 0: no window, k <= q)
  base, non-causal:  |q - k| < W                    (W <= 0: every key)
  chunk lookback:    when lookback >= 0 the base is further restricted to
                     k >= ((q // C) - lookback) * C  (reading: the chunk limit is
                     AND-ed with the window; the page says chunking restricts the
                     base mask)
  image:             q and k inside the same range [s, e] (inclusive, absolute
                     positions, valid only when s < e) and k >= q - W + 1
                     (clamped to the window's left edge only; no right clamp)
  allowed = (base or image) and 0 <= k < seq_len.
"""
import numpy as np


def allowed_ref(q, k, seq_len, window, causal, chunk_size, chunk_lookback, ranges):
    """Scalar form of the definition, for brute force on tiny inputs."""
    if k < 0 or k >= seq_len:
        return False
    if causal:
        base = k <= q and (window <= 0 or k >= q - window + 1)
    else:
        base = window <= 0 or abs(q - k) < window
    if chunk_lookback >= 0:
        base = base and k >= ((q // chunk_size) - chunk_lookback) * chunk_size
    image = False
    for s, e in ranges:
        if s < e and s <= q <= e and s <= k <= e and (window <= 0 or k >= q - window + 1):
            image = True
    return base or image


def allowed_rows(q_abs, seq_len, window, causal, chunk_size, chunk_lookback, ranges,
                 key_begin=0, key_end=None):
    """Vectorised form: bool [len(q_abs), seq_len] (same definition, optionally
    intersected with a key range [key_begin, key_end))."""
    q = np.asarray(q_abs, dtype=np.int64)[:, None]
    k = np.arange(seq_len, dtype=np.int64)[None, :]
    if causal:
        base = k <= q
        if window > 0:
            base = base & (k >= q - window + 1)
    else:
        base = np.abs(q - k) < window if window > 0 else np.ones_like(k >= q)
    if chunk_lookback >= 0:
        base = base & (k >= ((q // chunk_size) - chunk_lookback) * chunk_size)
    image = np.zeros_like(base)
    q_min, q_max = (int(q.min()), int(q.max())) if q.size else (0, -1)
    for s, e in ranges:
        if s < e and s <= q_max and e >= q_min:   # ranges no row lies in add nothing
            inr = (q >= s) & (q <= e) & (k >= s) & (k <= e)
            if window > 0:
                inr = inr & (k >= q - window + 1)
            image |= inr
    out = base | image
    if key_end is None:
        key_end = seq_len
    out &= (k >= key_begin) & (k < key_end)
    return out


def row_interval_ref(q, seq_len, window, causal, chunk_size, chunk_lookback, ranges):
    """(first, last) allowed key of row q, or None when the row allows nothing;
    used only by tests that check every row's allowed set is one interval."""
    m = allowed_rows([q], seq_len, window, causal, chunk_size, chunk_lookback, ranges)[0]
    idx = np.nonzero(m)[0]
    if len(idx) == 0:
        return None
    return int(idx[0]), int(idx[-1])
