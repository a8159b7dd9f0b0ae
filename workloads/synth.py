"""Seeded synthetic workloads.

Each workload is drawn from ``numpy.random.default_rng(seed)`` with the draws in
the order documented on each maker below, so that the same seed gives the same
tensors on every machine.  Values are N(0, 1) rounded to bfloat16 (round to
nearest even) and kept both as raw bf16 bit patterns (what the GPU receives) and
as float32 (exactly representable, what the oracle upcasts to float64).

Shapes follow the workloads of the pages:
  * vLLM PR #53147 summary (prhub), "Motivation": a Gemma-4 multimodal serving
    load of 60 images per request and a 16,550-token mean prefix;
  * the same page, "Key source snippet": a 4096-token geometry with a
    1024-token window and 32-token tiles;
  * vllm-ascend slot-mapping article, section 5: 2 requests of 5 tokens,
    block size 128, 8192 padded tokens;
  * MLA DCP decode notes (PR #16977), "Terms" and section 3.1: a 512-wide latent
    plus a 64-wide rope part, history/current partials merged by LSE.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

CONFIG_NAMES = {
    1: "tiny_prefill_256",
    2: "gemma_mm_prefill_16550",
    3: "batched_chunked_prefill_8seq",
    4: "noncausal_chunk_lookback_2x4096",
    5: "mla_splitkv_decode_b64",
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if not np.isfinite(x).all():
        raise ValueError("only finite values are rounded")
    u = x.view(np.uint32)
    r = (u >> 16) & np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u  # finite inputs stay below 2**32 after adding at most 0x8000
    r >>= 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _normal_bf16(rng: np.random.Generator, shape) -> np.ndarray:
    return f32_to_bf16_bits(rng.standard_normal(size=shape, dtype=np.float32))


@dataclass
class Workload:
    """One batch of synthetic input for the paged attention path.

    Token layout: the new tokens of request ``r`` occupy rows
    ``query_start_loc[r] : query_start_loc[r+1]`` of ``q_bits``; their logical
    positions are ``context_lens[r] + 0 .. query_lens[r]-1``.
    ``k_bits[r]`` / ``v_bits[r]`` hold the logical (un-paged) keys and values of
    request ``r`` for positions ``0 .. seq_lens[r]-1``; ``v_bits`` is None for
    the latent (MLA) layout, where V is the first ``head_dim_v`` columns of K.
    """

    name: str
    seed: int
    num_seqs: int
    query_lens: np.ndarray          # int64 [R]
    context_lens: np.ndarray        # int64 [R]
    seq_lens: np.ndarray            # int64 [R]
    query_start_loc: np.ndarray     # int32 [R+1]
    positions: np.ndarray           # int64 [N]
    max_num_tokens: int
    block_size: int
    num_blocks: int                 # physical pool size
    block_table: np.ndarray         # int32 [R, stride]; unused entries -1
    num_q_heads: int
    num_kv_heads: int
    head_dim_qk: int
    head_dim_v: int
    window: int
    causal: bool
    chunk_size: int
    chunk_lookback: int             # < 0: off
    mm_ranges: np.ndarray           # int32 [R, max_mm_ranges, 2], inclusive; (0,0) pads
    scale: float
    q_bits: np.ndarray              # uint16 [N, Hq, Dqk]
    k_bits: List[np.ndarray]        # uint16 [seq_len, Hkv, Dqk] per request
    v_bits: Optional[List[np.ndarray]]  # uint16 [seq_len, Hkv, Dv] per request, or None
    key_ranges: Optional[np.ndarray] = None   # int32 [S, R, 2] history splits, or None
    current_ranges: Optional[np.ndarray] = None  # int32 [1, R, 2], or None
    tile_size_geometry: int = 32
    notes: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def num_tokens(self) -> int:
        return int(self.query_start_loc[-1])

    @property
    def max_mm_ranges(self) -> int:
        return int(self.mm_ranges.shape[1])

    def q_f32(self) -> np.ndarray:
        return bf16_bits_to_f32(self.q_bits)

    def k_f32(self, r: int) -> np.ndarray:
        return bf16_bits_to_f32(self.k_bits[r])

    def v_f32(self, r: int) -> np.ndarray:
        if self.v_bits is None:
            return bf16_bits_to_f32(self.k_bits[r][..., : self.head_dim_v])
        return bf16_bits_to_f32(self.v_bits[r])

    def ranges_of(self, r: int):
        """Inclusive (start, end) pairs of request r, padding included."""
        return [(int(s), int(e)) for s, e in self.mm_ranges[r]]


def _block_tables(rng, seq_lens, block_size, stride=None):
    """Partition a randomly permuted pool of exactly enough physical blocks."""
    need = [-(-int(L) // block_size) for L in seq_lens]
    pool = int(sum(need))
    perm = rng.permutation(pool).astype(np.int32)
    stride = max(need) if stride is None else stride
    bt = np.full((len(seq_lens), stride), -1, dtype=np.int32)
    off = 0
    for r, n in enumerate(need):
        bt[r, :n] = perm[off: off + n]
        off += n
    return bt, pool


def _place_ranges(rng, total: int, lengths: List[int]) -> List[tuple]:
    """Non-overlapping inclusive ranges of the given lengths inside [0, total).

    Lengths that no longer fit are dropped (last first); the free tokens are
    spread into len+1 gaps by sorted uniform cut points.
    """
    lengths = list(lengths)
    while lengths and sum(lengths) > total:
        lengths.pop()
    n = len(lengths)
    if n == 0:
        return []
    free = total - sum(lengths)
    cuts = np.sort(rng.integers(0, free + 1, size=n))
    gaps = np.diff(np.concatenate([[0], cuts]))
    out = []
    pos = 0
    for g, ln in zip(gaps, lengths):
        pos += int(g)
        out.append((pos, pos + ln - 1))
        pos += ln
    return out


def _pack_ranges(per_seq: List[List[tuple]], max_ranges: int) -> np.ndarray:
    arr = np.zeros((len(per_seq), max(max_ranges, 1), 2), dtype=np.int32)
    for r, lst in enumerate(per_seq):
        for i, (s, e) in enumerate(lst):
            arr[r, i] = (s, e)
    return arr


def _assemble(name, seed, rng, query_lens, context_lens, block_size, hq, hkv, dqk, dv,
              window, causal, chunk_size, chunk_lookback, ranges_per_seq, max_ranges,
              max_num_tokens=None, latent=False, scale=None, bt_stride=None, notes=""):
    """Draw block tables, then Q, then K (and V) per request, in that order."""
    query_lens = np.asarray(query_lens, dtype=np.int64)
    context_lens = np.asarray(context_lens, dtype=np.int64)
    seq_lens = query_lens + context_lens
    qsl = np.zeros(len(query_lens) + 1, dtype=np.int32)
    qsl[1:] = np.cumsum(query_lens)
    positions = np.concatenate(
        [np.arange(c, c + q, dtype=np.int64) for c, q in zip(context_lens, query_lens)]
    ) if len(query_lens) else np.zeros(0, dtype=np.int64)
    n = int(qsl[-1])
    bt, pool = _block_tables(rng, seq_lens, block_size, bt_stride)
    q_bits = _normal_bf16(rng, (n, hq, dqk))
    k_bits, v_bits = [], ([] if not latent else None)
    for L in seq_lens:
        k_bits.append(_normal_bf16(rng, (int(L), hkv, dqk)))
        if not latent:
            v_bits.append(_normal_bf16(rng, (int(L), hkv, dv)))
    return Workload(
        name=name, seed=seed, num_seqs=len(query_lens), query_lens=query_lens,
        context_lens=context_lens, seq_lens=seq_lens, query_start_loc=qsl,
        positions=positions, max_num_tokens=int(max_num_tokens if max_num_tokens else n),
        block_size=block_size, num_blocks=pool, block_table=bt, num_q_heads=hq,
        num_kv_heads=hkv, head_dim_qk=dqk, head_dim_v=dv, window=window, causal=causal,
        chunk_size=chunk_size, chunk_lookback=chunk_lookback,
        mm_ranges=_pack_ranges(ranges_per_seq, max_ranges),
        scale=float(scale if scale is not None else 1.0 / np.sqrt(dqk)),
        q_bits=q_bits, k_bits=k_bits, v_bits=v_bits, notes=notes,
    )


def make_config(cfg: int, decode_splits: int = 8) -> Workload:
    """The five synthetic workloads; seed = 1000 + cfg.

    1 tiny prefill: 1 x 256 tokens, causal, W 64, block 16 (pool = permutation
      of 16 blocks), Hq 4 / Hkv 2, D 64, one image [64, 127], padded to 320.
    2 Gemma-style multimodal prefill: 1 x 16,550 tokens, causal, W 1024, Hq 16 /
      Hkv 8, D 256, block 16.  60 images of 256 tokens: leading text 64 + x0,
      gaps 1 + x_i, trailing x60, x ~ Multinomial(1067, 61 equal cells).
    3 batched chunked prefill: 8 requests, context U{0..4096}, chunk
      U{256..2048} (pair redrawn while the total is below 512), causal, W 512,
      Hq 8 / Hkv 1, D 128, block 16, 0-6 images of U{64..512} tokens each
      anywhere in [0, total), slot mapping padded to 16,384.
    4 non-causal with chunk lookback: 2 x 4096, W 1024, chunk 512, lookback 1,
      Hq 8 / Hkv 8, D 128, block 16, 4 images per request (three of U{64..512},
      one of U{1025..1536}, i.e. longer than the window), order shuffled.
    5 MLA-shaped split-KV decode: 64 requests x 1 new token, context length
      L ~ U{4096..32768} keys including the new one, 128 heads on one latent KV
      head of width 576 (V = first 512 columns), block 64, scale 1/sqrt(576);
      history keys [0, L-1) cut into ``decode_splits`` contiguous pieces at
      multiples of 64, current key [L-1, L).
    Draw order per config: the structural draws listed above, then the block
    table permutation, then Q, then K (and V) request by request.
    """
    seed = 1000 + cfg
    rng = np.random.default_rng(seed)
    name = CONFIG_NAMES[cfg]
    if cfg == 1:
        return _assemble(name, seed, rng, [256], [0], 16, 4, 2, 64, 64, 64, True, 0, -1,
                         [[(64, 127)]], 1, max_num_tokens=320)
    if cfg == 2:
        x = rng.multinomial(1067, [1.0 / 61] * 61)
        ranges = []
        pos = 64 + int(x[0])
        for i in range(60):
            ranges.append((pos, pos + 255))
            pos += 256
            if i < 59:
                pos += 1 + int(x[i + 1])
        assert pos + int(x[60]) == 16550
        return _assemble(name, seed, rng, [16550], [0], 16, 16, 8, 256, 256, 1024, True, 0, -1,
                         [ranges], 60)
    if cfg == 3:
        ctxs, chunks, ranges = [], [], []
        for _ in range(8):
            while True:
                c = int(rng.integers(0, 4097))
                q = int(rng.integers(256, 2049))
                if c + q >= 512:
                    break
            ctxs.append(c)
            chunks.append(q)
            nimg = int(rng.integers(0, 7))
            lens = [int(v) for v in rng.integers(64, 513, size=nimg)]
            ranges.append(_place_ranges(rng, c + q, lens))
        return _assemble(name, seed, rng, chunks, ctxs, 16, 8, 1, 128, 128, 512, True, 0, -1,
                         ranges, 6, max_num_tokens=16384)
    if cfg == 4:
        ranges = []
        for _ in range(2):
            lens = [int(v) for v in rng.integers(64, 513, size=3)] + [int(rng.integers(1025, 1537))]
            lens = [lens[i] for i in rng.permutation(4)]
            ranges.append(_place_ranges(rng, 4096, lens))
        return _assemble(name, seed, rng, [4096, 4096], [0, 0], 16, 8, 8, 128, 128, 1024, False,
                         512, 1, ranges, 4)
    if cfg == 5:
        lens = [int(v) for v in rng.integers(4096, 32769, size=64)]
        w = _assemble(name, seed, rng, [1] * 64, [L - 1 for L in lens], 64, 128, 1, 576, 512,
                      0, True, 0, -1, [[] for _ in lens], 1, latent=True,
                      scale=1.0 / np.sqrt(576.0))
        w.key_ranges = decode_split_ranges(w.seq_lens, decode_splits)
        w.current_ranges = np.stack(
            [np.stack([w.seq_lens - 1, w.seq_lens], axis=1)]).astype(np.int32)
        return w
    raise ValueError(f"unknown config {cfg}")


def decode_split_ranges(seq_lens, splits: int, align: int = 64) -> np.ndarray:
    """History key ranges [0, L-1) cut into ``splits`` pieces at multiples of
    ``align``; pieces past the end are empty (begin == end)."""
    out = np.zeros((splits, len(seq_lens), 2), dtype=np.int32)
    for r, L in enumerate(seq_lens):
        hist = int(L) - 1
        piece = -(-hist // splits)
        piece = -(-piece // align) * align
        for j in range(splits):
            b = min(j * piece, hist)
            e = min((j + 1) * piece, hist)
            out[j, r] = (b, e)
    return out


def make_small_case(seed: int, *, num_seqs=2, max_len=300, hq=4, hkv=2, d=64, dv=None,
                    block_size=16, window=None, causal=None, chunk=None, max_ranges=3,
                    latent=False) -> Workload:
    """A random small workload for property and parity tests.

    Draw order: per request (context, query length), then per request the
    image count and lengths and their placement, then window / causal / chunk
    choices not fixed by the caller, then block table, Q, K (and V).
    """
    rng = np.random.default_rng(seed)
    dv = d if dv is None else dv
    ctxs, qls, ranges = [], [], []
    for _ in range(num_seqs):
        total = int(rng.integers(1, max_len + 1))
        ql = int(rng.integers(1, total + 1))
        ctxs.append(total - ql)
        qls.append(ql)
    for r in range(num_seqs):
        total = ctxs[r] + qls[r]
        nimg = int(rng.integers(0, max_ranges + 1))
        lens = [int(v) for v in rng.integers(1, max(2, total // 2) + 1, size=nimg)]
        ranges.append(_place_ranges(rng, total, lens))
    if window is None:
        window = int(rng.choice([0, 1, 7, 16, 33, 64, 100]))
    if causal is None:
        causal = bool(rng.integers(0, 2))
    if chunk is None:
        chunk = (int(rng.choice([16, 32, 64])), int(rng.integers(0, 3))) if rng.integers(0, 3) == 0 else (0, -1)
    return _assemble(f"small_{seed}", seed, rng, qls, ctxs, block_size, hq, hkv, d, dv, window,
                     causal, chunk[0], chunk[1], ranges, max_ranges, latent=latent,
                     max_num_tokens=int(sum(qls)) + int(rng.integers(0, 64)))


def make_slot_batch(num_reqs: int, len_lo: int, len_hi: int, block_size: int, seed: int):
    """A large slot-mapping batch (not one of the five workloads): request
    lengths U{len_lo..len_hi}, every position of each request new, block tables
    a random permutation of an exactly sized pool (unused entries -1).
    Draw order: lengths, then the permutation.  Returns (query_start_loc int32
    [R+1], positions int64 [N], block_table int32 [R, stride])."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(len_lo, len_hi + 1, size=num_reqs)
    bt, _ = _block_tables(rng, lens, block_size)
    qsl = np.zeros(num_reqs + 1, dtype=np.int32)
    qsl[1:] = np.cumsum(lens)
    n = int(qsl[-1])
    # position of token t of request r = t - qsl[r]
    pos = np.arange(n, dtype=np.int64) - np.repeat(qsl[:-1].astype(np.int64), lens)
    return qsl, pos, bt
