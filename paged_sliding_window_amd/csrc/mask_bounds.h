// The mask and the per-query-block tile interval, as device functions shared by
// the attention kernels and the tile-bounds test export.
//
// Mask: vLLM PR #53147 summary, "Implementation breakdown" items 1-2 and
// "Review highlights": the window-clamped image mask is OR-ed onto the base
// (causal or bidirectional) window, optionally restricted by a chunk lookback.
// Tile interval: the same page, "Key source snippet" (union of the base window
// and every image range intersecting the block, converted to KV tiles), taking
// the lower bound from the block's first row so no allowed key is dropped.
#pragma once
#include <stdint.h>

namespace psw {

struct MaskGeom {
  int window;          // > 0 sliding window, <= 0 none
  int causal;          // 1 causal base, 0 bidirectional base
  int chunk_size;      // used when chunk_lookback >= 0
  int chunk_lookback;  // < 0 off
};

__host__ __device__ inline int64_t floordiv64(int64_t a, int64_t b) {
  int64_t q = a / b;
  return (q * b != a && ((a < 0) != (b < 0))) ? q - 1 : q;
}

struct TileRange {
  int lo, hi, max_seq_prefix_len;
};

// ranges: this request's [max_ranges][2] inclusive (start, end); nullptr = no images.
__host__ __device__ inline TileRange tile_bounds(int context_len, int seq_len, int query_len,
                                                 int q_block, int tile, int block_m, int block_q,
                                                 int queries_per_kv, const MaskGeom& g,
                                                 const int32_t* ranges, int max_ranges) {
  const bool use_mm = ranges != nullptr && max_ranges > 0;
  const int64_t qpos_lo = (int64_t)q_block * block_q;
  int64_t qpos_hi = qpos_lo + (block_m - 1) / queries_per_kv;
  if (qpos_hi > query_len - 1) qpos_hi = query_len - 1;
  const int64_t q_lo = context_len + qpos_lo, q_hi = context_len + qpos_hi;
  int64_t msp = (use_mm || !g.causal) ? seq_len : (q_hi + 1 < seq_len ? q_hi + 1 : seq_len);
  const int num_tiles = (int)((msp + tile - 1) / tile);
  TileRange r;
  r.max_seq_prefix_len = (int)msp;
  if (qpos_lo >= query_len) {
    r.lo = 0;
    r.hi = 0;
    return r;
  }
  if (g.window > 0) {
    int64_t first = g.chunk_lookback >= 0
                        ? (floordiv64(q_lo, g.chunk_size) - g.chunk_lookback) * g.chunk_size
                        : q_lo - g.window + 1;
    int64_t last = g.causal ? q_hi : q_hi + g.window - 1;
    if (use_mm) {
      for (int i = 0; i < max_ranges; ++i) {
        const int64_t s = ranges[2 * i], e = ranges[2 * i + 1];
        if (s < e && s <= q_hi && e >= q_lo) {
          const int64_t lo_img = s > q_lo - g.window + 1 ? s : q_lo - g.window + 1;
          if (lo_img < first) first = lo_img;
          if (e > last) last = e;
        }
      }
      if (last > seq_len - 1) last = seq_len - 1;
    }
    int64_t lo = floordiv64(first, tile);
    if (lo < 0) lo = 0;
    int64_t hi = floordiv64(last, tile) + 1;
    if (hi > num_tiles) hi = num_tiles;
    r.lo = (int)lo;
    r.hi = (int)hi;
  } else {
    r.lo = 0;
    r.hi = num_tiles;
  }
  return r;
}

// Allowed keys of absolute query q as one closed interval [lo, hi] (empty when
// lo > hi).  The base window and each image interval containing q both contain
// k = q, so their union is a single interval; it is then cut to
// [key_begin, key_end) and [0, seq_len).
__host__ __device__ inline void row_interval(int64_t q, int seq_len, const MaskGeom& g,
                                             const int32_t* ranges, int max_ranges,
                                             int key_begin, int key_end, int64_t& lo,
                                             int64_t& hi) {
  int64_t b_lo = g.window > 0 ? q - g.window + 1 : (int64_t)INT32_MIN;
  if (g.chunk_lookback >= 0) {
    const int64_t c = (floordiv64(q, g.chunk_size) - g.chunk_lookback) * g.chunk_size;
    if (c > b_lo) b_lo = c;
  }
  int64_t b_hi = g.causal ? q : (g.window > 0 ? q + g.window - 1 : (int64_t)INT32_MAX);
  if (ranges != nullptr) {
    for (int i = 0; i < max_ranges; ++i) {
      const int64_t s = ranges[2 * i], e = ranges[2 * i + 1];
      if (s < e && s <= q && q <= e) {
        int64_t l = s;
        if (g.window > 0 && q - g.window + 1 > l) l = q - g.window + 1;
        if (l < b_lo) b_lo = l;
        if (e > b_hi) b_hi = e;
      }
    }
  }
  if (b_lo < key_begin) b_lo = key_begin;
  if (b_lo < 0) b_lo = 0;
  if (b_hi > (int64_t)key_end - 1) b_hi = (int64_t)key_end - 1;
  if (b_hi > (int64_t)seq_len - 1) b_hi = (int64_t)seq_len - 1;
  lo = b_lo;
  hi = b_hi;
}

}  // namespace psw
