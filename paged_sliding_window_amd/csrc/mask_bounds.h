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

// A request's image ranges ([n][2] inclusive (start, end); r == nullptr: none).
// each(f) calls f(start, end) for every range in order; minmax(f, mn, mx)
// lowers mn / raises mx to the (lo, hi) that f(start, end, lo, hi) reports for
// every range it accepts (returns true for).
struct RangesPtr {
  const int32_t* r;
  int n;
  template <class F>
  __host__ __device__ void each(F&& f) const {
    for (int i = 0; i < n; ++i) f(r[2 * i], r[2 * i + 1]);
  }
  // each(f) restricted to ranges that may contain q (here: all of them)
  template <class F>
  __host__ __device__ void each_near(int q, F&& f) const {
    each(f);
  }
  template <class F>
  __host__ __device__ void minmax(F&& f, int64_t& mn, int64_t& mx) const {
    for (int i = 0; i < n; ++i) {
      int lo, hi;
      if (f(r[2 * i], r[2 * i + 1], lo, hi)) {
        if (lo < mn) mn = lo;
        if (hi > mx) mx = hi;
      }
    }
  }
};

// The same visits for a pointer that is uniform across the wave, with all 64
// lanes active: the ranges are read 64 at a time with one vector load (lane i
// holds range base + i) instead of a chain of dependent scalar loads, one per
// range, and tested in parallel across the lanes.
struct RangesWave {
  const int32_t* r;
  int n;
  // each(f) for the ranges that intersect [min q, max q] over the wave (the
  // others cannot contain any lane's q): lane i tests range base + i, and only
  // the ranges the ballot selects are walked, in order
  template <class F>
  __device__ void each_near(int q, F&& f) const {
    const int lane = __lane_id();
    int qmn = q, qmx = q;
    for (int o = 32; o > 0; o >>= 1) {
      const int a = __shfl_xor(qmn, o, 64), b = __shfl_xor(qmx, o, 64);
      qmn = a < qmn ? a : qmn;
      qmx = b > qmx ? b : qmx;
    }
    for (int base = 0; base < n; base += 64) {
      int sv = 0, ev = 0;
      if (base + lane < n) {
        sv = r[2 * (base + lane)];
        ev = r[2 * (base + lane) + 1];
      }
      uint64_t m = __ballot(sv < ev && sv <= qmx && ev >= qmn);
      while (m != 0) {
        const int i = __builtin_ctzll(m);
        m &= m - 1;
        f(__builtin_amdgcn_readlane(sv, i), __builtin_amdgcn_readlane(ev, i));
      }
    }
  }
  // f must not depend on the lane: lane i evaluates range base + i, and the
  // accepted (lo, hi) are reduced over the wave
  template <class F>
  __device__ void minmax(F&& f, int64_t& mn, int64_t& mx) const {
    const int lane = __lane_id();
    int bmn = INT32_MAX, bmx = INT32_MIN;
    for (int base = 0; base < n; base += 64) {
      int lo, hi;
      if (base + lane < n && f(r[2 * (base + lane)], r[2 * (base + lane) + 1], lo, hi)) {
        bmn = lo < bmn ? lo : bmn;
        bmx = hi > bmx ? hi : bmx;
      }
    }
    for (int o = 32; o > 0; o >>= 1) {
      const int a = __shfl_xor(bmn, o, 64), b = __shfl_xor(bmx, o, 64);
      bmn = a < bmn ? a : bmn;
      bmx = b > bmx ? b : bmx;
    }
    bmn = __builtin_amdgcn_readfirstlane(bmn);
    bmx = __builtin_amdgcn_readfirstlane(bmx);
    if (bmn <= bmx) {  // some range was accepted
      if (bmn < mn) mn = bmn;
      if (bmx > mx) mx = bmx;
    }
  }
};

// rg: this request's image ranges (RangesPtr or RangesWave).
template <class R>
__host__ __device__ inline TileRange tile_bounds_r(int context_len, int seq_len, int query_len,
                                                   int q_block, int tile, int block_m,
                                                   int block_q, int queries_per_kv,
                                                   const MaskGeom& g, const R& rg) {
  const bool use_mm = rg.r != nullptr && rg.n > 0;
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
      // positions and q_lo - window + 1 fit in 32 bits
      const int qh = (int)q_hi, ql = (int)q_lo, wl = (int)(q_lo - g.window + 1);
      rg.minmax(
          [=](int s, int e, int& lo_img, int& hi_img) {
            if (!(s < e && s <= qh && e >= ql)) return false;
            lo_img = s > wl ? s : wl;
            hi_img = e;
            return true;
          },
          first, last);
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

__host__ __device__ inline TileRange tile_bounds(int context_len, int seq_len, int query_len,
                                                 int q_block, int tile, int block_m, int block_q,
                                                 int queries_per_kv, const MaskGeom& g,
                                                 const int32_t* ranges, int max_ranges) {
  return tile_bounds_r(context_len, seq_len, query_len, q_block, tile, block_m, block_q,
                       queries_per_kv, g, RangesPtr{ranges, max_ranges});
}

// Allowed keys of absolute query q as one closed interval [lo, hi] (empty when
// lo > hi).  The base window and each image interval containing q both contain
// k = q, so their union is a single interval; it is then cut to
// [key_begin, key_end) and [0, seq_len).
template <class R>
__host__ __device__ inline void row_interval_r(int64_t q, int seq_len, const MaskGeom& g,
                                               const R& rg, int key_begin, int key_end,
                                               int64_t& lo, int64_t& hi) {
  int64_t b_lo = g.window > 0 ? q - g.window + 1 : (int64_t)INT32_MIN;
  if (g.chunk_lookback >= 0) {
    const int64_t c = (floordiv64(q, g.chunk_size) - g.chunk_lookback) * g.chunk_size;
    if (c > b_lo) b_lo = c;
  }
  int64_t b_hi = g.causal ? q : (g.window > 0 ? q + g.window - 1 : (int64_t)INT32_MAX);
  if (rg.r != nullptr) {
    // 32-bit walk: q and the image bounds are positions; the lower end of a
    // window that starts before position 0 only matters as "<= s"
    const int q32 = (int)q;
    const int wl = g.window > 0 ? (int)(q - g.window + 1 > INT32_MIN ? q - g.window + 1 : INT32_MIN)
                                : INT32_MIN;
    int lo32 = INT32_MAX, hi32 = INT32_MIN;
    rg.each_near(q32, [&](int s, int e) {
      if (s < e && s <= q32 && q32 <= e) {
        const int l = wl > s ? wl : s;
        lo32 = l < lo32 ? l : lo32;
        hi32 = e > hi32 ? e : hi32;
      }
    });
    if (lo32 <= hi32) {
      if (lo32 < b_lo) b_lo = lo32;
      if (hi32 > b_hi) b_hi = hi32;
    }
  }
  if (b_lo < key_begin) b_lo = key_begin;
  if (b_lo < 0) b_lo = 0;
  if (b_hi > (int64_t)key_end - 1) b_hi = (int64_t)key_end - 1;
  if (b_hi > (int64_t)seq_len - 1) b_hi = (int64_t)seq_len - 1;
  lo = b_lo;
  hi = b_hi;
}

__host__ __device__ inline void row_interval(int64_t q, int seq_len, const MaskGeom& g,
                                             const int32_t* ranges, int max_ranges,
                                             int key_begin, int key_end, int64_t& lo,
                                             int64_t& hi) {
  row_interval_r(q, seq_len, g, RangesPtr{ranges, max_ranges}, key_begin, key_end, lo, hi);
}

}  // namespace psw
