// Split-KV decode attention for the latent (MLA-shaped) cache: every query head
// reads one shared 576-wide latent row per key, and V is that row's first 512
// columns (MLA DCP decode study notes, vllm-ascend PR #16977: "Terms" for MLA;
// sections 1.1 and 3.1 for the history/current partials that each emit an
// output and an LSE; code blocks B and C for the two partial calls).
//
// Work items are (new token, key split) pairs; item i owns the KV tiles of its
// query row inside its split's key range.  Decode batches mix requests whose
// lengths differ by 8x, so one workgroup per item leaves most CUs idle while
// the longest items finish.  Instead the launch is balanced over the global
// tile sequence (items in order, each item's tiles in order):
//   1. decode_plan_kernel writes the exclusive prefix sum of tiles per item;
//   2. workgroup w of G takes the tiles [w * per, (w + 1) * per), per = ceil(T / G),
//      which may cover the end of one item, whole items and the start of another.
//      An item that lies inside one workgroup's range is written to the output
//      directly; otherwise each workgroup writes its piece (normalised O in bf16
//      and its LSE) to workspace slot 2w (the item began before the range) or
//      2w + 1 (the item begins inside the range and continues past it);
//   3. decode_merge_kernel merges the pieces of every item that spans several
//      workgroups by their LSEs, and writes 0 / -inf for items without tiles.
//
// Inside a workgroup, 128 query heads per KV head (decode_full_kernel): four
// waves, one per SIMD, wave w owns heads [32 w, 32 w + 32) over the whole row:
//   * tiles of 32 keys are gathered once per workgroup into LDS with
//     direct-to-LDS 16-byte loads in a three-deep ring; LDS-DMA instruction c
//     moves the 16-wide k-chunk c of all 32 keys as one block, so a K read for
//     k-chunk c and the transposed V reads are a lane base plus an immediate.
//     The DMA of tile t + 2 is spread over the score MFMAs of tile t (issued all
//     at once after the barrier, the four waves stall on the shared address
//     unit), and the block-table entry of a tile is read a tile ahead;
//   * S^T[32 keys][32 heads] = K Q^T over all 36 k-chunks, Q in registers;
//   * online softmax, then O^T += V^T P^T over all 512 output columns, V^T read
//     out of the same K tile with ds_read_b64_tr_b16.  The 16 output blocks
//     (256 fp32 per lane) live in the AGPRs, managed by inline assembly;
//   * the running max moves only when it grows by more than 2^8 (log2 units).
// With 32 or 64 heads per KV head (decode_attention_kernel) two waves share a
// 32-head block: wave (hb, 0) sums k-chunks 0..17 and wave (hb, 1) k-chunks
// 18..35, the halves are exchanged through LDS and added in the same order by
// both, both run the same softmax, and wave (hb, d) accumulates output columns
// [256 d, 256 d + 256).
// The mask (window, image ranges, key range of the split) is applied exactly
// as in the prefill kernel; one query position per item makes it uniform.
#include <mutex>
#include <type_traits>

#include "asm_ops.h"
#include "device_common.h"
#include "psw_internal.h"

namespace psw {

namespace dec {
constexpr int kD = 576, kDV = 512;
constexpr int kTile = 32;                   // keys per tile
constexpr int kKChunks = kD / 16;           // 36 MFMA k-chunks of 16 columns
constexpr int kHalfChunks = kKChunks / 2;   // 18 per wave of a pair
constexpr int kBlock = 1024 + 128;          // LDS bytes per k-chunk block (padded)
constexpr int kTileBytes = kKChunks * kBlock;
constexpr int kOBlocks = kDV / 2 / 32;      // 8 blocks of 32 output columns per wave
constexpr int kPlanThreads = 1024;
}  // namespace dec

// One (token, split) work item: its request and the tiles / keys its row may see.
struct DecodeItem {
  int token, split, seq, seq_len, t_lo, t_hi, row_lo, row_hi;
};

// WAVE: called by a whole wave for one item (all lanes active), so the image
// ranges are walked in the wave form; otherwise one item per thread.
template <bool WAVE>
__device__ __forceinline__ DecodeItem decode_item(const AttnParams& p, int item) {
  DecodeItem d;
  d.token = item / p.num_splits;
  d.split = item - d.token * p.num_splits;
  int s_lo = 0, s_hi = p.num_seqs - 1;
  while (s_lo < s_hi) {
    const int mid = (s_lo + s_hi + 1) >> 1;
    if (p.query_start_loc[mid] <= d.token) s_lo = mid; else s_hi = mid - 1;
  }
  d.seq = s_lo;
  const int q_start = p.query_start_loc[d.seq];
  const int query_len = p.query_start_loc[d.seq + 1] - q_start;
  const int qpos = d.token - q_start;
  d.seq_len = p.seq_lens[d.seq];
  const int ctx = d.seq_len - query_len;
  const int32_t* ranges =
      p.mm_ranges ? p.mm_ranges + (int64_t)d.seq * p.max_mm_ranges * 2 : nullptr;
  int key_begin = 0, key_end = d.seq_len;
  if (p.key_ranges) {
    const int64_t kr = ((int64_t)d.split * p.num_seqs + d.seq) * 2;
    key_begin = max(0, p.key_ranges[kr]);
    key_end = min(d.seq_len, p.key_ranges[kr + 1]);
  }
  using R = std::conditional_t<WAVE, RangesWave, RangesPtr>;
  const R rg{ranges, p.max_mm_ranges};
  int64_t lo64, hi64;
  row_interval_r((int64_t)ctx + qpos, d.seq_len, p.geom, rg, key_begin, key_end, lo64, hi64);
  if (lo64 <= hi64) {
    // the row's allowed keys are one interval; its tiles are inside the query
    // block's tile bounds, which are kept as the outer limit
    const TileRange tr = tile_bounds_r(ctx, d.seq_len, query_len, qpos, dec::kTile,
                                       p.queries_per_kv, 1, p.queries_per_kv, p.geom, rg);
    d.row_lo = (int)lo64;
    d.row_hi = (int)hi64;
    d.t_lo = max(tr.lo, d.row_lo / dec::kTile);
    d.t_hi = min(tr.hi, d.row_hi / dec::kTile + 1);
  } else {
    d.row_lo = INT32_MAX;
    d.row_hi = INT32_MIN;
    d.t_lo = d.t_hi = 0;
  }
  if (d.t_hi < d.t_lo) d.t_hi = d.t_lo;
  PSW_DCHECK(8, d.t_lo >= 0 &&
                    (d.t_lo == d.t_hi || (int64_t)(d.t_hi - 1) * dec::kTile < d.seq_len) &&
                    (d.row_lo > d.row_hi || (d.row_lo >= 0 && d.row_hi < d.seq_len)));
  return d;
}

// prefix[i] = number of tiles of items 0..i-1, prefix[items] = total (one workgroup).
__global__ __launch_bounds__(dec::kPlanThreads) void decode_plan_kernel(const AttnParams p,
                                                                        int32_t* prefix) {
  constexpr int kWaves = dec::kPlanThreads / kWave;
  __shared__ int wave_sum[kWaves];
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int items = p.num_tokens * p.num_splits;
  int carry = 0;
  for (int base = 0; base < items; base += dec::kPlanThreads) {
    const int it = base + tid;
    int cnt = 0;
    if (it < items) {
      const DecodeItem d = decode_item<false>(p, it);
      cnt = d.t_hi - d.t_lo;
    }
    int x = cnt;  // inclusive scan inside the wave
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int y = __shfl_up(x, off, kWave);
      if (lane >= off) x += y;
    }
    if (lane == kWave - 1) wave_sum[wave] = x;
    __syncthreads();
    if (wave == 0) {
      int v = lane < kWaves ? wave_sum[lane] : 0;
#pragma unroll
      for (int off = 1; off < kWaves; off <<= 1) {
        const int y = __shfl_up(v, off, kWave);
        if (lane >= off) v += y;
      }
      if (lane < kWaves) wave_sum[lane] = v;
    }
    __syncthreads();
    if (it < items) prefix[it] = carry + (wave > 0 ? wave_sum[wave - 1] : 0) + x - cnt;
    carry += wave_sum[kWaves - 1];
    __syncthreads();
  }
  if (tid == 0) prefix[items] = carry;
}

// Slot (16 bytes) of key row r, column half hh (columns 8*hh..8*hh+7 of a
// k-chunk) inside a k-chunk block.  Rows of the second half are rotated by 4 so
// that the 4 rows x 2 halves of a transposed read hit 8 distinct bank groups.
__device__ __forceinline__ int dec_slot(int r, int hh) { return 32 * hh + ((r + 4 * hh) & 31); }

__device__ __forceinline__ void dec_dma16(const void* gsrc, void* lds_dst) {
  __builtin_amdgcn_global_load_lds(
      (const __attribute__((address_space(1))) void*)gsrc,
      (__attribute__((address_space(3))) void*)(lds_void*)lds_dst, 16, 0, 0);
}

namespace dec {
// A vector load the compiler does not track (so it adds no vmcnt(0) waits of
// its own around the LDS-DMA pipeline): the result may be used only after
// vm_wait_tied<N>(), which waits until at most N vector-memory operations of
// this wave are outstanding (loads complete in issue order) and ties the
// register to that point.  The memory clobber keeps the load in program order
// with the LDS-DMA instructions.
__device__ __forceinline__ int load_i32_async(const int32_t* ptr) {
  int r;
  asm volatile("global_load_dword %0, %1, off" : "=v"(r) : "v"(ptr) : "memory");
  return r;
}
template <int N>
__device__ __forceinline__ void vm_wait_tied(int& r) {
  asm volatile("s_waitcnt vmcnt(%1)" : "+v"(r) : "i"(N));
}

}  // namespace dec

// Where the stream-K pieces live inside the caller's workspace.
struct DecodeWork {
  const int32_t* prefix;  // [items + 1]
  uint16_t* piece_o;      // bf16 [groups][2 * grid][heads per group][kDV]
  float* piece_lse;       // [groups][2 * grid][heads per group]
  int grid;               // workgroups per head group
};

// NB: 32-head MFMA blocks per wave; HG: head groups per workgroup.  The
// workgroup has 2 * HG waves, wave (hg, dh) owns heads [hg * NB * 32, +NB * 32)
// of the group and the d-half dh; one wave per SIMD, so each wave has the whole
// register file (the O accumulators live in AGPRs).  UNIFORM_BT: the block size
// is >= 32, so every 32-key tile lies inside one KV block whose table entry is
// read with one scalar load; the tile ring is then three deep.
template <int NB, int HG, bool UNIFORM_BT>
__global__ __launch_bounds__(HG * 128)
__attribute__((amdgpu_waves_per_eu((HG * 2 + 3) / 4, (HG * 2 + 3) / 4)))
void decode_attention_kernel(const AttnParams p, const DecodeWork wk) {
  using namespace dec;
  constexpr int kWaves = 2 * HG;
  constexpr int kHeads = HG * NB * 32;              // heads per workgroup
  // LDS-DMA instructions per tile: waves below kDmaExtra issue one more
  constexpr int kDmaPerWave = kKChunks / kWaves;
  constexpr int kDmaExtra = kKChunks % kWaves;
  constexpr int kBufs = UNIFORM_BT ? 3 : 2;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  float* xs = reinterpret_cast<float*>(smem + kBufs * kTileBytes);  // [wave][NB][4][64][4]

  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);  // uniform: keep it scalar
  const int half = lane >> 5;
  const int hg = wave >> 1, dh = wave & 1;
  const int G = wk.grid;
  const int groups = gridDim.y;
  const int logical = xcd_logical_id(blockIdx.x + gridDim.x * blockIdx.y, G * groups);
  const int w = logical % G;       // neighbouring w share items: keep them on one XCD
  const int group = logical / G;
  const int head0 = group * kHeads;
  const int kvh = head0 / p.queries_per_kv;

  const int items = p.num_tokens * p.num_splits;
  const int total = wk.prefix[items];
  const int per = max(1, (total + G - 1) / G);
  const int g0 = w * per, g1 = min(total, g0 + per);
  if (g0 >= g1) return;
  // first item with tiles at or after g0: the last item whose prefix is <= g0
  int it;
  {
    int lo = 0, hi = items - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (wk.prefix[mid] <= g0) lo = mid; else hi = mid - 1;
    }
    it = lo;
  }

  const int hl0 = hg * NB * 32 + (lane & 31);  // head (inside the group) of block 0
  const int64_t slot_pitch = (int64_t)p.num_kv_heads * kD;
  const uint16_t* kbase = p.k_cache + (int64_t)kvh * kD;
  const int bs_log2 = p.block_size_log2;
  const int bs_mask = (1 << bs_log2) - 1;
  const float c2 = p.scale_log2;
  // this lane's DMA slot: key row and column half within every k-chunk block
  const int dma_hh = lane >> 5;
  const int dma_row = (lane - 4 * dma_hh) & 31;
  // transposed V reads: group of 16 lanes covers 4 keys x 16 columns
  const int tr_key = half * 4 + ((lane & 15) >> 2);   // + 16 j (+ 8 for the upper 4 keys)
  const int tr_g = (lane >> 4) & 1;                    // which 16 of a 32-column block
  const int tr_hh = (lane & 3) >> 1, tr_in = (lane & 1) * 8;
  const int dcol = dh * (kDV / 2) + half * 4;

  bf16x8 qf[NB][kHalfChunks];
  int q_token = -1;
  int g = g0;
  while (true) {
    const int p0 = wk.prefix[it], p1 = wk.prefix[it + 1];
    PSW_DCHECK(11, p0 <= p1);
    const DecodeItem d = decode_item<true>(p, it);
    // previous item: all waves done with LDS, all stores and loads retired
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (d.token != q_token) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const uint16_t* qrow = p.q + ((int64_t)d.token * p.num_q_heads + head0 + hl0 + nb * 32) * kD +
                               dh * (kHalfChunks * 16) + half * 8;
#pragma unroll
        for (int c = 0; c < kHalfChunks; ++c)
          qf[nb][c] = *reinterpret_cast<const bf16x8*>(qrow + c * 16);
      }
      q_token = d.token;
    }
    const int t_first = d.t_lo + (g - p0);
    const int t_end = d.t_lo + (min(g1, p1) - p0);
    const int seq_len = d.seq_len;
    const int row_lo = d.row_lo, row_hi = d.row_hi;
    const int32_t* bt = p.block_table + (int64_t)d.seq * p.block_table_stride;

    f32x16 o[NB][kOBlocks];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int b = 0; b < kOBlocks; ++b) o[nb][b] = f32x16{};
    float m_run[NB], l_run[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      m_run[nb] = -INFINITY;
      l_run[nb] = 0.f;
    }

    // the LDS-DMA of one tile: this wave moves k-chunks wave, wave + kWaves, ...
    // Rows past the last key repeat the last key (finite values, masked later).
    auto issue_tile = [&](int tile, int buf) {
      const int first = tile * kTile;
      const uint16_t* src;
      if constexpr (UNIFORM_BT) {
        // uniform tile base + a per-lane 32-bit offset (row, column half)
        const int blk = load_uniform_i32(bt + (first >> bs_log2));
        PSW_DCHECK(9, blk >= 0);
        const char* tile_base = reinterpret_cast<const char*>(
            kbase + (((int64_t)blk << bs_log2) + (first & bs_mask)) * slot_pitch);
        const uint32_t row = (uint32_t)min(dma_row, seq_len - 1 - first);
        src = reinterpret_cast<const uint16_t*>(
            tile_base + (row * (uint32_t)slot_pitch + (uint32_t)dma_hh * 8u) * 2u);
      } else {
        const int key = min(first + dma_row, seq_len - 1);
        const int blk = bt[key >> bs_log2];
        PSW_DCHECK(9, blk >= 0);
        src = kbase + (((int64_t)blk << bs_log2) + (key & bs_mask)) * slot_pitch + dma_hh * 8;
      }
      char* dst = smem + buf * kTileBytes;
#pragma unroll
      for (int i = 0; i < kDmaPerWave; ++i) {
        const int c = i * kWaves + wave;
        dec_dma16(src + c * 16, dst + c * kBlock);
      }
      if constexpr (kDmaExtra != 0) {
        const int c = kDmaPerWave * kWaves + wave;
        if (wave < kDmaExtra) dec_dma16(src + c * 16, dst + c * kBlock);
      }
    };

    issue_tile(t_first, 0);
    if (kBufs == 3 && t_first + 1 < t_end) issue_tile(t_first + 1, 1);

    for (int t = t_first; t < t_end; ++t) {
      const int buf = (t - t_first) % kBufs;
      if constexpr (kBufs == 3) {
        // tile t landed; tile t + 1 (issued after it) may still be in flight
        if (t + 1 >= t_end) __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        else if (kDmaExtra != 0 && wave < kDmaExtra)
          __builtin_amdgcn_s_waitcnt(waitcnt_vm(kDmaPerWave + 1));
        else __builtin_amdgcn_s_waitcnt(waitcnt_vm(kDmaPerWave));
      } else {
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
      }
      lds_barrier();
      // the buffer tile t + kBufs - 1 goes to was last read in iteration t - 1
      if (t + kBufs - 1 < t_end) issue_tile(t + kBufs - 1, (buf + kBufs - 1) % kBufs);
      const char* kt = smem + buf * kTileBytes;

      f32x16 s[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) s[nb] = f32x16{};
      {
        const char* arow = kt + dec_slot(lane & 31, half) * 16 + dh * kHalfChunks * kBlock;
        bf16x8 a = *reinterpret_cast<const bf16x8*>(arow);
#pragma unroll
        for (int c = 0; c < kHalfChunks; ++c) {
          bf16x8 a_next = a;
          if (c + 1 < kHalfChunks) a_next = *reinterpret_cast<const bf16x8*>(arow + (c + 1) * kBlock);
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) s[nb] = mfma32(a, qf[nb][c], s[nb]);
          a = a_next;
        }
      }
      // exchange of the two d-halves: layout [wave][NB][4][lane][4 floats]
      {
        f32x4* mine = reinterpret_cast<f32x4*>(xs) + wave * NB * 4 * kWave + lane;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            mine[(nb * 4 + i) * kWave] =
                f32x4{s[nb][4 * i], s[nb][4 * i + 1], s[nb][4 * i + 2], s[nb][4 * i + 3]};
      }
      lds_barrier();
      {
        const f32x4* other =
            reinterpret_cast<const f32x4*>(xs) + (wave ^ 1) * NB * 4 * kWave + lane;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const f32x4 part = other[(nb * 4 + i) * kWave];
            // both waves of the pair add the halves in the same order
#pragma unroll
            for (int k = 0; k < 4; ++k)
              s[nb][4 * i + k] = dh == 0 ? s[nb][4 * i + k] + part[k] : part[k] + s[nb][4 * i + k];
          }
      }

      const int base = t * kTile;
      if (!(base >= row_lo && base + kTile - 1 <= row_hi)) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int k = base + (i / 4) * 8 + half * 4 + (i % 4);
          const bool ok = k >= row_lo && k <= row_hi;
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) s[nb][i] = ok ? s[nb][i] : -INFINITY;
        }
      }
      bf16x8 pf[NB][2];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        float mx = s[nb][0];
#pragma unroll
        for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[nb][i]);
        mx = fmaxf(mx, swap_halves(mx)) * c2;
        if (__ballot(mx > m_run[nb] + 8.f) != 0) {
          const float m_new = fmaxf(m_run[nb], mx);
          const float alpha = m_new == -INFINITY ? 1.f : fast_exp2(m_run[nb] - m_new);
          l_run[nb] *= alpha;
#pragma unroll
          for (int b = 0; b < kOBlocks; ++b) o[nb][b] *= alpha;
          m_run[nb] = m_new;
        }
        const float m_sub = m_run[nb] == -INFINITY ? 0.f : m_run[nb];
        float psum = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          s[nb][i] = fast_exp2(fmaf(s[nb][i], c2, -m_sub));
          psum += s[nb][i];
        }
        l_run[nb] += psum;
        pf[nb][0] = to_bf16x8(s[nb][0], s[nb][1], s[nb][2], s[nb][3], s[nb][4], s[nb][5],
                              s[nb][6], s[nb][7]);
        pf[nb][1] = to_bf16x8(s[nb][8], s[nb][9], s[nb][10], s[nb][11], s[nb][12], s[nb][13],
                              s[nb][14], s[nb][15]);
      }

      // O^T += V^T P^T.  Output columns dh*256 + b*32 + [0, 32) come from
      // k-chunk block 2 * (dh*8 + b) + tr_g; step st = 2b + j covers keys
      // [16 j, 16 j + 16).  The two transposed reads of step st + 1 are in
      // flight while the MFMA of step st runs.
      {
        const uint32_t vbase = lds_addr(kt + (2 * dh * kOBlocks + tr_g) * kBlock + tr_in);
        uint32_t va[2][2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          va[j][0] = vbase + dec_slot(16 * j + tr_key, tr_hh) * 16;
          va[j][1] = vbase + dec_slot(16 * j + tr_key + 8, tr_hh) * 16;
        }
        constexpr int kSteps = 2 * kOBlocks;
        bf16x4 vr[2][2];
        vr[0][0] = lds_read_tr4_async(va[0][0]);
        vr[0][1] = lds_read_tr4_async(va[0][1]);
#pragma unroll
        for (int st = 0; st < kSteps; ++st) {
          const int b = st >> 1, j = st & 1, cur = st & 1;
          if (st + 1 < kSteps) {
            const int bn = (st + 1) >> 1, jn = (st + 1) & 1;
            vr[cur ^ 1][0] = lds_read_tr4_async(va[jn][0] + bn * 2 * kBlock);
            vr[cur ^ 1][1] = lds_read_tr4_async(va[jn][1] + bn * 2 * kBlock);
            lds_wait_tr<2>(vr[cur][0], vr[cur][1]);
          } else {
            lds_wait_tr<0>(vr[cur][0], vr[cur][1]);
          }
          const bf16x8 vt = cat8(vr[cur][0], vr[cur][1]);
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) o[nb][b] = mfma32(vt, pf[nb][j], o[nb][b]);
        }
      }
    }

    const bool complete = p0 >= g0 && p1 <= g1;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int hl = hl0 + nb * 32;
      const float l_tot = l_run[nb] + swap_halves(l_run[nb]);
      const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
      const float lse_val = l_tot > 0.f ? (m_run[nb] + fast_log2(l_tot)) * kLn2 : -INFINITY;
      if (complete) {
        // the whole item is in this workgroup's range: final result
        const int64_t orow =
            ((int64_t)d.split * p.num_tokens + d.token) * p.num_q_heads + head0 + hl;
        const int64_t e0 = orow * kDV + dcol;
#pragma unroll
        for (int b = 0; b < kOBlocks; ++b)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            store_out4(p.out, e0 + b * 32 + q * 8, p.out_dtype, o[nb][b][4 * q] * inv,
                       o[nb][b][4 * q + 1] * inv, o[nb][b][4 * q + 2] * inv,
                       o[nb][b][4 * q + 3] * inv);
        if (p.lse != nullptr && dh == 0 && half == 0) p.lse[orow] = lse_val;
      } else {
        // a piece of an item shared with neighbouring workgroups
        const int slot = p0 < g0 ? 2 * w : 2 * w + 1;
        const int64_t prow = ((int64_t)group * 2 * G + slot) * kHeads + hl;
#pragma unroll
        for (int b = 0; b < kOBlocks; ++b)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            store_out4(wk.piece_o, prow * kDV + dcol + b * 32 + q * 8, kOutBf16,
                       o[nb][b][4 * q] * inv, o[nb][b][4 * q + 1] * inv,
                       o[nb][b][4 * q + 2] * inv, o[nb][b][4 * q + 3] * inv);
        if (dh == 0 && half == 0) wk.piece_lse[prow] = lse_val;
      }
    }

    g = min(g1, p1);
    if (g >= g1) break;
    ++it;
    while (wk.prefix[it + 1] <= g) ++it;  // skip items without tiles
  }
}

// Full-width variant for 128 query heads: 4 waves, one per SIMD, wave w owns
// heads [32 w, 32 w + 32) over the whole row: S^T over all 36 k-chunks (Q held
// in registers, 144 VGPRs) and O^T over all 512 output columns (256 AGPRs), so
// no half-scores are exchanged and no softmax is computed twice.  Each wave
// has 68 MFMAs per tile, against one softmax, one barrier and nine LDS-DMA
// instructions; the K and V^T reads run a few steps ahead of their MFMAs.
template <bool UNIFORM_BT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void decode_full_kernel(const AttnParams p, const DecodeWork wk) {
  using namespace dec;
  constexpr int kWaves = 4;
  constexpr int kHeads = 128;
  constexpr int kDmaPerWave = kKChunks / kWaves;  // 9
  static_assert(kDmaPerWave * kWaves == kKChunks, "k-chunks split evenly over the waves");
  constexpr int kOB = kDV / 32;                    // 16 output blocks of 32 columns
  constexpr int kBufs = UNIFORM_BT ? 3 : 2;
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);  // uniform: keep it scalar
  const int half = lane >> 5;
  const int G = wk.grid;
  const int groups = gridDim.y;
  const int logical = xcd_logical_id(blockIdx.x + gridDim.x * blockIdx.y, G * groups);
  const int w = logical % G;       // neighbouring w share items: keep them on one XCD
  const int group = logical / G;
  const int head0 = group * kHeads;
  const int kvh = head0 / p.queries_per_kv;

  const int items = p.num_tokens * p.num_splits;
  const int total = wk.prefix[items];
  const int per = max(1, (total + G - 1) / G);
  const int g0 = w * per, g1 = min(total, g0 + per);
  if (g0 >= g1) return;
  int it;
  {
    int lo = 0, hi = items - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (wk.prefix[mid] <= g0) lo = mid; else hi = mid - 1;
    }
    it = lo;
  }

  const int hl = wave * 32 + (lane & 31);  // head of this lane inside the group
  const int64_t slot_pitch = (int64_t)p.num_kv_heads * kD;
  const uint16_t* kbase = p.k_cache + (int64_t)kvh * kD;
  const int bs_log2 = p.block_size_log2;
  const int bs_mask = (1 << bs_log2) - 1;
  const float c2 = p.scale_log2;
  const int dma_hh = lane >> 5;
  const int dma_row = (lane - 4 * dma_hh) & 31;
  const int tr_key = half * 4 + ((lane & 15) >> 2);
  const int tr_g = (lane >> 4) & 1;
  const int tr_hh = (lane & 3) >> 1, tr_in = (lane & 1) * 8;
  const int dcol = half * 4;
  const uint32_t smem0 = lds_addr(smem);
  const uint32_t k_lane = (uint32_t)(dec_slot(lane & 31, half) * 16);
  uint32_t v_lane[2][2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    v_lane[j][0] = (uint32_t)(tr_g * kBlock + tr_in + dec_slot(16 * j + tr_key, tr_hh) * 16);
    v_lane[j][1] = (uint32_t)(tr_g * kBlock + tr_in + dec_slot(16 * j + tr_key + 8, tr_hh) * 16);
  }

  int g = g0;
  while (true) {
    const int p0 = wk.prefix[it], p1 = wk.prefix[it + 1];
    PSW_DCHECK(11, p0 <= p1);
    const DecodeItem d = decode_item<true>(p, it);
    // previous item: all waves done with LDS, all stores and loads retired
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    // Q is loaded per item (not kept across items: the registers are needed
    // by the epilogue)
    bf16x8 qf[kKChunks];
    {
      const uint16_t* qrow = p.q + ((int64_t)d.token * p.num_q_heads + head0 + hl) * kD + half * 8;
#pragma unroll
      for (int c = 0; c < kKChunks; ++c) qf[c] = *reinterpret_cast<const bf16x8*>(qrow + c * 16);
    }
    const int t_first = d.t_lo + (g - p0);
    const int t_end = d.t_lo + (min(g1, p1) - p0);
    const int seq_len = d.seq_len;
    const int row_lo = d.row_lo, row_hi = d.row_hi;
    const int32_t* bt = p.block_table + (int64_t)d.seq * p.block_table_stride;

    oacc_zero<0, 256>();
    float m_run = -INFINITY, l_run = 0.f;

    // The LDS-DMA of one tile: this wave moves k-chunks wave, wave + 4, ...
    // Rows past the last key repeat the last key (finite values, masked later).
    // dma_src() gives this lane's source row for the tile; chunk c then adds
    // c * 16 elements.
    auto dma_src = [&](int tile, int blk) __attribute__((always_inline)) {
      const int first = tile * kTile;
      if constexpr (UNIFORM_BT) {
        // uniform block entry blk + a per-lane 32-bit offset (row, column half)
        PSW_DCHECK(9, blk >= 0);
        const char* tile_base = reinterpret_cast<const char*>(
            kbase + (((int64_t)blk << bs_log2) + (first & bs_mask)) * slot_pitch);
        const uint32_t row = (uint32_t)min(dma_row, seq_len - 1 - first);
        return reinterpret_cast<const uint16_t*>(
            tile_base + (row * (uint32_t)slot_pitch + (uint32_t)dma_hh * 8u) * 2u);
      } else {
        const int key = min(first + dma_row, seq_len - 1);
        const int b = bt[key >> bs_log2];
        PSW_DCHECK(9, b >= 0);
        return kbase + (((int64_t)b << bs_log2) + (key & bs_mask)) * slot_pitch + dma_hh * 8;
      }
    };
    auto dma_chunk = [&](const uint16_t* src, int buf, int i) __attribute__((always_inline)) {
      const int c = i * kWaves + wave;
      dec_dma16(src + c * 16, smem + buf * kTileBytes + c * kBlock);
    };
    auto issue_tile = [&](int tile, int buf, int blk) __attribute__((always_inline)) {
      const uint16_t* src = dma_src(tile, blk);
#pragma unroll
      for (int i = 0; i < kDmaPerWave; ++i) dma_chunk(src, buf, i);
    };

    // UNIFORM_BT: a 3-deep ring.  In iteration t the DMA of tile t + 2 is
    // spread over the score MFMAs (all four waves issuing their nine
    // instructions at once stall on the shared address unit).  Past the last
    // tile the ring reloads the last tile into the free buffer, so that every
    // iteration has the same outstanding operations.  The block-table entry of
    // tile u + 1 is read with an untracked vector load just before the DMA of
    // tile u and consumed an iteration later; a scalar load there would be
    // waited for on the spot.
    auto bt_entry = [&](int tile) __attribute__((always_inline)) {
      return load_i32_async(bt + ((min(tile, t_end - 1) * kTile) >> bs_log2));
    };
    int bt_next = 0;
    if constexpr (UNIFORM_BT) {
      issue_tile(t_first, 0, load_uniform_i32(bt + ((t_first * kTile) >> bs_log2)));
      const int t1 = min(t_first + 1, t_end - 1);
      const int blk1 = load_uniform_i32(bt + ((t1 * kTile) >> bs_log2));
      bt_next = bt_entry(t_first + 2);
      issue_tile(t1, 1, blk1);
    } else {
      issue_tile(t_first, 0, 0);
    }

    for (int t = t_first; t < t_end; ++t) {
      const int buf = (t - t_first) % kBufs;
      const int nbuf = (buf + kBufs - 1) % kBufs;  // last read in iteration t - 1
      const uint16_t* nsrc = nullptr;
      if constexpr (UNIFORM_BT) {
        // tile t landed; the entry load and the nine DMAs issued after it
        // (tile t + 1, or a repeat of the last tile) may still be in flight
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(kDmaPerWave + 1));
        lds_barrier();
        vm_wait_tied<kDmaPerWave>(bt_next);  // older than the 9 DMAs of tile t + 1
        const int blk = __builtin_amdgcn_readfirstlane(bt_next);
        bt_next = bt_entry(t + 3);
        nsrc = dma_src(min(t + 2, t_end - 1), blk);
      } else {
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        lds_barrier();
        if (t + 1 < t_end) issue_tile(t + 1, nbuf, 0);
      }
      const uint32_t kt = smem0 + (uint32_t)(buf * kTileBytes);

      // S^T[32 keys][32 heads] over the 36 k-chunks, K reads KA ahead (with
      // one wave per SIMD only the wave's own reads in flight hide the LDS
      // latency); with UNIFORM_BT one DMA instruction of tile t + 2 after
      // every fourth MFMA
      f32x16 s;
      {
        constexpr int N = kKChunks, KA = 7;
        const uint32_t ka = kt + k_lane;
        bf16x8 kf[KA + 1];
        static_for<KA>([&](auto cc) {
          constexpr int c = decltype(cc)::value;
          kf[c] = lds_read_b128_at<c * kBlock>(ka);
        });
        static_for<N>([&](auto cc) {
          constexpr int c = decltype(cc)::value;
          constexpr int issued = c + KA < N ? c + KA : N;
          lds_wait<issued - 1 - c>(kf[c % (KA + 1)]);
          if constexpr (c == 0) s = mfma32_vgpr_first(kf[0], qf[0]);
          else mfma32_vgpr(s, kf[c % (KA + 1)], qf[c]);
          if constexpr (c + KA < N)
            kf[(c + KA) % (KA + 1)] = lds_read_b128_at<(c + KA) * kBlock>(ka);
          if constexpr (UNIFORM_BT && c % 4 == 0) dma_chunk(nsrc, nbuf, c / 4);
        });
        mfma_vgpr_settle(s);
      }

      const int base = t * kTile;
      if (!(base >= row_lo && base + kTile - 1 <= row_hi)) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int k = base + (i / 4) * 8 + half * 4 + (i % 4);
          s[i] = (k >= row_lo && k <= row_hi) ? s[i] : -INFINITY;
        }
      }
      float mx = s[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[i]);
      mx = pair_max(mx) * c2;
      if (__ballot(mx > m_run + 8.f) != 0) {
        const float m_new = fmaxf(m_run, mx);
        const float alpha = m_new == -INFINITY ? 1.f : fast_exp2(m_run - m_new);
        l_run *= alpha;
        oacc_scale<0, 256>(alpha);
        m_run = m_new;
      }
      const float m_sub = m_run == -INFINITY ? 0.f : m_run;
#pragma unroll
      for (int i = 0; i < 16; ++i) s[i] = fast_exp2(fmaf(s[i], c2, -m_sub));
      const bf16x8 pf0 = to_bf16x8(s[0], s[1], s[2], s[3], s[4], s[5], s[6], s[7]);
      const bf16x8 pf1 = to_bf16x8(s[8], s[9], s[10], s[11], s[12], s[13], s[14], s[15]);
      const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
      static_for<4>([&](auto ii) {
        constexpr int i = decltype(ii)::value;
        l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf0, pf0, 2 * i, 2 * i + 1),
                                                ones, l_run, false);
        l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf1, pf1, 2 * i, 2 * i + 1),
                                                ones, l_run, false);
      });

      // O^T += V^T P^T: step st covers output block b = st % 16 (columns 32 b +
      // [0, 32), k-chunks 2 b + tr_g) and keys 16 j + [0, 16), j = st / 16;
      // the transposed reads run VA steps ahead
      {
        constexpr int N = 2 * kOB, VA = 4;
        bf16x4 vr[VA + 1][2];
        auto read_v = [&](auto ss) __attribute__((always_inline)) {
          constexpr int st = decltype(ss)::value;
          constexpr int j = st / kOB, bo = (st % kOB) * 2 * kBlock;
          vr[st % (VA + 1)][0] = lds_read_tr4_at<bo>(kt + v_lane[j][0]);
          vr[st % (VA + 1)][1] = lds_read_tr4_at<bo>(kt + v_lane[j][1]);
        };
        static_for<VA>(read_v);
        static_for<N>([&](auto ss) {
          constexpr int st = decltype(ss)::value;
          constexpr int issued = st + VA < N ? st + VA : N;
          lds_wait<2 * (issued - 1 - st)>(vr[st % (VA + 1)][0], vr[st % (VA + 1)][1]);
          oacc_mfma<st % kOB>(cat8(vr[st % (VA + 1)][0], vr[st % (VA + 1)][1]),
                              st / kOB == 0 ? pf0 : pf1);
          if constexpr (st + VA < N) read_v(std::integral_constant<int, st + VA>{});
        });
      }
    }

    const bool complete = p0 >= g0 && p1 <= g1;
    const float l_tot = pair_sum(l_run);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const float lse_val = l_tot > 0.f ? (m_run + fast_log2(l_tot)) * kLn2 : -INFINITY;
    // final rows of an item inside this workgroup's range, else a piece of an
    // item shared with neighbouring workgroups (bf16, merged later)
    const int64_t orow = ((int64_t)d.split * p.num_tokens + d.token) * p.num_q_heads + head0 + hl;
    const int64_t prow = ((int64_t)group * 2 * G + (p0 < g0 ? 2 * w : 2 * w + 1)) * kHeads + hl;
    // pieces are bf16 (half the bytes of fp32 to write and merge: the attention
    // call measured 1.5 % faster; their rounding is that of a bf16 output);
    // final rows take the caller's output type
    void* dst = complete ? p.out : static_cast<void*>(wk.piece_o);
    const int64_t e0 = (complete ? orow : prow) * kDV + dcol;
    const int odt = complete ? p.out_dtype : kOutBf16;
    oacc_settle();
    static_for<kOB>([&](auto bb) {
      constexpr int b = decltype(bb)::value;
      const f32x16 v = oacc_get<b>();
#pragma unroll
      for (int q = 0; q < 4; ++q)
        store_out4(dst, e0 + b * 32 + q * 8, odt, v[4 * q] * inv, v[4 * q + 1] * inv,
                   v[4 * q + 2] * inv, v[4 * q + 3] * inv);
    });
    if (half == 0) {
      if (!complete) wk.piece_lse[prow] = lse_val;
      else if (p.lse != nullptr) p.lse[orow] = lse_val;
    }

    g = min(g1, p1);
    if (g >= g1) break;
    ++it;
    while (wk.prefix[it + 1] <= g) ++it;  // skip items without tiles
  }
}

// One wave per (item, head): merge the pieces of items that span several
// workgroups (LSE-weighted, as the combine step does), and write 0 / -inf for
// items without tiles.  Items inside one workgroup's range are already final.
__global__ __launch_bounds__(256) void decode_merge_kernel(const AttnParams p, const DecodeWork wk,
                                                           int heads_per_group) {
  using namespace dec;
  const int lane = threadIdx.x % kWave;
  const int64_t row = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave;
  const int items = p.num_tokens * p.num_splits;
  if (row >= (int64_t)items * p.num_q_heads) return;
  const int item = (int)(row / p.num_q_heads);
  const int head = (int)(row - (int64_t)item * p.num_q_heads);
  const int group = head / heads_per_group, hl = head - group * heads_per_group;
  const int G = wk.grid;
  const int total = wk.prefix[items];
  const int per = max(1, (total + G - 1) / G);
  const int p0 = wk.prefix[item], p1 = wk.prefix[item + 1];
  const int token = item / p.num_splits, split = item - token * p.num_splits;
  const int64_t orow = ((int64_t)split * p.num_tokens + token) * p.num_q_heads + head;
  const int wf = p0 / per, wl = p1 > p0 ? (p1 - 1) / per : wf;
  PSW_DCHECK(11, p0 <= p1);
  PSW_DCHECK(10, p1 <= p0 || (wf >= 0 && wl < G));
  if (p1 > p0 && wf == wl) return;  // written by its workgroup

  const int n = p1 > p0 ? wl - wf + 1 : 0;
  auto piece_row = [&](int k) -> int64_t {
    const int slot = k == 0 ? 2 * wf + 1 : 2 * (wf + k);
    return ((int64_t)group * 2 * G + slot) * heads_per_group + hl;
  };
  float M = -INFINITY;
  for (int k = lane; k < n; k += kWave) M = fmaxf(M, wk.piece_lse[piece_row(k)]);
  M = wave_max(M);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  if (M != -INFINITY) {
    for (int base = 0; base < n; base += kWave) {
      const int k = base + lane;
      const float wt_lane = k < n ? __expf(wk.piece_lse[piece_row(k)] - M) : 0.f;
      wsum += wave_sum(wt_lane);
      const int cnt = min(kWave, n - base);
      for (int j = 0; j < cnt; ++j) {
        const float wt = __builtin_bit_cast(
            float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wt_lane), j));
        float v[8];
        load8<kOutBf16>(wk.piece_o, piece_row(base + j) * kDV + lane * 8, v);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += wt * v[i];
      }
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  const int64_t e0 = orow * kDV + lane * 8;
  store_out4(p.out, e0, p.out_dtype, acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
  store_out4(p.out, e0 + 4, p.out_dtype, acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv);
  if (p.lse != nullptr && lane == 0) p.lse[orow] = wsum > 0.f ? M + __logf(wsum) : -INFINITY;
}

bool decode_supported(const AttnParams& p) {
  return p.head_dim_qk == dec::kD && p.head_dim_v == dec::kDV && p.v_cache == p.k_cache &&
         p.queries_per_kv % 32 == 0;
}

namespace {

int heads_per_workgroup(const AttnParams& p) {
  // as many query heads of one KV head per workgroup as the shapes allow
  if (p.queries_per_kv % 128 == 0) return 128;
  if (p.queries_per_kv % 64 == 0) return 64;
  return 32;
}

// Workgroups per head group: one per CU (each holds a whole CU's LDS budget).
int decode_grid(const AttnParams& p) {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
      cus = v;
  }
  const int groups = p.num_q_heads / heads_per_workgroup(p);
  return max(1, cus / max(1, groups));
}

constexpr int64_t align256(int64_t v) { return (v + 255) & ~int64_t(255); }

struct DecodeLayout {
  int64_t prefix_off, lse_off, o_off, bytes;
};

DecodeLayout decode_layout(const AttnParams& p, int grid) {
  const int64_t items = (int64_t)p.num_tokens * p.num_splits;
  const int64_t pieces = (int64_t)2 * grid * p.num_q_heads;  // over all head groups
  DecodeLayout l;
  l.prefix_off = 0;
  l.lse_off = align256((items + 1) * 4);
  l.o_off = l.lse_off + align256(pieces * 4);
  l.bytes = l.o_off + pieces * dec::kDV * 2;
  return l;
}

template <int NB, int HG, bool UNIFORM_BT>
hipError_t launch_decode_t(const AttnParams& p, const DecodeWork& wk, hipStream_t stream) {
  constexpr int kBufs = UNIFORM_BT ? 3 : 2;
  const size_t lds = kBufs * dec::kTileBytes + (size_t)(2 * HG) * NB * 16 * kWave * sizeof(float);
  auto kern = decode_attention_kernel<NB, HG, UNIFORM_BT>;
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(kern, dim3(wk.grid, p.num_q_heads / (HG * NB * 32)), dim3(HG * 128), lds,
                     stream, p, wk);
  return hipGetLastError();
}

template <bool UNIFORM_BT>
hipError_t launch_decode_full(const AttnParams& p, const DecodeWork& wk, hipStream_t stream) {
  constexpr int kBufs = UNIFORM_BT ? 3 : 2;
  const size_t lds = kBufs * dec::kTileBytes;
  auto kern = decode_full_kernel<UNIFORM_BT>;
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(kern, dim3(wk.grid, p.num_q_heads / 128), dim3(256), lds, stream, p, wk);
  return hipGetLastError();
}

template <bool UNIFORM_BT>
hipError_t launch_decode_shape(const AttnParams& p, int heads, const DecodeWork& wk,
                               hipStream_t stream) {
  if (heads == 128) return launch_decode_full<UNIFORM_BT>(p, wk, stream);
  // 64 heads as two 32-head groups of two waves each: one group of 64 heads per
  // wave pair needs more than the register file and spills inside its loop
  // (4x slower when measured)
  if (heads == 64) return launch_decode_t<1, 2, UNIFORM_BT>(p, wk, stream);
  return launch_decode_t<1, 1, UNIFORM_BT>(p, wk, stream);
}

}  // namespace

int64_t decode_workspace_bytes(const AttnParams& p) {
  return decode_layout(p, decode_grid(p)).bytes;
}

// Scratch of the allocation-free attention entry point: the latent decode's
// workspace (tile prefix and the pieces of shared items) at a fixed place in
// device memory.  Every device the library runs on holds its own copy from
// module load until the process ends.  Nothing in it needs clearing between
// calls: the plan kernel writes the whole prefix, and the merge reads only
// pieces the same call's attention kernel wrote.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

hipError_t scratch_device_ptr(void** ptr) {
  // In host code `scratch` is only a stand-in for the device symbol: its
  // address on each device comes from hipGetSymbolAddress, taken once per
  // device with that device current, and is used instead of the name.
  constexpr int kMaxDevices = 64;
  static std::mutex mutex;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mutex);
  if (addr[dev] == nullptr) {
    void* a = nullptr;
    e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (a == nullptr || (reinterpret_cast<uintptr_t>(a) & 255) != 0) return hipErrorInvalidSymbol;
    addr[dev] = a;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_attention_decode(const AttnParams& p, void* workspace, hipStream_t stream) {
  if (p.num_tokens == 0 || p.num_splits == 0) return hipSuccess;
  const int grid = decode_grid(p);
  const DecodeLayout l = decode_layout(p, grid);
  char* ws = static_cast<char*>(workspace);
  DecodeWork wk;
  wk.prefix = reinterpret_cast<const int32_t*>(ws + l.prefix_off);
  wk.piece_lse = reinterpret_cast<float*>(ws + l.lse_off);
  wk.piece_o = reinterpret_cast<uint16_t*>(ws + l.o_off);
  wk.grid = grid;
  hipLaunchKernelGGL(decode_plan_kernel, dim3(1), dim3(dec::kPlanThreads), 0, stream, p,
                     reinterpret_cast<int32_t*>(ws + l.prefix_off));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int hpw = heads_per_workgroup(p);
  // a 32-key tile lies inside one KV block when blocks hold at least 32 keys
  if (p.block_size_log2 >= 5) e = launch_decode_shape<true>(p, hpw, wk, stream);
  else e = launch_decode_shape<false>(p, hpw, wk, stream);
  if (e != hipSuccess) return e;
  const int64_t rows = (int64_t)p.num_tokens * p.num_splits * p.num_q_heads;
  hipLaunchKernelGGL(decode_merge_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream,
                     p, wk, hpw);
  return hipGetLastError();
}

PSW_DEBUG_TAKE(debug_take_decode)

}  // namespace psw
