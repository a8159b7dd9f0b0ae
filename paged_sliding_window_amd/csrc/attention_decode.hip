// Split-KV decode attention for the latent (MLA-shaped) cache: every query head
// reads one shared 576-wide latent row per key, and V is that row's first 512
// columns (MLA DCP decode study notes, vllm-ascend PR #16977: "Terms" for MLA;
// sections 1.1 and 3.1 for the history/current partials that each emit an
// output and an LSE; code blocks B and C for the two partial calls).
//
// One workgroup = one new token x NHB * 32 query heads x one key split, with
// two waves per 32-head block:
//   * tiles of 32 keys are gathered once per workgroup into LDS with
//     direct-to-LDS 16-byte loads, double buffered (tile t+1 and the block-table
//     reads of tile t+2 are in flight while tile t is computed).  LDS-DMA
//     instruction c moves the 16-wide k-chunk c of all 32 keys as one block, so
//     a K read for k-chunk c and the transposed V reads are a lane base plus an
//     immediate;
//   * S^T[32 keys][32 heads] = K Q^T is split over the 576-long dot product:
//     wave (hb, 0) sums k-chunks 0..17 and wave (hb, 1) k-chunks 18..35, each
//     with its Q fragments in registers; the halves are exchanged through LDS
//     and both waves add them in the same order, so they hold identical scores;
//   * both waves run the same online softmax; wave (hb, d) then accumulates
//     O^T += V^T P^T for output columns [256 d, 256 d + 256), reading V^T out of
//     the same K tile with ds_read_b64_tr_b16;
//   * the running max moves only when it grows by more than 2^8 (log2 units).
// The mask (window, image ranges, key range of the split) is applied exactly
// as in the prefill kernel; one query position per workgroup makes it uniform.
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
}  // namespace dec

// Slot (16 bytes) of key row r, column half hh (columns 8*hh..8*hh+7 of a
// k-chunk) inside a k-chunk block.  Rows of the second half are rotated by 4 so
// that the 4 rows x 2 halves of a transposed read hit 8 distinct bank groups.
__device__ __forceinline__ int dec_slot(int r, int hh) { return 32 * hh + ((r + 4 * hh) & 31); }

__device__ __forceinline__ void dec_dma16(const void* gsrc, void* lds_dst) {
  __builtin_amdgcn_global_load_lds(
      (const __attribute__((address_space(1))) void*)gsrc,
      (__attribute__((address_space(3))) void*)(lds_void*)lds_dst, 16, 0, 0);
}

template <int NHB>
__global__ __launch_bounds__(NHB * 128) void decode_attention_kernel(const AttnParams p) {
  using namespace dec;
  constexpr int kWaves = 2 * NHB;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  float* xs = reinterpret_cast<float*>(smem + 2 * kTileBytes);  // [kWaves][4][64][4]

  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int half = lane >> 5;
  const int hb = wave >> 1, dh = wave & 1;
  const int token = blockIdx.x;
  const int head0 = blockIdx.y * (NHB * 32);
  const int split = blockIdx.z;
  const int qpk = p.queries_per_kv;
  const int kvh = head0 / qpk;

  int s_lo = 0, s_hi = p.num_seqs - 1;
  while (s_lo < s_hi) {
    const int mid = (s_lo + s_hi + 1) >> 1;
    if (p.query_start_loc[mid] <= token) s_lo = mid; else s_hi = mid - 1;
  }
  const int seq = s_lo;
  const int q_start = p.query_start_loc[seq];
  const int query_len = p.query_start_loc[seq + 1] - q_start;
  const int qpos = token - q_start;
  const int seq_len = p.seq_lens[seq];
  const int ctx = seq_len - query_len;
  const int32_t* ranges = p.mm_ranges ? p.mm_ranges + (int64_t)seq * p.max_mm_ranges * 2 : nullptr;
  int key_begin = 0, key_end = seq_len;
  if (p.key_ranges) {
    key_begin = max(0, p.key_ranges[((int64_t)split * p.num_seqs + seq) * 2]);
    key_end = min(seq_len, p.key_ranges[((int64_t)split * p.num_seqs + seq) * 2 + 1]);
  }
  const TileRange tr = tile_bounds(ctx, seq_len, query_len, qpos, kTile, qpk, 1, qpk, p.geom,
                                   ranges, p.max_mm_ranges);
  const int t_lo = max(tr.lo, key_begin / kTile);
  const int t_hi = min(tr.hi, (key_end + kTile - 1) / kTile);

  int row_lo = INT32_MAX, row_hi = INT32_MIN;
  {
    int64_t lo64, hi64;
    row_interval((int64_t)ctx + qpos, seq_len, p.geom, ranges, p.max_mm_ranges, key_begin,
                 key_end, lo64, hi64);
    if (lo64 <= hi64) {
      row_lo = (int)lo64;
      row_hi = (int)hi64;
    }
  }

  const int head = head0 + hb * 32 + (lane & 31);
  bf16x8 qf[kHalfChunks];
  {
    const uint16_t* qrow =
        p.q + ((int64_t)token * p.num_q_heads + head) * kD + dh * (kHalfChunks * 16) + half * 8;
#pragma unroll
    for (int c = 0; c < kHalfChunks; ++c) qf[c] = *reinterpret_cast<const bf16x8*>(qrow + c * 16);
  }

  f32x16 o[kOBlocks];
#pragma unroll
  for (int b = 0; b < kOBlocks; ++b) o[b] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  if (t_lo < t_hi) {
    const int64_t slot_pitch = (int64_t)p.num_kv_heads * kD;
    const uint16_t* kbase = p.k_cache + (int64_t)kvh * kD;
    const int32_t* bt = p.block_table + (int64_t)seq * p.block_table_stride;
    const int bs_log2 = p.block_size_log2;
    const int bs_mask = (1 << bs_log2) - 1;
    const float c2 = p.scale_log2;

    // lane l < 32 holds the physical block of key (tile * 32 + l)
    auto fetch_block = [&](int tile) -> int {
      const int key = min(tile * kTile + (lane & 31), seq_len - 1);
      return bt[key >> bs_log2];
    };
    // this lane's DMA slot: key row and column half within every k-chunk block
    const int dma_hh = lane >> 5;
    const int dma_row = (lane - 4 * dma_hh) & 31;
    auto issue_tile = [&](int tile, int buf, int blk_of_lane) {
      const int key = min(tile * kTile + dma_row, seq_len - 1);
      const int blk = __shfl(blk_of_lane, dma_row, kWave);
      const uint16_t* src = kbase + (((int64_t)blk << bs_log2) + (key & bs_mask)) * slot_pitch +
                            dma_hh * 8;
      char* dst = smem + buf * kTileBytes;
#pragma unroll
      for (int i = 0; i < kKChunks / kWaves; ++i) {
        const int c = i * kWaves + wave;
        dec_dma16(src + c * 16, dst + c * kBlock);
      }
      if constexpr (kKChunks % kWaves != 0) {
        const int c = (kKChunks / kWaves) * kWaves + wave;
        if (wave < kKChunks % kWaves) dec_dma16(src + c * 16, dst + c * kBlock);
      }
    };

    int blk_next = fetch_block(t_lo);
    issue_tile(t_lo, 0, blk_next);
    if (t_lo + 1 < t_hi) blk_next = fetch_block(t_lo + 1);

    // transposed V reads: group of 16 lanes covers 4 keys x 16 columns
    const int tr_key = half * 4 + ((lane & 15) >> 2);   // + 16 j (+ 8 for the upper 4 keys)
    const int tr_g = (lane >> 4) & 1;                    // which 16 of a 32-column block
    const int tr_hh = (lane & 3) >> 1, tr_in = (lane & 1) * 8;

    for (int t = t_lo; t < t_hi; ++t) {
      const int buf = (t - t_lo) & 1;
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (t + 1 < t_hi) {
        issue_tile(t + 1, buf ^ 1, blk_next);
        if (t + 2 < t_hi) blk_next = fetch_block(t + 2);
      }
      const char* kt = smem + buf * kTileBytes;

      f32x16 s = f32x16{};
      {
        const char* arow = kt + dec_slot(lane & 31, half) * 16;
#pragma unroll
        for (int c = 0; c < kHalfChunks; ++c) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(arow + (dh * kHalfChunks + c) * kBlock);
          s = mfma32(a, qf[c], s);
        }
      }
      // exchange of the two halves: layout [wave][4][lane][4 floats]
      {
        f32x4* mine = reinterpret_cast<f32x4*>(xs) + wave * 4 * kWave + lane;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          mine[i * kWave] = f32x4{s[4 * i], s[4 * i + 1], s[4 * i + 2], s[4 * i + 3]};
      }
      __syncthreads();
      {
        const f32x4* other = reinterpret_cast<const f32x4*>(xs) + (wave ^ 1) * 4 * kWave + lane;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const f32x4 part = other[i * kWave];
          // both waves of the pair add the halves in the same order
#pragma unroll
          for (int k = 0; k < 4; ++k)
            s[4 * i + k] = dh == 0 ? s[4 * i + k] + part[k] : part[k] + s[4 * i + k];
        }
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
      mx = fmaxf(mx, swap_halves(mx)) * c2;
      if (__ballot(mx > m_run + 8.f) != 0) {
        const float m_new = fmaxf(m_run, mx);
        const float alpha = m_new == -INFINITY ? 1.f : fast_exp2(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int b = 0; b < kOBlocks; ++b) o[b] *= alpha;
        m_run = m_new;
      }
      const float m_sub = m_run == -INFINITY ? 0.f : m_run;
      float psum = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        s[i] = fast_exp2(fmaf(s[i], c2, -m_sub));
        psum += s[i];
      }
      l_run += psum;
      const bf16x8 pf0 = to_bf16x8(s[0], s[1], s[2], s[3], s[4], s[5], s[6], s[7]);
      const bf16x8 pf1 = to_bf16x8(s[8], s[9], s[10], s[11], s[12], s[13], s[14], s[15]);

#pragma unroll
      for (int b = 0; b < kOBlocks; ++b) {
        // output columns dh*256 + b*32 + [0, 32): k-chunk block 2 * (dh*8 + b) + tr_g
        const char* blk = kt + (2 * (dh * kOBlocks + b) + tr_g) * kBlock + tr_in;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int ka = 16 * j + tr_key, kb2 = ka + 8;
          const bf16x4 lo = lds_read_tr4(reinterpret_cast<const __bf16*>(blk + dec_slot(ka, tr_hh) * 16));
          const bf16x4 hi = lds_read_tr4(reinterpret_cast<const __bf16*>(blk + dec_slot(kb2, tr_hh) * 16));
          o[b] = mfma32(cat8(lo, hi), j == 0 ? pf0 : pf1, o[b]);
        }
      }
    }
  }

  const float l_tot = l_run + swap_halves(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const int64_t orow = ((int64_t)split * p.num_tokens + token) * p.num_q_heads + head;
  const int dcol = dh * (kDV / 2) + half * 4;
  if (p.out_f32) {
    float* dst = static_cast<float*>(p.out) + orow * kDV + dcol;
#pragma unroll
    for (int b = 0; b < kOBlocks; ++b)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<float4*>(dst + b * 32 + g * 8) =
            make_float4(o[b][4 * g] * inv, o[b][4 * g + 1] * inv, o[b][4 * g + 2] * inv,
                        o[b][4 * g + 3] * inv);
  } else {
    uint16_t* dst = static_cast<uint16_t*>(p.out) + orow * kDV + dcol;
#pragma unroll
    for (int b = 0; b < kOBlocks; ++b)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<bf16x4*>(dst + b * 32 + g * 8) =
            to_bf16x4(o[b][4 * g] * inv, o[b][4 * g + 1] * inv, o[b][4 * g + 2] * inv,
                      o[b][4 * g + 3] * inv);
  }
  if (p.lse != nullptr && dh == 0 && half == 0)
    p.lse[orow] = l_tot > 0.f ? (m_run + fast_log2(l_tot)) * kLn2 : -INFINITY;
}

bool decode_supported(const AttnParams& p) {
  return p.head_dim_qk == dec::kD && p.head_dim_v == dec::kDV && p.v_cache == p.k_cache &&
         p.queries_per_kv % 32 == 0;
}

template <int NHB>
static hipError_t launch_decode_t(const AttnParams& p, hipStream_t stream) {
  const size_t lds = 2 * dec::kTileBytes + (size_t)(2 * NHB) * 16 * kWave * sizeof(float);
  auto kern = decode_attention_kernel<NHB>;
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(kern, dim3(p.num_tokens, p.num_q_heads / (NHB * 32), p.num_splits),
                     dim3(NHB * 128), lds, stream, p);
  return hipGetLastError();
}

hipError_t launch_attention_decode(const AttnParams& p, hipStream_t stream) {
  if (p.num_tokens == 0) return hipSuccess;
  // as many 32-head blocks per workgroup as one KV head's query group allows
  if (p.queries_per_kv % 128 == 0) return launch_decode_t<4>(p, stream);
  if (p.queries_per_kv % 64 == 0) return launch_decode_t<2>(p, stream);
  return launch_decode_t<1>(p, stream);
}

}  // namespace psw
