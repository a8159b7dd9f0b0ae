// Split-KV decode attention for the latent (MLA-shaped) cache: every query head
// reads one shared 576-wide latent row per key, and V is that row's first 512
// columns (MLA DCP decode study notes, vllm-ascend PR #16977: "Terms" for MLA;
// sections 1.1 and 3.1 for the history/current partials that each emit an
// output and an LSE; code blocks B and C for the two partial calls).
//
// One workgroup = one new token x 32 query heads x one key split; 4 waves.
//   * a tile of 32 keys is gathered once into LDS (row-major [key][576]);
//   * S^T[32 keys][32 rows] is split over the 576-long dot product: wave w owns
//     k-chunks [9w, 9w+9) with its Q fragments in registers, writes its partial
//     sums to LDS, and every wave adds the four partials (same order in every
//     wave, so all waves hold identical scores);
//   * every wave runs the same online softmax, then O^T += V^T P^T for its own
//     128-column slice of the 512-wide output, reading V^T out of the same K
//     tile with ds_read_b64_tr_b16.
// Keys of a split outside the allowed interval of the row are masked exactly as
// in the prefill kernel (the window / image machinery applies unchanged).
#include "device_common.h"
#include "psw_internal.h"

namespace psw {

namespace dec {
constexpr int kD = 576, kDV = 512;
constexpr int kWaves = 4, kThreads = kWaves * kWave;
constexpr int kRows = 32;            // query heads per workgroup
constexpr int kTile = 32;            // keys per tile
constexpr int kKStride = kD + 8;     // LDS pitch in bf16
constexpr int kChunksPerWave = kD / 16 / kWaves;  // 9
constexpr int kOBlocksPerWave = kDV / 32 / kWaves;  // 4
constexpr int kLoadChunks = (kTile * kD / 8 + kThreads - 1) / kThreads;  // 9
}  // namespace dec

__global__ __launch_bounds__(dec::kThreads) void decode_attention_kernel(const AttnParams p) {
  using namespace dec;
  __shared__ __attribute__((aligned(16))) __bf16 k_lds[kTile * kKStride];
  __shared__ __attribute__((aligned(16))) float s_part[kWaves][16][kWave];

  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int half = lane >> 5;
  const int token = blockIdx.x;
  const int head0 = blockIdx.y * kRows;
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

  const int head = head0 + (lane & 31);
  bf16x8 qf[kChunksPerWave];
  {
    const uint16_t* qrow =
        p.q + ((int64_t)token * p.num_q_heads + head) * kD + wave * (kChunksPerWave * 16) + half * 8;
#pragma unroll
    for (int c = 0; c < kChunksPerWave; ++c) qf[c] = *reinterpret_cast<const bf16x8*>(qrow + c * 16);
  }

  f32x16 o[kOBlocksPerWave];
#pragma unroll
  for (int b = 0; b < kOBlocksPerWave; ++b) o[b] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  const int64_t slot_pitch = (int64_t)p.num_kv_heads * kD;
  const uint16_t* kbase = p.k_cache + (int64_t)kvh * kD;
  const int32_t* bt = p.block_table + (int64_t)seq * p.block_table_stride;
  const int bs_log2 = p.block_size_log2;
  const int bs_mask = (1 << bs_log2) - 1;
  const float c2 = p.scale_log2;
  const int tr_row = half * 4 + ((lane & 15) >> 2);
  const int tr_col = wave * (kOBlocksPerWave * 32) + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  for (int t = t_lo; t < t_hi; ++t) {
    const int tile_base = t * kTile;
    uint4 kreg[kLoadChunks];
#pragma unroll
    for (int i = 0; i < kLoadChunks; ++i) {
      const int c = i * kThreads + tid;
      const int row = c / (kD / 8), col = (c % (kD / 8)) * 8;
      const int key = tile_base + row;
      kreg[i] = make_uint4(0, 0, 0, 0);
      if (row < kTile && key < seq_len) {
        const int64_t slot = ((int64_t)bt[key >> bs_log2] << bs_log2) + (key & bs_mask);
        kreg[i] = *reinterpret_cast<const uint4*>(kbase + slot * slot_pitch + col);
      }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kLoadChunks; ++i) {
      const int c = i * kThreads + tid;
      const int row = c / (kD / 8), col = (c % (kD / 8)) * 8;
      if (row < kTile) *reinterpret_cast<uint4*>(&k_lds[row * kKStride + col]) = kreg[i];
    }
    __syncthreads();

    f32x16 sp = f32x16{};
#pragma unroll
    for (int c = 0; c < kChunksPerWave; ++c) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(
          &k_lds[(lane & 31) * kKStride + (wave * kChunksPerWave + c) * 16 + half * 8]);
      sp = mfma32(a, qf[c], sp);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) s_part[wave][i][lane] = sp[i];
    __syncthreads();
    f32x16 s = f32x16{};
#pragma unroll
    for (int w = 0; w < kWaves; ++w)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[i] += s_part[w][i][lane];

    const bool full = tile_base >= row_lo && tile_base + kTile - 1 <= row_hi;
    if (!full) {  // one query row per workgroup: uniform branch
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int k = tile_base + (i / 4) * 8 + half * 4 + (i % 4);
        s[i] = (k >= row_lo && k <= row_hi) ? s[i] : -INFINITY;
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[i]);
    mx = fmaxf(mx, swap_halves(mx));
    const float m_new = fmaxf(m_run, mx * c2);
    const float m_sub = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_sub);
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      s[i] = fast_exp2(fmaf(s[i], c2, -m_sub));
      psum += s[i];
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int b = 0; b < kOBlocksPerWave; ++b) o[b] *= alpha;
    const bf16x8 pf0 = to_bf16x8(s[0], s[1], s[2], s[3], s[4], s[5], s[6], s[7]);
    const bf16x8 pf1 = to_bf16x8(s[8], s[9], s[10], s[11], s[12], s[13], s[14], s[15]);
#pragma unroll
    for (int b = 0; b < kOBlocksPerWave; ++b) {
      const __bf16* src0 = &k_lds[tr_row * kKStride + b * 32 + tr_col];
      const __bf16* src1 = src0 + 16 * kKStride;
      o[b] = mfma32(cat8(lds_read_tr4(src0), lds_read_tr4(src0 + 8 * kKStride)), pf0, o[b]);
      o[b] = mfma32(cat8(lds_read_tr4(src1), lds_read_tr4(src1 + 8 * kKStride)), pf1, o[b]);
    }
  }

  const float l_tot = l_run + swap_halves(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const int64_t orow = ((int64_t)split * p.num_tokens + token) * p.num_q_heads + head;
  const int dcol = wave * (kOBlocksPerWave * 32) + half * 4;
  if (p.out_f32) {
    float* dst = static_cast<float*>(p.out) + orow * kDV + dcol;
#pragma unroll
    for (int b = 0; b < kOBlocksPerWave; ++b)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<float4*>(dst + b * 32 + g * 8) =
            make_float4(o[b][4 * g] * inv, o[b][4 * g + 1] * inv, o[b][4 * g + 2] * inv,
                        o[b][4 * g + 3] * inv);
  } else {
    uint16_t* dst = static_cast<uint16_t*>(p.out) + orow * kDV + dcol;
#pragma unroll
    for (int b = 0; b < kOBlocksPerWave; ++b)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<bf16x4*>(dst + b * 32 + g * 8) =
            to_bf16x4(o[b][4 * g] * inv, o[b][4 * g + 1] * inv, o[b][4 * g + 2] * inv,
                      o[b][4 * g + 3] * inv);
  }
  if (p.lse != nullptr && wave == 0 && half == 0)
    p.lse[orow] = l_tot > 0.f ? (m_run + fast_log2(l_tot)) * kLn2 : -INFINITY;
}

bool decode_supported(const AttnParams& p) {
  return p.head_dim_qk == dec::kD && p.head_dim_v == dec::kDV && p.v_cache == p.k_cache &&
         p.num_q_heads % dec::kRows == 0 && p.queries_per_kv % dec::kRows == 0;
}

hipError_t launch_attention_decode(const AttnParams& p, hipStream_t stream) {
  if (p.num_tokens == 0) return hipSuccess;
  hipLaunchKernelGGL(decode_attention_kernel,
                     dim3(p.num_tokens, p.num_q_heads / dec::kRows, p.num_splits),
                     dim3(dec::kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace psw
