// Paged prefill attention under the sliding window OR-ed with window-clamped
// image ranges, visiting only the KV tiles of each query block's union interval
// (vLLM PR #53147 summary, "Implementation breakdown" and "Key source snippet").
//
// Work decomposition (gfx950, wave64):
//   * one workgroup = one query block x one KV head x one key split; 4 waves,
//     32 rows each, 128 rows = (128 / queries_per_kv) positions x the query heads
//     of that KV head (rows position-major), so a K/V tile staged in LDS serves
//     every query head sharing it;
//   * KV tiles of 64 keys, gathered from the paged cache through the block table
//     with 16-byte loads (each key's row is contiguous) and staged in LDS in the
//     cache's own [key][dim] layout;
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16: K from LDS as the A operand,
//     Q held in registers as the B operand, so each lane ends up holding 32
//     scores of ONE query row (the other 32 keys of the row sit in lane ^ 32);
//     the online softmax then needs a single cross-half exchange per tile;
//   * O^T += V^T P^T: P^T comes straight from the S^T accumulators (converted
//     to bf16), V^T is read out of the row-major V tile with ds_read_b64_tr_b16,
//     and O^T keeps one query row per lane, so the rescale is per lane;
//   * per-element masking only on tiles that are not entirely inside every
//     row's allowed interval (each row's allowed keys form one interval).
#include "device_common.h"
#include "psw_internal.h"

namespace psw {

template <int D, int DV>
struct PrefillShape {
  static constexpr int kWaves = 4;
  static constexpr int kThreads = kWaves * kWave;
  static constexpr int kRowsPerWave = 32;
  static constexpr int kBlockM = kWaves * kRowsPerWave;
  static constexpr int kTile = 64;
  static constexpr int kKStride = D + 8;  // LDS row pitch in bf16 (16 B of padding)
  static constexpr int kVStride = DV + 8;
  static constexpr int kQFrags = D / 16;
  static constexpr int kOBlocks = DV / 32;
  static constexpr int kKChunks = kTile * D / 8 / kThreads;
  static constexpr int kVChunks = kTile * DV / 8 / kThreads;
  static_assert(kKChunks >= 1 && kVChunks >= 1, "tile too small for the workgroup");
};

template <int D, int DV>
__global__ __launch_bounds__(256) void prefill_attention_kernel(const AttnParams p) {
  using S = PrefillShape<D, DV>;
  __shared__ __attribute__((aligned(16))) __bf16 k_lds[S::kTile * S::kKStride];
  __shared__ __attribute__((aligned(16))) __bf16 v_lds[S::kTile * S::kVStride];

  const int tid = threadIdx.x;
  const int lane = tid % kWave, wave = tid / kWave;
  const int half = lane >> 5;
  const int kvh = blockIdx.y, split = blockIdx.z;
  const int qpk = p.queries_per_kv;
  const int block_q = S::kBlockM / qpk;

  // ---- request and query block of this workgroup --------------------------
  // Query blocks of request s occupy grid slots [qsl[s] / block_q + s, ...).
  const int x = blockIdx.x;
  int s_lo = 0, s_hi = p.num_seqs - 1;
  while (s_lo < s_hi) {
    const int mid = (s_lo + s_hi + 1) >> 1;
    if (p.query_start_loc[mid] / block_q + mid <= x) s_lo = mid; else s_hi = mid - 1;
  }
  const int seq = s_lo;
  const int q_start = p.query_start_loc[seq];
  const int query_len = p.query_start_loc[seq + 1] - q_start;
  const int q_block = x - (q_start / block_q + seq);
  if (q_block * block_q >= query_len) return;
  const int seq_len = p.seq_lens[seq];
  const int ctx = seq_len - query_len;
  const int32_t* ranges = p.mm_ranges ? p.mm_ranges + (int64_t)seq * p.max_mm_ranges * 2 : nullptr;
  int key_begin = 0, key_end = seq_len;
  if (p.key_ranges) {
    key_begin = max(0, p.key_ranges[((int64_t)split * p.num_seqs + seq) * 2]);
    key_end = min(seq_len, p.key_ranges[((int64_t)split * p.num_seqs + seq) * 2 + 1]);
  }
  const TileRange tr = tile_bounds(ctx, seq_len, query_len, q_block, S::kTile, block_q * qpk,
                                   block_q, qpk, p.geom, ranges, p.max_mm_ranges);
  const int t_lo = max(tr.lo, key_begin / S::kTile);
  const int t_hi = min(tr.hi, (key_end + S::kTile - 1) / S::kTile);

  // ---- this lane's query row ----------------------------------------------
  const int r = wave * S::kRowsPerWave + (lane & 31);
  const int pos_in_blk = r / qpk;
  const int head = kvh * qpk + (r - pos_in_blk * qpk);
  const int qpos = q_block * block_q + pos_in_blk;
  const bool row_valid = pos_in_blk < block_q && qpos < query_len;
  const int64_t token = (int64_t)q_start + qpos;
  int row_lo = INT32_MAX, row_hi = INT32_MIN;
  if (row_valid) {
    int64_t lo64, hi64;
    row_interval((int64_t)ctx + qpos, seq_len, p.geom, ranges, p.max_mm_ranges, key_begin,
                 key_end, lo64, hi64);
    if (lo64 <= hi64) {
      row_lo = (int)lo64;
      row_hi = (int)hi64;
    }
  }

  bf16x8 qf[S::kQFrags];
  {
    const uint16_t* qrow = p.q + (token * p.num_q_heads + head) * D + half * 8;
#pragma unroll
    for (int c = 0; c < S::kQFrags; ++c) {
      if (row_valid) qf[c] = *reinterpret_cast<const bf16x8*>(qrow + c * 16);
      else qf[c] = bf16x8{};
    }
  }

  f32x16 o[S::kOBlocks];
#pragma unroll
  for (int b = 0; b < S::kOBlocks; ++b) o[b] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  const bool latent = p.v_cache == p.k_cache;
  const int64_t k_slot_pitch = (int64_t)p.num_kv_heads * D;
  const int64_t v_slot_pitch = latent ? k_slot_pitch : (int64_t)p.num_kv_heads * DV;
  const uint16_t* kbase = p.k_cache + (int64_t)kvh * D;
  const uint16_t* vbase = p.v_cache + (int64_t)kvh * (latent ? D : DV);
  const int32_t* bt = p.block_table + (int64_t)seq * p.block_table_stride;
  const int bs_log2 = p.block_size_log2;
  const int bs_mask = (1 << bs_log2) - 1;
  const float c2 = p.scale_log2;

  for (int t = t_lo; t < t_hi; ++t) {
    const int tile_base = t * S::kTile;
    uint4 kreg[S::kKChunks], vreg[S::kVChunks];
#pragma unroll
    for (int i = 0; i < S::kKChunks; ++i) {
      const int c = i * S::kThreads + tid;
      const int row = c / (D / 8), col = (c % (D / 8)) * 8;
      const int key = tile_base + row;
      kreg[i] = make_uint4(0, 0, 0, 0);
      if (key < seq_len) {
        const int64_t slot = ((int64_t)bt[key >> bs_log2] << bs_log2) + (key & bs_mask);
        kreg[i] = *reinterpret_cast<const uint4*>(kbase + slot * k_slot_pitch + col);
      }
    }
#pragma unroll
    for (int i = 0; i < S::kVChunks; ++i) {
      const int c = i * S::kThreads + tid;
      const int row = c / (DV / 8), col = (c % (DV / 8)) * 8;
      const int key = tile_base + row;
      vreg[i] = make_uint4(0, 0, 0, 0);
      if (key < seq_len) {
        const int64_t slot = ((int64_t)bt[key >> bs_log2] << bs_log2) + (key & bs_mask);
        vreg[i] = *reinterpret_cast<const uint4*>(vbase + slot * v_slot_pitch + col);
      }
    }
    __syncthreads();  // every wave is done reading the previous tile
#pragma unroll
    for (int i = 0; i < S::kKChunks; ++i) {
      const int c = i * S::kThreads + tid;
      const int row = c / (D / 8), col = (c % (D / 8)) * 8;
      *reinterpret_cast<uint4*>(&k_lds[row * S::kKStride + col]) = kreg[i];
    }
#pragma unroll
    for (int i = 0; i < S::kVChunks; ++i) {
      const int c = i * S::kThreads + tid;
      const int row = c / (DV / 8), col = (c % (DV / 8)) * 8;
      *reinterpret_cast<uint4*>(&v_lds[row * S::kVStride + col]) = vreg[i];
    }
    __syncthreads();

    // S^T[key][row] for the two 32-key halves of the tile
    f32x16 s0 = f32x16{}, s1 = f32x16{};
#pragma unroll
    for (int c = 0; c < S::kQFrags; ++c) {
      const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(
          &k_lds[(lane & 31) * S::kKStride + c * 16 + half * 8]);
      const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(
          &k_lds[(32 + (lane & 31)) * S::kKStride + c * 16 + half * 8]);
      s0 = mfma32(a0, qf[c], s0);
      s1 = mfma32(a1, qf[c], s1);
    }

    const bool full = tile_base >= row_lo && tile_base + S::kTile - 1 <= row_hi;
    if (__ballot(!full) != 0) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int k0 = tile_base + (i / 4) * 8 + half * 4 + (i % 4);
        const int k1 = k0 + 32;
        s0[i] = (k0 >= row_lo && k0 <= row_hi) ? s0[i] : -INFINITY;
        s1[i] = (k1 >= row_lo && k1 <= row_hi) ? s1[i] : -INFINITY;
      }
    }

    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, fmaxf(s0[i], s1[i]));
    mx = fmaxf(mx, swap_halves(mx));
    const float m_new = fmaxf(m_run, mx * c2);
    const float m_sub = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_sub);
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      s0[i] = fast_exp2(fmaf(s0[i], c2, -m_sub));
      s1[i] = fast_exp2(fmaf(s1[i], c2, -m_sub));
      psum += s0[i] + s1[i];
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int b = 0; b < S::kOBlocks; ++b) o[b] *= alpha;

    bf16x8 pf[2][2];
    pf[0][0] = to_bf16x8(s0[0], s0[1], s0[2], s0[3], s0[4], s0[5], s0[6], s0[7]);
    pf[0][1] = to_bf16x8(s0[8], s0[9], s0[10], s0[11], s0[12], s0[13], s0[14], s0[15]);
    pf[1][0] = to_bf16x8(s1[0], s1[1], s1[2], s1[3], s1[4], s1[5], s1[6], s1[7]);
    pf[1][1] = to_bf16x8(s1[8], s1[9], s1[10], s1[11], s1[12], s1[13], s1[14], s1[15]);

    const int tr_row = half * 4 + ((lane & 15) >> 2);
    const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
    for (int b = 0; b < S::kOBlocks; ++b) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int row0 = kb * 32 + 16 * j + tr_row;
          const __bf16* src = &v_lds[row0 * S::kVStride + b * 32 + tr_col];
          const bf16x8 a = cat8(lds_read_tr4(src), lds_read_tr4(src + 8 * S::kVStride));
          o[b] = mfma32(a, pf[kb][j], o[b]);
        }
      }
    }
  }

  // ---- epilogue ------------------------------------------------------------
  const float l_tot = l_run + swap_halves(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (row_valid) {
    const int64_t orow = ((int64_t)split * p.num_tokens + token) * p.num_q_heads + head;
    if (p.out_f32) {
      float* dst = static_cast<float*>(p.out) + orow * DV + half * 4;
#pragma unroll
      for (int b = 0; b < S::kOBlocks; ++b)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *reinterpret_cast<float4*>(dst + b * 32 + g * 8) =
              make_float4(o[b][4 * g] * inv, o[b][4 * g + 1] * inv, o[b][4 * g + 2] * inv,
                          o[b][4 * g + 3] * inv);
    } else {
      uint16_t* dst = static_cast<uint16_t*>(p.out) + orow * DV + half * 4;
#pragma unroll
      for (int b = 0; b < S::kOBlocks; ++b)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *reinterpret_cast<bf16x4*>(dst + b * 32 + g * 8) =
              to_bf16x4(o[b][4 * g] * inv, o[b][4 * g + 1] * inv, o[b][4 * g + 2] * inv,
                        o[b][4 * g + 3] * inv);
    }
    if (p.lse != nullptr && half == 0)
      p.lse[orow] = l_tot > 0.f ? (m_run + fast_log2(l_tot)) * kLn2 : -INFINITY;
  }
}

bool prefill_supported(int head_dim_qk, int head_dim_v, int queries_per_kv, bool latent) {
  if (latent || queries_per_kv < 1 || queries_per_kv > 128) return false;
  return head_dim_qk == head_dim_v &&
         (head_dim_qk == 64 || head_dim_qk == 128 || head_dim_qk == 256);
}

template <int D, int DV>
static hipError_t launch_prefill_t(const AttnParams& p, hipStream_t stream) {
  using S = PrefillShape<D, DV>;
  const int block_q = S::kBlockM / p.queries_per_kv;
  const int gx = p.num_tokens / block_q + p.num_seqs;
  if (gx == 0) return hipSuccess;
  hipLaunchKernelGGL((prefill_attention_kernel<D, DV>), dim3(gx, p.num_kv_heads, p.num_splits),
                     dim3(S::kThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_attention_prefill(const AttnParams& p, hipStream_t stream) {
  switch (p.head_dim_qk) {
    case 64: return launch_prefill_t<64, 64>(p, stream);
    case 128: return launch_prefill_t<128, 128>(p, stream);
    case 256: return launch_prefill_t<256, 256>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace psw
