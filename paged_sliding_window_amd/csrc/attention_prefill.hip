// Paged prefill attention under the sliding window OR-ed with window-clamped
// image ranges, visiting only the KV tiles of each query block's union interval
// (vLLM PR #53147 summary, "Implementation breakdown" and "Key source snippet").
//
// Work decomposition (gfx950, wave64):
//   * one workgroup = one query block x one KV head x one key split; 4 waves of
//     32 rows each.  Rows are (position, query head of this KV head) in
//     position-major order, so one K/V tile in LDS serves every query head that
//     shares it (GQA).  Workgroups are ordered so each XCD walks consecutive
//     query blocks of one KV head (their K/V windows overlap);
//   * two workgroups share a CU, so each SIMD runs two waves whose tile
//     barriers are independent: one wave's softmax overlaps the other's MFMAs
//     (a single 8-wave workgroup keeps both waves of a SIMD in the same phase);
//   * KV tiles of 32 keys are gathered from the paged cache through the block
//     table with direct-to-LDS 16-byte loads (global_load_lds_dwordx4), double
//     buffered (68 KB per workgroup at head dim 256): the loads of tile t+1 and
//     the block-table reads of tile t+2 are in flight while tile t is computed.  Each load instruction writes whole
//     rows as one block and blocks are padded (K by 16 bytes, V by 64), so the
//     K reads below and the transposed V reads hit distinct banks while every
//     LDS address stays a lane base plus an immediate;
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16: K from LDS as the A operand, Q
//     held in registers as the B operand, so each lane ends up holding 32 scores
//     of ONE query row (the row's other 32 keys sit in lane ^ 32) and the online
//     softmax needs a single cross-half exchange per tile;
//   * O^T += V^T P^T: P^T comes straight from the S^T accumulators (rounded to
//     bf16), V^T is read out of the row-major V tile with ds_read_b64_tr_b16, and
//     O^T keeps one query row per lane, so rescaling is per lane;
//   * the running max is only moved when a tile's max exceeds it by more than
//     2^8 (log2 units); otherwise P may reach 256, still exact in bf16/fp32, and
//     the O rescale is skipped for the whole wave;
//   * per-element masking only on tiles not entirely inside every row's allowed
//     interval (each row's allowed keys form one interval).
#include "device_common.h"
#include "psw_internal.h"

namespace psw {

template <int D, int DV>
struct PrefillShape {
  static constexpr int kWaves = 4;
  static constexpr int kThreads = kWaves * kWave;
  static constexpr int kRowsPerWave = 32;
  static constexpr int kBlockM = kWaves * kRowsPerWave;
  static constexpr int kTile = 32;
  static constexpr int kKChunks = D / 8;   // 16-byte chunks per K row
  static constexpr int kVChunks = DV / 8;
  // LDS layout of a tile: one LDS-DMA instruction moves 1 KB = kRowsPerInstr
  // whole rows (rows g, g + kInstrPerTile, ...), written as one block; blocks
  // are kKBlock / kVBlock bytes apart.  The 16 extra bytes per K block put 16
  // consecutive rows read at the same column in 16 distinct bank groups; the
  // 64 extra bytes per V block do the same for the 4 rows x 4 chunks of a
  // transposed read.  Every LDS address is a per-lane base plus immediates.
  static constexpr int kRowsPerInstr = 1024 / (D * 2);
  static constexpr int kInstrPerTile = kTile / kRowsPerInstr;
  static constexpr int kInstrPerWave = kInstrPerTile / kWaves;
  static constexpr int kKBlock = 1024 + 16;
  static constexpr int kVBlock = 1024 + 64;
  static constexpr int kQFrags = D / 16;
  static constexpr int kOBlocks = DV / 32;
  static constexpr int kKBytes = kInstrPerTile * kKBlock;
  static constexpr int kVBytes = kInstrPerTile * kVBlock;
  static_assert(D == DV, "K and V tiles share the row-to-instruction mapping");
  static_assert(kRowsPerInstr * D * 2 == 1024 && kInstrPerWave * kWaves == kInstrPerTile,
                "tile rows must split evenly into LDS-DMA instructions and waves");
  static_assert(2 * (kKBytes + kVBytes) <= 160 * 1024, "double buffer exceeds LDS");
};

// Byte offset of tile row r inside a K or V tile buffer.
template <class S>
__device__ __forceinline__ int lds_row(int r, int block_bytes) {
  return (r % S::kInstrPerTile) * block_bytes + (r / S::kInstrPerTile) * (1024 / S::kRowsPerInstr);
}

__device__ __forceinline__ void lds_dma16(const void* gsrc, void* lds_dst) {
  __builtin_amdgcn_global_load_lds(
      (const __attribute__((address_space(1))) void*)gsrc,
      (__attribute__((address_space(3))) void*)(lds_void*)lds_dst, 16, 0, 0);
}

template <int D, int DV>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void
prefill_attention_kernel(const AttnParams p) {
  using S = PrefillShape<D, DV>;
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);  // uniform: keep it scalar
  const int half = lane >> 5;
  const int qpk = p.queries_per_kv;
  const int block_q = S::kBlockM / qpk;

  // ---- request and query block of this workgroup --------------------------
  // Logical work item (x fastest, then KV head, then split), spread so that
  // each XCD walks consecutive query blocks of one KV head.
  const int nx = gridDim.x, ny = gridDim.y;
  const int logical = xcd_logical_id(blockIdx.x + nx * (blockIdx.y + ny * blockIdx.z),
                                     nx * ny * gridDim.z);
  const int x = logical % nx;
  const int kvh = (logical / nx) % ny, split = logical / (nx * ny);
  // Query blocks of request s occupy slots [qsl[s] / block_q + s, ...) of x.
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
  // the wave's common interval: 32-key halves inside it need no per-element mask
  int wave_lo = row_valid ? row_lo : INT32_MIN, wave_hi = row_valid ? row_hi : INT32_MAX;
  for (int o = 32; o > 0; o >>= 1) {
    wave_lo = max(wave_lo, __shfl_xor(wave_lo, o, kWave));
    wave_hi = min(wave_hi, __shfl_xor(wave_hi, o, kWave));
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

  if (t_lo < t_hi) {
    const bool latent = p.v_cache == p.k_cache;
    const int64_t k_slot_pitch = (int64_t)p.num_kv_heads * D;
    const int64_t v_slot_pitch = latent ? k_slot_pitch : (int64_t)p.num_kv_heads * DV;
    const uint16_t* kbase = p.k_cache + (int64_t)kvh * D;
    const uint16_t* vbase = p.v_cache + (int64_t)kvh * (latent ? D : DV);
    const int32_t* bt = p.block_table + (int64_t)seq * p.block_table_stride;
    const int bs_log2 = p.block_size_log2;
    const int bs_mask = (1 << bs_log2) - 1;
    const float c2 = p.scale_log2;

    // LDS-DMA instruction g moves rows g + kInstrPerTile * q, q = lane / (D / 8),
    // 16-byte chunk lane % (D / 8) of each, into the block at g * k/vBlock.  A
    // wave issues instructions g = wave * kInstrPerWave + i, so a lane's rows in
    // a tile are the consecutive keys r0 + i: when blocks hold at least
    // kInstrPerWave keys they share one block, whose table entry the lane
    // prefetches (fetch_block) and whose addresses differ by one slot pitch.
    const int dma_q = lane / (D / 8), dma_ch = lane % (D / 8);
    const int r0 = wave * S::kInstrPerWave + S::kInstrPerTile * dma_q;
    const bool group_in_block = (1 << bs_log2) >= S::kInstrPerWave;
    // block of this lane's first row in the tile (clamped to the last key)
    auto fetch_block = [&](int tile) -> int {
      const int key = min(tile * S::kTile + r0, seq_len - 1);
      return bt[key >> bs_log2];
    };
    auto issue_tile = [&](int tile, int buf, int blk_of_lane) {
      char* kt = smem + buf * (S::kKBytes + S::kVBytes);
      char* vt = kt + S::kKBytes;
      const int first = tile * S::kTile;
      if (group_in_block && first + S::kTile <= seq_len) {
        const int64_t cache_row = ((int64_t)blk_of_lane << bs_log2) + ((first + r0) & bs_mask);
        const uint16_t* ks = kbase + cache_row * k_slot_pitch + dma_ch * 8;
        const uint16_t* vs = vbase + cache_row * v_slot_pitch + dma_ch * 8;
#pragma unroll
        for (int i = 0; i < S::kInstrPerWave; ++i) {
          const int g = wave * S::kInstrPerWave + i;
          lds_dma16(ks + i * k_slot_pitch, kt + g * S::kKBlock);
          lds_dma16(vs + i * v_slot_pitch, vt + g * S::kVBlock);
        }
      } else {
        // last tile (rows past the end repeat the last key: finite data, masked
        // out) or blocks smaller than a lane's row group: one lookup per row
#pragma unroll
        for (int i = 0; i < S::kInstrPerWave; ++i) {
          const int g = wave * S::kInstrPerWave + i;
          const int key = min(first + r0 + i, seq_len - 1);
          const int64_t cache_row = ((int64_t)bt[key >> bs_log2] << bs_log2) + (key & bs_mask);
          lds_dma16(kbase + cache_row * k_slot_pitch + dma_ch * 8, kt + g * S::kKBlock);
          lds_dma16(vbase + cache_row * v_slot_pitch + dma_ch * 8, vt + g * S::kVBlock);
        }
      }
    };

    int blk_next = fetch_block(t_lo);
    issue_tile(t_lo, 0, blk_next);
    if (t_lo + 1 < t_hi) blk_next = fetch_block(t_lo + 1);

    const int tr_row = half * 4 + ((lane & 15) >> 2);
    const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);  // bf16 column in a 32-block

    for (int t = t_lo; t < t_hi; ++t) {
      const int buf = (t - t_lo) & 1;
      // this wave's LDS-DMA loads of tile t and its block-table read have
      // landed; the barrier extends that to every wave and fences the reads of
      // the other buffer (tile t-1) before it is refilled
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (t + 1 < t_hi) {
        issue_tile(t + 1, buf ^ 1, blk_next);
        if (t + 2 < t_hi) blk_next = fetch_block(t + 2);
      }
      const char* kt = smem + buf * (S::kKBytes + S::kVBytes);
      const char* vt = kt + S::kKBytes;

#pragma unroll
      for (int kb = 0; kb < S::kTile / 32; ++kb) {
        const int base = t * S::kTile + kb * 32;
        // S^T[key][row] for 32 keys
        f32x16 s = f32x16{};
        const int kr = kb * 32 + (lane & 31);
#pragma unroll
        for (int c = 0; c < S::kQFrags; ++c) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(
              kt + lds_row<S>(kr, S::kKBlock) + (2 * c + half) * 16);
          s = mfma32(a, qf[c], s);
        }
        if (!(base >= wave_lo && base + 31 <= wave_hi)) {
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
        // move the running max only when it grows by more than 2^8
        if (__ballot(mx > m_run + 8.f) != 0) {
          const float m_new = fmaxf(m_run, mx);
          // 0 when only m_run is -inf; 1 for a row that is still fully masked
          const float alpha = m_new == -INFINITY ? 1.f : fast_exp2(m_run - m_new);
          l_run *= alpha;
#pragma unroll
          for (int b = 0; b < S::kOBlocks; ++b) o[b] *= alpha;
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
        // O^T += V^T P^T, output columns b*32 + [0, 32), keys kb*32 + 16 j + [0, 16)
        // in step st = 2b + j.  The transposed reads of step st + 1 are issued
        // before the MFMA of step st (and, unlike the builtin, do not make the
        // compiler wait for the prefetch of tile t + 1 still in flight).
        {
          const uint32_t vcol = lds_addr(vt + tr_col * 2);
          uint32_t va[2][2];
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const int ra = kb * 32 + 16 * j + tr_row;
            va[j][0] = vcol + lds_row<S>(ra, S::kVBlock);
            va[j][1] = vcol + lds_row<S>(ra + 8, S::kVBlock);
          }
          constexpr int kSteps = 2 * S::kOBlocks;
          bf16x4 vr[2][2];
          vr[0][0] = lds_read_tr4_async(va[0][0]);
          vr[0][1] = lds_read_tr4_async(va[0][1]);
#pragma unroll
          for (int st = 0; st < kSteps; ++st) {
            const int b = st >> 1, j = st & 1, cur = st & 1;
            if (st + 1 < kSteps) {
              const int bn = (st + 1) >> 1, jn = (st + 1) & 1;
              vr[cur ^ 1][0] = lds_read_tr4_async(va[jn][0] + bn * 64);
              vr[cur ^ 1][1] = lds_read_tr4_async(va[jn][1] + bn * 64);
              lds_wait_tr<2>(vr[cur][0], vr[cur][1]);
            } else {
              lds_wait_tr<0>(vr[cur][0], vr[cur][1]);
            }
            o[b] = mfma32(cat8(vr[cur][0], vr[cur][1]), j == 0 ? pf0 : pf1, o[b]);
          }
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
  const size_t lds = 2 * (S::kKBytes + S::kVBytes);
  auto kern = prefill_attention_kernel<D, DV>;
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(kern, dim3(gx, p.num_kv_heads, p.num_splits), dim3(S::kThreads), lds,
                     stream, p);
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
