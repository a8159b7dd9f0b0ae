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
//     barriers are independent.  A SIMD overlaps one wave's vector ALU work
//     (softmax) with the other wave's MFMAs, while inside one wave the two
//     serialise: the kernel keeps the vector instruction count per MFMA low;
//   * KV tiles of 32 keys are gathered from the paged cache through the block
//     table with direct-to-LDS 16-byte loads (global_load_lds_dwordx4), double
//     buffered: the loads of tile t+1 are in flight while tile t is computed.
//     The block-table entries of a tile are read one tile ahead, and a load's
//     address is a scalar base (block, row group) plus a 32-bit per-lane
//     offset, so issuing a tile costs a few vector instructions.  Each load instruction writes whole rows as one block and
//     blocks are padded (K by 16 bytes, V by 64), so the K reads and the
//     transposed V reads hit distinct banks while every LDS address is a lane
//     base plus an immediate;
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16: K from LDS as the A operand, Q
//     held in registers as the B operand, so each lane holds 16 scores of ONE
//     query row (the row's other 16 keys sit in lane ^ 32) and the online
//     softmax needs a single cross-half exchange per tile;
//   * O^T += V^T P^T: P^T comes straight from the S^T accumulators (rounded to
//     bf16), V^T is read out of the row-major V tile with ds_read_b64_tr_b16, and
//     O^T keeps one query row per lane, so rescaling is per lane.  The row sum
//     is taken over the same bf16 probabilities with v_dot2 (two per
//     instruction).  LDS reads run a few ahead of their MFMAs with explicit
//     waits;
//   * the running max is only moved when a tile's max exceeds it by more than
//     2^8 (log2 units); otherwise P may reach 256, still exact in bf16/fp32, and
//     the O rescale is skipped for the whole wave;
//   * a wave skips tiles outside the union of its rows' allowed intervals, and
//     masks per element only tiles not inside every row's interval (each row's
//     allowed keys form one interval);
//   * with the cache write fused in (FUSED), every workgroup reads keys at or
//     past its request's context length from the new K and V rows rather than
//     from the cache, so no workgroup waits for another's writes, and the
//     split-0 workgroup of a query block copies its tokens' new rows of its KV
//     head into their cache slots ([SLOT] section 1) after its tile loop (the
//     copy's loads overlap the output stores; copying before the loop instead
//     measured slower: all resident workgroups then move Q and the copy at once).
#include <type_traits>
#include <utility>

#include "asm_ops.h"
#include "device_common.h"
#include "psw_internal.h"

namespace psw {

template <int D, int WAVES, int STAGES, int TILE = 32>
struct PrefillShape {
  static constexpr int kD = D;
  static constexpr int kWaves = WAVES;
  static constexpr int kStages = STAGES;  // tile buffers in the LDS ring
  static constexpr int kThreads = kWaves * kWave;
  static constexpr int kRowsPerWave = 32;
  static constexpr int kBlockM = kWaves * kRowsPerWave;
  static constexpr int kTile = TILE;       // keys per tile: 32, or 64 (two 32-key score blocks)
  static constexpr int kKeyBlocks = kTile / 32;  // S^T accumulators of 32 keys
  static constexpr int kKeyGroups = kTile / 16;  // 16-key k-steps of the output product
  // 64-key tiles gather cached keys with one 64-bit address per lane (a lane's
  // rows of a tile are consecutive keys inside one cache block) instead of the
  // base + 32-bit offset form of 32-key tiles, whose rows lie in at most two blocks
  static constexpr bool kLaneDma = kTile > 32;
  // LDS layout of a tile: one LDS-DMA instruction moves 1 KB = kRowsPerInstr
  // whole rows (rows g, g + kInstrPerTile, ...), written as one block; blocks
  // are kKBlock / kVBlock bytes apart.  The 16 extra bytes per K block put 16
  // consecutive rows read at the same column in 16 distinct bank groups; the
  // 64 extra bytes per V block do the same for the 4 rows x 4 chunks of a
  // transposed read.
  static constexpr int kRowsPerInstr = 1024 / (D * 2);
  static constexpr int kInstrPerTile = kTile / kRowsPerInstr;
  static constexpr int kInstrPerWave = kInstrPerTile / kWaves;
  static constexpr int kVmPerTile = 2 * kInstrPerWave;  // vector-memory ops per wave per tile
  static constexpr int kKBlock = 1024 + 16;
  static constexpr int kVBlock = 1024 + 64;
  static constexpr int kKBytes = kInstrPerTile * kKBlock;
  static constexpr int kVBytes = kInstrPerTile * kVBlock;
  static constexpr int kBufBytes = kKBytes + kVBytes;
  static constexpr int kLdsBytes = kStages * kBufBytes;
  static constexpr int kQFrags = D / 16;   // MFMA k-steps of the score product
  static constexpr int kOBlocks = D / 32;  // 32-column output blocks
  static constexpr int kPvSteps = kKeyGroups * kOBlocks;
  static_assert(kTile == 32 || kTile == 64, "tile of 32 or 64 keys");
  static_assert(kKeyBlocks == 1 || 32 % kInstrPerTile == 0,
                "the second score block's rows sit at a fixed offset from the first's");
  static_assert(kRowsPerInstr * D * 2 == 1024 && kInstrPerWave >= 1 &&
                    kInstrPerWave * kWaves == kInstrPerTile,
                "tile rows must split evenly into LDS-DMA instructions and waves");
  static_assert(kStages >= 2 && kStages <= 4, "LDS ring depth");
  // two waves per SIMD: one workgroup of 8 waves or two of 4 per CU (160 KB LDS)
  static_assert(kLdsBytes * (8 / kWaves) <= 160 * 1024, "LDS of the resident workgroups");
};

// Byte offset of tile row r inside a K or V tile buffer.
template <class S>
__host__ __device__ constexpr int lds_row(int r, int block_bytes) {
  return (r % S::kInstrPerTile) * block_bytes + (r / S::kInstrPerTile) * (1024 / S::kRowsPerInstr);
}

// LDS byte offset, from the lane's first K read, of the score product's c-th
// K read: k-chunk c % kQFrags (16 columns, 32 bytes) of key block c / kQFrags
// (rows 32 kb + [0, 32), a fixed distance from block 0's rows).
template <class S>
__host__ __device__ constexpr int k_read_offset(int c) {
  return (c / S::kQFrags) * (lds_row<S>(32 % S::kTile, S::kKBlock) - lds_row<S>(0, S::kKBlock)) +
         (c % S::kQFrags) * 32;
}

__device__ __forceinline__ void lds_dma16(const void* gsrc, void* lds_dst) {
  __builtin_amdgcn_global_load_lds(
      (const __attribute__((address_space(1))) void*)gsrc,
      (__attribute__((address_space(3))) void*)(lds_void*)lds_dst, 16, 0, 0);
}

__device__ __forceinline__ float dot2_bf16(bf16x2 a, bf16x2 b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(a, b, c, false);
}

template <class S, bool FUSED>
__global__ __launch_bounds__(S::kThreads) __attribute__((amdgpu_waves_per_eu(2))) void
prefill_attention_kernel(const AttnParams p) {
  constexpr int D = S::kD;
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
  const RangesWave rg{ranges, p.max_mm_ranges};  // every lane is active here
  const TileRange tr = tile_bounds_r(ctx, seq_len, query_len, q_block, S::kTile, block_q * qpk,
                                     block_q, qpk, p.geom, rg);
  int t_lo = max(tr.lo, key_begin / S::kTile);
  int t_hi = min(tr.hi, (key_end + S::kTile - 1) / S::kTile);
  if (p.key_ranges == nullptr && p.num_splits > 1) {
    // segmented split: split s takes tiles [lo + s * seg, lo + (s + 1) * seg) of
    // the block's interval, seg = ceil(tiles / splits)
    const int n = max(0, t_hi - t_lo);
    const int seg = (n + p.num_splits - 1) / p.num_splits;
    const int s_lo = min(t_lo + split * seg, t_hi);
    t_hi = min(t_hi, s_lo + seg);
    t_lo = s_lo;
  }
  PSW_DCHECK(0, t_lo >= 0 && (t_lo >= t_hi || (int64_t)(t_hi - 1) * S::kTile < seq_len));

  // ---- this lane's query row ----------------------------------------------
  const int r = wave * S::kRowsPerWave + (lane & 31);
  const int pos_in_blk = r / qpk;
  const int head = kvh * qpk + (r - pos_in_blk * qpk);
  const int qpos = q_block * block_q + pos_in_blk;
  const bool row_valid = pos_in_blk < block_q && qpos < query_len;
  const int64_t token = (int64_t)q_start + qpos;
  int row_lo = INT32_MAX, row_hi = INT32_MIN;
  {
    // computed by every lane (the wave form of the range walk needs them all)
    int64_t lo64, hi64;
    row_interval_r((int64_t)ctx + qpos, seq_len, p.geom, rg, key_begin, key_end, lo64, hi64);
    if (row_valid && lo64 <= hi64) {
      row_lo = (int)lo64;
      row_hi = (int)hi64;
    }
  }
  PSW_DCHECK(2, row_lo > row_hi || (row_lo >= 0 && row_hi < seq_len));
  PSW_DCHECK(3, row_lo > row_hi || (p.key_ranges == nullptr && p.num_splits > 1) ||
                    ((int64_t)row_lo >= (int64_t)t_lo * S::kTile &&
                     (int64_t)row_hi < (int64_t)t_hi * S::kTile));
  // The wave's common interval (tiles inside it need no per-element mask) and
  // the union of its rows' intervals (tiles outside it are skipped).
  int wave_lo = row_valid ? row_lo : INT32_MIN, wave_hi = row_valid ? row_hi : INT32_MAX;
  int any_lo = row_lo, any_hi = row_hi;
  for (int o = 32; o > 0; o >>= 1) {
    wave_lo = max(wave_lo, __shfl_xor(wave_lo, o, kWave));
    wave_hi = min(wave_hi, __shfl_xor(wave_hi, o, kWave));
    any_lo = min(any_lo, __shfl_xor(any_lo, o, kWave));
    any_hi = max(any_hi, __shfl_xor(any_hi, o, kWave));
  }
  wave_lo = __builtin_amdgcn_readfirstlane(wave_lo);
  wave_hi = __builtin_amdgcn_readfirstlane(wave_hi);
  any_lo = __builtin_amdgcn_readfirstlane(any_lo);
  any_hi = __builtin_amdgcn_readfirstlane(any_hi);

  bf16x8 qf[S::kQFrags];
  {
    const uint16_t* qrow = p.q + (token * p.num_q_heads + head) * D + half * 8;
#pragma unroll
    for (int c = 0; c < S::kQFrags; ++c) {
      if (row_valid) qf[c] = *reinterpret_cast<const bf16x8*>(qrow + c * 16);
      else qf[c] = bf16x8{};
    }
    // Q has landed before any tile load is issued: otherwise the compiler
    // guards the first use of Q inside the tile loop with a wait for every
    // outstanding load, which would drain the tile prefetch on each iteration
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  }

  f32x16 o[S::kOBlocks];
#pragma unroll
  for (int b = 0; b < S::kOBlocks; ++b) o[b] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  if (t_lo < t_hi) {
    // K and V rows have the same pitch (head_dim_qk == head_dim_v here)
    const int64_t pitch = (int64_t)p.num_kv_heads * D * 2;  // bytes per cache slot
    const char* kbase = reinterpret_cast<const char*>(p.k_cache + (int64_t)kvh * D);
    const char* vbase = reinterpret_cast<const char*>(p.v_cache + (int64_t)kvh * D);
    const int32_t* bt = p.block_table + (int64_t)seq * p.block_table_stride;
    // Fused cache write: key k >= ctx is row new_row0 + k of k_new / v_new
    // (rows have a cache slot's pitch)
    const char* knew = FUSED ? reinterpret_cast<const char*>(p.k_new + (int64_t)kvh * D) : nullptr;
    const char* vnew = FUSED ? reinterpret_cast<const char*>(p.v_new + (int64_t)kvh * D) : nullptr;
    const int64_t new_row0 = (int64_t)q_start - ctx;
    const int bs_log2 = p.block_size_log2;
    const int bs_mask = (1 << bs_log2) - 1;
    const float c2 = p.scale_log2;

    // LDS-DMA instruction g moves rows g + kInstrPerTile * q, q = lane / (D / 8),
    // 16-byte chunk lane % (D / 8) of each.  Wave w issues g = w * kInstrPerWave
    // + i.  With blocks of >= 16 keys the 32 keys of a tile lie in one or two
    // blocks: keys [first, first + 16) in block b0 and the rest in b1 (the same
    // block for larger blocks), so lane row g + rq, rq = kInstrPerTile * q,
    // sits at seg(sel) + g * pitch + lane_off, with sel = (rq >= 16) when blocks
    // hold 16 keys and lane_off = (rq within its segment) * pitch + chunk * 16.
    const int dma_q = lane / (D / 8), dma_ch = lane % (D / 8);
    const int rq = S::kInstrPerTile * dma_q;
    const bool fast_blocks = bs_log2 >= 4;
    const bool two_segs = bs_log2 == 4;
    const bool lane_second = two_segs && rq >= 16;
    const uint32_t lane_off = (uint32_t)(((two_segs ? (rq & 15) : rq) * pitch) + dma_ch * 16);
    const uint32_t new_off = (uint32_t)(rq * pitch + dma_ch * 16);  // one run of rows

    // Block-table entries of the workgroup's tiles live in two registers:
    // lane l of ent0 / ent1 holds the entry of block blk0 + l / blk0 + 64 + l
    // (clamped to the request's last block), read before the tile loop, so the
    // loop issues no table loads of its own.  A tile whose blocks fall outside
    // the 128 held entries reloads the window (its use waits for every
    // outstanding load; only tile ranges longer than 128 blocks get there).
    const int last_blk = (seq_len - 1) >> bs_log2;
    int blk0 = 0, ent0 = 0, ent1 = 0;
    // The two loads and their wait are one assembly block: the compiler does
    // not track them, so it adds no wait of its own where the entries are
    // read (which would also wait for the tile loads in flight).
    auto load_window = [&](int b) __attribute__((always_inline)) {
      blk0 = b;
      const int32_t* a0 = bt + min(b + lane, last_blk);
      const int32_t* a1 = bt + min(b + 64 + lane, last_blk);
      asm volatile(
          "global_load_dword %0, %2, off\n\t"
          "global_load_dword %1, %3, off\n\t"
          "s_waitcnt vmcnt(0)"
          : "=&v"(ent0), "=&v"(ent1)
          : "v"(a0), "v"(a1)
          : "memory");
    };
    auto entry = [&](int rel) __attribute__((always_inline)) -> int {
      return rel < 64 ? __builtin_amdgcn_readlane(ent0, rel)
                      : __builtin_amdgcn_readlane(ent1, rel - 64);
    };
    // Fast path of a tile's DMA: every instruction is a scalar base (lo) plus
    // one 32-bit offset per lane (voff).
    struct DmaPlan {
      int64_t lo;
      uint32_t voff;
      bool fast;
      const char* kb;  // uniform K and V bases of this wave's first instruction
      const char* vb;
      const char* ka;  // 64-key tiles: this lane's K and V addresses for that instruction
      const char* va;
    };
    const int64_t wave_row = (int64_t)wave * S::kInstrPerWave * pitch;
    auto plan_tile = [&](int tile) __attribute__((always_inline)) {
      DmaPlan d;
      d.fast = false;
      const int first = tile * S::kTile;
      if constexpr (FUSED) {
        if (first >= ctx) {
          // every key of the tile is new: consecutive rows of k_new / v_new
          d.lo = (new_row0 + first) * pitch;
          d.voff = new_off;
          d.fast = first + S::kTile <= seq_len &&
                   (int64_t)(S::kTile + S::kInstrPerTile) * pitch + 1024 < ((int64_t)1 << 31);
          d.kb = knew + (d.lo + wave_row);
          d.vb = vnew + (d.lo + wave_row);
          if constexpr (S::kLaneDma) {
            d.ka = d.kb + d.voff;
            d.va = d.vb + d.voff;
          }
          return d;
        }
        if (first + S::kTile > ctx) return d;  // old and new keys: per-lane path
      }
      if (!fast_blocks) return d;
      if constexpr (S::kLaneDma) {
        // A lane's rows of the tile are keys first + rq + g, g < kInstrPerTile:
        // consecutive keys that sit in one block when blocks hold at least
        // kInstrPerTile keys (tiles start on multiples of 64).  The lane's
        // address is its block's entry (one of the tile's kRowsPerInstr row
        // groups, picked from uniform table reads) plus its row and chunk.
        if ((1 << bs_log2) < S::kInstrPerTile) return d;
        const int bf = first >> bs_log2, bl = (first + S::kTile - 1) >> bs_log2;
        if (bf < blk0 || bl - blk0 >= 128) load_window(bf);
        int e = 0;
        static_for<S::kRowsPerInstr>([&](auto qq) {
          constexpr int q = decltype(qq)::value;
          const int eq = entry(((first + q * S::kInstrPerTile) >> bs_log2) - blk0);
          e = dma_q == q ? eq : e;
        });
        PSW_DCHECK(1, first + S::kTile > seq_len || e >= 0);
        d.fast = first + S::kTile <= seq_len;
        const int64_t row =
            ((int64_t)e << bs_log2) + ((first + rq) & bs_mask) + wave * S::kInstrPerWave;
        d.ka = kbase + (row * pitch + dma_ch * 16);
        d.va = vbase + (row * pitch + dma_ch * 16);
        return d;
      }
      // with 16-key blocks keys [first, first + 16) sit in block b and the
      // rest in b + 1; larger blocks hold the whole tile
      const int b = first >> bs_log2;
      if (b < blk0 || b + 1 - blk0 >= 128) load_window(b);
      const int b0 = entry(b - blk0);
      const int b1 = two_segs ? entry(b + 1 - blk0) : b0;
      // byte offsets of the two segments in the cache (first row of each)
      const int64_t seg0 = (((int64_t)b0 << bs_log2) + (first & bs_mask)) * pitch;
      const int64_t seg1 = ((int64_t)b1 << bs_log2) * pitch;
      d.lo = two_segs ? min(seg0, seg1) : seg0;
      const int64_t delta = two_segs ? max(seg0, seg1) - d.lo : 0;
      // every lane offset (segment distance + row within the tile + chunk +
      // instruction row) must fit in 32 bits
      d.fast = first + S::kTile <= seq_len &&
               delta + (int64_t)(S::kTile + S::kInstrPerTile) * pitch + 1024 < ((int64_t)1 << 31);
      PSW_DCHECK(1, !d.fast || (b0 >= 0 && b1 >= 0));
      const bool lane_far = lane_second ? seg1 > seg0 : seg0 > seg1;
      d.voff = lane_off + (lane_far ? (uint32_t)delta : 0u);
      d.kb = kbase + (d.lo + wave_row);
      d.vb = vbase + (d.lo + wave_row);
      return d;
    };
    // instruction i of this wave (K, then V), fast path
    // instruction i: uniform base + one 32-bit lane offset (the segment
    // distance and i rows of the cache fit in 32 bits on the fast path)
    const uint32_t pitch32 = (uint32_t)pitch;
    auto dma_k = [&](const DmaPlan& d, int buf, int i) __attribute__((always_inline)) {
      const int g = wave * S::kInstrPerWave + i;
      char* dst = smem + buf * S::kBufBytes + g * S::kKBlock;
      if constexpr (S::kLaneDma) lds_dma16(d.ka + (int64_t)i * pitch, dst);
      else lds_dma16(d.kb + (uint32_t)(d.voff + (uint32_t)i * pitch32), dst);
    };
    auto dma_v = [&](const DmaPlan& d, int buf, int i) __attribute__((always_inline)) {
      const int g = wave * S::kInstrPerWave + i;
      char* dst = smem + buf * S::kBufBytes + S::kKBytes + g * S::kVBlock;
      if constexpr (S::kLaneDma) lds_dma16(d.va + (int64_t)i * pitch, dst);
      else lds_dma16(d.vb + (uint32_t)(d.voff + (uint32_t)i * pitch32), dst);
    };
    auto issue_tile = [&](int tile, int buf, const DmaPlan& d) __attribute__((always_inline)) {
      char* kt = smem + buf * S::kBufBytes;
      char* vt = kt + S::kKBytes;
      const int first = tile * S::kTile;
      if (d.fast) {
#pragma unroll
        for (int i = 0; i < S::kInstrPerWave; ++i) {
          dma_k(d, buf, i);
          dma_v(d, buf, i);
        }
      } else {
        // last tile (rows past the end repeat the last key: finite data,
        // masked out), blocks below 16 keys, or segments far apart: per-lane
        // 64-bit addresses and table reads
#pragma unroll
        for (int i = 0; i < S::kInstrPerWave; ++i) {
          const int g = wave * S::kInstrPerWave + i;
          const int key = min(first + g + rq, seq_len - 1);
          if (FUSED && key >= ctx) {
            const int64_t row = (new_row0 + key) * pitch + dma_ch * 16;
            lds_dma16(knew + row, kt + g * S::kKBlock);
            lds_dma16(vnew + row, vt + g * S::kVBlock);
            continue;
          }
          const int32_t blk = bt[key >> bs_log2];
          PSW_DCHECK(1, blk >= 0);
          const int64_t row = (((int64_t)blk << bs_log2) + (key & bs_mask)) * pitch + dma_ch * 16;
          lds_dma16(kbase + row, kt + g * S::kKBlock);
          lds_dma16(vbase + row, vt + g * S::kVBlock);
        }
      }
    };

    const int tr_row = half * 4 + ((lane & 15) >> 2);
    const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);  // bf16 column in a 32-block
    const uint32_t k_lane = (uint32_t)(lds_row<S>(lane & 31, S::kKBlock) + half * 16);
    const uint32_t v_lane = (uint32_t)(S::kKBytes + tr_col * 2);
    uint32_t v_rows[S::kKeyGroups][2];
#pragma unroll
    for (int j = 0; j < S::kKeyGroups; ++j) {
      v_rows[j][0] = v_lane + (uint32_t)lds_row<S>(16 * j + tr_row, S::kVBlock);
      v_rows[j][1] = v_lane + (uint32_t)lds_row<S>(16 * j + tr_row + 8, S::kVBlock);
    }
    const uint32_t smem0 = lds_addr(smem);
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

    // Pipeline over a ring of NS tile buffers: the DMA plan of tile u is made
    // in iteration u - NS (after its output MFMAs are issued) and its DMA is
    // issued in iteration u - NS + 1, spread over the score MFMAs, so up to
    // NS - 1 tiles are in flight while one is computed.
    constexpr int NS = S::kStages;
    if (fast_blocks) load_window((t_lo * S::kTile) >> bs_log2);
#pragma unroll
    for (int j = 0; j < NS - 1; ++j)
      if (t_lo + j < t_hi) issue_tile(t_lo + j, j, plan_tile(t_lo + j));
    DmaPlan nd;  // plan of tile t + NS - 1
    nd.fast = false;
    if (t_lo + NS - 1 < t_hi) nd = plan_tile(t_lo + NS - 1);

    int buf = 0;  // (t - t_lo) % NS
    for (int t = t_lo; t < t_hi; ++t, buf = buf + 1 == NS ? 0 : buf + 1) {
      // this wave's LDS-DMA loads of tile t have landed once at most the loads
      // of the tiles issued after it (up to NS - 2, kVmPerTile each, more on
      // the per-lane path) are outstanding; the barrier extends that to every
      // wave and fences the reads of tile t - 1's buffer before it is refilled
      const int later = min(NS - 2, t_hi - 1 - t);
      if (NS >= 4 && later >= 2) __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * S::kVmPerTile));
      else if (NS >= 3 && later >= 1) __builtin_amdgcn_s_waitcnt(waitcnt_vm(S::kVmPerTile));
      else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
      lds_barrier();
      const int base = t * S::kTile;
      const bool skip = base > any_hi || base + S::kTile - 1 < any_lo;  // no row of the wave sees it
      // Tile tn goes to the buffer tile t - 1 used.  The fast-path DMA is
      // spread over the score MFMAs below (all waves issuing right after the
      // barrier stall on the shared address unit); the other cases issue it
      // here.
      const int tn = t + NS - 1;
      const int bn = buf == 0 ? NS - 1 : buf - 1;
      if (tn < t_hi && (!nd.fast || skip)) issue_tile(tn, bn, nd);
      const bool inter = tn < t_hi && nd.fast;
      if (skip) {
        if (tn + 1 < t_hi) nd = plan_tile(tn + 1);
        continue;
      }
      const uint32_t kt = smem0 + (uint32_t)(buf * S::kBufBytes);

      // S^T[key][row] for each 32-key block of the tile (its own accumulator);
      // MFMA c reads k-chunk c % kQFrags of key block c / kQFrags, K reads
      // KA ahead.  Two copies of the sequence, with and without the DMA of
      // tile tn, so that no branch sits between the MFMAs.
      f32x16 s[S::kKeyBlocks];
      auto score = [&](auto with_dma) __attribute__((always_inline)) {
        constexpr bool DMA = decltype(with_dma)::value;
        constexpr int NQ = S::kQFrags, N = NQ * S::kKeyBlocks, KA = 3;
        const uint32_t ka = kt + k_lane;
        bf16x8 kf[KA + 1];
        static_for<KA>([&](auto cc) {
          constexpr int c = decltype(cc)::value;
          kf[c] = lds_read_b128_at<k_read_offset<S>(c)>(ka);
        });
#pragma unroll
        for (int kb = 0; kb < S::kKeyBlocks; ++kb) s[kb] = f32x16{};
        static_for<N>([&](auto cc) {
          constexpr int c = decltype(cc)::value;
          constexpr int issued = c + KA < N ? c + KA : N;
          lds_wait<issued - 1 - c>(kf[c % (KA + 1)]);
          s[c / NQ] = mfma32(kf[c % (KA + 1)], qf[c % NQ], s[c / NQ]);
          if constexpr (c + KA < N)
            kf[(c + KA) % (KA + 1)] = lds_read_b128_at<k_read_offset<S>(c + KA)>(ka);
          constexpr int step = N / S::kInstrPerWave;
          if constexpr (DMA && c % step == 0) dma_k(nd, bn, c / step);
          if constexpr (DMA && c % step == step / 2) dma_v(nd, bn, c / step);
        });
      };
      if (inter) score(std::true_type{});
      else score(std::false_type{});
      if (!(base >= wave_lo && base + S::kTile - 1 <= wave_hi)) {
#pragma unroll
        for (int kb = 0; kb < S::kKeyBlocks; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int k = base + 32 * kb + (i / 4) * 8 + half * 4 + (i % 4);
            s[kb][i] = (k >= row_lo && k <= row_hi) ? s[kb][i] : -INFINITY;
          }
      }
      float mx = s[0][0];
#pragma unroll
      for (int kb = 0; kb < S::kKeyBlocks; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (kb > 0 || i > 0) mx = fmaxf(mx, s[kb][i]);
      mx = pair_max(mx) * c2;
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
      // P^T in bf16, one B operand per 16-key group: keys 16 j + [0, 16) are
      // elements 8 (j % 2) .. + 8 of key block j / 2's accumulator
      bf16x8 pf[S::kKeyGroups];
#pragma unroll
      for (int kb = 0; kb < S::kKeyBlocks; ++kb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) s[kb][i] = fast_exp2(fmaf(s[kb][i], c2, -m_sub));
        pf[2 * kb] = to_bf16x8(s[kb][0], s[kb][1], s[kb][2], s[kb][3], s[kb][4], s[kb][5],
                               s[kb][6], s[kb][7]);
        pf[2 * kb + 1] = to_bf16x8(s[kb][8], s[kb][9], s[kb][10], s[kb][11], s[kb][12],
                                   s[kb][13], s[kb][14], s[kb][15]);
      }
      // row sum over the bf16 probabilities the output product uses
      static_for<4>([&](auto ii) {
        constexpr int i = decltype(ii)::value;
#pragma unroll
        for (int j = 0; j < S::kKeyGroups; ++j)
          l_run = dot2_bf16(__builtin_shufflevector(pf[j], pf[j], 2 * i, 2 * i + 1), ones, l_run);
      });

      // O^T += V^T P^T: step st covers output columns b*32 + [0, 32) and keys
      // 16 j + [0, 16), j = st / kOBlocks, b = st % kOBlocks; the transposed
      // reads run VA steps ahead
      {
        constexpr int N = S::kPvSteps, VA = 2;
        bf16x4 vr[VA + 1][2];
        auto read_v = [&](auto ss) __attribute__((always_inline)) {
          constexpr int st = decltype(ss)::value;
          constexpr int j = st / S::kOBlocks, bo = (st % S::kOBlocks) * 64;
          vr[st % (VA + 1)][0] = lds_read_tr4_at<bo>(kt + v_rows[j][0]);
          vr[st % (VA + 1)][1] = lds_read_tr4_at<bo>(kt + v_rows[j][1]);
        };
        static_for<VA>(read_v);
        static_for<N>([&](auto ss) {
          constexpr int st = decltype(ss)::value;
          constexpr int issued = st + VA < N ? st + VA : N;
          lds_wait<2 * (issued - 1 - st)>(vr[st % (VA + 1)][0], vr[st % (VA + 1)][1]);
          o[st % S::kOBlocks] = mfma32(cat8(vr[st % (VA + 1)][0], vr[st % (VA + 1)][1]),
                                       pf[st / S::kOBlocks], o[st % S::kOBlocks]);
          if constexpr (st + VA < N) read_v(std::integral_constant<int, st + VA>{});
        });
      }
      if (tn + 1 < t_hi) nd = plan_tile(tn + 1);  // in the shadow of the last MFMAs
    }
  }

  // ---- epilogue ------------------------------------------------------------
  const float l_tot = pair_sum(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  // Fused cache write: 16-byte chunk c of this workgroup's copy is chunk
  // c % (D / 8) of the K (then V) row of token c / (D / 4), KV head kvh.  A
  // pass moves up to kCopyPass chunks per thread, loaded together; the first
  // pass's loads are issued before the output stores.
  constexpr int kCh = D / 8, kCopyPass = D == 256 ? 16 : 8;
  const int copy_tokens =
      FUSED && split == 0 ? min(block_q, query_len - q_block * block_q) : 0;
  const int copy_total = copy_tokens * 2 * kCh;
  const int64_t copy_tok0 = (int64_t)q_start + q_block * block_q;
  using CopyBuf = bf16x8[FUSED ? kCopyPass : 1];
  using CopySlots = int32_t[FUSED ? kCopyPass : 1];
  auto copy_load = [&](int c0, CopyBuf& cbuf, CopySlots& cslot) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kCopyPass; ++i) {
      const int c = c0 + i * S::kThreads + tid;
      if (c < copy_total) {
        const int tok = c / (2 * kCh), rem = c - tok * 2 * kCh;
        const int64_t elem = ((copy_tok0 + tok) * p.num_kv_heads + kvh) * D + (rem % kCh) * 8;
        cbuf[i] = *reinterpret_cast<const bf16x8*>((rem < kCh ? p.k_new : p.v_new) + elem);
        cslot[i] = p.slot_mapping[copy_tok0 + tok];
      }
    }
  };
  auto copy_store = [&](int c0, const CopyBuf& cbuf, const CopySlots& cslot)
                        __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kCopyPass; ++i) {
      const int c = c0 + i * S::kThreads + tid;
      if (c < copy_total) {
        const int rem = c % (2 * kCh);
        const int32_t sl = cslot[i];
        PSW_DCHECK(4, sl == -1 || (sl >= 0 && sl < p.num_slots));
        if (sl >= 0 && sl < p.num_slots) {
          const int64_t elem = ((int64_t)sl * p.num_kv_heads + kvh) * D + (rem % kCh) * 8;
          *reinterpret_cast<bf16x8*>((rem < kCh ? p.k_cache_w : p.v_cache_w) + elem) = cbuf[i];
        }
      }
    }
  };
  auto copy_rest = [&](int c0) __attribute__((always_inline)) {
    for (; c0 < copy_total; c0 += kCopyPass * S::kThreads) {
      CopyBuf cb;
      CopySlots cs;
      copy_load(c0, cb, cs);
      copy_store(c0, cb, cs);
    }
  };
  CopyBuf cb;
  CopySlots cs;
  if constexpr (FUSED) copy_load(0, cb, cs);

  if (row_valid) {
    const int64_t orow = ((int64_t)split * p.num_tokens + token) * p.num_q_heads + head;
    const int64_t e0 = orow * D + half * 4;
#pragma unroll
    for (int b = 0; b < S::kOBlocks; ++b)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        store_out4(p.out, e0 + b * 32 + g * 8, p.out_dtype, o[b][4 * g] * inv,
                   o[b][4 * g + 1] * inv, o[b][4 * g + 2] * inv, o[b][4 * g + 3] * inv);
    if (p.lse != nullptr && half == 0)
      p.lse[orow] = l_tot > 0.f ? (m_run + fast_log2(l_tot)) * kLn2 : -INFINITY;
  }
  if constexpr (FUSED) {
    copy_store(0, cb, cs);
    // more passes only with one or two query heads per KV head (64-128 tokens)
    copy_rest(kCopyPass * S::kThreads);
  }
}

bool prefill_supported(int head_dim_qk, int head_dim_v, int queries_per_kv, bool latent) {
  if (latent || queries_per_kv < 1 || queries_per_kv > 128) return false;
  return head_dim_qk == head_dim_v &&
         (head_dim_qk == 64 || head_dim_qk == 128 || head_dim_qk == 256);
}

// Launch shapes: two 4-wave workgroups per CU, two tile buffers each.  One
// 8-wave workgroup per CU with a four-deep ring (prefetch distance three
// tiles) measured no faster on the 16,550-token workload: the tile loads are
// not what the loop waits for.
template <class S, bool FUSED>
static hipError_t launch_prefill_t(const AttnParams& p, hipStream_t stream) {
  const int block_q = S::kBlockM / p.queries_per_kv;
  const int gx = p.num_tokens / block_q + p.num_seqs;
  if (gx == 0) return hipSuccess;
  const size_t lds = S::kLdsBytes;
  auto kern = prefill_attention_kernel<S, FUSED>;
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(kern, dim3(gx, p.num_kv_heads, p.num_splits), dim3(S::kThreads), lds,
                     stream, p);
  return hipGetLastError();
}

// Head dim 128 takes 64-key tiles when a query row spans more than 1,536 keys
// (no window, or a non-causal window of 769 or more): a tile's fixed work (its
// barrier, DMA plan, row-max exchange and rescale test) is then spread over
// twice the MFMAs (the 2 x 4096-token non-causal workload with W 1024: 0.079
// against 0.091 ms).  Shorter rows keep 32-key tiles: a 64-key tile wastes
// more keys at the window's edges, and its registers allow two resident
// workgroups per CU instead of three (the chunked W 512 workload: 0.056
// against 0.052 ms; a causal W 1024 one: equal).  The choice depends only on
// the call's mask geometry, so a call and its fused-write twin tile alike.
bool prefill_long_tiles(int head_dim, int window, int causal) {
  if (head_dim != 128) return false;
  if (window <= 0) return true;
  const int64_t span = causal ? (int64_t)window : 2 * (int64_t)window - 1;
  return span > 1536;
}

template <bool FUSED>
static hipError_t launch_prefill_d(const AttnParams& p, hipStream_t stream) {
  switch (p.head_dim_qk) {
    case 64: return launch_prefill_t<PrefillShape<64, 4, 2>, FUSED>(p, stream);
    case 128:
      if (prefill_long_tiles(128, p.geom.window, p.geom.causal))
        return launch_prefill_t<PrefillShape<128, 4, 2, 64>, FUSED>(p, stream);
      return launch_prefill_t<PrefillShape<128, 4, 2>, FUSED>(p, stream);
    case 256: return launch_prefill_t<PrefillShape<256, 4, 2>, FUSED>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_attention_prefill(const AttnParams& p, hipStream_t stream) {
  return p.k_new != nullptr ? launch_prefill_d<true>(p, stream)
                            : launch_prefill_d<false>(p, stream);
}

PSW_DEBUG_TAKE(debug_take_prefill)

}  // namespace psw
