// Slot mapping: vllm-ascend Triton operator deep dive, _compute_slot_mapping_kernel,
// sections 1, 2 and 4.3.  The page's design runs one program per request plus a
// dedicated padding program, and loads a bounded window of the block table per
// 1024-token tile.  Here the grid is flat over the padded token axis instead:
// each wave owns 64 x kSlotTokensPerThread consecutive tokens, finds the
// request of its first token with a 64-way search over query_start_loc (each
// round one load per lane and a ballot, two rounds for 4096 requests); each
// lane then finds its own first token's request among the 64 boundaries that
// follow, loaded one per lane and searched across the lanes (many short
// requests per wave, as in decode batches of one token per request), or
// beyond them by a galloping search, and crosses the boundaries inside its own
// tokens with the next few boundaries read ahead.  With at most 64 requests
// one load of query_start_loc (one start per lane) serves the search, the
// window and the read-ahead through lane shuffles.  A lane's block-table
// entries are loaded as one round after all its tokens' requests are known.
// Positions are read with 16-byte loads and slots (or -1) written with
// 16-byte stores, so every wave streams contiguous positions and slots.
// Block-table entries are read per token; consecutive tokens of a request hit
// the same cache line, which plays the role of the page's bounded window.
#include <type_traits>

#include "psw_internal.h"

namespace psw {

constexpr int kSlotThreads = 256;
constexpr int kSlotTokensPerThread = 8;  // a multiple of 4
static_assert(kSlotTokensPerThread % 4 == 0, "whole 16-byte stores");
constexpr int kWaveLanes = 64;
constexpr int kSlotChunks = 1;  // consecutive chunks of 64 x kSlotTokensPerThread per wave

// Largest r in [0, num_reqs) with qsl[r] <= t (qsl non-decreasing, qsl[0] = 0
// <= t): the candidate interval shrinks 64-fold per round, every lane testing
// one evenly spaced candidate.  t is the same in every lane.
__device__ __forceinline__ int find_request_wave(const int32_t* __restrict__ qsl, int num_reqs,
                                                 int t, int lane) {
  int lo = 0, n = num_reqs;  // the answer lies in [lo, lo + n)
  while (n > 1) {
    const int step = (n + kWaveLanes - 1) / kWaveLanes;
    const int r = lo + lane * step;
    const bool ok = lane * step < n && qsl[r] <= t;
    // lane 0 tests qsl[lo] <= t (qsl[0] = 0 <= t): never empty; the bit is
    // forced so that a malformed qsl still keeps the search in range
    const uint64_t m = __ballot(ok) | 1ull;
    const int k = 63 - __builtin_clzll(m);
    const int nlo = lo + k * step;
    n = min(step, lo + n - nlo);
    lo = nlo;
  }
  return lo;
}

// Moves r forward to the request of token t, given qsl[r] <= t and next =
// qsl[r + 1] (INT32_MAX past the last request); empty requests are skipped.
// One step covers the usual case of at most one boundary; past that the
// search gallops (probing r + 2, r + 3, r + 5, ...) and then halves, so a
// lane k requests past the wave's first one pays O(log k) dependent loads.
__device__ __forceinline__ void seek_request(const int32_t* __restrict__ qsl, int num_reqs,
                                             int64_t t, int& r, int& next) {
  if (t < next) return;
  ++r;  // qsl[r] = next <= t
  next = r + 1 < num_reqs ? qsl[r + 1] : INT32_MAX;
  if (t < next) return;
  // invariant: qsl[lo] <= t < v_hi = qsl[hi] (hi == num_reqs: past the end)
  int lo = r + 1, step = 1, hi, v_hi = INT32_MAX;
  for (;;) {
    hi = lo + step;
    if (hi >= num_reqs) {
      hi = num_reqs;
      break;
    }
    const int v = qsl[hi];
    if (v > t) {
      v_hi = v;
      break;
    }
    lo = hi;
    step <<= 1;
  }
  while (hi - lo > 1) {
    const int mid = lo + ((hi - lo) >> 1);
    const int v = qsl[mid];
    if (v <= t) lo = mid;
    else {
      hi = mid;
      v_hi = v;
    }
  }
  r = lo;
  next = v_hi;
}

// Geometry of the context-parallel and circular modes ([SLOT] sections 2.2,
// 3.1 and 4.2), validated on the host.  pow2: every size below is a power of
// two and the *_log2 fields hold their logarithms (shifts and masks instead
// of divisions).
struct SlotGeom {
  int block_size, kv_block, blocks_per_kv, world, rank, inter;
  int pow2, bs_log2, kvb_log2, world_log2, inter_log2, bpk_log2;
};

enum SlotMode { kSlotPlain = 0, kSlotCp = 1, kSlotCircular = 2 };

// Logical block and offset of position p (p >= 0, below 2^31) on this rank:
// false when another rank owns it.
template <int MODE, bool POW2>
__device__ __forceinline__ bool cp_place(uint32_t p, const SlotGeom& g, uint32_t& lb,
                                         uint32_t& off) {
  if constexpr (MODE == kSlotCircular) {
    // the circular cache keeps every position in logical block 0
    lb = 0;
    off = POW2 ? (p & (uint32_t)(g.block_size - 1)) : p % (uint32_t)g.block_size;
    return true;
  } else if constexpr (POW2) {
    // step 1: virtual block of the world's physical blocks
    const int vbs_log2 = g.kvb_log2 + g.world_log2;
    const uint32_t vb = p >> vbs_log2, vo = p & ((1u << vbs_log2) - 1u);
    // step 2: owner of the position's interleave segment
    if (((vo >> g.inter_log2) & (uint32_t)(g.world - 1)) != (uint32_t)g.rank) return false;
    // step 3: this rank's segments of the virtual block, end to end
    const uint32_t local = ((vo >> (g.world_log2 + g.inter_log2)) << g.inter_log2) |
                           (vo & (uint32_t)(g.inter - 1));
    // step 4: logical block and offset
    lb = (vb << g.bpk_log2) + (local >> g.bs_log2);
    off = local & (uint32_t)(g.block_size - 1);
    return true;
  } else {
    const uint32_t vbs = (uint32_t)g.kv_block * (uint32_t)g.world;
    const uint32_t vb = p / vbs, vo = p - vb * vbs;
    const uint32_t seg = vo / (uint32_t)g.inter;
    if (seg % (uint32_t)g.world != (uint32_t)g.rank) return false;
    const uint32_t wi = (uint32_t)g.world * (uint32_t)g.inter;
    const uint32_t local = (vo / wi) * (uint32_t)g.inter + (vo - seg * (uint32_t)g.inter);
    const uint32_t lbl = local / (uint32_t)g.block_size;
    lb = vb * (uint32_t)g.blocks_per_kv + lbl;
    off = local - lbl * (uint32_t)g.block_size;
    return true;
  }
}

// One chunk of 64 x kSlotTokensPerThread tokens starting at wave_t0.  r and
// next carry this lane's request (and the first token of the request after
// it) from one chunk of the wave to the next; have_r is false until the
// wave's request has been searched once.
template <int MODE, bool POW2>
__device__ __forceinline__ void slot_chunk(
    const int32_t* __restrict__ qsl, int num_reqs, const int64_t* __restrict__ positions,
    int num_tokens, const int32_t* __restrict__ block_table, int stride, int block_size,
    int32_t* __restrict__ out, int max_num_tokens, const SlotGeom& g, int64_t wave_t0, int lane,
    int& r, int& next, bool& have_r) {
  const int64_t t0 = wave_t0 + (int64_t)lane * kSlotTokensPerThread;
  int32_t res[kSlotTokensPerThread];
  int64_t pos[kSlotTokensPerThread];
  const bool full = t0 + kSlotTokensPerThread <= num_tokens;
  if (full && (((uintptr_t)(positions + t0)) & 15) == 0) {
    const int4* p4 = reinterpret_cast<const int4*>(positions + t0);
#pragma unroll
    for (int q = 0; q < kSlotTokensPerThread / 2; ++q) {
      const int4 a = p4[q];
      pos[2 * q] = ((int64_t)(uint32_t)a.x) | ((int64_t)a.y << 32);
      pos[2 * q + 1] = ((int64_t)(uint32_t)a.z) | ((int64_t)a.w << 32);
    }
  } else {
#pragma unroll
    for (int j = 0; j < kSlotTokensPerThread; ++j)
      pos[j] = (t0 + j < num_tokens) ? positions[t0 + j] : 0;
  }
  // the wave's first token's request (uniform), searched once per wave, when
  // it has real tokens; later chunks continue from each lane's request
  int32_t win[kSlotTokensPerThread];
  bool have_win = false;  // win[] already holds this lane's next boundaries
  if (!have_r && num_reqs > 0 && wave_t0 < num_tokens) {
    // (uniform branch: every lane of the wave takes it)
    // The 64 boundaries after the wave's request, one per lane: a lane whose
    // first token lies within them finds its request by a binary search over
    // the lanes (the boundaries are non-decreasing), so batches of short
    // requests, such as decode steps of one token per request, need no chain
    // of dependent loads.  `next` is the first token of the request after the
    // lane's (kept in a register: read again only when a lane crosses into it).
    int32_t wq;
    const bool small = num_reqs <= kWaveLanes;
    if (small) {
      // At most 64 requests: every start in one load, qsl[lane]; the wave's
      // request (the last start at or below its first token) by a ballot, and
      // the boundaries after it by lane shuffles
      const int32_t v = lane < num_reqs ? qsl[lane] : INT32_MAX;
      r = 63 - __builtin_clzll(__ballot((int64_t)v <= wave_t0) | 1ull);
      const int src = r + 1 + lane;
      const int32_t sv = __shfl(v, min(src, kWaveLanes - 1), kWaveLanes);
      wq = src < num_reqs ? sv : INT32_MAX;
    } else {
      r = find_request_wave(qsl, num_reqs, (int)wave_t0, lane);
      const int wj = r + 1 + lane;
      wq = wj < num_reqs ? qsl[wj] : INT32_MAX;
    }
    int cnt = 0;  // boundaries of the window at or below t0 (a prefix of it)
#pragma unroll
    for (int step = 32; step > 0; step >>= 1) {
      const int32_t v = __shfl(wq, cnt + step - 1, kWaveLanes);
      if ((int64_t)v <= t0) cnt += step;
    }
    const int32_t last = __shfl(wq, kWaveLanes - 1, kWaveLanes);
    if (cnt == kWaveLanes - 1 && (int64_t)last <= t0) cnt = kWaveLanes;
    const int32_t nx = __shfl(wq, cnt & (kWaveLanes - 1), kWaveLanes);
    r += cnt;
    if (cnt < kWaveLanes) next = nx;
    else next = r + 1 < num_reqs ? qsl[r + 1] : INT32_MAX;  // past the window: read on
    if (small) {
      // the window holds every later boundary: the lane's next ones,
      // qsl[r + 1 + k], are window lanes cnt + k (past the window: none)
#pragma unroll
      for (int k = 0; k < kSlotTokensPerThread; ++k) {
        const int32_t x = __shfl(wq, min(cnt + k, kWaveLanes - 1), kWaveLanes);
        win[k] = cnt + k < kWaveLanes ? x : INT32_MAX;
      }
      have_win = true;
    }
    have_r = true;
  }
  // this lane's first token's request
  if (num_reqs > 0 && have_r && t0 < num_tokens) seek_request(qsl, num_reqs, t0, r, next);
  bool done = false;
  if constexpr (MODE == kSlotPlain && POW2) {
    // Common case: the thread's tokens are all real, inside one request, at
    // consecutive positions p0 .. p0 + n - 1 below 2^31.  They then span at
    // most two blocks (n <= block size) or a few, and the table entries of the
    // first and last are all that is read; anything else takes the general
    // path below.
    if (full && num_reqs > 0) {
      PSW_DCHECK(16, r >= 0 && r < num_reqs && qsl[r] <= t0);
      bool run = t0 + kSlotTokensPerThread <= next && pos[0] >= 0 &&
                 pos[0] + kSlotTokensPerThread - 1 <= INT32_MAX &&
                 kSlotTokensPerThread <= block_size;
#pragma unroll
      for (int j = 1; j < kSlotTokensPerThread; ++j) run = run && pos[j] == pos[0] + j;
      if (run) {
        const uint32_t p0 = (uint32_t)pos[0], mask = (uint32_t)(block_size - 1);
        const uint32_t lb0 = p0 >> g.bs_log2;
        const uint32_t lb1 = (p0 + kSlotTokensPerThread - 1) >> g.bs_log2;  // lb0 or lb0 + 1
        const int64_t row = (int64_t)r * stride;
        const int32_t b0 = lb0 < (uint32_t)stride ? block_table[row + lb0] : -1;
        const int32_t b1 = lb1 == lb0 ? b0 : (lb1 < (uint32_t)stride ? block_table[row + lb1] : -1);
#pragma unroll
        for (int j = 0; j < kSlotTokensPerThread; ++j) {
          const uint32_t pj = p0 + j;
          const bool second = (pj >> g.bs_log2) != lb0;
          const int32_t b = second ? b1 : b0;
          res[j] = b >= 0 ? (int32_t)(((uint32_t)b << g.bs_log2) + (pj & mask)) : -1;
        }
        done = true;
      }
    }
  }
  // General path: the lane's next boundaries qsl[rw + 1 + k], read together
  // (or taken from the window above), serve its tokens' crossings (one token
  // per request needs one per token); more crossings than that (empty
  // requests) read on
  const int rw = r;
  PSW_DCHECK(16, !have_win || t0 >= num_tokens || t0 < next);
  if (!done && num_reqs > 0 && t0 < num_tokens && !have_win) {
#pragma unroll
    for (int k = 0; k < kSlotTokensPerThread; ++k)
      win[k] = rw + 1 + k < num_reqs ? qsl[rw + 1 + k] : INT32_MAX;
  }
  // First each token's request and its table element (tix, -1 when the
  // token maps to -1) with its offset inside the block, then the table
  // entries of all the lane's tokens as one round of independent loads: a
  // load per token inside the request walk would wait for each in turn (a
  // decode batch of one token per request takes this path on every lane).
  int64_t tix[kSlotTokensPerThread], toff[kSlotTokensPerThread];
#pragma unroll
  for (int j = 0; j < kSlotTokensPerThread && !done; ++j) {
    const int64_t t = t0 + j;
    tix[j] = -1;
    toff[j] = 0;
    if (t < num_tokens && num_reqs > 0) {
      while (t >= next) {  // crossing into the next request (empty ones skipped)
        ++r;
        const int k = r - rw;  // >= 1
        int32_t nx = INT32_MAX;
        if (k < kSlotTokensPerThread) {
#pragma unroll
          for (int i = 1; i < kSlotTokensPerThread; ++i) nx = k == i ? win[i] : nx;
        } else {
          nx = r + 1 < num_reqs ? qsl[r + 1] : INT32_MAX;
        }
        next = nx;
      }
      PSW_DCHECK(16, r >= 0 && r < num_reqs && qsl[r] <= t && (r + 1 == num_reqs || t < qsl[r + 1]));
      const int64_t p = pos[j];
      if constexpr (MODE == kSlotPlain && POW2) {
        // power-of-two blocks: shift and mask of the 32-bit position (the
        // slot's low 32 bits are those of the 64-bit product below)
        if (p >= 0 && p <= INT32_MAX) {
          const uint32_t lb = (uint32_t)p >> g.bs_log2;
          if (lb < (uint32_t)stride) {
            tix[j] = (int64_t)r * stride + lb;
            toff[j] = (uint32_t)p & (uint32_t)(block_size - 1);
          }
        }
      } else if constexpr (MODE == kSlotPlain) {
        if (p >= 0) {
          const int64_t lb = p / block_size;
          if (lb < stride) {
            tix[j] = (int64_t)r * stride + lb;
            toff[j] = p - lb * block_size;
          }
        }
      } else {
        uint32_t lb, off;
        if (p >= 0 && p <= INT32_MAX && cp_place<MODE, POW2>((uint32_t)p, g, lb, off) &&
            lb < (uint32_t)stride) {
          // step 5 below: physical block through the table
          tix[j] = (int64_t)r * stride + lb;
          toff[j] = off;
        }
      }
    }
  }
  if (!done) {
    int32_t b[kSlotTokensPerThread];
#pragma unroll
    for (int j = 0; j < kSlotTokensPerThread; ++j) b[j] = tix[j] >= 0 ? block_table[tix[j]] : -1;
#pragma unroll
    for (int j = 0; j < kSlotTokensPerThread; ++j)
      res[j] = b[j] >= 0 ? (int32_t)(b[j] * (int64_t)block_size + toff[j]) : -1;
  }
  if (t0 + kSlotTokensPerThread <= max_num_tokens && (((uintptr_t)(out + t0)) & 15) == 0) {
#pragma unroll
    for (int q = 0; q < kSlotTokensPerThread / 4; ++q)
      reinterpret_cast<int4*>(out + t0)[q] =
          make_int4(res[4 * q], res[4 * q + 1], res[4 * q + 2], res[4 * q + 3]);
  } else {
#pragma unroll
    for (int j = 0; j < kSlotTokensPerThread; ++j)
      if (t0 + j < max_num_tokens) out[t0 + j] = res[j];
  }
}

// Each wave maps kSlotChunks consecutive chunks (the request search is done
// once per wave and carried forward).
template <int MODE, bool POW2>
__global__ __launch_bounds__(kSlotThreads) void slot_mapping_kernel(
    const int32_t* __restrict__ qsl, int num_reqs, const int64_t* __restrict__ positions,
    int num_tokens, const int32_t* __restrict__ block_table, int stride, int block_size,
    int32_t* __restrict__ out, int max_num_tokens, const SlotGeom g) {
  const int lane = threadIdx.x % kWaveLanes;
  constexpr int64_t kChunkTokens = (int64_t)kWaveLanes * kSlotTokensPerThread;
  const int64_t wave = (int64_t)blockIdx.x * (kSlotThreads / kWaveLanes) + threadIdx.x / kWaveLanes;
  int r = 0, next = INT32_MAX;
  bool have_r = false;
  for (int c = 0; c < kSlotChunks; ++c) {
    const int64_t wave_t0 = (wave * kSlotChunks + c) * kChunkTokens;
    if (wave_t0 >= max_num_tokens) break;  // the rest of the wave's chunks are past the end
    slot_chunk<MODE, POW2>(qsl, num_reqs, positions, num_tokens, block_table, stride, block_size,
                           out, max_num_tokens, g, wave_t0, lane, r, next, have_r);
  }
}

template <int MODE, bool POW2>
static hipError_t launch_slot_t(const int32_t* qsl, int num_reqs, const int64_t* positions,
                                int num_tokens, const int32_t* block_table, int stride,
                                int block_size, int32_t* out, int max_num_tokens,
                                const SlotGeom& g, hipStream_t stream) {
  const int64_t per_block = (int64_t)kSlotThreads * kSlotTokensPerThread * kSlotChunks;
  const int grid = (int)((max_num_tokens + per_block - 1) / per_block);
  hipLaunchKernelGGL((slot_mapping_kernel<MODE, POW2>), dim3(grid), dim3(kSlotThreads), 0, stream,
                     qsl, num_reqs, positions, num_tokens, block_table, stride, block_size, out,
                     max_num_tokens, g);
  return hipGetLastError();
}

static int ilog2_exact(int v) {  // log2 of a power of two, else -1
  if (v < 1 || (v & (v - 1)) != 0) return -1;
  int l = 0;
  while ((1 << l) < v) ++l;
  return l;
}

hipError_t launch_slot_mapping(const int32_t* qsl, int num_reqs, const int64_t* positions,
                               int num_tokens, const int32_t* block_table, int stride,
                               int block_size, int32_t* out, int max_num_tokens,
                               hipStream_t stream) {
  if (max_num_tokens == 0) return hipSuccess;
  SlotGeom g{};
  g.block_size = block_size;
  g.bs_log2 = ilog2_exact(block_size);
  if (g.bs_log2 >= 0)
    return launch_slot_t<kSlotPlain, true>(qsl, num_reqs, positions, num_tokens, block_table,
                                           stride, block_size, out, max_num_tokens, g, stream);
  return launch_slot_t<kSlotPlain, false>(qsl, num_reqs, positions, num_tokens, block_table,
                                          stride, block_size, out, max_num_tokens, g, stream);
}


hipError_t launch_slot_mapping_cp(const int32_t* qsl, int num_reqs, const int64_t* positions,
                                  int num_tokens, const int32_t* block_table, int stride,
                                  int block_size, int kv_cache_block_size, int cp_world_size,
                                  int cp_rank, int cp_interleave, bool circular, int32_t* out,
                                  int max_num_tokens, hipStream_t stream) {
  if (max_num_tokens == 0) return hipSuccess;
  SlotGeom g{};
  g.block_size = block_size;
  g.kv_block = kv_cache_block_size;
  g.blocks_per_kv = kv_cache_block_size / block_size;
  g.world = cp_world_size;
  g.rank = cp_rank;
  g.inter = cp_interleave;
  g.bs_log2 = ilog2_exact(block_size);
  g.kvb_log2 = ilog2_exact(kv_cache_block_size);
  g.world_log2 = ilog2_exact(cp_world_size);
  g.inter_log2 = ilog2_exact(cp_interleave);
  g.bpk_log2 = ilog2_exact(g.blocks_per_kv);
  g.pow2 = g.bs_log2 >= 0 && g.kvb_log2 >= 0 && g.world_log2 >= 0 && g.inter_log2 >= 0 &&
           g.bpk_log2 >= 0;
  auto go = [&](auto mode, auto pow2) {
    return launch_slot_t<decltype(mode)::value, decltype(pow2)::value>(
        qsl, num_reqs, positions, num_tokens, block_table, stride, block_size, out,
        max_num_tokens, g, stream);
  };
  using P = std::integral_constant<int, kSlotPlain>;
  using C = std::integral_constant<int, kSlotCp>;
  using R = std::integral_constant<int, kSlotCircular>;
  using T = std::true_type;
  using F = std::false_type;
  if (circular) return g.bs_log2 >= 0 ? go(R{}, T{}) : go(R{}, F{});
  // one rank: the interleave is the identity and the mapping is the plain one
  if (cp_world_size == 1) return g.bs_log2 >= 0 ? go(P{}, T{}) : go(P{}, F{});
  return g.pow2 ? go(C{}, T{}) : go(C{}, F{});
}

PSW_DEBUG_TAKE(debug_take_slot_mapping)

}  // namespace psw
