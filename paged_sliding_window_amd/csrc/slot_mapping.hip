// Slot mapping: vllm-ascend Triton operator deep dive, _compute_slot_mapping_kernel,
// sections 1, 2 and 4.3.  The page's design runs one program per request plus a
// dedicated padding program, and loads a bounded window of the block table per
// 1024-token tile.  Here the grid is flat over the padded token axis instead:
// each wave owns 64 x kSlotTokensPerThread consecutive tokens, finds the
// request of its first token with a 64-way search over query_start_loc (each
// round one load per lane and a ballot, two rounds for 4096 requests), and
// each lane then walks forward over the few request boundaries inside its own
// tokens.  Positions are read with 16-byte loads and slots (or -1) written
// with 16-byte stores, so every wave streams contiguous positions and slots.
// Block-table entries are read per token; consecutive tokens of a request hit
// the same cache line, which plays the role of the page's bounded window.
#include "psw_internal.h"

namespace psw {

constexpr int kSlotThreads = 256;
#ifndef SLOT_TPT
#define SLOT_TPT 4
#endif
constexpr int kSlotTokensPerThread = SLOT_TPT;  // a multiple of 4
static_assert(kSlotTokensPerThread % 4 == 0, "whole 16-byte stores");
constexpr int kWaveLanes = 64;

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
    const uint64_t m = __ballot(ok);  // lane 0 tests qsl[lo] <= t: never empty
    const int k = 63 - __builtin_clzll(m);
    const int nlo = lo + k * step;
    n = min(step, lo + n - nlo);
    lo = nlo;
  }
  return lo;
}

__global__ __launch_bounds__(kSlotThreads) void slot_mapping_kernel(
    const int32_t* __restrict__ qsl, int num_reqs, const int64_t* __restrict__ positions,
    int num_tokens, const int32_t* __restrict__ block_table, int stride, int block_size,
    int32_t* __restrict__ out, int max_num_tokens) {
  const int lane = threadIdx.x % kWaveLanes;
  const int64_t wave_t0 = ((int64_t)blockIdx.x * kSlotThreads + (threadIdx.x - lane)) *
                          kSlotTokensPerThread;
  if (wave_t0 >= max_num_tokens) return;  // whole wave past the end
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
  // the wave's first token's request (uniform), when it has real tokens
  int r = (num_reqs > 0 && wave_t0 < num_tokens)
              ? find_request_wave(qsl, num_reqs, (int)wave_t0, lane)
              : 0;
#pragma unroll
  for (int j = 0; j < kSlotTokensPerThread; ++j) {
    const int64_t t = t0 + j;
    res[j] = -1;
    if (t < num_tokens && num_reqs > 0) {
      while (r + 1 < num_reqs && qsl[r + 1] <= t) ++r;  // crossing into the next request
      const int64_t p = pos[j];
      if (p >= 0) {
        const int64_t lb = p / block_size;
        if (lb < stride) {
          const int32_t b = block_table[(int64_t)r * stride + lb];
          if (b >= 0) res[j] = (int32_t)(b * (int64_t)block_size + (p - lb * block_size));
        }
      }
    }
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

hipError_t launch_slot_mapping(const int32_t* qsl, int num_reqs, const int64_t* positions,
                               int num_tokens, const int32_t* block_table, int stride,
                               int block_size, int32_t* out, int max_num_tokens,
                               hipStream_t stream) {
  if (max_num_tokens == 0) return hipSuccess;
  const int64_t threads = (max_num_tokens + kSlotTokensPerThread - 1) / kSlotTokensPerThread;
  const int grid = (int)((threads + kSlotThreads - 1) / kSlotThreads);
  hipLaunchKernelGGL(slot_mapping_kernel, dim3(grid), dim3(kSlotThreads), 0, stream, qsl,
                     num_reqs, positions, num_tokens, block_table, stride, block_size, out,
                     max_num_tokens);
  return hipGetLastError();
}

}  // namespace psw
