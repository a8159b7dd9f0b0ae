// Slot mapping: vllm-ascend Triton operator deep dive, _compute_slot_mapping_kernel,
// sections 1, 2 and 4.3.  The page's design runs one program per request plus a
// dedicated padding program, and loads a bounded window of the block table per
// 1024-token tile.  Here the grid is flat over the padded token axis instead:
// each thread owns consecutive tokens, finds its request by binary search over
// query_start_loc (L2-resident, a few dozen bytes per request), reads its
// positions with 16-byte loads and writes its slots (or -1) with one 16-byte
// store, so every wave streams contiguous positions and slots.  Block-table
// entries are read per token; consecutive tokens of a request hit the same
// cache line, which plays the role of the page's bounded window.
#include "psw_internal.h"

namespace psw {

constexpr int kSlotThreads = 256;
constexpr int kSlotTokensPerThread = 4;

__device__ __forceinline__ int find_request(const int32_t* __restrict__ qsl, int num_reqs, int t) {
  // largest r in [0, num_reqs) with qsl[r] <= t
  int lo = 0, hi = num_reqs - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (qsl[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__global__ __launch_bounds__(kSlotThreads) void slot_mapping_kernel(
    const int32_t* __restrict__ qsl, int num_reqs, const int64_t* __restrict__ positions,
    int num_tokens, const int32_t* __restrict__ block_table, int stride, int block_size,
    int32_t* __restrict__ out, int max_num_tokens) {
  const int64_t t0 = ((int64_t)blockIdx.x * kSlotThreads + threadIdx.x) * kSlotTokensPerThread;
  if (t0 >= max_num_tokens) return;
  int32_t res[kSlotTokensPerThread];
  int64_t pos[kSlotTokensPerThread];
  const bool full = t0 + kSlotTokensPerThread <= num_tokens;
  if (full && (((uintptr_t)(positions + t0)) & 15) == 0) {
    const int4* p4 = reinterpret_cast<const int4*>(positions + t0);
    int4 a = p4[0], b = p4[1];
    pos[0] = ((int64_t)(uint32_t)a.x) | ((int64_t)a.y << 32);
    pos[1] = ((int64_t)(uint32_t)a.z) | ((int64_t)a.w << 32);
    pos[2] = ((int64_t)(uint32_t)b.x) | ((int64_t)b.y << 32);
    pos[3] = ((int64_t)(uint32_t)b.z) | ((int64_t)b.w << 32);
  } else {
#pragma unroll
    for (int j = 0; j < kSlotTokensPerThread; ++j)
      pos[j] = (t0 + j < num_tokens) ? positions[t0 + j] : 0;
  }
  int r = (num_reqs > 0 && t0 < num_tokens) ? find_request(qsl, num_reqs, (int)t0) : 0;
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
    *reinterpret_cast<int4*>(out + t0) = make_int4(res[0], res[1], res[2], res[3]);
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
