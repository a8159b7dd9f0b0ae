// Write new K/V rows into the paged cache at their slots (vllm-ascend slot
// mapping article, section 1: the slot id addresses a token's K/V vector; the
// pad slot -1 is never written, nor is any slot outside the cache).  One thread copies one 16-byte chunk; the
// chunk index runs fastest along the head dimension so each wave moves whole
// contiguous rows.
#include "psw_internal.h"

namespace psw {

constexpr int kKvThreads = 256;

__global__ __launch_bounds__(kKvThreads) void kv_cache_write_kernel(
    const uint4* __restrict__ k_new, const uint4* __restrict__ v_new,
    const int32_t* __restrict__ slots, int64_t num_tokens, int hkv, int dk16, int dv16,
    uint4* __restrict__ k_cache, uint4* __restrict__ v_cache, int64_t num_slots) {
  const int64_t k_row = (int64_t)hkv * dk16;  // 16-byte chunks per token of K
  const int64_t v_row = (int64_t)hkv * dv16;
  const int64_t k_total = num_tokens * k_row;
  const int64_t total = k_total + (v_new ? num_tokens * v_row : 0);
  for (int64_t i = (int64_t)blockIdx.x * kKvThreads + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * kKvThreads) {
    if (i < k_total) {
      const int64_t t = i / k_row, c = i - t * k_row;
      const int32_t s = slots[t];
      PSW_DCHECK(17, s == -1 || (s >= 0 && s < num_slots));
      if (s >= 0 && s < num_slots) k_cache[(int64_t)s * k_row + c] = k_new[i];
    } else {
      const int64_t j = i - k_total;
      const int64_t t = j / v_row, c = j - t * v_row;
      const int32_t s = slots[t];
      if (s >= 0 && s < num_slots) v_cache[(int64_t)s * v_row + c] = v_new[j];
    }
  }
}

hipError_t launch_kv_cache_write(const uint16_t* k_new, const uint16_t* v_new,
                                 const int32_t* slots, int num_tokens, int num_kv_heads,
                                 int head_dim_k, int head_dim_v, uint16_t* k_cache,
                                 uint16_t* v_cache, int64_t num_slots, hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  const int dk16 = head_dim_k / 8, dv16 = v_new ? head_dim_v / 8 : 0;
  const int64_t total = (int64_t)num_tokens * num_kv_heads * (dk16 + dv16);
  int64_t grid = (total + kKvThreads - 1) / kKvThreads;
  if (grid > 65536) grid = 65536;
  hipLaunchKernelGGL(kv_cache_write_kernel, dim3((unsigned)grid), dim3(kKvThreads), 0, stream,
                     reinterpret_cast<const uint4*>(k_new), reinterpret_cast<const uint4*>(v_new),
                     slots, (int64_t)num_tokens, num_kv_heads, dk16, dv16,
                     reinterpret_cast<uint4*>(k_cache), reinterpret_cast<uint4*>(v_cache),
                     num_slots);
  return hipGetLastError();
}

PSW_DEBUG_TAKE(debug_take_kv_write)

}  // namespace psw
