// Merge split-KV partials by log-sum-exp: MLA DCP decode study notes
// (vllm-ascend PR #16977), "Terms" (LSE), section 1.1 (two partials, each with
// output and LSE, merge into one softmax over all keys) and code block D (the
// merge reads the received history shards and the local current partial in
// place, with no packing).  Here the partials arrive as an array of pointers
// passed by value in the kernel arguments, so nothing is packed either.
//
// One wave per row: lane p reads lse_p, the wave reduces max and weight sum,
// then each lane accumulates eight consecutive output columns over the partials
// (16-byte loads of bf16 / fp16, 32-byte loads of fp32 partials).
#include "device_common.h"
#include "psw_internal.h"

namespace psw {

constexpr int kCombineWaves = 4;

template <int PART, int OUT>
__global__ __launch_bounds__(kCombineWaves * kWave) void lse_combine_kernel(
    const CombineArgs parts, int num_partials, int64_t num_rows, int head_dim_v,
    void* __restrict__ out, float* __restrict__ out_lse) {
  const int lane = threadIdx.x % kWave;
  const int64_t row = (int64_t)blockIdx.x * kCombineWaves + threadIdx.x / kWave;
  if (row >= num_rows) return;
  float l = -INFINITY;
  if (lane < num_partials) l = parts.lse[lane][row];
  const float M = wave_max(l);
  float w = (lane < num_partials && M != -INFINITY) ? __expf(l - M) : 0.f;
  const float den = wave_sum(w);
  const float inv = den > 0.f ? 1.f / den : 0.f;
  for (int d0 = lane * 8; d0 < head_dim_v; d0 += kWave * 8) {
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int p = 0; p < num_partials; ++p) {
      // readlane ignores EXEC: lanes outside this column loop still hold weights
      const float wp = __builtin_bit_cast(
          float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), p));
      float v[8];
      load8<PART>(parts.out[p], row * head_dim_v + d0, v);
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] += wp * v[j];
    }
    const int64_t e0 = row * head_dim_v + d0;
    store_out4(out, e0, OUT, acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
    store_out4(out, e0 + 4, OUT, acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv);
  }
  if (out_lse != nullptr && lane == 0)
    out_lse[row] = den > 0.f ? M + __logf(den) : -INFINITY;
}

template <int PART>
static void launch_combine_out(const CombineArgs& parts, int num_partials, int64_t num_rows,
                               int head_dim_v, void* out, int out_dtype, float* out_lse,
                               dim3 grid, dim3 block, hipStream_t stream) {
  if (out_dtype == kOutF32)
    hipLaunchKernelGGL((lse_combine_kernel<PART, kOutF32>), grid, block, 0, stream, parts,
                       num_partials, num_rows, head_dim_v, out, out_lse);
  else if (out_dtype == kOutF16)
    hipLaunchKernelGGL((lse_combine_kernel<PART, kOutF16>), grid, block, 0, stream, parts,
                       num_partials, num_rows, head_dim_v, out, out_lse);
  else
    hipLaunchKernelGGL((lse_combine_kernel<PART, kOutBf16>), grid, block, 0, stream, parts,
                       num_partials, num_rows, head_dim_v, out, out_lse);
}

hipError_t launch_lse_combine(const CombineArgs& parts, int num_partials, int partial_dtype,
                              int64_t num_rows, int head_dim_v, void* out, int out_dtype,
                              float* out_lse, hipStream_t stream) {
  if (num_rows == 0) return hipSuccess;
  const dim3 grid((unsigned)((num_rows + kCombineWaves - 1) / kCombineWaves));
  const dim3 block(kCombineWaves * kWave);
  if (partial_dtype == kOutF32)
    launch_combine_out<kOutF32>(parts, num_partials, num_rows, head_dim_v, out, out_dtype,
                                out_lse, grid, block, stream);
  else if (partial_dtype == kOutF16)
    launch_combine_out<kOutF16>(parts, num_partials, num_rows, head_dim_v, out, out_dtype,
                                out_lse, grid, block, stream);
  else
    launch_combine_out<kOutBf16>(parts, num_partials, num_rows, head_dim_v, out, out_dtype,
                                 out_lse, grid, block, stream);
  return hipGetLastError();
}

}  // namespace psw
