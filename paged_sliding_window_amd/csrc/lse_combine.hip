// Merge split-KV partials by log-sum-exp: MLA DCP decode study notes
// (vllm-ascend PR #16977), "Terms" (LSE), section 1.1 (two partials, each with
// output and LSE, merge into one softmax over all keys) and code block D (the
// merge reads the received history shards and the local current partial in
// place, with no packing).  Here the partials arrive as an array of pointers
// passed by value in the kernel arguments, so nothing is packed either.
//
// One wave per row: lane p reads lse_p, the wave reduces max and weight sum,
// then each lane accumulates eight consecutive output columns over the partials
// (16-byte loads of bf16, 32-byte loads of fp32 partials).
#include "device_common.h"
#include "psw_internal.h"

namespace psw {

constexpr int kCombineWaves = 4;

template <bool PART_F32, bool OUT_F32>
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
      if (PART_F32) {
        const float4* src =
            reinterpret_cast<const float4*>(static_cast<const float*>(parts.out[p]) +
                                            row * head_dim_v + d0);
        float4 a = src[0], b = src[1];
        acc[0] += wp * a.x; acc[1] += wp * a.y; acc[2] += wp * a.z; acc[3] += wp * a.w;
        acc[4] += wp * b.x; acc[5] += wp * b.y; acc[6] += wp * b.z; acc[7] += wp * b.w;
      } else {
        const uint4 v = *reinterpret_cast<const uint4*>(
            static_cast<const uint16_t*>(parts.out[p]) + row * head_dim_v + d0);
        const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[2 * j] += wp * __builtin_bit_cast(float, u[j] << 16);
          acc[2 * j + 1] += wp * __builtin_bit_cast(float, u[j] & 0xffff0000u);
        }
      }
    }
    if (OUT_F32) {
      float4* dst = reinterpret_cast<float4*>(static_cast<float*>(out) + row * head_dim_v + d0);
      dst[0] = make_float4(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
      dst[1] = make_float4(acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv);
    } else {
      bf16x8 o = to_bf16x8(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv,
                           acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv);
      *reinterpret_cast<bf16x8*>(static_cast<uint16_t*>(out) + row * head_dim_v + d0) = o;
    }
  }
  if (out_lse != nullptr && lane == 0)
    out_lse[row] = den > 0.f ? M + __logf(den) : -INFINITY;
}

hipError_t launch_lse_combine(const CombineArgs& parts, int num_partials, int partial_f32,
                              int64_t num_rows, int head_dim_v, void* out, int out_f32,
                              float* out_lse, hipStream_t stream) {
  if (num_rows == 0) return hipSuccess;
  const dim3 grid((unsigned)((num_rows + kCombineWaves - 1) / kCombineWaves));
  const dim3 block(kCombineWaves * kWave);
  if (partial_f32 && out_f32)
    hipLaunchKernelGGL((lse_combine_kernel<true, true>), grid, block, 0, stream, parts,
                       num_partials, num_rows, head_dim_v, out, out_lse);
  else if (partial_f32)
    hipLaunchKernelGGL((lse_combine_kernel<true, false>), grid, block, 0, stream, parts,
                       num_partials, num_rows, head_dim_v, out, out_lse);
  else if (out_f32)
    hipLaunchKernelGGL((lse_combine_kernel<false, true>), grid, block, 0, stream, parts,
                       num_partials, num_rows, head_dim_v, out, out_lse);
  else
    hipLaunchKernelGGL((lse_combine_kernel<false, false>), grid, block, 0, stream, parts,
                       num_partials, num_rows, head_dim_v, out, out_lse);
  return hipGetLastError();
}

}  // namespace psw
