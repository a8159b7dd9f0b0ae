// V-up projection of the merged latent attention output: MLA DCP decode study
// notes (vllm-ascend PR #16977), "Terms" (the attention output over the
// latent vectors is projected back to each head's V dimension), section 1.1
// (the merged output is batch-major) and code block A (one batched product
// per head, no transposes of the data):
//
//     out[t, h, :] = x[t, h, :] @ W_UV[h]      x [T, H, R], W_UV [H, R, Dv], out [T, H, Dv]
//
// One workgroup computes 64 tokens x 64 output columns of one head with
// v_mfma_f32_32x32x16_bf16 (fp32 accumulation): the head's W_UV columns are
// copied into LDS with direct-to-LDS loads (rows of 64 columns, 128 B) and
// read transposed with ds_read_b64_tr_b16 as the A operand (32 output columns
// x 16 rows of R), while x supplies the B operand straight from global memory
// (16 contiguous bytes of one token's row per lane and k-step), so the
// product out^T = W_UV^T x^T lands one token per lane.  Wave w takes output
// columns 32 (w & 1) .. + 32 and tokens 32 (w >> 1) .. + 32.
#include "asm_ops.h"
#include "device_common.h"
#include "psw_internal.h"

namespace psw {

namespace vup {
constexpr int kThreads = 256;
constexpr int kCols = 64;     // output columns per workgroup
constexpr int kTokens = 64;   // tokens per workgroup
constexpr int kRowBytes = kCols * 2;
}  // namespace vup

__device__ __forceinline__ void vup_dma16(const void* gsrc, void* lds_dst) {
  __builtin_amdgcn_global_load_lds(
      (const __attribute__((address_space(1))) void*)gsrc,
      (__attribute__((address_space(3))) void*)(lds_void*)lds_dst, 16, 0, 0);
}

template <int R>
__global__ __launch_bounds__(vup::kThreads) void vup_projection_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, uint16_t* __restrict__ out,
    int num_tokens, int num_heads, int dv) {
  using namespace vup;
  constexpr int kSteps = R / 16;          // MFMA k-steps
  constexpr int kInstr = R / 8;           // LDS-DMA instructions (8 rows of 128 B each)
  constexpr int kPerWave = kInstr / 4;
  static_assert(kPerWave * 4 == kInstr, "rows split evenly over the waves");
  static_assert(kSteps * 16 * kRowBytes <= 65536, "LDS offsets fit the 16-bit immediate");
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int lane = threadIdx.x % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int half = lane >> 5;
  const int ncb = dv / kCols;
  const int h = blockIdx.x / ncb, cb = blockIdx.x - h * ncb;
  const int64_t row_bytes = (int64_t)dv * 2;  // one row of W_UV[h]

  // W_UV[h][:, 64 cb .. 64 cb + 64) -> LDS: instruction g moves rows 8 g .. 8 g + 7,
  // lane l row 8 g + l / 8, 16-byte chunk l % 8
  {
    const char* wb = reinterpret_cast<const char*>(w + (int64_t)h * R * dv + cb * kCols);
    const int64_t lane_off = (lane >> 3) * row_bytes + (lane & 7) * 16;
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
      const int g = wave * kPerWave + i;
      vup_dma16(wb + (int64_t)(8 * g) * row_bytes + lane_off, smem + g * 1024);
    }
  }

  // this lane's token and its k-chunks 16 s + 8 half .. + 8 (the B operand)
  const int t = blockIdx.y * kTokens + (wave >> 1) * 32 + (lane & 31);
  const bool valid = t < num_tokens;
  bf16x8 xf[kSteps];
  {
    const uint16_t* xr = x + ((int64_t)(valid ? t : 0) * num_heads + h) * R + half * 8;
#pragma unroll
    for (int s = 0; s < kSteps; ++s)
      xf[s] = valid ? *reinterpret_cast<const bf16x8*>(xr + 16 * s) : bf16x8{};
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // this wave's copies and x rows have landed
  lds_barrier();                              // every wave's copies are visible

  // A operand: W_UV^T for columns 32 (w & 1) + [0, 32) and rows 16 s + [0, 16):
  // two transposed reads give a lane rows 8 half + [0, 4) and + [4, 8) of its
  // column, the k order of the B operand
  const int tr_row = half * 8 + ((lane & 15) >> 2);
  const int tr_col = (wave & 1) * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const uint32_t a0 = lds_addr(smem) + (uint32_t)(tr_row * kRowBytes + tr_col * 2);
  f32x16 acc = f32x16{};
  constexpr int RA = 2;  // transposed reads run RA k-steps ahead
  bf16x4 ar[RA + 1][2];
  auto read_a = [&](auto ss) __attribute__((always_inline)) {
    constexpr int s = decltype(ss)::value;
    ar[s % (RA + 1)][0] = lds_read_tr4_at<s * 16 * kRowBytes>(a0);
    ar[s % (RA + 1)][1] = lds_read_tr4_at<s * 16 * kRowBytes + 4 * kRowBytes>(a0);
  };
  static_for<RA>(read_a);
  static_for<kSteps>([&](auto ss) {
    constexpr int s = decltype(ss)::value;
    constexpr int issued = s + RA < kSteps ? s + RA : kSteps;
    lds_wait<2 * (issued - 1 - s)>(ar[s % (RA + 1)][0], ar[s % (RA + 1)][1]);
    acc = mfma32(cat8(ar[s % (RA + 1)][0], ar[s % (RA + 1)][1]), xf[s], acc);
    if constexpr (s + RA < kSteps) read_a(std::integral_constant<int, s + RA>{});
  });

  // acc[i]: output column (i / 4) * 8 + 4 half + i % 4 of the wave's 32, token t
  if (valid) {
    uint16_t* o = out + ((int64_t)t * num_heads + h) * dv + cb * kCols + (wave & 1) * 32 + half * 4;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<bf16x4*>(o + q * 8) =
          to_bf16x4(acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]);
  }
}

bool vup_supported(int kv_lora_rank, int v_head_dim) {
  return (kv_lora_rank == 128 || kv_lora_rank == 256 || kv_lora_rank == 512) &&
         v_head_dim >= vup::kCols && v_head_dim % vup::kCols == 0;
}

template <int R>
static hipError_t launch_vup_t(const uint16_t* x, const uint16_t* w, uint16_t* out, int T, int H,
                               int dv, hipStream_t stream) {
  const size_t lds = (size_t)R * vup::kRowBytes;
  auto kern = vup_projection_kernel<R>;
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (attr != hipSuccess) return attr;
  dim3 grid((unsigned)(H * (dv / vup::kCols)), (unsigned)((T + vup::kTokens - 1) / vup::kTokens));
  hipLaunchKernelGGL(kern, grid, dim3(vup::kThreads), lds, stream, x, w, out, T, H, dv);
  return hipGetLastError();
}

hipError_t launch_vup_projection(const uint16_t* x, const uint16_t* w, uint16_t* out,
                                 int num_tokens, int num_heads, int kv_lora_rank, int v_head_dim,
                                 hipStream_t stream) {
  if (num_tokens == 0 || num_heads == 0) return hipSuccess;
  switch (kv_lora_rank) {
    case 128: return launch_vup_t<128>(x, w, out, num_tokens, num_heads, v_head_dim, stream);
    case 256: return launch_vup_t<256>(x, w, out, num_tokens, num_heads, v_head_dim, stream);
    case 512: return launch_vup_t<512>(x, w, out, num_tokens, num_heads, v_head_dim, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace psw
