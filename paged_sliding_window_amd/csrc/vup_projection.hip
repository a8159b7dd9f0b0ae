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

// LSE combine and V-up projection in one launch (the two steps that end the
// decode, [DCP] code blocks D and A): the workgroup of (head h, 64 output
// columns, 64 tokens) first merges its 64 tokens' latent rows of head h from
// the P partials into LDS, with the combine kernel's arithmetic (the same max,
// weights, tree order of the weight sum, fused multiply-adds in partial order
// and bf16 rounding), so the merged row, its LSE and the projection equal
// those of psw_lse_combine followed by psw_vup_projection bit for bit; then
// projects them as vup_projection_kernel does, with the B operand read from
// LDS.  The workgroups of the first 64-column block also write the merged rows
// (when asked) and their LSEs.
namespace vup {
constexpr int kMaxFusedPartials = 16;
}

template <int R, int PART>
__global__ __launch_bounds__(vup::kThreads) void combine_vup_kernel(
    const CombineArgs parts, int num_partials, const uint16_t* __restrict__ w,
    uint16_t* __restrict__ out, float* __restrict__ out_lse, uint16_t* __restrict__ merged,
    int num_tokens, int num_heads, int dv) {
  using namespace vup;
  constexpr int kSteps = R / 16;
  constexpr int kInstr = R / 8;
  constexpr int kPerWave = kInstr / 4;
  constexpr int kChunks = R / 8;                  // 16-byte chunks of one latent row
  constexpr int kXPitch = R * 2 + 16;             // LDS bytes per merged row (padded)
  constexpr int kWBytes = kSteps * 16 * kRowBytes;
  constexpr int kXBytes = kTokens * kXPitch;
  constexpr int kWts = kMaxFusedPartials + 1;     // per token: P weights, then 1 / sum
  static_assert(kPerWave * 4 == kInstr && (kTokens * kChunks) % kThreads == 0, "shapes");
  extern __shared__ __attribute__((aligned(16))) char smem[];
  char* xs = smem + kWBytes;
  float* wts = reinterpret_cast<float*>(smem + kWBytes + kXBytes);

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int half = lane >> 5;
  const int ncb = dv / kCols;
  // the column blocks of one (head, token block) merge the same rows: give
  // them neighbouring logical ids, which share an XCD and so its L2 (the
  // second merge then reads the partials from L2 rather than HBM)
  const int logical = xcd_logical_id(blockIdx.x + gridDim.x * blockIdx.y, gridDim.x * gridDim.y);
  const int bx = logical % gridDim.x;
  const int h = bx / ncb, cb = bx - h * ncb;
  const int64_t row_bytes = (int64_t)dv * 2;
  const int tok0 = (logical / gridDim.x) * kTokens;

  // W_UV[h][:, 64 cb .. + 64) -> LDS, as in vup_projection_kernel
  {
    const char* wb = reinterpret_cast<const char*>(w + (int64_t)h * R * dv + cb * kCols);
    const int64_t lane_off = (lane >> 3) * row_bytes + (lane & 7) * 16;
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
      const int g = wave * kPerWave + i;
      vup_dma16(wb + (int64_t)(8 * g) * row_bytes + lane_off, smem + g * 1024);
    }
  }

  // weights of the 64 tokens' rows (one thread per token)
  if (tid < kTokens) {
    const int t = tok0 + tid;
    float wv[kMaxFusedPartials];
    float M = -INFINITY, inv = 0.f;
    if (t < num_tokens) {
      const int64_t row = (int64_t)t * num_heads + h;
      float l[kMaxFusedPartials];
#pragma unroll
      for (int p = 0; p < kMaxFusedPartials; ++p) {
        l[p] = p < num_partials ? parts.lse[p][row] : -INFINITY;
        M = fmaxf(M, l[p]);
      }
#pragma unroll
      for (int p = 0; p < kMaxFusedPartials; ++p)
        wv[p] = (p < num_partials && M != -INFINITY) ? __expf(l[p] - M) : 0.f;
      // the sum in the order of the combine kernel's butterfly over 64 lanes
      // (the levels 32 and 16 add zeros for P <= 16)
      float a[kMaxFusedPartials];
#pragma unroll
      for (int p = 0; p < kMaxFusedPartials; ++p) a[p] = wv[p];
#pragma unroll
      for (int o = kMaxFusedPartials / 2; o > 0; o >>= 1)
#pragma unroll
        for (int i = 0; i < o; ++i) a[i] = a[i] + a[i + o];
      const float den = a[0];
      inv = den > 0.f ? 1.f / den : 0.f;
      if (cb == 0 && out_lse != nullptr) out_lse[row] = den > 0.f ? M + __logf(den) : -INFINITY;
    } else {
#pragma unroll
      for (int p = 0; p < kMaxFusedPartials; ++p) wv[p] = 0.f;
    }
#pragma unroll
    for (int p = 0; p < kMaxFusedPartials; ++p) wts[tid * kWts + p] = wv[p];
    wts[tid * kWts + kMaxFusedPartials] = inv;
  }
  __syncthreads();

  // merged rows: chunk c of the workgroup is chunk c % kChunks of token c / kChunks;
  // a thread takes chunks tid + kThreads * i, kBatch at a time, and for each
  // partial issues the batch's loads together before accumulating them
  constexpr int kPer = kTokens * kChunks / kThreads;
  constexpr int kBatch = kPer < 8 ? kPer : 8;
  static_assert(kPer % kBatch == 0, "whole batches");
#pragma unroll 1
  for (int b0 = 0; b0 < kPer; b0 += kBatch) {
    int64_t e[kBatch];
    int tls[kBatch];
    bool ok[kBatch];
    float acc[kBatch][8];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int c = tid + kThreads * (b0 + i);
      tls[i] = c / kChunks;
      const int t = tok0 + tls[i];
      ok[i] = t < num_tokens;
      e[i] = ((int64_t)(ok[i] ? t : 0) * num_heads + h) * R + (c - tls[i] * kChunks) * 8;
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[i][j] = 0.f;
    }
    for (int p = 0; p < num_partials; ++p) {
      const void* src = parts.out[p];
      float v[kBatch][8];
#pragma unroll
      for (int i = 0; i < kBatch; ++i) load8<PART>(src, e[i], v[i]);
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        const float wp = wts[tls[i] * kWts + p];
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] += wp * v[i][j];
      }
    }
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const float inv = wts[tls[i] * kWts + kMaxFusedPartials];
      bf16x8 x8 = to_bf16x8(acc[i][0] * inv, acc[i][1] * inv, acc[i][2] * inv, acc[i][3] * inv,
                            acc[i][4] * inv, acc[i][5] * inv, acc[i][6] * inv, acc[i][7] * inv);
      if (!ok[i]) x8 = bf16x8{};
      else if (cb == 0 && merged != nullptr) *reinterpret_cast<bf16x8*>(merged + e[i]) = x8;
      const int c = tid + kThreads * (b0 + i);
      *reinterpret_cast<bf16x8*>(xs + tls[i] * kXPitch + (c - tls[i] * kChunks) * 16) = x8;
    }
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // this wave's W_UV copies have landed
  __syncthreads();                            // every wave's copies and merged rows

  // the B operand: this lane's token and its k-chunks 16 s + 8 half .. + 8
  const int tl = (wave >> 1) * 32 + (lane & 31);
  const int t = tok0 + tl;
  bf16x8 xf[kSteps];
#pragma unroll
  for (int s = 0; s < kSteps; ++s)
    xf[s] = *reinterpret_cast<const bf16x8*>(xs + tl * kXPitch + (16 * s + 8 * half) * 2);

  const int tr_row = half * 8 + ((lane & 15) >> 2);
  const int tr_col = (wave & 1) * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const uint32_t a0 = lds_addr(smem) + (uint32_t)(tr_row * kRowBytes + tr_col * 2);
  f32x16 acc = f32x16{};
  constexpr int RA = 2;
  bf16x4 ar[RA + 1][2];
  auto read_a = [&](auto ss) __attribute__((always_inline)) {
    constexpr int s = decltype(ss)::value;
    ar[s % (RA + 1)][0] = lds_read_tr4_at<s * 16 * kRowBytes>(a0);
    ar[s % (RA + 1)][1] = lds_read_tr4_at<s * 16 * kRowBytes + 4 * kRowBytes>(a0);
  };
  // the merged rows are in registers before the transposed reads start (the
  // explicit waits below count only those)
  __builtin_amdgcn_s_waitcnt(waitcnt_lgkm(0));
  static_for<RA>(read_a);
  static_for<kSteps>([&](auto ss) {
    constexpr int s = decltype(ss)::value;
    constexpr int issued = s + RA < kSteps ? s + RA : kSteps;
    lds_wait<2 * (issued - 1 - s)>(ar[s % (RA + 1)][0], ar[s % (RA + 1)][1]);
    acc = mfma32(cat8(ar[s % (RA + 1)][0], ar[s % (RA + 1)][1]), xf[s], acc);
    if constexpr (s + RA < kSteps) read_a(std::integral_constant<int, s + RA>{});
  });

  if (t < num_tokens) {
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

template <int R, int PART>
static hipError_t launch_combine_vup_t(const CombineArgs& parts, int P, const uint16_t* w,
                                       uint16_t* out, float* out_lse, uint16_t* merged, int T,
                                       int H, int dv, hipStream_t stream) {
  const size_t lds = (size_t)R * vup::kRowBytes + (size_t)vup::kTokens * (R * 2 + 16) +
                     (size_t)vup::kTokens * (vup::kMaxFusedPartials + 1) * sizeof(float);
  auto kern = combine_vup_kernel<R, PART>;
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (attr != hipSuccess) return attr;
  dim3 grid((unsigned)(H * (dv / vup::kCols)), (unsigned)((T + vup::kTokens - 1) / vup::kTokens));
  hipLaunchKernelGGL(kern, grid, dim3(vup::kThreads), lds, stream, parts, P, w, out, out_lse,
                     merged, T, H, dv);
  return hipGetLastError();
}

template <int PART>
static hipError_t launch_combine_vup_p(const CombineArgs& parts, int P, const uint16_t* w,
                                       uint16_t* out, float* out_lse, uint16_t* merged, int T,
                                       int H, int R, int dv, hipStream_t stream) {
  switch (R) {
    case 128: return launch_combine_vup_t<128, PART>(parts, P, w, out, out_lse, merged, T, H, dv, stream);
    case 256: return launch_combine_vup_t<256, PART>(parts, P, w, out, out_lse, merged, T, H, dv, stream);
    case 512: return launch_combine_vup_t<512, PART>(parts, P, w, out, out_lse, merged, T, H, dv, stream);
    default: return hipErrorInvalidValue;
  }
}

int combine_vup_max_partials() { return vup::kMaxFusedPartials; }

hipError_t launch_combine_vup(const CombineArgs& parts, int num_partials, int partial_dtype,
                              const uint16_t* w, uint16_t* out, float* out_lse, uint16_t* merged,
                              int num_tokens, int num_heads, int kv_lora_rank, int v_head_dim,
                              hipStream_t stream) {
  if (num_tokens == 0 || num_heads == 0) return hipSuccess;
  if (partial_dtype == kOutF32)
    return launch_combine_vup_p<kOutF32>(parts, num_partials, w, out, out_lse, merged,
                                         num_tokens, num_heads, kv_lora_rank, v_head_dim, stream);
  if (partial_dtype == kOutF16)
    return launch_combine_vup_p<kOutF16>(parts, num_partials, w, out, out_lse, merged,
                                         num_tokens, num_heads, kv_lora_rank, v_head_dim, stream);
  return launch_combine_vup_p<kOutBf16>(parts, num_partials, w, out, out_lse, merged, num_tokens,
                                        num_heads, kv_lora_rank, v_head_dim, stream);
}

}  // namespace psw
