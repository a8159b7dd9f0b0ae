// Device-side vocabulary shared by the gfx950 kernels: vector types, the two
// bf16 MFMA shapes, the LDS transpose read, and small wave helpers.
//
// Lane layouts (checked on gfx950 with an in-bounds probe):
//   v_mfma_f32_32x32x16_bf16  A[32][16]: lane l holds row l%32, k = (l/32)*8 .. +8
//                             B[16][32]: lane l holds col l%32, k = (l/32)*8 .. +8
//                             C[32][32]: lane l, reg i -> row (i/4)*8 + (l/32)*4 + i%4, col l%32
//   ds_read_b64_tr_b16        inside each 16-lane group, result element j of lane i is
//                             element i%4 of the 4 halfwords read by lane 4*j + i/4.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace psw {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// Element types of outputs and partials (the psw_dtype values of the C ABI).
constexpr int kOutBf16 = 0, kOutF32 = 1, kOutF16 = 2;

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLog2eHost = 1.4426950408889634f;

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Four bf16 read "transposed" out of LDS (see the layout note above).
__device__ __forceinline__ bf16x4 lds_read_tr4(const __bf16* p) {
  i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)((__attribute__((address_space(3))) char*)(
          (lds_void*)(p))));
  return __builtin_bit_cast(bf16x4, v);
}

// 32-bit LDS address of a pointer into shared memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)(p);
}

// The same transposed read issued as inline assembly.  With the builtin the
// compiler cannot tell the read apart from LDS-DMA writes still in flight and
// waits for every outstanding vector-memory load (vmcnt(0)) before it, which
// stalls a loop that prefetches the next tiles with LDS-DMA.  The compiler does
// not track this read: consume the result only after lds_wait_tr<N>(), which
// waits until at most N LDS operations of this wave are outstanding (LDS
// operations complete in issue order) and ties the registers to that wait.
__device__ __forceinline__ bf16x4 lds_read_tr4_async(uint32_t addr) {
  i16x4 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(r) : "v"(addr));
  return __builtin_bit_cast(bf16x4, r);
}

template <int N>
__device__ __forceinline__ void lds_wait_tr(bf16x4& a, bf16x4& b) {
  static_assert(N == 0 || N == 2 || N == 4, "lgkmcnt value");
  if constexpr (N == 0) asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a), "+v"(b));
  else if constexpr (N == 2) asm volatile("s_waitcnt lgkmcnt(2)" : "+v"(a), "+v"(b));
  else asm volatile("s_waitcnt lgkmcnt(4)" : "+v"(a), "+v"(b));
}

__device__ __forceinline__ bf16x8 cat8(const bf16x4& a, const bf16x4& b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Round eight fp32 to bf16 (nearest even) with v_cvt_pk_bf16_f32.
__device__ __forceinline__ bf16x8 to_bf16x8(float a0, float a1, float a2, float a3, float a4,
                                             float a5, float a6, float a7) {
  bf16x2 p0 = __builtin_convertvector((f32x2){a0, a1}, bf16x2);
  bf16x2 p1 = __builtin_convertvector((f32x2){a2, a3}, bf16x2);
  bf16x2 p2 = __builtin_convertvector((f32x2){a4, a5}, bf16x2);
  bf16x2 p3 = __builtin_convertvector((f32x2){a6, a7}, bf16x2);
  bf16x4 q0 = __builtin_shufflevector(p0, p1, 0, 1, 2, 3);
  bf16x4 q1 = __builtin_shufflevector(p2, p3, 0, 1, 2, 3);
  return cat8(q0, q1);
}

__device__ __forceinline__ bf16x4 to_bf16x4(float a0, float a1, float a2, float a3) {
  bf16x2 p0 = __builtin_convertvector((f32x2){a0, a1}, bf16x2);
  bf16x2 p1 = __builtin_convertvector((f32x2){a2, a3}, bf16x2);
  return __builtin_shufflevector(p0, p1, 0, 1, 2, 3);
}

__device__ __forceinline__ f16x4 to_f16x4(float a0, float a1, float a2, float a3) {
  return f16x4{(_Float16)a0, (_Float16)a1, (_Float16)a2, (_Float16)a3};
}

// Four consecutive output elements starting at element `elem` of `base`, stored
// in the output type `dtype` (uniform across the wave).
__device__ __forceinline__ void store_out4(void* base, int64_t elem, int dtype, float a0, float a1,
                                           float a2, float a3) {
  if (dtype == kOutF32)
    *reinterpret_cast<float4*>(static_cast<float*>(base) + elem) = make_float4(a0, a1, a2, a3);
  else if (dtype == kOutF16)
    *reinterpret_cast<f16x4*>(static_cast<_Float16*>(base) + elem) = to_f16x4(a0, a1, a2, a3);
  else
    *reinterpret_cast<bf16x4*>(static_cast<uint16_t*>(base) + elem) = to_bf16x4(a0, a1, a2, a3);
}

// Eight consecutive elements of a partial, widened to fp32.
template <int PART>
__device__ __forceinline__ void load8(const void* base, int64_t elem, float (&v)[8]) {
  if constexpr (PART == kOutF32) {
    const float4* src = reinterpret_cast<const float4*>(static_cast<const float*>(base) + elem);
    const float4 a = src[0], b = src[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else if constexpr (PART == kOutF16) {
    const f16x8 h = *reinterpret_cast<const f16x8*>(static_cast<const _Float16*>(base) + elem);
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = (float)h[j];
  } else {
    const uint4 u4 = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + elem);
    const uint32_t u[4] = {u4.x, u4.y, u4.z, u4.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = __builtin_bit_cast(float, u[j] << 16);
      v[2 * j + 1] = __builtin_bit_cast(float, u[j] & 0xffff0000u);
    }
  }
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __builtin_bit_cast(float, (uint32_t)b << 16);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Workgroup barrier for LDS data: this wave's LDS reads and writes retire
// (lgkmcnt) before the barrier, and the memory clobber keeps the compiler from
// moving memory accesses across it.  Unlike __syncthreads() it does not wait
// for vector-memory operations, so LDS-DMA tile prefetches stay in flight; a
// tile's own DMA is waited for with an explicit vmcnt before the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// s_waitcnt immediate that waits until at most n vector-memory operations of
// this wave are outstanding (expcnt and lgkmcnt left alone).
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }
// s_waitcnt operand waiting for LDS / scalar-memory operations only (lgkmcnt <= n)
constexpr int waitcnt_lgkm(int n) { return 0xF | (0x7 << 4) | ((n & 0xF) << 8) | (0x3 << 14); }

__device__ __forceinline__ int load_uniform_i32(const int32_t* ptr) {
  return *(const __attribute__((address_space(4))) int32_t*)ptr;
}

// Workgroups are handed to the 8 XCDs round-robin by linear id (id % 8), and
// each XCD has its own L2.  This bijection gives XCD x the contiguous range of
// logical ids [x * q + min(x, r), ...) (q = n / 8, r = n % 8), so neighbouring
// logical work items, which read overlapping K/V, share one L2.
constexpr int kNumXcd = 8;
__device__ __forceinline__ int xcd_logical_id(int lin, int n) {
  const int xcd = lin % kNumXcd, local = lin / kNumXcd;
  const int q = n / kNumXcd, r = n % kNumXcd;
  return xcd < r ? xcd * (q + 1) + local : r * (q + 1) + (xcd - r) * q + local;
}

__device__ __forceinline__ float swap_halves(float x) {  // value of lane l ^ 32
  return __shfl_xor(x, 32, kWave);
}

// max / sum of the values of lanes l and l ^ 32, in every lane, with one
// v_permlane32_swap (a VALU instruction) instead of an LDS permute.  The swap
// leaves the low half's value in one register and the high half's in the
// other in both halves, so both lanes of a pair get the same result, added in
// the same order.
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float wave_max(float x) {
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, kWave));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, kWave);
  return x;
}

}  // namespace psw
