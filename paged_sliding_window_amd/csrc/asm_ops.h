// Instruction-level helpers shared by the attention kernels: compile-time
// loops, LDS reads the compiler does not track, and MFMAs whose accumulators
// live in AGPRs (or in VGPRs) under inline assembly.
#pragma once
#include <utility>

#include "device_common.h"

namespace psw {

// Compile-time loop: f(std::integral_constant<int, I>) for I = 0 .. N-1.
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// LDS reads the compiler does not track (with the builtins it cannot tell them
// apart from LDS-DMA writes still in flight and waits for every outstanding
// vector-memory load first): the result may be consumed only after
// lds_wait<N>() on it, which waits until at most N LDS operations of this wave
// are outstanding (they complete in issue order; outstanding scalar loads only
// make the wait longer) and ties the registers to that point.
template <int OFF>
__device__ __forceinline__ bf16x8 lds_read_b128_at(uint32_t addr) {
  bf16x8 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  return r;
}
template <int OFF>
__device__ __forceinline__ bf16x4 lds_read_tr4_at(uint32_t addr) {
  i16x4 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  return __builtin_bit_cast(bf16x4, r);
}
template <int N>
__device__ __forceinline__ void lds_wait(bf16x8& a) {
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(a) : "i"(N < 15 ? N : 15));
}
template <int N>
__device__ __forceinline__ void lds_wait(bf16x4& a, bf16x4& b) {
  asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(a), "+v"(b) : "i"(N < 15 ? N : 15));
}

// Output accumulators in AGPRs: block b (32 output columns x 32 rows or
// heads, the MFMA's 16 result registers) is a[16 b .. 16 b + 15].  Only the inline
// assembly below writes or reads them: a kernel using them keeps its other
// values below 256 VGPRs, so the compiler allocates no AGPR of its own (a
// build check verifies this), and the clobber of a255 makes it reserve all
// 256.  The compiler does not see the MFMAs inside the assembly, so the wait
// states it would insert are written out: two before an MFMA whose sources a
// VALU instruction may just have written, and 16 or more between an MFMA and
// a VALU read of its result.
template <int FIRST, int COUNT>
__device__ __forceinline__ void oacc_zero() {
  asm volatile(
      ".set psw_r, %0\n.rept %1\n"
      "v_accvgpr_write_b32 a[psw_r], 0\n"
      ".set psw_r, psw_r + 1\n.endr" :: "i"(FIRST), "i"(COUNT) : "a255");
}
template <int B>
__device__ __forceinline__ void oacc_mfma(const bf16x8& a, const bf16x8& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 a[%2:%3], %0, %1, a[%2:%3]"
               :: "v"(a), "v"(b), "i"(16 * B), "i"(16 * B + 15));
}
__device__ __forceinline__ void oacc_settle() {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" ::: "memory");
}
// accumulators FIRST .. FIRST + COUNT - 1 times alpha, two at a time
template <int FIRST, int COUNT>
__device__ __forceinline__ void oacc_scale(float alpha) {
  static_assert(COUNT % 2 == 0, "pairs of accumulators");
  float t0, t1;
  asm volatile(
      "s_nop 7\n\ts_nop 7\n\ts_nop 3\n"
      ".set psw_r, %3\n.rept %4\n"
      "v_accvgpr_read_b32 %0, a[psw_r]\n"
      "v_accvgpr_read_b32 %1, a[psw_r + 1]\n"
      "v_mul_f32 %0, %0, %2\n"
      "v_mul_f32 %1, %1, %2\n"
      "v_accvgpr_write_b32 a[psw_r], %0\n"
      "v_accvgpr_write_b32 a[psw_r + 1], %1\n"
      ".set psw_r, psw_r + 2\n.endr"
      : "=&v"(t0), "=&v"(t1)
      : "v"(alpha), "i"(FIRST), "i"(COUNT / 2));
}
// accumulator block B as 16 floats; the memory clobber keeps the stores of
// earlier blocks before these reads
template <int B>
__device__ __forceinline__ f32x16 oacc_get() {
  f32x16 v;
  static_for<16>([&](auto ii) {
    constexpr int i = decltype(ii)::value;
    float x;
    asm volatile("v_accvgpr_read_b32 %0, a[%1]" : "=v"(x) : "i"(16 * B + i) : "memory");
    v[i] = x;
  });
  return v;
}

// MFMAs as inline assembly with the accumulator in VGPRs (the builtin could
// put it in AGPRs beside the output accumulators).  The compiler does not see
// these as MFMAs, so the wait states it would insert are written here: two
// before each MFMA (a VALU write of a source operand), and after the chain
// enough for the VALU to read the result.  The s_nop before a dependent MFMA
// overlaps the previous MFMA's execution.
__device__ __forceinline__ f32x16 mfma32_vgpr_first(const bf16x8& a, const bf16x8& b) {
  f32x16 d;
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0"
               : "=&v"(d) : "v"(a), "v"(b));
  return d;
}
__device__ __forceinline__ void mfma32_vgpr(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
               : "+v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_vgpr_settle(f32x16& d) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(d));
}

}  // namespace psw
