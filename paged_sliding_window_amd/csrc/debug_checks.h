// Debug checks of the kernels' internal invariants (builds with PSW_DEBUG).
//
// PSW_DCHECK(id, cond) sets bit `id` of this translation unit's device word
// when `cond` is false and lets the kernel go on: a trap would end the
// process's GPU work, while a recorded bit is read back (and cleared) by
// psw_debug_take_failures() after the work is done.  The bit is set with a
// vector atomic OR.  Release builds compile every check away (`cond` is not
// evaluated), so a check must have no side effects.
//
// Check ids (bit numbers), each an invariant that holds for inputs meeting
// the C ABI's preconditions:
//   0  prefill: the workgroup's tile range [t_lo, t_hi) lies inside the
//      request's keys
//   1  prefill: every block-table entry a tile's loads use is a valid block
//      (>= 0)
//   2  prefill: a valid row's allowed keys lie in [0, seq_len)
//   3  prefill, unless the tile loop is cut into segmented splits: every valid
//      row's allowed keys lie inside the workgroup's tile range (the tile
//      bounds never cut an allowed key)
//   4  prefill with the fused cache write: a slot other than -1 lies in
//      [0, num_slots)
//   8  decode: an item's allowed keys and tile range lie inside its request
//   9  decode: every block-table entry a tile's loads use is a valid block
//   10 decode: a piece of a shared item lies inside the workspace's pieces
//   11 decode: the per-item tile prefix never decreases
//   16 slot mapping: the request found for a token holds that token
//   17 KV write: a slot other than -1 lies in [0, num_slots)
#pragma once
#include <hip/hip_runtime.h>

#ifdef PSW_DEBUG
namespace psw {
static __device__ unsigned int debug_word;
}
#define PSW_DCHECK(id, cond)                                                              \
  do {                                                                                    \
    if (!(cond)) __hip_atomic_fetch_or(&::psw::debug_word, 1u << (id), __ATOMIC_RELAXED, \
                                       __HIP_MEMORY_SCOPE_AGENT);                         \
  } while (0)
// Host function `name`: this translation unit's word on the current device,
// then cleared (the caller has synchronised the device).
#define PSW_DEBUG_TAKE(name)                                                               \
  hipError_t name(unsigned* out) {                                                         \
    unsigned v = 0, zero = 0;                                                              \
    hipError_t e = hipMemcpyFromSymbol(&v, HIP_SYMBOL(::psw::debug_word), sizeof v, 0,     \
                                       hipMemcpyDeviceToHost);                             \
    if (e == hipSuccess)                                                                   \
      e = hipMemcpyToSymbol(HIP_SYMBOL(::psw::debug_word), &zero, sizeof zero, 0,          \
                            hipMemcpyHostToDevice);                                        \
    *out = v;                                                                              \
    return e;                                                                              \
  }
#else
#define PSW_DCHECK(id, cond) \
  do {                       \
  } while (0)
#define PSW_DEBUG_TAKE(name)         \
  hipError_t name(unsigned* out) {   \
    *out = 0;                        \
    return hipSuccess;               \
  }
#endif
