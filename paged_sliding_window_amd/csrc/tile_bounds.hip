// Test export of the tile interval: vLLM PR #53147 summary, "Key source
// snippet" (a one-program helper kernel calls the production bounds routine
// and stores loop_lo, loop_hi and max_seq_prefix_len).  This kernel calls the
// same psw::tile_bounds the attention kernels use.
#include "psw_internal.h"

namespace psw {

__global__ void tile_bounds_kernel(const int32_t* __restrict__ qsl,
                                   const int32_t* __restrict__ seq_lens,
                                   const int32_t* __restrict__ mm_ranges, int max_mm_ranges,
                                   int queries_per_kv, MaskGeom geom, int tile, int block_m,
                                   int block_q, const int32_t* __restrict__ seq_idx,
                                   const int32_t* __restrict__ q_block_idx, int n,
                                   int32_t* __restrict__ out) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int s = seq_idx[i];
  const int query_len = qsl[s + 1] - qsl[s];
  const int seq_len = seq_lens[s];
  const int32_t* ranges = mm_ranges ? mm_ranges + (int64_t)s * max_mm_ranges * 2 : nullptr;
  const TileRange r = tile_bounds(seq_len - query_len, seq_len, query_len, q_block_idx[i], tile,
                                  block_m, block_q, queries_per_kv, geom, ranges, max_mm_ranges);
  out[3 * i] = r.lo;
  out[3 * i + 1] = r.hi;
  out[3 * i + 2] = r.max_seq_prefix_len;
}

hipError_t launch_tile_bounds(const int32_t* qsl, const int32_t* seq_lens,
                              const int32_t* mm_ranges, int max_mm_ranges, int queries_per_kv,
                              MaskGeom geom, int tile, int block_m, int block_q,
                              const int32_t* seq_idx, const int32_t* q_block_idx, int n,
                              int32_t* out, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(tile_bounds_kernel, dim3((n + 127) / 128), dim3(128), 0, stream, qsl,
                     seq_lens, mm_ranges, max_mm_ranges, queries_per_kv, geom, tile, block_m,
                     block_q, seq_idx, q_block_idx, n, out);
  return hipGetLastError();
}

}  // namespace psw
