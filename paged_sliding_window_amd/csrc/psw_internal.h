// Launchers behind the C ABI (implemented next to their kernels).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "debug_checks.h"
#include "mask_bounds.h"

namespace psw {

// Everything the attention kernels read, already validated on the host.
struct AttnParams {
  const uint16_t* q;
  const uint16_t* k_cache;
  const uint16_t* v_cache;  // == k_cache for the latent layout
  const int32_t* block_table;
  const int32_t* query_start_loc;
  const int32_t* seq_lens;
  const int32_t* mm_ranges;   // nullptr: no images
  const int32_t* key_ranges;  // nullptr: one split over [0, seq_len)
  void* out;
  float* lse;
  int num_seqs, num_tokens, num_q_heads, num_kv_heads, queries_per_kv;
  int head_dim_qk, head_dim_v;
  int block_size_log2, block_table_stride, max_mm_ranges;
  MaskGeom geom;
  int num_splits;
  int out_dtype;  // kOutBf16, kOutF32 or kOutF16 (the psw_dtype values)
  float scale_log2;  // softmax scale * log2(e)
  // Cache write fused into the prefill (psw_swa_mm_attention_kv_write); k_new
  // is nullptr for the plain call.  New rows are [num_tokens, num_kv_heads, D].
  const uint16_t* k_new;
  const uint16_t* v_new;
  const int32_t* slot_mapping;
  uint16_t* k_cache_w;  // the caches, written (same memory as k_cache / v_cache)
  uint16_t* v_cache_w;
  int64_t num_slots;
};

hipError_t launch_slot_mapping(const int32_t* qsl, int num_reqs, const int64_t* positions,
                               int num_tokens, const int32_t* block_table, int stride,
                               int block_size, int32_t* out, int max_num_tokens,
                               hipStream_t stream);

// Context-parallel rank / circular-cache variant (geometry validated by the caller).
hipError_t launch_slot_mapping_cp(const int32_t* qsl, int num_reqs, const int64_t* positions,
                                  int num_tokens, const int32_t* block_table, int stride,
                                  int block_size, int kv_cache_block_size, int cp_world_size,
                                  int cp_rank, int cp_interleave, bool circular, int32_t* out,
                                  int max_num_tokens, hipStream_t stream);

hipError_t launch_kv_cache_write(const uint16_t* k_new, const uint16_t* v_new,
                                 const int32_t* slots, int num_tokens, int num_kv_heads,
                                 int head_dim_k, int head_dim_v, uint16_t* k_cache,
                                 uint16_t* v_cache, int64_t num_slots, hipStream_t stream);

constexpr int kMaxPartials = 64;
struct CombineArgs {
  const void* out[kMaxPartials];
  const float* lse[kMaxPartials];
};
hipError_t launch_lse_combine(const CombineArgs& parts, int num_partials, int partial_dtype,
                              int64_t num_rows, int head_dim_v, void* out, int out_dtype,
                              float* out_lse, hipStream_t stream);

// V-up projection: out[t, h, :] = x[t, h, :] @ w[h] (bf16 in and out, fp32 accumulation).
bool vup_supported(int kv_lora_rank, int v_head_dim);
// LSE combine of P <= combine_vup_max_partials() latent partials followed by the
// V-up projection, in one launch (merged rows optional, LSEs optional).
int combine_vup_max_partials();
hipError_t launch_combine_vup(const CombineArgs& parts, int num_partials, int partial_dtype,
                              const uint16_t* w, uint16_t* out, float* out_lse, uint16_t* merged,
                              int num_tokens, int num_heads, int kv_lora_rank, int v_head_dim,
                              hipStream_t stream);
hipError_t launch_vup_projection(const uint16_t* x, const uint16_t* w, uint16_t* out,
                                 int num_tokens, int num_heads, int kv_lora_rank, int v_head_dim,
                                 hipStream_t stream);

hipError_t launch_tile_bounds(const int32_t* qsl, const int32_t* seq_lens,
                              const int32_t* mm_ranges, int max_mm_ranges, int queries_per_kv,
                              MaskGeom geom, int tile, int block_m, int block_q,
                              const int32_t* seq_idx, const int32_t* q_block_idx, int n,
                              int32_t* out, hipStream_t stream);

// Returns hipErrorInvalidValue (not launched) when no kernel fits the shape.
bool prefill_supported(int head_dim_qk, int head_dim_v, int queries_per_kv, bool latent);
hipError_t launch_attention_prefill(const AttnParams& p, hipStream_t stream);

bool decode_supported(const AttnParams& p);
// Bytes of device workspace the latent decode needs on the current device.
int64_t decode_workspace_bytes(const AttnParams& p);
hipError_t launch_attention_decode(const AttnParams& p, void* workspace, hipStream_t stream);

// Device scratch of the allocation-free entry point (one per device, this many
// bytes): its address on the current device, looked up on first use.
constexpr int64_t kScratchBytes = (int64_t)66 << 20;
hipError_t scratch_device_ptr(void** ptr);

// Failed debug checks recorded on the current device by each translation
// unit's kernels since the last call, then cleared (0 outside PSW_DEBUG
// builds); the caller synchronises the device first.
hipError_t debug_take_prefill(unsigned* out);
hipError_t debug_take_decode(unsigned* out);
hipError_t debug_take_slot_mapping(unsigned* out);
hipError_t debug_take_kv_write(unsigned* out);

}  // namespace psw
