// extern "C" entry points of libpsw.so: host-side validation of scalars and
// pointer presence, then one or more kernel launches on the caller's stream.
// Nothing here allocates or synchronises.
#include <cmath>
#include <cstdio>
#include <cstring>
#include <cstdarg>
#include <mutex>

#include "psw.h"
#include "device_common.h"
#include "psw_internal.h"

namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_last_error[0] = '\0';
  return PSW_OK;
}

int check_hip(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(PSW_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool is_pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }
bool known_dtype(int d) { return d == PSW_BF16 || d == PSW_F32 || d == PSW_F16; }
static_assert(PSW_BF16 == psw::kOutBf16 && PSW_F32 == psw::kOutF32 && PSW_F16 == psw::kOutF16,
              "kernel dtype codes are the ABI's");
int log2i(int v) {
  int l = 0;
  while ((1 << l) < v) ++l;
  return l;
}

}  // namespace

extern "C" {

int psw_abi_version(void) { return PSW_ABI_VERSION; }

const char* psw_status_string(int status) {
  switch (status) {
    case PSW_OK: return "ok";
    case PSW_ERR_INVALID: return "invalid argument";
    case PSW_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case PSW_ERR_HIP: return "HIP launch error";
    default: return "unknown status";
  }
}

const char* psw_last_error(void) { return g_last_error; }

int psw_slot_mapping(const int32_t* query_start_loc, int32_t num_reqs, const int64_t* positions,
                     int32_t num_tokens, const int32_t* block_table, int32_t block_table_stride,
                     int32_t block_size, int32_t* slot_mapping, int32_t max_num_tokens,
                     void* stream) {
  if (num_reqs < 0 || num_tokens < 0)
    return fail(PSW_ERR_INVALID, "num_reqs (%d) and num_tokens (%d) must be >= 0", num_reqs,
                num_tokens);
  if (block_table_stride < 1 || block_size < 1)
    return fail(PSW_ERR_INVALID, "block_table_stride (%d) and block_size (%d) must be >= 1",
                block_table_stride, block_size);
  if (max_num_tokens < num_tokens)
    return fail(PSW_ERR_INVALID, "max_num_tokens (%d) < num_tokens (%d)", max_num_tokens,
                num_tokens);
  if (max_num_tokens > 0 && slot_mapping == nullptr)
    return fail(PSW_ERR_INVALID, "slot_mapping is NULL");
  if (num_tokens > 0 && (positions == nullptr || query_start_loc == nullptr ||
                         (num_reqs > 0 && block_table == nullptr)))
    return fail(PSW_ERR_INVALID, "query_start_loc, positions and block_table are required");
  return check_hip(psw::launch_slot_mapping(query_start_loc, num_reqs, positions, num_tokens,
                                            block_table, block_table_stride, block_size,
                                            slot_mapping, max_num_tokens, (hipStream_t)stream),
                   "slot_mapping");
}

int psw_slot_mapping_cp(const int32_t* query_start_loc, int32_t num_reqs,
                        const int64_t* positions, int32_t num_tokens,
                        const int32_t* block_table, int32_t block_table_stride,
                        int32_t block_size, int32_t kv_cache_block_size,
                        int32_t cp_world_size, int32_t cp_rank, int32_t cp_interleave,
                        int32_t circular, int32_t* slot_mapping, int32_t max_num_tokens,
                        void* stream) {
  if (num_reqs < 0 || num_tokens < 0)
    return fail(PSW_ERR_INVALID, "num_reqs (%d) and num_tokens (%d) must be >= 0", num_reqs,
                num_tokens);
  if (block_table_stride < 1 || block_size < 1)
    return fail(PSW_ERR_INVALID, "block_table_stride (%d) and block_size (%d) must be >= 1",
                block_table_stride, block_size);
  if (kv_cache_block_size < 1 || kv_cache_block_size % block_size != 0)
    return fail(PSW_ERR_INVALID, "kv_cache_block_size (%d) must be a positive multiple of "
                "block_size (%d)", kv_cache_block_size, block_size);
  if (cp_world_size < 1 || cp_rank < 0 || cp_rank >= cp_world_size)
    return fail(PSW_ERR_INVALID, "cp_rank (%d) must lie in [0, cp_world_size = %d)", cp_rank,
                cp_world_size);
  if (cp_interleave < 1 || kv_cache_block_size % cp_interleave != 0)
    return fail(PSW_ERR_INVALID, "cp_interleave (%d) must divide kv_cache_block_size (%d)",
                cp_interleave, kv_cache_block_size);
  if ((int64_t)kv_cache_block_size * cp_world_size >= ((int64_t)1 << 31))
    return fail(PSW_ERR_INVALID, "kv_cache_block_size * cp_world_size must be below 2^31");
  if (circular != 0 && circular != 1)
    return fail(PSW_ERR_INVALID, "circular must be 0 or 1, got %d", circular);
  if (circular && cp_world_size != 1)
    return fail(PSW_ERR_INVALID, "a circular cache is not allowed with cp_world_size %d > 1",
                cp_world_size);
  if (max_num_tokens < num_tokens)
    return fail(PSW_ERR_INVALID, "max_num_tokens (%d) < num_tokens (%d)", max_num_tokens,
                num_tokens);
  if (max_num_tokens > 0 && slot_mapping == nullptr)
    return fail(PSW_ERR_INVALID, "slot_mapping is NULL");
  if (num_tokens > 0 && (positions == nullptr || query_start_loc == nullptr ||
                         (num_reqs > 0 && block_table == nullptr)))
    return fail(PSW_ERR_INVALID, "query_start_loc, positions and block_table are required");
  return check_hip(psw::launch_slot_mapping_cp(query_start_loc, num_reqs, positions, num_tokens,
                                               block_table, block_table_stride, block_size,
                                               kv_cache_block_size, cp_world_size, cp_rank,
                                               cp_interleave, circular != 0, slot_mapping,
                                               max_num_tokens, (hipStream_t)stream),
                   "slot_mapping_cp");
}

int psw_kv_cache_write(const void* k_new, const void* v_new, const int32_t* slot_mapping,
                       int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim_k,
                       int32_t head_dim_v, void* k_cache, void* v_cache, int64_t num_slots,
                       void* stream) {
  if (num_tokens < 0 || num_kv_heads < 1 || num_slots < 0)
    return fail(PSW_ERR_INVALID, "bad counts: num_tokens %d num_kv_heads %d num_slots %lld",
                num_tokens, num_kv_heads, (long long)num_slots);
  if (head_dim_k < 8 || head_dim_k % 8 != 0)
    return fail(PSW_ERR_INVALID, "head_dim_k (%d) must be a positive multiple of 8", head_dim_k);
  if ((v_new == nullptr) != (v_cache == nullptr))
    return fail(PSW_ERR_INVALID, "v_new and v_cache must both be given or both be NULL");
  if (v_new != nullptr && (head_dim_v < 8 || head_dim_v % 8 != 0))
    return fail(PSW_ERR_INVALID, "head_dim_v (%d) must be a positive multiple of 8", head_dim_v);
  if (num_tokens > 0 && (k_new == nullptr || slot_mapping == nullptr || k_cache == nullptr))
    return fail(PSW_ERR_INVALID, "k_new, slot_mapping and k_cache are required");
  return check_hip(psw::launch_kv_cache_write(
                       static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new),
                       slot_mapping, num_tokens, num_kv_heads, head_dim_k, head_dim_v,
                       static_cast<uint16_t*>(k_cache), static_cast<uint16_t*>(v_cache),
                       num_slots, (hipStream_t)stream),
                   "kv_cache_write");
}

static int fill_geometry(const psw_attn_args* a, psw::AttnParams& p, bool need_tensors,
                         bool need_pointers = true) {
  if (a == nullptr) return fail(PSW_ERR_INVALID, "args is NULL");
  if (a->struct_size != (int32_t)sizeof(psw_attn_args))
    return fail(PSW_ERR_INVALID, "struct_size %d != sizeof(psw_attn_args) %d", a->struct_size,
                (int)sizeof(psw_attn_args));
  if (a->num_seqs < 0 || a->num_tokens < 0 || a->num_q_heads < 1 || a->num_kv_heads < 1)
    return fail(PSW_ERR_INVALID, "bad counts: seqs %d tokens %d q_heads %d kv_heads %d",
                a->num_seqs, a->num_tokens, a->num_q_heads, a->num_kv_heads);
  if (a->num_q_heads % a->num_kv_heads != 0)
    return fail(PSW_ERR_INVALID, "num_q_heads %d is not a multiple of num_kv_heads %d",
                a->num_q_heads, a->num_kv_heads);
  if (a->max_mm_ranges < 0 || (a->mm_ranges != nullptr && a->max_mm_ranges == 0))
    return fail(PSW_ERR_INVALID, "max_mm_ranges %d inconsistent with mm_ranges", a->max_mm_ranges);
  if (a->chunk_lookback >= 0 && a->chunk_size < 1)
    return fail(PSW_ERR_INVALID, "chunk_size %d must be >= 1 with chunk_lookback %d",
                a->chunk_size, a->chunk_lookback);
  if (need_pointers && a->num_seqs > 0 && (a->query_start_loc == nullptr || a->seq_lens == nullptr))
    return fail(PSW_ERR_INVALID, "query_start_loc and seq_lens are required");
  if (need_tensors) {
    if (a->head_dim_qk < 16 || a->head_dim_v < 16)
      return fail(PSW_ERR_INVALID, "head dims %d/%d too small", a->head_dim_qk, a->head_dim_v);
    if (!is_pow2(a->block_size))
      return fail(PSW_ERR_INVALID, "block_size %d must be a power of two", a->block_size);
    if (a->block_table_stride < 1)
      return fail(PSW_ERR_INVALID, "block_table_stride %d must be >= 1", a->block_table_stride);
    if (a->num_splits < 1)
      return fail(PSW_ERR_INVALID, "num_splits %d must be >= 1", a->num_splits);
    if (!known_dtype(a->out_dtype))
      return fail(PSW_ERR_INVALID, "out_dtype %d unknown", a->out_dtype);
    if (!(a->scale > 0.f) || !std::isfinite(a->scale))
      return fail(PSW_ERR_INVALID, "scale must be finite and > 0");
    if (need_pointers && a->num_tokens > 0 && (a->q == nullptr || a->k_cache == nullptr ||
                              a->block_table == nullptr || a->out == nullptr))
      return fail(PSW_ERR_INVALID, "q, k_cache, block_table and out are required");
  }
  p.q = static_cast<const uint16_t*>(a->q);
  p.k_cache = static_cast<const uint16_t*>(a->k_cache);
  p.v_cache = a->v_cache ? static_cast<const uint16_t*>(a->v_cache) : p.k_cache;
  p.block_table = a->block_table;
  p.query_start_loc = a->query_start_loc;
  p.seq_lens = a->seq_lens;
  p.mm_ranges = a->max_mm_ranges > 0 ? a->mm_ranges : nullptr;
  p.key_ranges = a->key_ranges;
  p.out = a->out;
  p.lse = a->lse;
  p.num_seqs = a->num_seqs;
  p.num_tokens = a->num_tokens;
  p.num_q_heads = a->num_q_heads;
  p.num_kv_heads = a->num_kv_heads;
  p.queries_per_kv = a->num_q_heads / a->num_kv_heads;
  p.head_dim_qk = a->head_dim_qk;
  p.head_dim_v = a->head_dim_v;
  p.block_size_log2 = is_pow2(a->block_size) ? log2i(a->block_size) : 0;
  p.block_table_stride = a->block_table_stride;
  p.max_mm_ranges = a->max_mm_ranges;
  p.geom.window = a->window;
  p.geom.causal = a->causal ? 1 : 0;
  p.geom.chunk_size = a->chunk_size;
  p.geom.chunk_lookback = a->chunk_lookback;
  p.num_splits = a->num_splits;
  p.out_dtype = a->out_dtype;
  p.scale_log2 = a->scale * psw::kLog2eHost;
  return PSW_OK;
}

// Workspace the call needs for these arguments on the current device (0: none).
static int64_t workspace_needed(const psw_attn_args* args, const psw::AttnParams& p) {
  const bool latent = args->v_cache == nullptr;
  if (latent && psw::decode_supported(p) && p.num_tokens > 0 && p.num_seqs > 0)
    return psw::decode_workspace_bytes(p);
  return 0;
}

int psw_attention_workspace_size(const psw_attn_args* args, int64_t* bytes) {
  if (bytes == nullptr) return fail(PSW_ERR_INVALID, "bytes is NULL");
  psw::AttnParams p{};
  int st = fill_geometry(args, p, true, false);
  if (st != PSW_OK) return st;
  *bytes = workspace_needed(args, p);
  return ok();
}

}  // extern "C"

namespace {

// Host checks of one attention call; on PSW_OK, p holds its parameters, latent
// says which kernel family runs it and empty that there is nothing to launch.
// With caller_workspace false the call's workspace is the library's scratch
// instead of args->workspace (which is then ignored).
int prepare_attention(const psw_attn_args* args, psw::AttnParams& p, bool& latent, bool& empty,
                      int64_t& workspace_used, bool caller_workspace = true) {
  int st = fill_geometry(args, p, true);
  if (st != PSW_OK) return st;
  latent = args->v_cache == nullptr;
  empty = p.num_tokens == 0 || p.num_seqs == 0;
  workspace_used = 0;
  if (latent && args->key_ranges == nullptr && args->num_splits > 1)
    return fail(PSW_ERR_UNSUPPORTED, "segmented splits (num_splits %d without key_ranges) are "
                "for the prefill shapes; the latent decode balances its own work",
                args->num_splits);
  if (empty) return PSW_OK;
  const int64_t need = workspace_needed(args, p);
  if (!caller_workspace && need > psw::kScratchBytes)
    return fail(PSW_ERR_INVALID,
                "this call needs %lld bytes of scratch; the allocation-free entry point has "
                "%lld (fewer tokens or splits per call, or psw_swa_mm_attention with a "
                "workspace)", (long long)need, (long long)psw::kScratchBytes);
  if (caller_workspace && need > 0 &&
      (args->workspace == nullptr || args->workspace_bytes < need ||
       (reinterpret_cast<uintptr_t>(args->workspace) & 255) != 0))
    return fail(PSW_ERR_INVALID,
                "workspace of %lld bytes (256-byte aligned) required, got %lld at %p",
                (long long)need, (long long)args->workspace_bytes, args->workspace);
  workspace_used = need;
  if (latent && psw::decode_supported(p)) return PSW_OK;
  if (psw::prefill_supported(p.head_dim_qk, p.head_dim_v, p.queries_per_kv, latent)) return PSW_OK;
  return fail(PSW_ERR_UNSUPPORTED,
              "no kernel for head dims %d/%d, %d query heads per KV head, %s V",
              p.head_dim_qk, p.head_dim_v, p.queries_per_kv, latent ? "latent" : "separate");
}

// Enqueues a call that prepare_attention accepted, with `workspace` as its
// workspace (args->workspace, or the library's scratch).
int launch_prepared(const psw_attn_args* args, const psw::AttnParams& p, bool latent,
                    hipStream_t stream, void* workspace) {
  if (latent && psw::decode_supported(p))
    return check_hip(psw::launch_attention_decode(p, workspace, stream), "attention(decode)");
  return check_hip(psw::launch_attention_prefill(p, stream), "attention(prefill)");
}

int launch_prepared(const psw_attn_args* args, const psw::AttnParams& p, bool latent,
                    hipStream_t stream) {
  return launch_prepared(args, p, latent, stream, args->workspace);
}

}  // namespace

extern "C" {

int psw_swa_mm_attention(const psw_attn_args* args, void* stream) {
  psw::AttnParams p{};
  bool latent = false, empty = false;
  int64_t ws = 0;
  int st = prepare_attention(args, p, latent, empty, ws);
  if (st != PSW_OK) return st;
  if (empty) return ok();
  return launch_prepared(args, p, latent, (hipStream_t)stream);
}

int psw_swa_mm_attention_noalloc(const psw_attn_args* args, void* stream) {
  psw::AttnParams p{};
  bool latent = false, empty = false;
  int64_t need = 0;
  int st = prepare_attention(args, p, latent, empty, need, /*caller_workspace=*/false);
  if (st != PSW_OK) return st;
  if (empty) return ok();
  void* scratch = nullptr;
  if (need > 0 && (st = check_hip(psw::scratch_device_ptr(&scratch), "scratch address")) != PSW_OK)
    return st;
  return launch_prepared(args, p, latent, (hipStream_t)stream, scratch);
}

int psw_swa_mm_attention_kv_write(const psw_attn_args* args, const void* k_new,
                                  const void* v_new, const int32_t* slot_mapping,
                                  int64_t num_slots, void* stream) {
  psw::AttnParams p{};
  bool latent = false, empty = false;
  int64_t ws = 0;
  int st = prepare_attention(args, p, latent, empty, ws);
  if (st != PSW_OK) return st;
  if (latent)
    return fail(PSW_ERR_UNSUPPORTED, "the fused cache write serves the prefill shapes; write a "
                "latent cache with psw_kv_cache_write");
  if (num_slots < 0) return fail(PSW_ERR_INVALID, "num_slots %lld < 0", (long long)num_slots);
  if (empty) return ok();
  if (k_new == nullptr || v_new == nullptr || slot_mapping == nullptr || args->v_cache == nullptr)
    return fail(PSW_ERR_INVALID, "k_new, v_new, slot_mapping and v_cache are required");
  p.k_new = static_cast<const uint16_t*>(k_new);
  p.v_new = static_cast<const uint16_t*>(v_new);
  p.slot_mapping = slot_mapping;
  p.k_cache_w = const_cast<uint16_t*>(p.k_cache);
  p.v_cache_w = const_cast<uint16_t*>(p.v_cache);
  p.num_slots = num_slots;
  return check_hip(psw::launch_attention_prefill(p, (hipStream_t)stream),
                   "attention(prefill, cache write)");
}

int psw_lse_combine(const void* const* partial_out, const float* const* partial_lse,
                    int32_t num_partials, int32_t partial_dtype, int64_t num_rows,
                    int32_t head_dim_v, void* out, int32_t out_dtype, float* out_lse,
                    void* stream) {
  if (num_partials < 1 || num_partials > psw::kMaxPartials)
    return fail(PSW_ERR_INVALID, "num_partials %d outside [1, %d]", num_partials,
                psw::kMaxPartials);
  if (num_rows < 0) return fail(PSW_ERR_INVALID, "num_rows < 0");
  if (head_dim_v < 8 || head_dim_v % 8 != 0 || head_dim_v > 1024)
    return fail(PSW_ERR_INVALID, "head_dim_v %d must be a multiple of 8 in [8, 1024]", head_dim_v);
  if (!known_dtype(partial_dtype) || !known_dtype(out_dtype))
    return fail(PSW_ERR_INVALID, "unknown dtype (partials %d, output %d)", partial_dtype,
                out_dtype);
  if (partial_out == nullptr || partial_lse == nullptr)
    return fail(PSW_ERR_INVALID, "partial pointer arrays are required");
  psw::CombineArgs parts{};
  for (int i = 0; i < num_partials; ++i) {
    if (num_rows > 0 && (partial_out[i] == nullptr || partial_lse[i] == nullptr))
      return fail(PSW_ERR_INVALID, "partial %d is NULL", i);
    parts.out[i] = partial_out[i];
    parts.lse[i] = partial_lse[i];
  }
  if (num_rows > 0 && out == nullptr) return fail(PSW_ERR_INVALID, "out is NULL");
  return check_hip(psw::launch_lse_combine(parts, num_partials, partial_dtype, num_rows,
                                           head_dim_v, out, out_dtype,
                                           out_lse, (hipStream_t)stream),
                   "lse_combine");
}

}  // extern "C"

namespace {

// Fork and join events of psw_decode_two_streams, made once per device on its
// first call there and kept until the process ends.  The mutex makes the
// record / wait sequence of one call atomic with respect to other threads.
constexpr int kMaxDevices = 64;
std::mutex g_events_mutex;
hipEvent_t g_fork[kMaxDevices], g_join[kMaxDevices];

int device_events(hipEvent_t& fork, hipEvent_t& join) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(PSW_ERR_HIP, "no current device below %d", kMaxDevices);
  if (g_fork[dev] == nullptr) {
    hipEvent_t f = nullptr, j = nullptr;
    hipError_t e = hipEventCreateWithFlags(&f, hipEventDisableTiming);
    if (e != hipSuccess) return check_hip(e, "hipEventCreateWithFlags");
    e = hipEventCreateWithFlags(&j, hipEventDisableTiming);
    if (e != hipSuccess) {
      (void)hipEventDestroy(f);
      return check_hip(e, "hipEventCreateWithFlags");
    }
    g_fork[dev] = f;
    g_join[dev] = j;
  }
  fork = g_fork[dev];
  join = g_join[dev];
  return PSW_OK;
}

bool overlap(const void* a, int64_t na, const void* b, int64_t nb) {
  if (a == nullptr || b == nullptr || na <= 0 || nb <= 0) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + (uintptr_t)nb && y < x + (uintptr_t)na;
}

}  // namespace

extern "C" {

int psw_decode_two_streams(const psw_attn_args* history, const psw_attn_args* current,
                           void* out, int32_t out_dtype, float* out_lse, void* main_stream,
                           void* side_stream) {
  psw::AttnParams ph{}, pc{};
  bool latent_h = false, latent_c = false, empty_h = false, empty_c = false;
  int64_t ws_h = 0, ws_c = 0;
  int st = prepare_attention(history, ph, latent_h, empty_h, ws_h);
  if (st != PSW_OK) return st;
  st = prepare_attention(current, pc, latent_c, empty_c, ws_c);
  if (st != PSW_OK) return st;
  if (history->num_tokens != current->num_tokens ||
      history->num_q_heads != current->num_q_heads || history->head_dim_v != current->head_dim_v)
    return fail(PSW_ERR_INVALID, "history and current disagree in tokens, query heads or V dim");
  if (history->out_dtype != current->out_dtype)
    return fail(PSW_ERR_INVALID, "history and current partials must share one dtype");
  if (!known_dtype(out_dtype))
    return fail(PSW_ERR_INVALID, "out_dtype %d unknown", out_dtype);
  const int num_partials = history->num_splits + current->num_splits;
  if (num_partials > psw::kMaxPartials)
    return fail(PSW_ERR_INVALID, "%d partials, at most %d", num_partials, psw::kMaxPartials);
  const int dv = history->head_dim_v;
  if (dv % 8 != 0 || dv > 1024)
    return fail(PSW_ERR_INVALID, "head_dim_v %d must be a multiple of 8 in [8, 1024]", dv);
  const int64_t rows = (int64_t)history->num_tokens * history->num_q_heads;
  if (rows == 0) return ok();
  if (history->num_seqs == 0 || current->num_seqs == 0)
    return fail(PSW_ERR_INVALID, "%d tokens but no sequences: the combine would read unwritten "
                "partials", history->num_tokens);
  if (out == nullptr) return fail(PSW_ERR_INVALID, "out is NULL");
  if (history->lse == nullptr || current->lse == nullptr)
    return fail(PSW_ERR_INVALID, "both calls must write their LSE");

  // partial s of a call: its out and lse advanced by s slices of rows
  const void* po[psw::kMaxPartials];
  const float* pl[psw::kMaxPartials];
  const size_t elt = history->out_dtype == PSW_F32 ? 4 : 2;
  int n = 0;
  for (const psw_attn_args* a : {history, current})
    for (int s = 0; s < a->num_splits; ++s, ++n) {
      po[n] = static_cast<const char*>(a->out) + (size_t)s * rows * dv * elt;
      pl[n] = a->lse + (size_t)s * rows;
    }

  hipStream_t ms = (hipStream_t)main_stream, ss = (hipStream_t)side_stream;
  std::lock_guard<std::mutex> lock(g_events_mutex);
  if (ms == ss) {
    if (!empty_h && (st = launch_prepared(history, ph, latent_h, ms)) != PSW_OK) return st;
    if (!empty_c && (st = launch_prepared(current, pc, latent_c, ms)) != PSW_OK) return st;
  } else {
    hipEvent_t fork = nullptr, join = nullptr;
    if ((st = device_events(fork, join)) != PSW_OK) return st;
    // One workspace used by both calls orders the current call after the
    // history call's use of it; separate workspaces let the two run together.
    const bool shared = overlap(history->workspace, ws_h, current->workspace, ws_c);
    if (!shared && (st = check_hip(hipEventRecord(fork, ms), "hipEventRecord")) != PSW_OK)
      return st;
    if (!empty_h && (st = launch_prepared(history, ph, latent_h, ms)) != PSW_OK) return st;
    if (shared && (st = check_hip(hipEventRecord(fork, ms), "hipEventRecord")) != PSW_OK)
      return st;
    if ((st = check_hip(hipStreamWaitEvent(ss, fork, 0), "hipStreamWaitEvent")) != PSW_OK)
      return st;
    if (!empty_c && (st = launch_prepared(current, pc, latent_c, ss)) != PSW_OK) return st;
    if ((st = check_hip(hipEventRecord(join, ss), "hipEventRecord")) != PSW_OK) return st;
    // with several ranks, the exchange of history partials is enqueued here on
    // the main stream, overlapping the current call on the side stream
    if ((st = check_hip(hipStreamWaitEvent(ms, join, 0), "hipStreamWaitEvent")) != PSW_OK)
      return st;
  }
  return psw_lse_combine(po, pl, num_partials, history->out_dtype, rows, dv, out, out_dtype,
                         out_lse, main_stream);
}

int psw_vup_projection(const void* x, const void* w_uv, void* out, int32_t num_tokens,
                       int32_t num_heads, int32_t kv_lora_rank, int32_t v_head_dim,
                       void* stream) {
  if (num_tokens < 0 || num_heads < 0 || kv_lora_rank < 1 || v_head_dim < 1)
    return fail(PSW_ERR_INVALID, "num_tokens %d, num_heads %d, kv_lora_rank %d, v_head_dim %d",
                num_tokens, num_heads, kv_lora_rank, v_head_dim);
  if (!psw::vup_supported(kv_lora_rank, v_head_dim))
    return fail(PSW_ERR_UNSUPPORTED, "kv_lora_rank %d / v_head_dim %d (need 128, 256 or 512 / a "
                "multiple of 64)", kv_lora_rank, v_head_dim);
  if (num_tokens > 0 && num_heads > 0 && (x == nullptr || w_uv == nullptr || out == nullptr))
    return fail(PSW_ERR_INVALID, "x, w_uv and out are required");
  return check_hip(psw::launch_vup_projection(static_cast<const uint16_t*>(x),
                                              static_cast<const uint16_t*>(w_uv),
                                              static_cast<uint16_t*>(out), num_tokens, num_heads,
                                              kv_lora_rank, v_head_dim, (hipStream_t)stream),
                   "vup_projection");
}

int psw_lse_combine_vup(const void* const* partial_out, const float* const* partial_lse,
                        int32_t num_partials, int32_t partial_dtype, const void* w_uv,
                        void* out, float* out_lse, void* merged, int32_t num_tokens,
                        int32_t num_heads, int32_t kv_lora_rank, int32_t v_head_dim,
                        void* stream) {
  const int max_p = psw::combine_vup_max_partials();
  if (num_partials < 1 || num_partials > max_p)
    return fail(PSW_ERR_INVALID, "num_partials %d outside [1, %d]", num_partials, max_p);
  if (num_tokens < 0 || num_heads < 0 || kv_lora_rank < 1 || v_head_dim < 1)
    return fail(PSW_ERR_INVALID, "num_tokens %d, num_heads %d, kv_lora_rank %d, v_head_dim %d",
                num_tokens, num_heads, kv_lora_rank, v_head_dim);
  if (!known_dtype(partial_dtype))
    return fail(PSW_ERR_INVALID, "unknown partial dtype %d", partial_dtype);
  if (!psw::vup_supported(kv_lora_rank, v_head_dim))
    return fail(PSW_ERR_UNSUPPORTED, "kv_lora_rank %d / v_head_dim %d (need 128, 256 or 512 / a "
                "multiple of 64)", kv_lora_rank, v_head_dim);
  const bool work = num_tokens > 0 && num_heads > 0;
  if (work && (partial_out == nullptr || partial_lse == nullptr))
    return fail(PSW_ERR_INVALID, "partial pointer arrays are required");
  psw::CombineArgs parts{};
  for (int i = 0; work && i < num_partials; ++i) {
    if (partial_out[i] == nullptr || partial_lse[i] == nullptr)
      return fail(PSW_ERR_INVALID, "partial %d is NULL", i);
    parts.out[i] = partial_out[i];
    parts.lse[i] = partial_lse[i];
  }
  if (work && (w_uv == nullptr || out == nullptr))
    return fail(PSW_ERR_INVALID, "w_uv and out are required");
  return check_hip(psw::launch_combine_vup(parts, num_partials, partial_dtype,
                                           static_cast<const uint16_t*>(w_uv),
                                           static_cast<uint16_t*>(out), out_lse,
                                           static_cast<uint16_t*>(merged), num_tokens, num_heads,
                                           kv_lora_rank, v_head_dim, (hipStream_t)stream),
                   "lse_combine_vup");
}

int psw_debug_take_failures(uint32_t* mask) {
  if (mask == nullptr) return fail(PSW_ERR_INVALID, "mask is NULL");
  *mask = 0;
#ifndef PSW_DEBUG
  return fail(PSW_ERR_UNSUPPORTED, "not a debug build (compile the library with PSW_DEBUG)");
#else
  if (const int st = check_hip(hipDeviceSynchronize(), "debug checks (synchronize)"); st != PSW_OK)
    return st;
  unsigned total = 0;
  for (auto take : {psw::debug_take_prefill, psw::debug_take_decode, psw::debug_take_slot_mapping,
                    psw::debug_take_kv_write}) {
    unsigned v = 0;
    if (const int st = check_hip(take(&v), "debug checks (read)"); st != PSW_OK) return st;
    total |= v;
  }
  *mask = total;
  return ok();
#endif
}

int psw_tile_bounds(const psw_attn_args* geometry, int32_t tile_size, int32_t block_m,
                    int32_t block_q, const int32_t* seq_idx, const int32_t* q_block_idx,
                    int32_t num_queries, int32_t* out, void* stream) {
  psw::AttnParams p{};
  int st = fill_geometry(geometry, p, false);
  if (st != PSW_OK) return st;
  if (tile_size < 1 || block_m < 1 || block_q < 1 || num_queries < 0)
    return fail(PSW_ERR_INVALID, "tile_size %d block_m %d block_q %d num_queries %d", tile_size,
                block_m, block_q, num_queries);
  if (num_queries > 0 && (seq_idx == nullptr || q_block_idx == nullptr || out == nullptr))
    return fail(PSW_ERR_INVALID, "seq_idx, q_block_idx and out are required");
  return check_hip(psw::launch_tile_bounds(p.query_start_loc, p.seq_lens, p.mm_ranges,
                                           p.max_mm_ranges, p.queries_per_kv, p.geom, tile_size,
                                           block_m, block_q, seq_idx, q_block_idx, num_queries,
                                           out, (hipStream_t)stream),
                   "tile_bounds");
}

}  // extern "C"
