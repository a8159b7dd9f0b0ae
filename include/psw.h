/*
 * psw.h - C ABI of libpsw.so: paged sliding-window attention with window-clamped
 * image (multimodal-prefix) ranges on AMD Instinct MI355X (gfx950).
 *
 * The pages this library follows (cited by title and section):
 *   [SWA-MM] vLLM PR #53147 summary (prhub.com.cn): sliding-window tile pruning
 *            restored under a window-clamped multimodal-prefix mask.
 *   [SLOT]   vllm-ascend Triton operator deep dive: _compute_slot_mapping_kernel
 *            (0539edu.com): logical position -> physical KV-cache slot.
 *   [DCP]    MLA DCP decode two-stream overlap and V-up fusion study notes,
 *            vllm-ascend PR #16977: history/current partials merged by LSE.
 *
 * Conventions shared by every entry point
 *   - Tensor arguments are DEVICE pointers into memory the caller owns and keeps
 *     alive until the enqueued work has finished. Arrays of pointers and the
 *     argument struct itself are HOST memory, read before the call returns.
 *   - `stream` is a hipStream_t (NULL: the legacy default stream). Every call
 *     only enqueues work on it: no device allocation, no host synchronisation
 *     (psw_decode_two_streams also creates two HIP events per device, once).
 *   - Scalars and pointer presence are validated on the host. When a check
 *     fails (PSW_ERR_INVALID, PSW_ERR_UNSUPPORTED) nothing is enqueued and
 *     outputs are untouched; PSW_ERR_HIP means a launch failed, possibly after
 *     earlier launches of the same call were enqueued. Device-resident data
 *     (offsets, positions, table entries) is NOT validated; the preconditions
 *     listed per call are the caller's to keep.
 *   - All tensors are dense and row-major (last dimension contiguous).
 *   - bf16 is IEEE bfloat16 (raw 16-bit patterns), fp32 is IEEE binary32.
 */
#ifndef PSW_H
#define PSW_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PSW_ABI_VERSION 8

enum psw_status {
  PSW_OK = 0,
  PSW_ERR_INVALID = -1,      /* bad scalar, missing pointer, inconsistent sizes */
  PSW_ERR_UNSUPPORTED = -2,  /* valid request this build has no kernel for */
  PSW_ERR_HIP = -3           /* a HIP launch failed; see psw_last_error() */
};

/* Element types of outputs and partials.  fp16 is IEEE binary16; conversions to
   bf16 and fp16 round to nearest even. */
enum psw_dtype { PSW_BF16 = 0, PSW_F32 = 1, PSW_F16 = 2 };

/* Returns PSW_ABI_VERSION. */
int psw_abi_version(void);

/* Static text for a status code. */
const char* psw_status_string(int status);

/* Detail of the last error raised on the calling host thread ("" if none). */
const char* psw_last_error(void);

/*
 * psw_slot_mapping - [SLOT] sections 1, 2, 4 and 5.1.
 * For request r and every token t in [query_start_loc[r], query_start_loc[r+1]):
 *     slot_mapping[t] = block_table[r * block_table_stride + pos / block_size] * block_size
 *                       + pos % block_size,          pos = positions[t]
 * and slot_mapping[t] = -1 (the pad slot id) for t in [num_tokens, max_num_tokens).
 * A token whose position is negative, whose logical block is >= block_table_stride,
 * or whose table entry is negative also gets -1.
 *   query_start_loc   int32 [num_reqs + 1], non-decreasing, query_start_loc[0] = 0,
 *                     query_start_loc[num_reqs] = num_tokens (device)
 *   positions         int64 [num_tokens], values below 2^31 (device)
 *   block_table       int32 [num_reqs, block_table_stride] (device)
 *   slot_mapping      int32 [max_num_tokens] output (device)
 * Errors: PSW_ERR_INVALID if num_reqs < 0, num_tokens < 0, block_table_stride < 1,
 * block_size < 1, max_num_tokens < num_tokens, or a needed pointer is NULL.
 */
int psw_slot_mapping(const int32_t* query_start_loc, int32_t num_reqs,
                     const int64_t* positions, int32_t num_tokens,
                     const int32_t* block_table, int32_t block_table_stride,
                     int32_t block_size, int32_t* slot_mapping, int32_t max_num_tokens,
                     void* stream);

/*
 * psw_slot_mapping_cp - [SLOT] section 3.1 (steps 1-5 of the context-parallel
 * interleave), section 2.2 (circular cache) and section 4.2 (parameters).
 * The slot mapping of ONE context-parallel rank: with V = kv_cache_block_size *
 * cp_world_size, a token at position pos >= 0 of request r belongs to rank
 *     ((pos % V) / cp_interleave) % cp_world_size
 * and, on its own rank, gets
 *     local   = ((pos % V) / (cp_world_size * cp_interleave)) * cp_interleave
 *               + (pos % V) % cp_interleave
 *     logical = (pos / V) * (kv_cache_block_size / block_size) + local / block_size
 *     slot    = block_table[r * block_table_stride + logical] * block_size
 *               + local % block_size
 * while tokens owned by another rank get -1.  With circular = 1 (a circular
 * cache; the page allows it only without context parallelism) every position
 * uses logical block 0 and offset pos % block_size.  As in psw_slot_mapping: a
 * negative position (or one of 2^31 and above), a logical block
 * >= block_table_stride or a negative table entry gives -1, and
 * [num_tokens, max_num_tokens) is filled with -1.  cp_world_size = 1 is exactly
 * psw_slot_mapping.
 *   query_start_loc, positions, block_table, slot_mapping: as psw_slot_mapping (device)
 *   kv_cache_block_size  tokens per physical KV block, a multiple of block_size
 *   cp_world_size, cp_rank  ranks of the context-parallel group and this rank
 *   cp_interleave        tokens per interleave segment, dividing kv_cache_block_size
 * Errors: PSW_ERR_INVALID as psw_slot_mapping, and if kv_cache_block_size is not a
 * positive multiple of block_size, cp_world_size < 1, cp_rank outside
 * [0, cp_world_size), cp_interleave < 1 or not a divisor of kv_cache_block_size,
 * kv_cache_block_size * cp_world_size >= 2^31, circular not 0 or 1, or circular
 * with cp_world_size > 1.
 */
int psw_slot_mapping_cp(const int32_t* query_start_loc, int32_t num_reqs,
                        const int64_t* positions, int32_t num_tokens,
                        const int32_t* block_table, int32_t block_table_stride,
                        int32_t block_size, int32_t kv_cache_block_size,
                        int32_t cp_world_size, int32_t cp_rank, int32_t cp_interleave,
                        int32_t circular, int32_t* slot_mapping, int32_t max_num_tokens,
                        void* stream);

/*
 * psw_kv_cache_write - [SLOT] section 1 (the slot id addresses a token's K/V
 * vector in the paged cache).  For every token t with slot s = slot_mapping[t] >= 0:
 *     k_cache[s, h, :] = k_new[t, h, :]   and   v_cache[s, h, :] = v_new[t, h, :]
 * Slots equal to -1 (padding) are skipped, and so is any slot outside
 * [0, num_slots), which a PSW_DEBUG build also records as failed check 17.
 *   k_new    bf16 [num_tokens, num_kv_heads, head_dim_k]      (device)
 *   v_new    bf16 [num_tokens, num_kv_heads, head_dim_v] or NULL (latent caches
 *            keep V inside K; then v_cache must be NULL too)     (device)
 *   k_cache  bf16 [num_slots, num_kv_heads, head_dim_k], slot = block * block_size
 *            + offset, i.e. the [num_blocks, block_size, heads, dim] layout (device)
 *   v_cache  bf16 [num_slots, num_kv_heads, head_dim_v] or NULL      (device)
 * Preconditions: every slot_mapping[t] is -1 or in [0, num_slots); no two tokens
 * share a slot.  head dims must be multiples of 8.
 */
int psw_kv_cache_write(const void* k_new, const void* v_new, const int32_t* slot_mapping,
                       int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim_k,
                       int32_t head_dim_v, void* k_cache, void* v_cache, int64_t num_slots,
                       void* stream);

/*
 * psw_vup_projection - MLA DCP decode notes (vllm-ascend PR #16977), "Terms"
 * (the latent attention output is projected back to each head's V dimension),
 * section 1.1 (the merged output is batch-major) and code block A (one
 * batched product per head, no transposes):
 *     out[t, h, :] = x[t, h, :] @ w_uv[h]          fp32 accumulation, bf16 result
 *   x     bf16 [num_tokens, num_heads, kv_lora_rank], contiguous (device) - e.g. the
 *         psw_lse_combine output viewed as [tokens, heads, rank]
 *   w_uv  bf16 [num_heads, kv_lora_rank, v_head_dim], contiguous (device)
 *   out   bf16 [num_tokens, num_heads, v_head_dim], contiguous (device), caller-owned
 * Errors: PSW_ERR_INVALID for negative sizes or a NULL pointer with work to do;
 * PSW_ERR_UNSUPPORTED unless kv_lora_rank is 128, 256 or 512 and v_head_dim is a
 * positive multiple of 64.
 */
int psw_vup_projection(const void* x, const void* w_uv, void* out, int32_t num_tokens,
                       int32_t num_heads, int32_t kv_lora_rank, int32_t v_head_dim,
                       void* stream);

/*
 * psw_lse_combine_vup - the two steps that end the latent decode in one launch:
 * the LSE merge of psw_lse_combine ([DCP] "Terms", section 1.1, code block D)
 * over P partial latent outputs, then the V-up projection of psw_vup_projection
 * ([DCP] "Terms", section 1.1, code block A) of the merged rows:
 *     x[t, h, :] = sum_p w_p O_p[t, h, :] / sum_p w_p,   out[t, h, :] = x[t, h, :] @ w_uv[h]
 * Results are bit for bit those of psw_lse_combine (bf16 output) followed by
 * psw_vup_projection on its output; the merged rows are only written when
 * merged != NULL.
 *   partial_out  host array of P device pointers, each partial_dtype
 *                [num_tokens, num_heads, kv_lora_rank] (PSW_BF16, PSW_F16 or PSW_F32)
 *   partial_lse  host array of P device pointers, each fp32 [num_tokens, num_heads]
 *   w_uv         bf16 [num_heads, kv_lora_rank, v_head_dim] (device)
 *   out          bf16 [num_tokens, num_heads, v_head_dim] (device), caller-owned
 *   out_lse      fp32 [num_tokens, num_heads] or NULL: LSE of each merged row
 *   merged       bf16 [num_tokens, num_heads, kv_lora_rank] or NULL: the merged rows
 * The partials are read in place.  Errors: PSW_ERR_INVALID for P outside
 * [1, 16], negative sizes, an unknown dtype or a NULL pointer with work to do;
 * PSW_ERR_UNSUPPORTED unless kv_lora_rank is 128, 256 or 512 and v_head_dim is
 * a positive multiple of 64.
 */
int psw_lse_combine_vup(const void* const* partial_out, const float* const* partial_lse,
                        int32_t num_partials, int32_t partial_dtype, const void* w_uv,
                        void* out, float* out_lse, void* merged, int32_t num_tokens,
                        int32_t num_heads, int32_t kv_lora_rank, int32_t v_head_dim,
                        void* stream);

/*
 * Arguments of psw_swa_mm_attention and psw_tile_bounds.
 *
 * Mask ([SWA-MM] "Implementation breakdown" items 1-2, "Key source snippet",
 * "Review highlights").  For request r, new token i has absolute position
 * q = context_len + i with context_len = seq_lens[r] - query_len.  Key k in
 * [0, seq_lens[r]) is allowed iff  base(q, k) OR image(q, k):
 *   base, causal != 0:  q - window + 1 <= k <= q  (window <= 0: k <= q)
 *   base, causal == 0:  |q - k| < window           (window <= 0: every key)
 *   chunk_lookback >= 0 further restricts base to k >= ((q / chunk_size) - chunk_lookback) * chunk_size
 *   image: some range [s, e] of the request (inclusive, absolute, used only when
 *          s < e) holds both q and k, and k >= q - window + 1 (when window > 0).
 * Query head h reads KV head h / (num_q_heads / num_kv_heads).
 * Output row (token t, head h) = softmax(scale * q . k over allowed keys) . v,
 * and lse = natural log of the sum of exp(scale * q . k) over those keys.
 * A row with no allowed key (within its split) gets output 0 and lse -inf.
 *
 * Split-KV partials ([DCP] sections 1.1 and 3.1): with key_ranges != NULL, split j
 * of request r only uses keys in [key_ranges[(j*num_seqs + r)*2], key_ranges[.. + 1]);
 * begin >= end is an empty split.  Partials are written to out[j] and lse[j] and are
 * merged afterwards with psw_lse_combine.
 */
typedef struct psw_attn_args {
  int32_t struct_size;            /* = sizeof(psw_attn_args) */
  const void* q;                  /* bf16 [num_tokens, num_q_heads, head_dim_qk] */
  const void* k_cache;            /* bf16 [num_slots, num_kv_heads, head_dim_qk] */
  const void* v_cache;            /* bf16 [num_slots, num_kv_heads, head_dim_v], or NULL:
                                     V = first head_dim_v columns of k_cache (latent) */
  const int32_t* block_table;     /* int32 [num_seqs, block_table_stride] */
  const int32_t* query_start_loc; /* int32 [num_seqs + 1] */
  const int32_t* seq_lens;        /* int32 [num_seqs], total keys incl. cached context */
  const int32_t* mm_ranges;       /* int32 [num_seqs, max_mm_ranges, 2] or NULL (no images) */
  const int32_t* key_ranges;      /* int32 [num_splits, num_seqs, 2], or NULL: one split, or
                                     segmented splits when num_splits > 1 (see below) */
  void* out;                      /* out_dtype [num_splits, num_tokens, num_q_heads, head_dim_v]:
                                     the final output, or the split partials in bf16, fp16
                                     or fp32 (normalised per split; LSE stays fp32) */
  float* lse;                     /* fp32 [num_splits, num_tokens, num_q_heads] or NULL */
  int32_t num_seqs, num_tokens, num_q_heads, num_kv_heads, head_dim_qk, head_dim_v;
  int32_t block_size, block_table_stride, max_mm_ranges;
  int32_t window;                 /* > 0: sliding window; <= 0: none */
  int32_t causal;                 /* 1: causal base; 0: bidirectional base */
  int32_t chunk_size, chunk_lookback;  /* chunk_lookback < 0: off */
  int32_t num_splits;             /* >= 1 */
  int32_t out_dtype;              /* PSW_BF16, PSW_F32 or PSW_F16 */
  float scale;                    /* softmax scale */
  void* workspace;                /* device scratch of >= psw_attention_workspace_size() bytes,
                                     256-byte aligned; may be NULL when that size is 0 */
  int64_t workspace_bytes;        /* size of workspace */
} psw_attn_args;

/*
 * psw_swa_mm_attention - paged attention under the mask above, visiting only the
 * KV tiles of each query block's union interval ([SWA-MM] "Key source snippet").
 * Supported: (head_dim_qk, head_dim_v) in {(64,64), (128,128), (256,256)} with
 * num_q_heads / num_kv_heads <= 128, and the latent decode shape (576, 512) with
 * v_cache == NULL and one KV head.  block_size must be a power of two.
 * Preconditions: query_start_loc non-decreasing from 0 to num_tokens;
 * 1 <= query_len <= seq_len for every request with new tokens; block-table
 * entries for every key below seq_len are valid blocks of the caches; image
 * ranges lie in [0, seq_len).
 * Splits.  With key_ranges, split s covers keys [key_ranges[s][r][0],
 * key_ranges[s][r][1]) of request r.  Without key_ranges and num_splits > 1
 * (segmented splits, [SWA-MM] "Key source snippet": the tile loop of a query
 * block is the unit of work), each query block's tile interval [lo, hi) is cut
 * into num_splits pieces of ceil((hi - lo) / num_splits) tiles, split s taking
 * the s-th (possibly empty); query blocks are 128 rows (128 / (num_q_heads /
 * num_kv_heads) positions of one request, rounded down) and tiles 32 keys, or 64
 * keys at head dim 128 when a row spans more than 1,536 keys (window <= 0, or
 * causal == 0 with window >= 769).  Either way each
 * split writes its partial output and LSE (-inf and a zero row where the split
 * sees no allowed key), and psw_lse_combine over the splits gives the unsplit
 * result.  Segmented splits serve the prefill shapes, whose work is one
 * workgroup per (query block, KV head, split); the latent decode balances its
 * own work and takes splits only as key ranges.
 * Errors: PSW_ERR_INVALID (struct_size mismatch, counts < 0, num_q_heads not a
 * multiple of num_kv_heads, block_size not a power of two, chunk_size < 1 with
 * chunk_lookback >= 0, num_splits < 1, NULL pointer, workspace missing,
 * misaligned or smaller than psw_attention_workspace_size()),
 * PSW_ERR_UNSUPPORTED (head dims / dtype combination without a kernel;
 * segmented splits with the latent decode shape).
 */
int psw_swa_mm_attention(const psw_attn_args* args, void* stream);

/*
 * psw_swa_mm_attention_noalloc - psw_swa_mm_attention for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops and
 * harnesses that forbid allocation.  Same arguments, kernels, results and
 * errors, except that the call's workspace (today only the latent decode uses
 * one) is a scratch array inside the library instead of args->workspace, which
 * is ignored with workspace_bytes; the caller still passes inputs and outputs.
 * The call itself allocates nothing (no hipMalloc / hipFree).
 * Limit: the scratch holds 66 MiB on each device, enough for the latent decode
 * with up to 128 query heads per workgroup on 256 CUs and up to 458,751
 * (token, split) items; a call needing more fails with PSW_ERR_INVALID and a
 * message, before anything is enqueued.  Every device the library runs on holds its copy of the
 * scratch from module load until the process ends; nothing in it needs
 * clearing between calls.  All calls on one device share that device's
 * scratch: calls that overlap in time on one device (two streams, two host
 * threads) race, and must be ordered by the caller.
 */
int psw_swa_mm_attention_noalloc(const psw_attn_args* args, void* stream);

/*
 * psw_swa_mm_attention_kv_write - the cache write of psw_kv_cache_write ([SLOT]
 * section 1) fused into a prefill call of psw_swa_mm_attention: one launch
 * that stores the new K and V rows in their cache slots and computes the
 * attention, reading the keys at or past each request's context length from
 * the new rows instead of the cache (so the attention never waits for the
 * write).  With the same arguments, the cache afterwards and the outputs are
 * exactly those of
 *     psw_kv_cache_write(k_new, v_new, slot_mapping, num_tokens, num_kv_heads,
 *                        head_dim_qk, head_dim_v, k_cache, v_cache, num_slots)
 *     psw_swa_mm_attention(args)
 * when the precondition below holds.
 *   args          as psw_swa_mm_attention, with separate K and V caches (the
 *                 prefill shapes); the caches args->k_cache / v_cache are written
 *   k_new, v_new  bf16 [num_tokens, num_kv_heads, head_dim] (device): row t holds
 *                 the key / value of new token t
 *   slot_mapping  int32 [num_tokens] (device): -1 (not stored) or a slot; slots
 *                 outside [0, num_slots) are skipped (a PSW_DEBUG build records
 *                 them as failed check 4)
 *   num_slots     rows of each cache (num_blocks * block_size)
 * Precondition (beyond psw_swa_mm_attention's): new token i of request r has
 * slot_mapping[query_start_loc[r] + i] = the slot the block table gives position
 * context_len + i, as psw_slot_mapping computes it, and no other token shares
 * it.  The kernel does not check this: a mapping that breaks it still writes
 * the cache as psw_kv_cache_write would, but the attention reads the new keys
 * from k_new / v_new, not from wherever the mapping put them.
 * Errors: psw_swa_mm_attention's; PSW_ERR_UNSUPPORTED for the latent decode
 * shape (its one new key per request is written with psw_kv_cache_write);
 * PSW_ERR_INVALID for num_slots < 0 or a NULL k_new, v_new or slot_mapping with
 * tokens to process.
 */
int psw_swa_mm_attention_kv_write(const psw_attn_args* args, const void* k_new,
                                  const void* v_new, const int32_t* slot_mapping,
                                  int64_t num_slots, void* stream);

/*
 * psw_attention_workspace_size - bytes of device workspace psw_swa_mm_attention
 * needs for these arguments on the calling thread's current device (stored in
 * *bytes; 0 when the call needs none).  Today only the latent decode uses it:
 * it balances all (token, split) items over one workgroup per CU and keeps the
 * per-item tile prefix and the pieces of items shared by several workgroups
 * there.  The size depends on num_tokens, num_splits, num_q_heads and the CU
 * count, not on device data.  The workspace holds no state between calls, but
 * two calls that overlap in time must not share one.
 * Errors: as psw_swa_mm_attention's argument checks; bytes == NULL is PSW_ERR_INVALID.
 */
int psw_attention_workspace_size(const psw_attn_args* args, int64_t* bytes);

/*
 * psw_lse_combine - [DCP] "Terms", section 1.1 and code block D: merge P partial
 * results row by row,  M = max_p lse_p,  w_p = exp(lse_p - M),
 *     out = sum_p w_p * O_p / sum_p w_p,   out_lse = M + log(sum_p w_p).
 * Partials with lse = -inf weigh 0; a row whose partials are all -inf gets 0 / -inf.
 *   partial_out   host array of P device pointers, each partial_dtype [num_rows, head_dim_v]
 *                 with partial_dtype PSW_BF16, PSW_F16 or PSW_F32 ([DCP] section 2.1: the
 *                 history partial reaches the merge in BF16/FP16 without a cast; section
 *                 3.2: the three history dtypes are all tested)
 *   partial_lse   host array of P device pointers, each fp32 [num_rows]
 *   out           out_dtype [num_rows, head_dim_v] (device), any of the three types;
 *                 out_lse fp32 [num_rows] or NULL
 * The partials are read in place (no packing).  1 <= P <= 64; head_dim_v a
 * multiple of 8 and at most 1024.
 */
int psw_lse_combine(const void* const* partial_out, const float* const* partial_lse,
                    int32_t num_partials, int32_t partial_dtype, int64_t num_rows,
                    int32_t head_dim_v, void* out, int32_t out_dtype, float* out_lse,
                    void* stream);

/*
 * psw_decode_two_streams - [DCP] section 2.1 (the stream swap), section 3.2 and
 * code blocks C and D: the history and current partials of a decode step on
 * two streams, joined before their LSE combine on the main stream.
 *   history   attention call over the history key ranges (num_splits partials),
 *             enqueued on main_stream
 *   current   attention call over the current key (its own partials), enqueued
 *             on side_stream
 *   out, out_dtype, out_lse  as psw_lse_combine, with num_rows = num_tokens x
 *             num_q_heads and head_dim_v of the two calls
 * Both calls are checked exactly as psw_swa_mm_attention checks one; they must
 * agree in num_tokens, num_q_heads, head_dim_v and out_dtype (the partial
 * dtype), both must write lse and, with tokens, have sequences, and together
 * hold at most 64 partials.  The
 * combine reads history's partials 0 .. S_h - 1 and then current's, in place.
 * Ordering: the side stream waits for an event recorded on main_stream, either
 * before the history call (the two workspaces are disjoint: the current call
 * sees everything enqueued on main_stream before this call and can run beside
 * the history call) or after it (the workspaces overlap: the current call runs
 * after the history call has finished with the shared workspace, as the pages
 * order it).  main_stream then waits for an event recorded on side_stream after
 * the current call, and runs the combine.  With main_stream == side_stream the
 * three steps run in order on that stream.  The exchange of history partials
 * between ranks, which the pages place on the main stream between the history
 * call and the join, has no counterpart on one GPU.
 * Tensors read or written on side_stream must stay alive until side_stream has
 * passed them.  On its first call on a device this function creates two HIP
 * events for that device (kept until the process ends); calls from several
 * threads enqueue one at a time.  Errors: as psw_swa_mm_attention and
 * psw_lse_combine; nothing is enqueued when a check fails.
 */
int psw_decode_two_streams(const psw_attn_args* history, const psw_attn_args* current,
                           void* out, int32_t out_dtype, float* out_lse, void* main_stream,
                           void* side_stream);

/*
 * psw_tile_bounds - the per-query-block tile interval the attention kernel uses,
 * exported for tests ([SWA-MM] "Key source snippet": the helper test kernel that
 * calls the production bounds routine and stores its three results).
 * For each query n: out[3n..3n+2] = (loop_lo, loop_hi, max_seq_prefix_len) of
 * request seq_idx[n], query block q_block_idx[n] (rows q_block*block_q .. +
 * (block_m - 1) / queries_per_kv), tiles of tile_size keys.  Uses geometry's
 * query_start_loc, seq_lens, mm_ranges, max_mm_ranges, num_q_heads, num_kv_heads,
 * window, causal, chunk_size, chunk_lookback; other fields are ignored.
 *   seq_idx, q_block_idx  int32 [num_queries] (device);  out int32 [num_queries, 3] (device)
 */
int psw_tile_bounds(const psw_attn_args* geometry, int32_t tile_size, int32_t block_m,
                    int32_t block_q, const int32_t* seq_idx, const int32_t* q_block_idx,
                    int32_t num_queries, int32_t* out, void* stream);

/*
 * psw_debug_take_failures - for testing the library itself, not part of the
 * method.  A build compiled with PSW_DEBUG has its kernels check their internal
 * invariants (tile ranges inside the request's keys, valid block-table entries
 * for every tile they load, tile bounds that contain every allowed key, the
 * request found for each token, KV slots inside the cache, the decode's work
 * split and workspace pieces) and record each failed check as a bit of a
 * per-device mask instead of trapping.  This call synchronises the current
 * device, stores the mask recorded there since the previous call (0 = every
 * check held; bit i = check i failed, the check list is in the library's
 * debug_checks.h) in *mask, and clears it.
 * Errors: PSW_ERR_INVALID for a NULL mask; PSW_ERR_UNSUPPORTED (and *mask = 0)
 * in builds without PSW_DEBUG; PSW_ERR_HIP if the synchronisation reports an
 * error.
 */
int psw_debug_take_failures(uint32_t* mask);

#ifdef __cplusplus
}
#endif

#endif /* PSW_H */
