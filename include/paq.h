/*
 * paq.h -- C ABI of the MI355X (gfx950) paged, quantized-KV attention library.
 *
 * Three operations over a block-paged KV cache stored as INT8, packed INT4 or
 * FP8 E4M3 with fp32 scales:
 *   kv_quant_append     quantize a step's new key/value rows into their slots
 *                       (kv_quant_append_rotary: rotary embedding first);
 *   paged_attn_decode   GQA decode (one new token per sequence), single pass or
 *                       split-KV ("flash decoding") with a log-sum-exp merge;
 *   paged_attn_prefill  ragged, causal, chunked prefill;
 *   paged_attn_decode_sparse  decode over caller-selected KV blocks;
 *   paged_attn_decode_host  the same decode on the host CPU, host-resident data.
 *
 * Problem statement (shared by all three; the cache shape with
 * cache_head_size is from "ONNX Runtime: INT4 Paged KV Cache", section 2; the
 * cumulative query lengths and their host copy are from "PagedAttention FA
 * path: exact max_query_len", section 1):
 *   query        (token_count, num_heads, head_size), dtype q_dtype
 *   out          (token_count, num_heads, head_size), dtype q_dtype
 *   key_cache,
 *   value_cache  (num_blocks, block_size, kv_num_heads, cache_head_size) bytes,
 *                cache_head_size = (head_size+1)/2 for INT4, head_size otherwise
 *   block_table  int32 (batch, max_blocks_per_seq): physical block of each
 *                logical block of each sequence (unused entries may hold any
 *                value; they are never read)
 *   cum_q        int32 (batch+1): rows cum_q[b]..cum_q[b+1]-1 of query/out
 *                belong to sequence b; q_len_b = cum_q[b+1]-cum_q[b] >= 0
 *   past_lens    int32 (batch): tokens of sequence b cached before this step
 *   k_scale,
 *   v_scale      fp32, (kv_num_heads, head_size) per channel or (kv_num_heads)
 *                per kv head
 *
 * Semantics.  A step's new rows are appended first (kv_quant_append on the same
 * stream); sequence b then holds kv_len_b = past_b + q_len_b tokens, token t at
 * row t % block_size of block block_table[b][t / block_size].  Query row i of
 * sequence b (0 <= i < q_len_b) attends to positions 0..past_b+i, query head h
 * to kv head h / (num_heads/kv_num_heads).  Scores are softmax_scale * q.k
 * (softmax_scale <= 0 selects 1/sqrt(head_size)); keys and values are
 * code * scale.  Sequences with q_len 0 produce no rows and cost no reads.
 *
 * Ownership.  Every pointer is owned by the caller.  Pointers named *_host are
 * host memory and are read synchronously inside the call (they may be freed
 * when it returns); all other array pointers are device memory that must stay
 * valid until the work queued on `stream` has finished.  `stream` is a
 * hipStream_t (NULL = the default stream).  The library never allocates or
 * frees device memory, never synchronizes the stream and keeps no state
 * between calls other than its loaded kernels.
 *
 * Errors.  Every check runs on the host before anything is launched: a
 * non-zero status means nothing was launched and nothing written.
 * paq_last_error() describes the most recent failure of the calling thread.
 * Preconditions that are NOT checked (device-resident data): block ids in
 * [0, num_blocks), device cum_q/past_lens equal to their host copies, finite
 * positive scales, finite inputs.  Key scales may lie far outside the 16-bit
 * ranges (tested over [2^-60, 2^100] per channel): the 16-bit kernels fold
 * k_scale / M into the query with M the power of two >= the kv head's largest
 * key scale, and keep softmax_scale * M in fp32; the products
 * softmax_scale * k_scale * |q . k codes| must stay below ~2^120.  Value
 * scales must keep the outputs inside the query dtype's range.
 */
#ifndef PAQ_H
#define PAQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PAQ_ABI_VERSION 1

enum paq_status {
  PAQ_OK = 0,
  PAQ_ERR_INVALID_ARG = 1, /* shapes, lengths, pointers or enums are wrong   */
  PAQ_ERR_UNSUPPORTED = 2, /* valid but not built: head_size, block_size...  */
  PAQ_ERR_WORKSPACE = 3,   /* split decode workspace missing or too small    */
  PAQ_ERR_HIP = 4          /* the HIP runtime refused a launch               */
};

enum paq_dtype { PAQ_DT_F32 = 0, PAQ_DT_F16 = 1, PAQ_DT_BF16 = 2 };

/* KV storage formats.
 * INT8: two's-complement byte, codes in [-127, 127].
 * INT4: two 4-bit two's-complement codes in [-7, 7] per byte ("ONNX Runtime:
 *       INT4 Paged KV Cache", section 2); channel 2j in the low nibble,
 *       channel 2j+1 in the high nibble.
 * FP8_E4M3: OCP E4M3 (bias 7, max 448, S.1111.111 NaN, no infinities). */
enum paq_kv_format { PAQ_KV_INT8 = 0, PAQ_KV_INT4 = 1, PAQ_KV_FP8_E4M3 = 2 };

enum paq_scale_mode { PAQ_SCALE_PER_CHANNEL = 0, PAQ_SCALE_PER_HEAD = 1 };

/* Which kernels a decode call runs (see paq_plan_decode). */
enum paq_path {
  PAQ_PATH_NONE = 0,         /* no rows: nothing is launched                    */
  PAQ_PATH_SINGLE = 1,       /* one pass per (sequence, kv head), 16-bit MFMA   */
  PAQ_PATH_SPLIT = 2,        /* split-KV chunks + log-sum-exp combine, MFMA     */
  PAQ_PATH_F32_SINGLE = 3,   /* portable fp32 kernel, one pass                  */
  PAQ_PATH_F32_SPLIT = 4,    /* portable fp32 kernel, split-KV + combine        */
  PAQ_PATH_PREFILL = 5,      /* MFMA prefill tiles                              */
  PAQ_PATH_F32_PREFILL = 6   /* portable fp32 kernel, one query row per group   */
};

/* Shape/format description shared by all calls. */
typedef struct paq_desc {
  int32_t batch;              /* sequences, >= 0                               */
  int32_t token_count;        /* rows of query/out (= cum_q[batch]), >= 0      */
  int32_t num_heads;          /* query heads, multiple of kv_num_heads         */
  int32_t kv_num_heads;       /* >= 1                                          */
  int32_t head_size;          /* 64 or 128                                     */
  int32_t block_size;         /* 16, 32, 64 or 128 tokens per block            */
  int32_t num_blocks;         /* blocks in each cache pool                     */
  int32_t max_blocks_per_seq; /* columns of block_table                        */
  int32_t q_dtype;            /* enum paq_dtype: query and output              */
  int32_t kv_format;          /* enum paq_kv_format                            */
  int32_t scale_mode;         /* enum paq_scale_mode                           */
} paq_desc;

/* Host-side plan of a call (introspection; the calls compute it themselves). */
typedef struct paq_plan {
  int32_t max_query_len;    /* exact max_b q_len_b, from the host cum_q        */
  int32_t max_kv_len;       /* max_b past_b + q_len_b over sequences with rows */
  int32_t active_seqs;      /* sequences with q_len > 0                        */
  int32_t work_units;       /* active_seqs * kv_num_heads                      */
  int32_t num_splits;       /* KV chunks per sequence (1 = single pass)        */
  int32_t path;             /* enum paq_path                                   */
  int32_t grid_x, grid_y, grid_z; /* launch grid of the main kernel            */
  int32_t reserved;
  uint64_t workspace_bytes; /* device workspace the call needs (split decode)  */
} paq_plan;

/* ABI version of the loaded library (PAQ_ABI_VERSION). */
int32_t paq_abi_version(void);

/* Static text for a status code. */
const char* paq_status_string(int32_t status);

/* Message describing the last failed call on this thread ("" if none). */
const char* paq_last_error(void);

/* Plan a decode call without launching anything (pure host code, usable
 * without a GPU).  num_splits: 0 = automatic (split when the work units
 * under-fill num_cus compute units and a sequence has more than one block,
 * mirroring the flash-decoding rule of "GQA GEMV decode", section 2), 1 = single
 * pass, > 1 = that many block-aligned chunks per sequence.  num_cus <= 0
 * queries the current device.  Returns a status; fills *plan on success. */
int32_t paq_plan_decode(const paq_desc* d, const int32_t* cum_q_host,
                        const int32_t* past_lens_host, int32_t num_splits,
                        int32_t num_cus, paq_plan* plan);

/* Plan a prefill call (exact max_query_len from the host cum_q, as in
 * "PagedAttention FA path: exact max_query_len", section 1). */
int32_t paq_plan_prefill(const paq_desc* d, const int32_t* cum_q_host,
                         const int32_t* past_lens_host, paq_plan* plan);

/* Device workspace bytes paged_attn_decode needs for these arguments (0 for a
 * single pass).  Returns 0 as well when the arguments are invalid. */
size_t paged_attn_decode_workspace_size(const paq_desc* d, const int32_t* cum_q_host,
                                        const int32_t* past_lens_host,
                                        int32_t num_splits);

/* GQA paged decode: every q_len_b must be 0 or 1.  Split-KV (path SPLIT) needs
 * `workspace` (device, 16-byte aligned) of at least
 * paged_attn_decode_workspace_size() bytes; it holds fp32 partial outputs and
 * log-sum-exps (one per output row, head and slice of plan.grid_z: a
 * workgroup of the 16-bit kernel merges its chunks first) and is overwritten.  fp32 queries take the portable fp32
 * kernel; fp16/bf16 queries take the MFMA kernel, which folds the per-channel
 * k_scale into the query ("ONNX Runtime: INT4 Paged KV Cache", section 3).
 * Returns PAQ_ERR_WORKSPACE if the workspace is missing or too small. */
int32_t paged_attn_decode(const paq_desc* d, const void* query, void* out,
                          const void* key_cache, const void* value_cache,
                          const float* k_scale, const float* v_scale,
                          const int32_t* block_table, const int32_t* cum_q,
                          const int32_t* past_lens, const int32_t* cum_q_host,
                          const int32_t* past_lens_host, float softmax_scale,
                          int32_t num_splits, void* workspace, size_t workspace_bytes,
                          void* stream);

/* Ragged causal prefill: any q_len_b >= 0.  The grid is sized from the exact
 * max_query_len of the host cum_q; if it is 0 nothing is launched. */
int32_t paged_attn_prefill(const paq_desc* d, const void* query, void* out,
                           const void* key_cache, const void* value_cache,
                           const float* k_scale, const float* v_scale,
                           const int32_t* block_table, const int32_t* cum_q,
                           const int32_t* past_lens, const int32_t* cum_q_host,
                           const int32_t* past_lens_host, float softmax_scale,
                           void* stream);

/* Quantize rows cum_q[b]..cum_q[b+1]-1 of key/value (token_count, kv_num_heads,
 * head_size; dtype kv_in_dtype) and store row i of sequence b at position
 * past_b + i.  code = clamp(round_half_even(fl32(x / s))) with +-127 (INT8),
 * +-7 (INT4), or E4M3 round-half-even saturating to +-448 (FP8); x / s is the
 * correctly rounded fp32 quotient.  Cache bytes of other positions are not
 * touched.  Needs ceil((past_b + q_len_b) / block_size) <= max_blocks_per_seq. */
int32_t kv_quant_append(const paq_desc* d, int32_t kv_in_dtype, const void* key,
                        const void* value, void* key_cache, void* value_cache,
                        const float* k_scale, const float* v_scale,
                        const int32_t* block_table, const int32_t* cum_q,
                        const int32_t* past_lens, const int32_t* cum_q_host,
                        const int32_t* past_lens_host, void* stream);

/* Block-sparse GQA decode ("INT8-KV Tensor-Core DynamicSparseAttention",
 * section 1; the page gives no selection rule, so the selection is an input):
 * the new token of sequence b attends to exactly the keys t < kv_len_b whose
 * logical block t / block_size is one of sel_blocks[b][0 .. num_sel[b]).
 *   sel_blocks   int32 (batch, max_sel), device: ascending logical block
 *                indices, each < ceil(kv_len_b / block_size) (not checked:
 *                device data, like block ids)
 *   num_sel      int32 (batch), device; num_sel_host its host copy, each in
 *                [1, min(max_sel, ceil(kv_len_b / block_size))] for sequences
 *                with a new row (checked on the host)
 * Runs a small kernel that turns the selection into a compact block table
 * and effective key counts, then the dense decode kernels over it (single
 * pass or split-KV with num_splits as for paged_attn_decode, planned on
 * num_sel_host * block_size keys).  `workspace` (device, 16-byte aligned)
 * must hold paged_attn_decode_sparse_workspace_size() bytes; it is
 * overwritten.  Otherwise as paged_attn_decode. */
int32_t paged_attn_decode_sparse(const paq_desc* d, const void* query, void* out,
                                 const void* key_cache, const void* value_cache,
                                 const float* k_scale, const float* v_scale,
                                 const int32_t* block_table, const int32_t* cum_q,
                                 const int32_t* past_lens, const int32_t* cum_q_host,
                                 const int32_t* past_lens_host, const int32_t* sel_blocks,
                                 const int32_t* num_sel, const int32_t* num_sel_host,
                                 int32_t max_sel, float softmax_scale, int32_t num_splits,
                                 void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes of paged_attn_decode_sparse (0 when the arguments are
 * invalid or there is nothing to do). */
size_t paged_attn_decode_sparse_workspace_size(const paq_desc* d, const int32_t* cum_q_host,
                                               const int32_t* past_lens_host,
                                               const int32_t* num_sel_host, int32_t max_sel,
                                               int32_t num_splits);

/* GQA decode on the host CPU over host-resident caches: the CPU workload of
 * "GQA GEMV decode" (sections 2-3).  Every pointer is HOST memory (including
 * block_table, cum_q and past_lens); nothing touches a GPU, and no GPU call
 * ever falls back to it.  A dedicated M = 1 kernel: each key row is
 * dequantized once and dotted with the G query heads of its kv head, each
 * value row accumulated with their softmax weights (fp32 throughout, online
 * softmax over 256-key tiles).  When active sequences x kv heads is below
 * num_threads, each sequence's keys are split into block-aligned chunks
 * (num_splits, 0 = automatic) run on separate threads and merged by their
 * log-sum-exps.  d->q_dtype must be PAQ_DT_F32 (PAQ_ERR_UNSUPPORTED
 * otherwise); q_len must be 0 or 1; num_threads 0 = the host's hardware
 * threads.  Blocks the calling thread until done. */
int32_t paged_attn_decode_host(const paq_desc* d, const float* query, float* out,
                               const void* key_cache, const void* value_cache,
                               const float* k_scale, const float* v_scale,
                               const int32_t* block_table, const int32_t* cum_q,
                               const int32_t* past_lens, float softmax_scale,
                               int32_t num_splits, int32_t num_threads);

/* kv_quant_append with rotary position embedding (RoPE) of the new rows first,
 * in the same launch.  The step just before attention; "PagedAttention FA
 * path: exact max_query_len" (sections 1-2) shows the rotary kernel dropping
 * rows when its grid came from the heuristic token_count - batch + 1 and a
 * sequence had no new token: this grid, like every grid here, comes from the
 * exact max_query_len of cum_q_host.
 *   query        (token_count, num_heads, head_size), dtype d->q_dtype, device;
 *                rotated in place (each element rounded half-even to q_dtype).
 *                NULL rotates the keys only.
 *   key, value   as for kv_quant_append; keys are rotated before they are
 *                quantized, values are appended unchanged.
 *   cos_cache,
 *   sin_cache    fp32 (max_position, rotary_dim / 2), device, 16-byte aligned:
 *                the angle of pair k at position p is [p * rotary_dim/2 + k].
 *   rotary_dim   channels 0..rotary_dim-1 rotate, the rest pass through; even,
 *                <= head_size (PAQ_ERR_INVALID_ARG otherwise) and a multiple of
 *                16 (PAQ_ERR_UNSUPPORTED otherwise).
 *   interleaved  0: pair k is channels (k, k + rotary_dim/2); 1: (2k, 2k+1).
 * Row i of sequence b has position past_b + i (the position its key is stored
 * at), which must be < max_position (checked on the host: PAQ_ERR_INVALID_ARG).
 * A pair (x, y) becomes x' = fl32(fl32(x*c) - fl32(y*s)), y' = fl32(fl32(y*c) +
 * fl32(x*s)), c and s its table entries: every product and sum rounded to fp32,
 * no fused multiply-add, so the key codes (quantized from x' as in
 * kv_quant_append) are reproducible bit for bit.  Same ownership, stream and
 * error rules as the other calls; query, key and value must not overlap. */
int32_t kv_quant_append_rotary(const paq_desc* d, int32_t kv_in_dtype, void* query,
                               const void* key, const void* value, void* key_cache,
                               void* value_cache, const float* k_scale, const float* v_scale,
                               const int32_t* block_table, const int32_t* cum_q,
                               const int32_t* past_lens, const int32_t* cum_q_host,
                               const int32_t* past_lens_host, const float* cos_cache,
                               const float* sin_cache, int32_t max_position,
                               int32_t rotary_dim, int32_t interleaved, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PAQ_H */
