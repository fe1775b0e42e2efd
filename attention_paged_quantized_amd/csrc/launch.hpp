// launch.hpp -- internal interface between the host library (paq_host.cpp) and
// the kernel translation units.  Every launcher assumes the host has already
// validated its arguments; it returns 0, or -1 for a format/dtype/shape
// combination it was not built for.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace paq {

struct AppendArgs {
  const void* key;
  const void* value;
  void* key_cache;
  void* value_cache;
  const float* k_scale;
  const float* v_scale;
  const int32_t* block_table;
  const int32_t* cum_q;
  const int32_t* past_lens;
  int batch, hkv, head_size, block_size, max_blocks;
  int kv_format, scale_mode, in_dtype;
  int max_query_len;   // exact, from the host cum_q
  int tokens_per_wg;
  // rotary variant only
  void* query;         // (token_count, num_heads, head_size) q_dtype, rotated in place; or null
  const float* cos_cache;   // (max_position, rotary_dim / 2)
  const float* sin_cache;
  int num_heads, q_dtype, rotary_dim, interleaved;
};

struct AttnArgs {
  const void* query;
  void* out;
  const uint8_t* key_cache;
  const uint8_t* value_cache;
  const float* k_scale;
  const float* v_scale;
  const int32_t* block_table;
  const int32_t* cum_q;
  const int32_t* past_lens;
  // fp32 kernel split-KV: partial outputs [T][H][S][D] and their log-sum-exps
  // as (raw maximum, log2 sum) pairs [T][H][S][2]; MFMA decode parts: partial
  // outputs [parts][H][D] and (raw maximum, sum) pairs [parts][H][2]
  float* part_o;
  float* part_lse;
  float* part_ml;
  int32_t* dec_counters; // MFMA decode: arrival counter per (sequence, head group), zero
  int batch, token_count, num_heads, hkv, head_size, block_size, max_blocks;
  int q_dtype, kv_format, scale_mode;
  int num_splits;       // 1 = single pass (no partials)
  int part_count;       // fp32 split-KV: partials per (row, head) in the workspace
  int grid_x;           // 1-D launch grid (MFMA decode and prefill: from the host plan)
  int pf_ntq;           // prefill: query tiles of every sequence if all have the same, else 0
  int pf_k_per_use;     // prefill: K codes converted per use (comparison variant)
  int max_query_len;    // exact, from the host cum_q
  int max_kv_len;       // longest sequence with new rows (host)
  int block_size_log2;  // block_size is a power of two
  // MFMA decode partition (host plan)
  int dec_mode;            // DEC_SINGLE / DEC_CHUNKS / DEC_STREAM
  int dec_waves;           // waves per workgroup (4 or 8)
  int dec_head_groups;     // kv_num_heads / heads per wave
  int dec_parts_per_seq;   // DEC_CHUNKS: parts of every sequence
  int dec_chunks_per_part; // DEC_CHUNKS: consecutive chunks per part
  long long dec_total_tiles;  // DEC_STREAM: 32-key tiles of all segments
  float softmax_scale;  // already resolved (> 0)
  // Decode with the step's append fused in (MFMA decode only): the new key
  // and value rows (token_count, kv_num_heads, head_size) in the query's
  // dtype, quantized into the caches by the wave that streams the tile
  // holding them; null for a plain decode.
  const void* new_key;
  const void* new_value;
  int new_rows_f32;     // MFMA decode: the new rows are fp32 (else the query's dtype)
};

// Launch geometry shared by the host planner and the launchers.
// Decode (MFMA): one wave serves this many adjacent kv heads -- 128 / row
// bytes (whole 128-byte lines per copied row segment), at most 2 (four heads
// per wave need more registers than a wave has: the 32-byte rows of INT4 at
// head size 64 are copied as 64-byte segments), and only as many as divide
// the kv head count (row bytes: head_size, or head_size / 2 for INT4).
inline int decode_heads_per_wave(int kv_format, int head_size, int hkv) {
  const int row = (kv_format == 1 /* INT4 */) ? head_size / 2 : head_size;
  int hw = row >= 128 ? 1 : (128 / row > 2 ? 2 : 128 / row);
  while (hw > 1 && hkv % hw) hw /= 2;
  return hw;
}
// MFMA decode partitions (see decode_mfma.hip).
enum { DEC_SINGLE = 0, DEC_CHUNKS = 1, DEC_STREAM = 2 };
// Arrival counters at the head of every decode workspace: one int32 per
// (sequence, head group) of a split call, zero before a call and after it.
constexpr int kDecCounters = 16384;
// Parts per sequence of the chunk partition, and workgroups of the balanced
// (stream) partition: at most about one per compute unit is useful (more
// workgroups per segment were measured slower), and the last piece to arrive
// reads the others' partials in rounds of 16.
constexpr int kDecMaxPartsPerSeq = 256;
constexpr size_t kDecCounterBytes = (size_t)kDecCounters * 4;
// Prefill (MFMA): workgroups of 4 waves x 32 / group tokens.  (Sequence, kv
// head) pair p runs on XCD p % 8 and needs ceil(q_len / tokens) query tiles;
// the 1-D grid is 8 x the largest per-XCD tile count, so no workgroup is
// launched for a tile past its sequence's new rows.
constexpr int kPrefillWaves = 4;
inline int prefill_tokens_per_workgroup(int group) { return kPrefillWaves * (32 / group); }
inline int prefill_grid(const int32_t* cum_q_host, int batch, int group, int hkv) {
  const int tok = prefill_tokens_per_workgroup(group);
  long items[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (long pr = 0; pr < (long)hkv * batch; ++pr) {
    const int b = (int)(pr / hkv);
    items[pr % 8] += (cum_q_host[b + 1] - cum_q_host[b] + tok - 1) / tok;
  }
  long m = 0;
  for (int x = 0; x < 8; ++x) m = items[x] > m ? items[x] : m;
  return (int)(8 * m);
}
// The common query-tile count of all sequences, or 0 when they differ.
inline int prefill_uniform_tiles(const int32_t* cum_q_host, int batch, int group) {
  const int tok = prefill_tokens_per_workgroup(group);
  int n = -1;
  for (int b = 0; b < batch; ++b) {
    const int t = (cum_q_host[b + 1] - cum_q_host[b] + tok - 1) / tok;
    if (n >= 0 && t != n) return 0;
    n = t;
  }
  return n > 0 ? n : 0;
}

int launch_quant_append(const AppendArgs& a, hipStream_t st);
int launch_rotary_append(const AppendArgs& a, hipStream_t st);
int launch_decode_f32(const AttnArgs& a, hipStream_t st);     // any q_len (portable)
int launch_decode_mfma(const AttnArgs& a, hipStream_t st);    // q_len in {0,1}
int launch_combine(const AttnArgs& a, hipStream_t st);
int launch_prefill_mfma(const AttnArgs& a, hipStream_t st);
// block-sparse decode: selected blocks -> compact table + effective past
int launch_sparse_compact(const int32_t* block_table, int max_blocks, const int32_t* sel,
                          const int32_t* num_sel, int max_sel, const int32_t* cum_q,
                          const int32_t* past_lens, int block_size, int batch, int32_t* compact,
                          int32_t* eff_past, hipStream_t st);
// block-sparse prefill: selected earlier blocks + the blocks holding new
// tokens -> compact table (row stride `stride`) + effective past
int launch_sparse_prefill_compact(const int32_t* block_table, int max_blocks, const int32_t* sel,
                                  const int32_t* num_sel, int max_sel, const int32_t* cum_q,
                                  const int32_t* past_lens, int block_size, int batch,
                                  int stride, int32_t* compact, int32_t* eff_past,
                                  hipStream_t st);

// Shape support of the MFMA kernels (host checks before choosing a path).
bool decode_mfma_supports(int head_size, int group, int block_size, int q_dtype);
// The portable fp32 kernel serves GQA groups up to this size.
constexpr int kF32KernelMaxGroup = 16;
bool prefill_mfma_supports(int head_size, int group, int block_size, int q_dtype);

}  // namespace paq
