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
  float* part_o;        // split-KV partial outputs [T][H][S][D] (fp32), or null
  float* part_lse;      // split-KV partial log-sum-exps [T][H][S], or null
  int batch, token_count, num_heads, hkv, head_size, block_size, max_blocks;
  int q_dtype, kv_format, scale_mode;
  int num_splits;       // 1 = single pass (no partials)
  int part_count;       // split-KV: partials per (row, head) in the workspace
  int grid_x;           // launch grid (1-D prefill: from the host plan)
  int pf_ntq;           // prefill: query tiles of every sequence if all have the same, else 0
  int max_query_len;    // exact, from the host cum_q
  int max_kv_len;       // longest sequence with new rows (host)
  int block_size_log2;  // block_size is a power of two
  int num_cus;          // compute units of the device (split-KV grid sizing)
  int split_chunks_per_wg;  // split-KV: consecutive chunks per workgroup (set by the launcher)
  float softmax_scale;  // already resolved (> 0)
};

// Launch geometry shared by the host planner and the launchers.
// Decode (MFMA): one wave serves this many adjacent kv heads -- 128 / row
// bytes when the kv head count allows, else the largest power of two that
// divides it (row bytes: head_size, or head_size / 2 for INT4).
inline int decode_heads_per_wave(int kv_format, int head_size, int hkv) {
  const int row = (kv_format == 1 /* INT4 */) ? head_size / 2 : head_size;
  int hw = row >= 128 ? 1 : 128 / row;
  while (hw > 1 && hkv % hw) hw /= 2;
  return hw;
}
// Decode split-KV: waves (one per chunk) per workgroup -- 8 when the grid
// still gives every compute unit a workgroup, else 4.
inline int decode_split_waves(int hkv, int heads_per_wave, int batch, int splits, int num_cus) {
  const long waves = (long)(hkv / heads_per_wave) * batch * splits;
  return waves >= 8L * (num_cus > 0 ? num_cus : 256) ? 8 : 4;
}
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

// Shape support of the MFMA kernels (host checks before choosing a path).
bool decode_mfma_supports(int head_size, int group, int block_size, int q_dtype);
bool prefill_mfma_supports(int head_size, int group, int block_size, int q_dtype);

}  // namespace paq
