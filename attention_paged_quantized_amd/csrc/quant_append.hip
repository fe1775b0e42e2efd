// quant_append.hip -- quantize a step's new key/value rows and scatter them
// into their block-paged cache slots (INT8, packed INT4 or FP8 E4M3).
//
// Cache layout (num_blocks, block_size, kv_num_heads, cache_head_size) with
// cache_head_size = (head_size+1)/2 for INT4 ("ONNX Runtime: INT4 Paged KV
// Cache", section 2).  Row i of sequence b (query-row cum_q[b]+i) goes to
// position t = past_b + i, i.e. block block_table[b][t / block_size], row
// t % block_size.
//
// Bit contract: code = clamp(rint(fl32(x / s))) with +-127 / +-7, or E4M3
// round-half-even saturating to +-448.  `x / s` is IEEE fp32 division (the
// library is built without fast-math, so it is correctly rounded).
//
// Memory-bound: a thread converts 8 consecutive channels of one kv head of K
// or V (one 16- or 32-byte load, one 8- or 4-byte store per token) for the
// tokens of its workgroup, eight tokens' loads in flight at a time.
#include "append.hpp"
#include "launch.hpp"

namespace paq {

constexpr int kAppendThreads = 256;

template <int KVF, int SM, typename TI>
__global__ __launch_bounds__(kAppendThreads) void quant_append_kernel(
    const TI* __restrict__ key, const TI* __restrict__ value, uint8_t* __restrict__ kcache,
    uint8_t* __restrict__ vcache, const float* __restrict__ kscale,
    const float* __restrict__ vscale, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ cum_q, const int32_t* __restrict__ past_lens, int hkv,
    int head_size, int block_size, int max_blocks, int tokens_per_wg) {
  const int b = blockIdx.y;
  // the lengths in one round trip (past is read before the exit test, so the
  // row loads below wait for one memory latency, not two)
  const int q0 = cum_q[b];
  const int qlen = cum_q[b + 1] - q0;
  const int past = past_lens[b];
  const int i_begin = blockIdx.x * tokens_per_wg;
  if (i_begin >= qlen) return;
  const int i_end = min(qlen, i_begin + tokens_per_wg);
  const int chunks_per_row = hkv * head_size / 8;           // per tensor
  const int chunk_per_tok = 2 * chunks_per_row;              // K and V
  const int C = (KVF == KV_INT4) ? head_size / 2 : head_size;
  // A thread keeps one chunk (8 channels of one kv head of K or V) and walks
  // the workgroup's tokens, kUnroll at a time with all their loads issued
  // before the first store; neighbouring lanes take neighbouring chunks.
  constexpr int kUnroll = 8;
  for (int c = threadIdx.x; c < chunk_per_tok; c += kAppendThreads) {
    const bool is_v = c >= chunks_per_row;
    const int cc = is_v ? c - chunks_per_row : c;
    const int h = cc / (head_size / 8), d0 = (cc % (head_size / 8)) * 8;
    const TI* src = (is_v ? value : key) + ((size_t)q0 * hkv + h) * head_size + d0;
    uint8_t* cache = (is_v ? vcache : kcache) + (size_t)h * C;
    const int32_t* table = block_table + (size_t)b * max_blocks;
    float s[8];
    load_scales8<SM>(is_v ? vscale : kscale, h, head_size, d0, s);
    auto dst = [&](int t, int blk) {
      return cache + ((size_t)blk * block_size + t % block_size) * hkv * C;
    };
    int i = i_begin;
    for (; i + kUnroll <= i_end; i += kUnroll) {
      float x[kUnroll][8];
      int blk[kUnroll];
#pragma unroll
      for (int j = 0; j < kUnroll; ++j) {
        load8(src + (size_t)(i + j) * hkv * head_size, x[j]);
        blk[j] = table[(past + i + j) / block_size];
      }
#pragma unroll
      for (int j = 0; j < kUnroll; ++j) store_codes8<KVF>(dst(past + i + j, blk[j]), d0, x[j], s);
    }
    for (; i < i_end; ++i) {
      float x[8];
      load8(src + (size_t)i * hkv * head_size, x);
      store_codes8<KVF>(dst(past + i, table[(past + i) / block_size]), d0, x, s);
    }
  }
}

template <int KVF, int SM>
static int launch_fmt(const AppendArgs& a, int in_dtype, dim3 grid, hipStream_t st) {
  switch (in_dtype) {
#define PAQ_APPEND_CASE(DTV, TYPE)                                                        \
  case DTV:                                                                              \
    hipLaunchKernelGGL((quant_append_kernel<KVF, SM, TYPE>), grid, dim3(kAppendThreads), \
                       0, st, (const TYPE*)a.key, (const TYPE*)a.value,                   \
                       (uint8_t*)a.key_cache, (uint8_t*)a.value_cache, a.k_scale,         \
                       a.v_scale, a.block_table, a.cum_q, a.past_lens, a.hkv,             \
                       a.head_size, a.block_size, a.max_blocks, a.tokens_per_wg);         \
    return 0;
    PAQ_APPEND_CASE(DT_F32, float)
    PAQ_APPEND_CASE(DT_F16, f16)
    PAQ_APPEND_CASE(DT_BF16, bf16)
#undef PAQ_APPEND_CASE
  }
  return -1;
}

int launch_quant_append(const AppendArgs& a, hipStream_t st) {
  dim3 grid((a.max_query_len + a.tokens_per_wg - 1) / a.tokens_per_wg, a.batch);
  const int key = a.kv_format * 2 + a.scale_mode;
  switch (key) {
    case KV_INT8 * 2 + SCALE_CHANNEL: return launch_fmt<KV_INT8, SCALE_CHANNEL>(a, a.in_dtype, grid, st);
    case KV_INT8 * 2 + SCALE_HEAD: return launch_fmt<KV_INT8, SCALE_HEAD>(a, a.in_dtype, grid, st);
    case KV_INT4 * 2 + SCALE_CHANNEL: return launch_fmt<KV_INT4, SCALE_CHANNEL>(a, a.in_dtype, grid, st);
    case KV_INT4 * 2 + SCALE_HEAD: return launch_fmt<KV_INT4, SCALE_HEAD>(a, a.in_dtype, grid, st);
    case KV_FP8 * 2 + SCALE_CHANNEL: return launch_fmt<KV_FP8, SCALE_CHANNEL>(a, a.in_dtype, grid, st);
    case KV_FP8 * 2 + SCALE_HEAD: return launch_fmt<KV_FP8, SCALE_HEAD>(a, a.in_dtype, grid, st);
  }
  return -1;
}

}  // namespace paq
