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
// Memory-bound: each thread converts 8 consecutive channels of one (token,
// kv head) row of K or V: one 16- or 32-byte load, one 8- or 4-byte store.
#include "device.hpp"
#include "launch.hpp"

namespace paq {

constexpr int kAppendThreads = 256;

template <typename T>
__device__ __forceinline__ void load8(const T* p, float (&x)[8]) {
  if constexpr (sizeof(T) == 2) {
    u32x4 v = *reinterpret_cast<const u32x4*>(p);
    const T* e = reinterpret_cast<const T*>(&v);
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = to_f32(e[i]);
  } else {
    f32x4 a = *reinterpret_cast<const f32x4*>(p);
    f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) { x[i] = a[i]; x[4 + i] = b[i]; }
  }
}

template <int KVF, int SM, typename TI>
__global__ __launch_bounds__(kAppendThreads) void quant_append_kernel(
    const TI* __restrict__ key, const TI* __restrict__ value, uint8_t* __restrict__ kcache,
    uint8_t* __restrict__ vcache, const float* __restrict__ kscale,
    const float* __restrict__ vscale, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ cum_q, const int32_t* __restrict__ past_lens, int hkv,
    int head_size, int block_size, int max_blocks, int tokens_per_wg) {
  const int b = blockIdx.y;
  const int q0 = cum_q[b];
  const int qlen = cum_q[b + 1] - q0;
  const int i_begin = blockIdx.x * tokens_per_wg;
  if (i_begin >= qlen) return;
  const int i_end = min(qlen, i_begin + tokens_per_wg);
  const int past = past_lens[b];
  const int chunks_per_row = hkv * head_size / 8;           // per tensor
  const int chunk_per_tok = 2 * chunks_per_row;              // K and V
  const int C = (KVF == KV_INT4) ? head_size / 2 : head_size;
  const int total = (i_end - i_begin) * chunk_per_tok;
  for (int idx = threadIdx.x; idx < total; idx += kAppendThreads) {
    const int tok = i_begin + idx / chunk_per_tok;
    int rem = idx % chunk_per_tok;
    const bool is_v = rem >= chunks_per_row;
    if (is_v) rem -= chunks_per_row;
    const int h = rem / (head_size / 8);
    const int d0 = (rem % (head_size / 8)) * 8;
    const TI* src = (is_v ? value : key) + ((size_t)(q0 + tok) * hkv + h) * head_size + d0;
    const float* sc = is_v ? vscale : kscale;
    float x[8];
    load8(src, x);
    float s[8];
    if constexpr (SM == SCALE_CHANNEL) {
      f32x4 a = *reinterpret_cast<const f32x4*>(sc + h * head_size + d0);
      f32x4 c = *reinterpret_cast<const f32x4*>(sc + h * head_size + d0 + 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) { s[i] = a[i]; s[4 + i] = c[i]; }
    } else {
      const float v = sc[h];
#pragma unroll
      for (int i = 0; i < 8; ++i) s[i] = v;
    }
    const int t = past + tok;
    const int blk = block_table[(size_t)b * max_blocks + t / block_size];
    uint8_t* dst = (is_v ? vcache : kcache) +
                   (((size_t)blk * block_size + t % block_size) * hkv + h) * C;
    if constexpr (KVF == KV_INT8) {
      uint32_t w0 = 0, w1 = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        w0 |= (uint32_t)(quant_int(x[i] / s[i], 127.0f) & 0xFF) << (8 * i);
        w1 |= (uint32_t)(quant_int(x[4 + i] / s[4 + i], 127.0f) & 0xFF) << (8 * i);
      }
      *reinterpret_cast<u32x2*>(dst + d0) = (u32x2){w0, w1};
    } else if constexpr (KVF == KV_INT4) {
      uint32_t w = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        w |= (uint32_t)(quant_int(x[i] / s[i], 7.0f) & 0xF) << (4 * i);
      *reinterpret_cast<uint32_t*>(dst + d0 / 2) = w;
    } else {
      uint32_t w0 = 0, w1 = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        w0 |= e4m3_encode(x[i] / s[i]) << (8 * i);
        w1 |= e4m3_encode(x[4 + i] / s[4 + i]) << (8 * i);
      }
      *reinterpret_cast<u32x2*>(dst + d0) = (u32x2){w0, w1};
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
