// rotary_append.hip -- rotary position embedding of a step's new query and key
// rows, fused with the quantize-and-append of keys and values.
//
// The rows are the ones the cumulative query lengths lay out, and the grid is
// sized from the exact max_query_len of the host cum_q ("PagedAttention FA
// path: exact max_query_len", sections 1-2: the heuristic bound dropped rotary
// rows whenever a sequence had no new token).  Row i of sequence b sits at
// position past_b + i, the position its key is stored at.
//
// Rotation: channels 0..rotary_dim-1 rotate in pairs -- (k, k + rotary_dim/2),
// or (2k, 2k+1) when interleaved -- by the caller's angle tables: a pair
// (x, y) at pair index k of position p becomes
//   x' = fl32(fl32(x * cos[p][k]) - fl32(y * sin[p][k]))
//   y' = fl32(fl32(y * cos[p][k]) + fl32(x * sin[p][k]))
// with every product and sum rounded to fp32 (no fused multiply-add), so the
// cache codes taken from x' / scale are reproducible bit for bit.  Channels
// from rotary_dim on pass through.  Queries are rounded half-even to their
// dtype and written back in place; keys go on to the quantizer of
// kv_quant_append; values are appended as they are.
//
// Memory-bound.  A work unit is 8 consecutive channels of one row (16 in the
// non-interleaved layout, where a unit takes both chunks a pair spans, so
// that the in-place query update never reads a chunk another lane writes).
#include "append.hpp"
#include "launch.hpp"

namespace paq {

constexpr int kRotThreads = 256;

// One pair, each product and sum rounded to fp32 on its own.
__device__ __forceinline__ void rotate_pair(float& x, float& y, float c, float s) {
#pragma clang fp contract(off)
  const float xc = x * c, ys = y * s, yc = y * c, xs = x * s;
  x = xc - ys;
  y = yc + xs;
}

// interleaved: pairs (2j, 2j+1) of one chunk at angles k0 .. k0+3
__device__ __forceinline__ void rotate_interleaved8(float (&x)[8], const float* cs,
                                                    const float* sn, int k0) {
  const f32x4 c = *reinterpret_cast<const f32x4*>(cs + k0);
  const f32x4 s = *reinterpret_cast<const f32x4*>(sn + k0);
#pragma unroll
  for (int j = 0; j < 4; ++j) rotate_pair(x[2 * j], x[2 * j + 1], c[j], s[j]);
}

// half layout: pairs (x[j], y[j]) of two chunks at angles k0 .. k0+7
__device__ __forceinline__ void rotate_half8(float (&x)[8], float (&y)[8], const float* cs,
                                             const float* sn, int k0) {
  const f32x4 c0 = *reinterpret_cast<const f32x4*>(cs + k0);
  const f32x4 c1 = *reinterpret_cast<const f32x4*>(cs + k0 + 4);
  const f32x4 s0 = *reinterpret_cast<const f32x4*>(sn + k0);
  const f32x4 s1 = *reinterpret_cast<const f32x4*>(sn + k0 + 4);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    rotate_pair(x[j], y[j], c0[j], s0[j]);
    rotate_pair(x[4 + j], y[4 + j], c1[j], s1[j]);
  }
}

// 8 consecutive elements, rounded half-even to T
template <typename T>
__device__ __forceinline__ void store8(T* p, const float (&x)[8]) {
  if constexpr (sizeof(T) == 2) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = (uint32_t)__builtin_bit_cast(uint16_t, from_f32<T>(x[2 * i])) |
             ((uint32_t)__builtin_bit_cast(uint16_t, from_f32<T>(x[2 * i + 1])) << 16);
    *reinterpret_cast<u32x4*>(p) = (u32x4){w[0], w[1], w[2], w[3]};
  } else {
    *reinterpret_cast<f32x4*>(p) = (f32x4){x[0], x[1], x[2], x[3]};
    *reinterpret_cast<f32x4*>(p + 4) = (f32x4){x[4], x[5], x[6], x[7]};
  }
}

// rotation unit u of one query row, in place
template <typename TQ>
__device__ __forceinline__ void rotate_query_unit(TQ* q, int u, int half, bool interleaved,
                                                  const float* cs, const float* sn) {
  const int d0 = 8 * u;
  float x[8];
  load8(q + d0, x);
  if (interleaved) {
    rotate_interleaved8(x, cs, sn, d0 / 2);
    store8(q + d0, x);
  } else {
    float y[8];
    load8(q + d0 + half, y);
    rotate_half8(x, y, cs, sn, d0);
    store8(q + d0, x);
    store8(q + d0 + half, y);
  }
}

template <int KVF, int SM, typename TI>
__global__ __launch_bounds__(kRotThreads) void rotary_append_kernel(AppendArgs a) {
  const int b = blockIdx.y;
  const int q0 = a.cum_q[b];
  const int qlen = a.cum_q[b + 1] - q0;
  const int past = a.past_lens[b];              // read beside the lengths
  const int i_begin = blockIdx.x * a.tokens_per_wg;
  if (i_begin >= qlen) return;
  const int i_end = min(qlen, i_begin + a.tokens_per_wg);
  const int D = a.head_size, rd = a.rotary_dim, hkv = a.hkv, half = rd / 2;
  const bool il = a.interleaved != 0;
  const int ur = il ? rd / 8 : rd / 16;                 // rotation units per head
  const int uk = ur + (D - rd) / 8;                      // key units per head
  const int nq = a.query ? a.num_heads * ur : 0;
  const int nk = hkv * uk, nv = hkv * (D / 8);
  const int per_tok = nq + nk + nv;
  const int C = (KVF == KV_INT4) ? D / 2 : D;
  const int total = (i_end - i_begin) * per_tok;
  for (int idx = threadIdx.x; idx < total; idx += kRotThreads) {
    const int tok = i_begin + idx / per_tok;
    int u = idx % per_tok;
    const int row = q0 + tok, pos = past + tok;
    const float* cs = a.cos_cache + (size_t)pos * half;
    const float* sn = a.sin_cache + (size_t)pos * half;
    if (u < nq) {                                        // query rotation, in place
      const int h = u / ur;
      const size_t off = ((size_t)row * a.num_heads + h) * D;
      switch (a.q_dtype) {
        case DT_F32: rotate_query_unit((float*)a.query + off, u % ur, half, il, cs, sn); break;
        case DT_F16: rotate_query_unit((f16*)a.query + off, u % ur, half, il, cs, sn); break;
        default: rotate_query_unit((bf16*)a.query + off, u % ur, half, il, cs, sn); break;
      }
      continue;
    }
    u -= nq;
    const bool is_v = u >= nk;
    if (is_v) u -= nk;
    const int h = is_v ? u / (D / 8) : u / uk;
    u = is_v ? u % (D / 8) : u % uk;
    const TI* src = (const TI*)(is_v ? a.value : a.key) + ((size_t)row * hkv + h) * D;
    uint8_t* crow = cache_row((uint8_t*)(is_v ? a.value_cache : a.key_cache), a.block_table, b,
                              a.max_blocks, pos, a.block_size, hkv, h, C);
    const float* scale = is_v ? a.v_scale : a.k_scale;
    float x[8], s[8];
    if (is_v || u >= ur) {                               // values, and key channels past rd
      const int d0 = is_v ? 8 * u : rd + 8 * (u - ur);
      load8(src + d0, x);
      load_scales8<SM>(scale, h, D, d0, s);
      store_codes8<KVF>(crow, d0, x, s);
    } else if (il) {
      const int d0 = 8 * u;
      load8(src + d0, x);
      rotate_interleaved8(x, cs, sn, d0 / 2);
      load_scales8<SM>(scale, h, D, d0, s);
      store_codes8<KVF>(crow, d0, x, s);
    } else {
      const int d0 = 8 * u, d1 = d0 + half;
      float y[8];
      load8(src + d0, x);
      load8(src + d1, y);
      rotate_half8(x, y, cs, sn, d0);
      load_scales8<SM>(scale, h, D, d0, s);
      store_codes8<KVF>(crow, d0, x, s);
      load_scales8<SM>(scale, h, D, d1, s);
      store_codes8<KVF>(crow, d1, y, s);
    }
  }
}

template <int KVF, int SM>
static int launch_rot_fmt(const AppendArgs& a, dim3 grid, hipStream_t st) {
  switch (a.in_dtype) {
    case DT_F32:
      hipLaunchKernelGGL((rotary_append_kernel<KVF, SM, float>), grid, dim3(kRotThreads), 0, st, a);
      return 0;
    case DT_F16:
      hipLaunchKernelGGL((rotary_append_kernel<KVF, SM, f16>), grid, dim3(kRotThreads), 0, st, a);
      return 0;
    case DT_BF16:
      hipLaunchKernelGGL((rotary_append_kernel<KVF, SM, bf16>), grid, dim3(kRotThreads), 0, st, a);
      return 0;
  }
  return -1;
}

int launch_rotary_append(const AppendArgs& a, hipStream_t st) {
  dim3 grid((a.max_query_len + a.tokens_per_wg - 1) / a.tokens_per_wg, a.batch);
  switch (a.kv_format * 2 + a.scale_mode) {
    case KV_INT8 * 2 + SCALE_CHANNEL: return launch_rot_fmt<KV_INT8, SCALE_CHANNEL>(a, grid, st);
    case KV_INT8 * 2 + SCALE_HEAD: return launch_rot_fmt<KV_INT8, SCALE_HEAD>(a, grid, st);
    case KV_INT4 * 2 + SCALE_CHANNEL: return launch_rot_fmt<KV_INT4, SCALE_CHANNEL>(a, grid, st);
    case KV_INT4 * 2 + SCALE_HEAD: return launch_rot_fmt<KV_INT4, SCALE_HEAD>(a, grid, st);
    case KV_FP8 * 2 + SCALE_CHANNEL: return launch_rot_fmt<KV_FP8, SCALE_CHANNEL>(a, grid, st);
    case KV_FP8 * 2 + SCALE_HEAD: return launch_rot_fmt<KV_FP8, SCALE_HEAD>(a, grid, st);
  }
  return -1;
}

}  // namespace paq
