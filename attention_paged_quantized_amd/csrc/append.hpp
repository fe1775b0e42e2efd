// append.hpp -- the per-chunk steps of appending new rows to the paged cache,
// shared by the plain and the rotary quantize-append kernels: 8 consecutive
// channels of one (token, kv head) row are loaded as fp32, divided by their
// scales and stored as codes (bit contract of kv_quant_append).
#pragma once

#include "device.hpp"

namespace paq {

// 8 consecutive elements (16-byte aligned for 16-bit types, 32-byte for fp32)
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

// the scales of channels d0..d0+7 of kv head h
template <int SM>
__device__ __forceinline__ void load_scales8(const float* __restrict__ sc, int h, int head_size,
                                             int d0, float (&s)[8]) {
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
}

// The code bytes of x / s for 8 consecutive channels, as stored: 8 bytes
// (INT8, FP8) or 4 (INT4, channel 2j in the low nibble); INT4 uses w[0] only.
template <int KVF>
__device__ __forceinline__ u32x2 codes8(const float (&x)[8], const float (&s)[8]) {
  if constexpr (KVF == KV_INT8) {
    uint32_t w0 = 0, w1 = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      w0 |= (uint32_t)(quant_int(x[i] / s[i], 127.0f) & 0xFF) << (8 * i);
      w1 |= (uint32_t)(quant_int(x[4 + i] / s[4 + i], 127.0f) & 0xFF) << (8 * i);
    }
    return (u32x2){w0, w1};
  } else if constexpr (KVF == KV_INT4) {
    uint32_t w = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      w |= (uint32_t)(quant_int(x[i] / s[i], 7.0f) & 0xF) << (4 * i);
    return (u32x2){w, 0u};
  } else {
    uint32_t w0 = 0, w1 = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      w0 |= e4m3_encode(x[i] / s[i]) << (8 * i);
      w1 |= e4m3_encode(x[4 + i] / s[4 + i]) << (8 * i);
    }
    return (u32x2){w0, w1};
  }
}

// codes of x / s for channels d0..d0+7 into the cache row `row` (C bytes)
template <int KVF>
__device__ __forceinline__ void store_codes8(uint8_t* row, int d0, const float (&x)[8],
                                             const float (&s)[8]) {
  const u32x2 w = codes8<KVF>(x, s);
  if constexpr (KVF == KV_INT4) *reinterpret_cast<uint32_t*>(row + d0 / 2) = w[0];
  else *reinterpret_cast<u32x2*>(row + d0) = w;
}

// The 4 code bytes [bo, bo + 4) of a cache row (channels bo..bo+3 for INT8
// and FP8, 2 bo..2 bo+7 for INT4) in two steps: the raw input elements and
// scales behind them, then the codes (the arithmetic of store_codes8).
struct Raw4 {
  u32x4 x[2];    // up to 8 input elements (fp32: 32 bytes)
  f32x4 s[2];    // their scales
};
template <int KVF, int SM, typename TI>
__device__ __forceinline__ void load_raw4(const TI* __restrict__ x_row,
                                          const float* __restrict__ sc, int h, int head_size,
                                          int bo, Raw4& r) {
  constexpr int N = KVF == KV_INT4 ? 8 : 4;                 // channels
  const int d0 = KVF == KV_INT4 ? 2 * bo : bo;
  const u32x4* xp = reinterpret_cast<const u32x4*>(x_row + d0);
  if constexpr (N * sizeof(TI) == 32) {
    r.x[0] = xp[0]; r.x[1] = xp[1];
  } else if constexpr (N * sizeof(TI) == 16) {
    r.x[0] = xp[0];
  } else {
    const u32x2 v = *reinterpret_cast<const u32x2*>(x_row + d0);
    r.x[0] = (u32x4){v[0], v[1], 0u, 0u};
  }
  if constexpr (SM == SCALE_CHANNEL) {
    const f32x4* sp = reinterpret_cast<const f32x4*>(sc + h * head_size + d0);
    r.s[0] = sp[0];
    if constexpr (N == 8) r.s[1] = sp[1];
  } else {
    const float v = sc[h];
    r.s[0] = (f32x4){v, v, v, v};
    r.s[1] = r.s[0];
  }
}
template <int KVF, typename TI>
__device__ __forceinline__ uint32_t codes4_from(const Raw4& r) {
  constexpr int N = KVF == KV_INT4 ? 8 : 4;
  const TI* e = reinterpret_cast<const TI*>(r.x);
  float x[8], s[8];
#pragma unroll
  for (int i = 0; i < N; ++i) {
    x[i] = to_f32(e[i]);
    s[i] = r.s[i / 4][i % 4];
  }
  if constexpr (KVF == KV_INT4) {
    return codes8<KVF>(x, s)[0];
  } else {
    uint32_t w = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t c = (KVF == KV_INT8) ? (uint32_t)(quant_int(x[i] / s[i], 127.0f) & 0xFF)
                                          : e4m3_encode(x[i] / s[i]);
      w |= c << (8 * i);
    }
    return w;
  }
}

// the cache row of position t of sequence b, kv head h
__device__ __forceinline__ uint8_t* cache_row(uint8_t* cache, const int32_t* __restrict__ block_table,
                                              int b, int max_blocks, int t, int block_size,
                                              int hkv, int h, int C) {
  const int blk = block_table[(size_t)b * max_blocks + t / block_size];
  return cache + (((size_t)blk * block_size + t % block_size) * hkv + h) * C;
}

}  // namespace paq
