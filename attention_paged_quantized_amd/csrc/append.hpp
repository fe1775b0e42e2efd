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

// codes of x / s for channels d0..d0+7 into the cache row `row` (C bytes)
template <int KVF>
__device__ __forceinline__ void store_codes8(uint8_t* row, int d0, const float (&x)[8],
                                             const float (&s)[8]) {
  if constexpr (KVF == KV_INT8) {
    uint32_t w0 = 0, w1 = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      w0 |= (uint32_t)(quant_int(x[i] / s[i], 127.0f) & 0xFF) << (8 * i);
      w1 |= (uint32_t)(quant_int(x[4 + i] / s[4 + i], 127.0f) & 0xFF) << (8 * i);
    }
    *reinterpret_cast<u32x2*>(row + d0) = (u32x2){w0, w1};
  } else if constexpr (KVF == KV_INT4) {
    uint32_t w = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      w |= (uint32_t)(quant_int(x[i] / s[i], 7.0f) & 0xF) << (4 * i);
    *reinterpret_cast<uint32_t*>(row + d0 / 2) = w;
  } else {
    uint32_t w0 = 0, w1 = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      w0 |= e4m3_encode(x[i] / s[i]) << (8 * i);
      w1 |= e4m3_encode(x[4 + i] / s[4 + i]) << (8 * i);
    }
    *reinterpret_cast<u32x2*>(row + d0) = (u32x2){w0, w1};
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
