// device.hpp -- gfx950 device helpers shared by the paged quantized-KV kernels:
// element types, exact code->fp16/bf16 conversions, the E4M3 encoder, wave
// reductions and the MFMA operand vector types.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace paq {

typedef _Float16 f16;
typedef __bf16 bf16;
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

enum { KV_INT8 = 0, KV_INT4 = 1, KV_FP8 = 2 };
enum { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };
enum { SCALE_CHANNEL = 0, SCALE_HEAD = 1 };

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <int DT> struct dtype_of;
template <> struct dtype_of<DT_F32> { typedef float type; };
template <> struct dtype_of<DT_F16> { typedef f16 type; };
template <> struct dtype_of<DT_BF16> { typedef bf16 type; };

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(f16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ f16 from_f32<f16>(float x) { return (f16)x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  // v_perm_b32: byte k of the result is byte sel[k] of the 8-byte value {hi:lo}
  return __builtin_amdgcn_perm(hi, lo, sel);
}

template <typename T> __device__ __forceinline__ T bitcast(uint32_t x) {
  return __builtin_bit_cast(T, x);
}

// ---------------------------------------------------------------------------
// Quantization (bit contract of kv_quant_append).
// ---------------------------------------------------------------------------

// Round-half-even of an fp32 value to an integer code, clamped to [-m, m].
__device__ __forceinline__ int quant_int(float q, float m) {
  float r = __builtin_rintf(q);
  r = fminf(fmaxf(r, -m), m);
  return (int)r;
}

// OCP E4M3 encode with round-half-even and saturation to +-448.  Exact bit
// manipulation of the fp32 input (NaN inputs are outside the contract).
__device__ __forceinline__ uint32_t e4m3_encode(float y) {
  uint32_t u = __builtin_bit_cast(uint32_t, y);
  uint32_t sign = (u >> 24) & 0x80u;
  uint32_t a = u & 0x7fffffffu;
  uint32_t code;
  if (a >= 0x43E80000u) {            // |y| >= 464 (or inf): rounds past 448
    code = 0x7Eu;
  } else if (a < 0x3C800000u) {      // |y| < 2^-6: subnormal grid, step 2^-9
    float s = __builtin_bit_cast(float, a) * 512.0f;   // exact scaling
    code = (uint32_t)__builtin_rintf(s);              // 0..8 (8 = smallest normal)
  } else {                            // normal: keep 3 of 23 mantissa bits, RNE
    uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u);
    code = (r >> 20) - (120u << 3);   // rebias exponent 127 -> 7
  }
  return sign | code;
}

// OCP E4M3 code -> fp32 (exact): normal values rebias the exponent 7 -> 127,
// subnormals are m * 2^-9.  NaN codes are never produced by the quantizer.
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  const uint32_t e = (c >> 3) & 0xFu, m = c & 7u;
  const float mag = e ? __builtin_bit_cast(float, ((e + 120u) << 23) | (m << 20))
                      : (float)m * 0x1p-9f;
  return (c & 0x80u) ? -mag : mag;
}

// ---------------------------------------------------------------------------
// Exact code -> fp16 conversions ("magic number" construction: the fp16 value
// with exponent field 25 (0x6400 = 1024.0) has unit spacing, so placing an
// unsigned integer u < 1024 in its mantissa bits gives exactly 1024 + u).
// ---------------------------------------------------------------------------

// Two signed bytes (already XOR-ed with 0x80, so u = code + 128) selected by
// `sel` -> fp16 pair (code0, code1).  sel picks bytes of x into bytes 0 and 2.
__device__ __forceinline__ f16x2 i8pair_to_f16x2(uint32_t x_biased, uint32_t sel02) {
  uint32_t m = perm(0x64646464u, x_biased, sel02);
  f16x2 v = bitcast<f16x2>(m);
  return v - (f16x2){(f16)1152.0f, (f16)1152.0f};
}

// Eight packed INT4 codes (two's-complement nibbles; nibble k of w is code k)
// -> four exact fp16 pairs o[0] = (c0, c4), o[1] = (c1, c5), o[2] = (c2, c6),
// o[3] = (c3, c7).  One v_bitop3 per pair computes, bit by bit,
// mask ? (w ^ k) : k, with k holding the 0x6400 exponent outside the nibble
// fields and the nibble's sign bit inside them: that places u = code + 8 in the
// mantissa of 1024.0 (nibbles 0, 2, 4, 6: value 1024 + u) or 16u there
// (nibbles 1, 3, 5, 7: value 1024 + 16u, scaled back by an exact fma).
__device__ __forceinline__ void int4x8_to_f16x2x4(uint32_t w, f16x2 (&o)[4]) {
  // truth table of (S1 ? S0 ^ S2 : S2) with S0, S1, S2 = 0xF0, 0xCC, 0xAA
  constexpr uint32_t kMaskedXor = 0x6A;
  const uint32_t w8 = w >> 8;
  const uint32_t p0 = __builtin_amdgcn_bitop3_b32(w, 0x000F000Fu, 0x64086408u, kMaskedXor);
  const uint32_t p1 = __builtin_amdgcn_bitop3_b32(w, 0x00F000F0u, 0x64806480u, kMaskedXor);
  const uint32_t p2 = __builtin_amdgcn_bitop3_b32(w8, 0x000F000Fu, 0x64086408u, kMaskedXor);
  const uint32_t p3 = __builtin_amdgcn_bitop3_b32(w8, 0x00F000F0u, 0x64806480u, kMaskedXor);
  const f16x2 lo_bias = (f16x2){(f16)-1032.0f, (f16)-1032.0f};
  const f16x2 hi_scale = (f16x2){(f16)0.0625f, (f16)0.0625f};
  const f16x2 hi_bias = (f16x2){(f16)-72.0f, (f16)-72.0f};
  o[0] = bitcast<f16x2>(p0) + lo_bias;
  o[1] = __builtin_elementwise_fma(bitcast<f16x2>(p1), hi_scale, hi_bias);
  o[2] = bitcast<f16x2>(p2) + lo_bias;
  o[3] = __builtin_elementwise_fma(bitcast<f16x2>(p3), hi_scale, hi_bias);
}

// The same eight codes as affine fp16 images without the final fixups:
// o[0], o[2] = 1032 + code (nibbles 0, 2, 4, 6), o[1], o[3] = 1152 + 16 code
// (nibbles 1, 3, 5, 7); one v_bitop3 per pair.
__device__ __forceinline__ void int4x8_to_f16x2x4_raw(uint32_t w, f16x2 (&o)[4]) {
  constexpr uint32_t kMaskedXor = 0x6A;
  const uint32_t w8 = w >> 8;
  o[0] = bitcast<f16x2>(__builtin_amdgcn_bitop3_b32(w, 0x000F000Fu, 0x64086408u, kMaskedXor));
  o[1] = bitcast<f16x2>(__builtin_amdgcn_bitop3_b32(w, 0x00F000F0u, 0x64806480u, kMaskedXor));
  o[2] = bitcast<f16x2>(__builtin_amdgcn_bitop3_b32(w8, 0x000F000Fu, 0x64086408u, kMaskedXor));
  o[3] = bitcast<f16x2>(__builtin_amdgcn_bitop3_b32(w8, 0x00F000F0u, 0x64806480u, kMaskedXor));
}

// E4M3 bytes at bits [8,16) and [24,32) of y -> fp16 pair holding value / 256
// (exact, subnormal for the smallest codes).
__device__ __forceinline__ f16x2 e4m3_hi_bytes_to_f16x2_raw(uint32_t y) {
  return bitcast<f16x2>((y & 0x80008000u) | ((y >> 1) & 0x3F803F80u));
}

// E4M3 bytes placed at bits [8,16) and [24,32) of y -> fp16 pair (exact):
// the fp16 with bits sign<<15 | (code&0x7F)<<7 equals value * 2^-8.
__device__ __forceinline__ f16x2 e4m3_hi_bytes_to_f16x2(uint32_t y) {
  uint32_t m = (y & 0x80008000u) | ((y >> 1) & 0x3F803F80u);
  f16x2 v = bitcast<f16x2>(m);
  return v * (f16x2){(f16)256.0f, (f16)256.0f};
}

// ---------------------------------------------------------------------------
// Wave (64-lane) reductions.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Reductions over the four 16-lane rows of a wave (lanes l, l^16, l^32, l^48).
__device__ __forceinline__ float rows_max(float v) {
  v = fmaxf(v, __shfl_xor(v, 16, 64));
  return fmaxf(v, __shfl_xor(v, 32, 64));
}
__device__ __forceinline__ float rows_sum(float v) {
  v += __shfl_xor(v, 16, 64);
  return v + __shfl_xor(v, 32, 64);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------
// Device-coherent stores and loads (agent-scope relaxed atomics: global_store /
// global_load with sc1, coherent across the XCDs' L2 caches) for the values
// one workgroup hands to another inside a launch.  Ordering comes from the
// writer waiting for its stores (s_waitcnt vmcnt(0)) before it signals, not
// from a fence: an agent-scope fence would write back and invalidate the whole
// L2 of the XCD.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void store_agent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_agent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wait_stores() {
  __builtin_amdgcn_s_waitcnt(0x0F70);            // vmcnt(0), other counters untouched
}

// ---------------------------------------------------------------------------
// Key-scale normaliser ("ONNX Runtime: INT4 Paged KV Cache", section 3: the
// per-channel key scale is folded into the query after dividing by a power of
// two of the kv head's largest scale, so the 16-bit operand cannot overflow).
// M = 2^e with e = ceil(log2 max|s|), capped at 127 (the largest fp32 power of
// two), so every finite scale -- FLT_MAX and subnormals included -- gives a
// finite M and s / M = ldexp(s, -e) exact with |s / M| < 2.  max|s| = 0 gives
// e = 0.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int scale_exponent(float smax) {
  if (!(smax > 0.f)) return 0;
  int ex;
  const float fr = frexpf(smax, &ex);                      // smax = fr * 2^ex, fr in [0.5, 1)
  return min(fr == 0.5f ? ex - 1 : ex, 127);
}

// scale_exponent of kv head g's key scales, computed by a whole workgroup
// (blockDim.x a multiple of 64, >= D; *slot is LDS scratch).  Every thread
// returns the same value.
// (key_scale_exponent_of: the same from the value this thread loaded -- its
// channel's |scale| for threads below D, else 0; the per-head |scale|)
template <int SM>
__device__ __forceinline__ int key_scale_exponent_of(float m, int* slot) {
  if constexpr (SM == SCALE_CHANNEL) {
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    if (threadIdx.x == 0) *slot = 0;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) atomicMax(slot, __float_as_int(m));
    __syncthreads();
    m = __int_as_float(*slot);
  }
  return scale_exponent(m);
}

template <int SM>
__device__ __forceinline__ int key_scale_exponent(const float* k_scale, int g, int D, int* slot) {
  float m;
  if constexpr (SM == SCALE_CHANNEL) {
    m = (int)threadIdx.x < D ? fabsf(k_scale[g * D + threadIdx.x]) : 0.f;
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    if (threadIdx.x == 0) *slot = 0;
    __syncthreads();
    // non-negative floats order like their bit patterns
    if ((threadIdx.x & 63) == 0) atomicMax(slot, __float_as_int(m));
    __syncthreads();
    m = __int_as_float(*slot);
  } else {
    m = fabsf(k_scale[g]);
  }
  return scale_exponent(m);
}

// The factor that turns a raw score (query' . key operand) into log2 units:
// softmax_scale * 2^e * log2(e) / key_operand_scale, clamped into
// [FLT_MIN, FLT_MAX].  Past FLT_MAX every score gap the raw scores can
// resolve is already a hard argmax; below FLT_MIN every logit is below
// 2^-100 and the softmax is uniform to fp32 precision.  Keeping the factor
// finite and positive is what lets the kernels form every exponent as
// (raw - raw_max) * factor without an infinity or a NaN.
__device__ __forceinline__ float score_factor_log2(float softmax_scale, int e, float key_op_scale) {
  const float r = ldexpf(softmax_scale * 1.4426950408889634f / key_op_scale, e);
  return fminf(fmaxf(r, 0x1p-126f), 0x1.fffffep127f);
}

// Softmax numerators 2^(c * (s - m) + e) in an fp16 P: s a raw score, m the
// running maximum of the raw scores, c the score factor (log2 units, finite,
// see score_factor_log2) and e the scale exponent of P.  While |c * m| stays
// below kHugeScoreLog2 they are computed as exp2(fma(s, c, e - c * m)): the
// exact product against the rounded c * m and the rounding of e - c * m each
// stay within 1/8, so with the lazy-maximum slack the argument stays under
// 15.5 and P under 2^16.  Past it (key scales far beyond the 16-bit ranges: a
// hard-argmax softmax) the difference s - m is taken first -- exact near the
// maximum (Sterbenz) -- and only then scaled, so no product of a huge factor
// and a huge score is ever formed and nothing overflows.
constexpr float kHugeScoreLog2 = 0x1p22f;
__device__ __forceinline__ float safe_score_arg(float s, float m, float c, float e) {
#pragma clang fp contract(off)
  return (s - m) * c + e;
}

}  // namespace paq
