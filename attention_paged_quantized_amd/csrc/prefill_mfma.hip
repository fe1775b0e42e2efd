// prefill_mfma.hip -- ragged, causal, chunked prefill over an INT8 / packed-INT4
// / FP8 paged cache on gfx950 matrix cores (v_mfma_f32_32x32x16).
//
// Grid (query tiles, kv heads, sequences), sized from the exact max_query_len
// of the host cum_q ("PagedAttention FA path: exact max_query_len", section
// 1); a tile past its sequence's q_len exits at once, so zero-token sequences
// cost one early exit.  Query tiles run heaviest-first (the last tiles of a
// sequence see the most keys).
//
// Workgroup = 4 waves = 32/G tokens per wave x the G query heads of one kv head:
// the GQA group is packed into the 32 MFMA query columns of every wave.
//
// Per 64-key KV tile ("FlashInfer FP8 KV-cache prefill", repack section: convert
// once into shared memory instead of per use):
//   * all 256 threads load the codes of the next tile while the current one is
//     computed, then convert them exactly to 16-bit values in LDS (double
//     buffered): K row-major, V transposed (channel-major) with keys in the order
//     the PV operand wants; 16-byte chunks are XOR-swizzled to avoid LDS bank
//     conflicts;
//   * S^T = K Q'^T: A = 32 keys x 16 channels of K, B = Q'^T (lane: query column
//     l%32), so every lane owns one query column and reduces its softmax row
//     with a single cross-lane exchange (lanes l and l^32);
//   * the 16 scores a lane holds per 32-key block are exactly the B operand of
//     two PV MFMAs (keys {8(r/4)+4(l/32)+r%4}), so P never moves between lanes;
//   * O^T += V^T P^T with fp16 P scaled by 2^7 under a lazily refreshed running
//     maximum (rescale only when a score exceeds it by more than 2^8);
//   * causal mask (row i sees keys <= past + i) only where a tile crosses the
//     diagonal; a wave skips the math of tiles entirely above its rows.
// Key scales: per-channel scales are folded into the query (power-of-two
// normaliser M_h >= max|s|, "ONNX Runtime: INT4 Paged KV Cache", section 3);
// per-head scales go into the score factor.  Value scales are applied in the
// epilogue.  QK runs in fp16, or in bf16 for bf16 queries with per-head scales
// (then both operands are exact); PV always runs in fp16 (codes are exact).
#include "device.hpp"
#include "launch.hpp"

namespace paq {

namespace {

constexpr int kPfWaves = 4;
constexpr int kPfThreads = kPfWaves * 64;
constexpr int kBN = 64;                      // keys per KV tile
constexpr float kPfSlack = 8.0f;             // lazy running-max slack (log2 units)
constexpr float kPfPScale = 128.0f;          // fp16 P = p * 2^7

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

template <typename T> struct mfma32;
template <> struct mfma32<f16> {
  typedef f16x8 vec;
  static __device__ __forceinline__ f32x16 run(vec a, vec b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};
template <> struct mfma32<bf16> {
  typedef bf16x8 vec;
  static __device__ __forceinline__ f32x16 run(vec a, vec b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

template <int KVF, int D> struct PfGeo {
  static constexpr int C = (KVF == KV_INT4) ? D / 2 : D;     // bytes per cache row
  static constexpr int CPU = (KVF == KV_INT4) ? 32 : 16;     // channels per 16-byte unit
  static constexpr int UPR = C / 16;                         // 16-byte units per row
  static constexpr int KUNITS = kBN * UPR;                   // K units per tile
  static constexpr int KU_PER_T = (KUNITS + kPfThreads - 1) / kPfThreads;   // per thread
  static constexpr int VUNITS = (kBN / 2) * UPR;             // V units (key pairs)
  static constexpr int VU_PER_T = (VUNITS + kPfThreads - 1) / kPfThreads;
  static constexpr int KROW = D * 2;                         // bytes of a K row in LDS
  static constexpr int KCH = D / 8;                          // 16-byte chunks per K row
  static constexpr int VROW = kBN * 2;                       // bytes of a V^T row in LDS
  static constexpr int TILE = kBN * KROW + D * VROW;         // one LDS buffer
};

// 16 raw code bytes -> 16 (or 32 for INT4) channel values, as 16-bit words of
// type T (exact conversions).
template <int KVF, typename T>
__device__ __forceinline__ void decode_unit(const u32x4& w, uint32_t (&out)[PfGeo<KVF, 128>::CPU / 2]);

// INT8 -> fp16 / bf16
template <>
__device__ __forceinline__ void decode_unit<KV_INT8, f16>(const u32x4& w, uint32_t (&out)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t x = w[i] ^ 0x80808080u;
    out[2 * i] = __builtin_bit_cast(uint32_t, i8pair_to_f16x2(x, 0x04010400u));
    out[2 * i + 1] = __builtin_bit_cast(uint32_t, i8pair_to_f16x2(x, 0x04030402u));
  }
}
// INT4 -> fp16 (32 channels; channel 2j low nibble of byte j)
template <>
__device__ __forceinline__ void decode_unit<KV_INT4, f16>(const u32x4& w, uint32_t (&out)[16]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // nibble k of w[i] is channel 8i+k; emit the pairs (2j, 2j+1) as fp16
    // 1024 + (code + 8) by the 0x6400 mantissa construction
    const uint32_t x = w[i] ^ 0x88888888u;
    const uint32_t p01 = ((x & 0xFu) | ((x << 12) & 0xF0000u)) | 0x64006400u;
    const uint32_t p23 = (((x >> 8) & 0xFu) | ((x << 4) & 0xF0000u)) | 0x64006400u;
    const uint32_t p45 = (((x >> 16) & 0xFu) | ((x >> 4) & 0xF0000u)) | 0x64006400u;
    const uint32_t p67 = (((x >> 24) & 0xFu) | ((x >> 12) & 0xF0000u)) | 0x64006400u;
    const f16x2 bias = (f16x2){(f16)1032.0f, (f16)1032.0f};
    out[4 * i] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, p01) - bias);
    out[4 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, p23) - bias);
    out[4 * i + 2] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, p45) - bias);
    out[4 * i + 3] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, p67) - bias);
  }
}
// FP8 E4M3 -> fp16 (exact)
template <>
__device__ __forceinline__ void decode_unit<KV_FP8, f16>(const u32x4& w, uint32_t (&out)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __builtin_bit_cast(uint32_t, e4m3_hi_bytes_to_f16x2(perm(w[i], w[i], 0x010C000Cu)));
    out[2 * i + 1] =
        __builtin_bit_cast(uint32_t, e4m3_hi_bytes_to_f16x2(perm(w[i], w[i], 0x030C020Cu)));
  }
}
// FP8 E4M3 -> bf16 (exact, via fp32)
template <>
__device__ __forceinline__ void decode_unit<KV_FP8, bf16>(const u32x4& w, uint32_t (&out)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const bf16 a = (bf16)e4m3_to_f32((w[i] >> (16 * j)) & 0xFFu);
      const bf16 b = (bf16)e4m3_to_f32((w[i] >> (16 * j + 8)) & 0xFFu);
      out[2 * i + j] = __builtin_bit_cast(uint32_t, (bf16x2){a, b});
    }
  }
}
// bf16 QK is only used with FP8 per-head scales; the other formats never ask
// for it, but the template must exist.
template <>
__device__ __forceinline__ void decode_unit<KV_INT8, bf16>(const u32x4& w, uint32_t (&out)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const bf16 a = (bf16)(float)(int8_t)((w[i] >> (16 * j)) & 0xFFu);
      const bf16 b = (bf16)(float)(int8_t)((w[i] >> (16 * j + 8)) & 0xFFu);
      out[2 * i + j] = __builtin_bit_cast(uint32_t, (bf16x2){a, b});
    }
}
template <>
__device__ __forceinline__ void decode_unit<KV_INT4, bf16>(const u32x4& w, uint32_t (&out)[16]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t byte = (w[i] >> (8 * j)) & 0xFFu;
      const bf16 a = (bf16)(float)((int)((byte & 0xFu) ^ 8u) - 8);
      const bf16 b = (bf16)(float)((int)((byte >> 4) ^ 8u) - 8);
      out[4 * i + j] = __builtin_bit_cast(uint32_t, (bf16x2){a, b});
    }
}

// Position of key k (0..63) of a tile inside a V^T row: within each 16-key
// chunk c, slot 8*eta + j holds key 16c + 8(j/4) + 4*eta + j%4.
__device__ __forceinline__ int vt_pos(int k) {
  const int c = k >> 4, k16 = k & 15;
  const int eta = (k16 >> 2) & 1;
  const int j = 4 * (k16 >> 3) + (k16 & 3);
  return 16 * c + 8 * eta + j;
}

template <int D, int KVF, int SM, typename TQ, typename TK>
__global__ __launch_bounds__(kPfThreads, 2) void prefill_mfma_kernel(
    AttnArgs a, const int32_t* __restrict__ block_table) {
  using Geo = PfGeo<KVF, D>;
  using MK = mfma32<TK>;
  typedef typename MK::vec kvec;
  constexpr int C = Geo::C;
  constexpr int NKK = D / 16;                   // QK MFMAs per 32-key block
  constexpr int NDT = D / 32;                   // output channel tiles
  const int G = a.num_heads / a.hkv;
  const int TPW = 32 / G;                       // tokens per wave
  const int TOK = kPfWaves * TPW;               // tokens per workgroup
  const int qt = gridDim.x - 1 - blockIdx.x;    // heaviest tiles first
  const int h = blockIdx.y, b = blockIdx.z;
  const int q0 = a.cum_q[b];
  const int qlen = a.cum_q[b + 1] - q0;
  const int tok0 = qt * TOK;
  if (tok0 >= qlen) return;
  const int past = a.past_lens[b];
  const int H = a.num_heads, hkv = a.hkv, bs = a.block_size, lbs = a.block_size_log2;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, eta = lane >> 5;     // query column, k-half
  const int32_t* __restrict__ table = block_table + (size_t)b * a.max_blocks;
  const uint32_t row_stride = (uint32_t)(hkv * C);
  const uint8_t* kbase = a.key_cache + (size_t)h * C;
  const uint8_t* vbase = a.value_cache + (size_t)h * C;

  // keys this workgroup needs and this wave's causal limit
  const int tok_end = min(qlen, tok0 + TOK);
  const int kv_end = past + tok_end;                          // exclusive
  const int ntiles = (kv_end + kBN - 1) / kBN;
  const int wtok_last = min(tok_end, tok0 + (wave + 1) * TPW) - 1;
  const int wave_lim = past + wtok_last;                      // last key any row of the wave sees

  __shared__ __attribute__((aligned(16))) uint8_t lds[2][Geo::TILE];

  // ---- staging: codes of a tile -> registers -> converted LDS tile ----
  u32x4 kraw[Geo::KU_PER_T], vraw[Geo::VU_PER_T][2];
  auto load_codes = [&](int kt) {
#pragma unroll
    for (int i = 0; i < Geo::KU_PER_T; ++i) {
      const int u = tid + i * kPfThreads;
      if (Geo::KUNITS % kPfThreads && u >= Geo::KUNITS) break;
      const int k = u / Geo::UPR, c = u % Geo::UPR;
      const int key = min(kt * kBN + k, kv_end - 1);
      const size_t off = ((size_t)table[key >> lbs] << lbs | (key & (bs - 1))) * row_stride;
      kraw[i] = *reinterpret_cast<const u32x4*>(kbase + off + 16 * c);
    }
#pragma unroll
    for (int i = 0; i < Geo::VU_PER_T; ++i) {
      const int u = tid + i * kPfThreads;
      if (Geo::VUNITS % kPfThreads && u >= Geo::VUNITS) break;
      const int m = u / Geo::UPR, c = u % Geo::UPR;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int key = min(kt * kBN + 2 * m + e, kv_end - 1);
        const size_t off = ((size_t)table[key >> lbs] << lbs | (key & (bs - 1))) * row_stride;
        vraw[i][e] = *reinterpret_cast<const u32x4*>(vbase + off + 16 * c);
      }
    }
  };
  auto store_tile = [&](int buf) {
    uint8_t* kl = lds[buf];
    uint8_t* vl = lds[buf] + kBN * Geo::KROW;
#pragma unroll
    for (int i = 0; i < Geo::KU_PER_T; ++i) {
      const int u = tid + i * kPfThreads;
      if (Geo::KUNITS % kPfThreads && u >= Geo::KUNITS) break;
      const int k = u / Geo::UPR, c = u % Geo::UPR;
      uint32_t w[Geo::CPU / 2];
      decode_unit<KVF, TK>(kraw[i], w);
      // channels [CPU*c, CPU*c + CPU) = 16-byte chunks CPU*c/8 ...
#pragma unroll
      for (int j = 0; j < Geo::CPU / 8; ++j) {
        const int chunk = (Geo::CPU / 8) * c + j;
        const int phys = chunk ^ (k & (Geo::KCH - 1));
        *reinterpret_cast<u32x4*>(kl + k * Geo::KROW + 16 * phys) =
            (u32x4){w[4 * j], w[4 * j + 1], w[4 * j + 2], w[4 * j + 3]};
      }
    }
#pragma unroll
    for (int i = 0; i < Geo::VU_PER_T; ++i) {
      const int u = tid + i * kPfThreads;
      if (Geo::VUNITS % kPfThreads && u >= Geo::VUNITS) break;
      const int m = u / Geo::UPR, c = u % Geo::UPR;
      uint32_t w0[Geo::CPU / 2], w1[Geo::CPU / 2];
      decode_unit<KVF, f16>(vraw[i][0], w0);
      decode_unit<KVF, f16>(vraw[i][1], w1);
      const int pos = vt_pos(2 * m);                       // even: keys 2m, 2m+1 adjacent
#pragma unroll
      for (int j = 0; j < Geo::CPU; ++j) {
        const int d = Geo::CPU * c + j;
        const uint32_t lo = (j & 1) ? (w0[j >> 1] >> 16) : (w0[j >> 1] & 0xFFFFu);
        const uint32_t hi = (j & 1) ? (w1[j >> 1] >> 16) : (w1[j >> 1] & 0xFFFFu);
        const int phys = (pos >> 3) ^ (d & 7);
        *reinterpret_cast<uint32_t*>(vl + d * Geo::VROW + 16 * phys + 2 * (pos & 7)) =
            lo | (hi << 16);
      }
    }
  };

  if (ntiles > 0) load_codes(0);

  // ---- query operand: Q'^T columns, fold of the key scale ----
  const int my_tok = min(tok0 + wave * TPW + n / G, qlen - 1);      // clamp padded rows
  const int hq = h * G + (n % G);
  const TQ* qrow = reinterpret_cast<const TQ*>(a.query) + ((size_t)(q0 + my_tok) * H + hq) * D;
  float Mh = 1.f;
  if constexpr (SM == SCALE_CHANNEL) {
    float smax = 0.f;
    for (int d = lane; d < D; d += 64) smax = fmaxf(smax, fabsf(a.k_scale[h * D + d]));
    smax = wave_max(smax);
    int ex;
    const float fr = frexpf(smax, &ex);
    Mh = (smax == 0.f) ? 1.f : ldexpf(1.f, fr == 0.5f ? ex - 1 : ex);
  }
  const float invM = 1.f / Mh;
  kvec qop[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    const u32x4 x = *reinterpret_cast<const u32x4*>(qrow + 16 * kk + 8 * eta);
    const TQ* e = reinterpret_cast<const TQ*>(&x);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float v = to_f32(e[j]);
      if constexpr (SM == SCALE_CHANNEL) v *= a.k_scale[h * D + 16 * kk + 8 * eta + j] * invM;
      qop[kk][j] = (TK)v;
    }
  }
  const float sk = (SM == SCALE_CHANNEL) ? Mh : a.k_scale[h];
  const float c2 = a.softmax_scale * sk * kLog2e;
  const int row_lim = past + my_tok;              // last key this query column sees

  float m_run = -INFINITY, l_run = 0.f;
  f32x16 o[NDT];
#pragma unroll
  for (int i = 0; i < NDT; ++i) o[i] = (f32x16){};

  if (ntiles > 0) store_tile(0);
  __syncthreads();

  for (int kt = 0; kt < ntiles; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < ntiles) load_codes(kt + 1);
    const int key0 = kt * kBN;
    if (key0 <= wave_lim) {
      const uint8_t* kl = lds[buf];
      const uint8_t* vl = lds[buf] + kBN * Geo::KROW;
      // S^T for the two 32-key blocks
      f32x16 s[2];
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        s[st] = (f32x16){};
        const int k = 32 * st + n;
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
          const int phys = (2 * kk + eta) ^ (k & (Geo::KCH - 1));
          const kvec kop = *reinterpret_cast<const kvec*>(kl + k * Geo::KROW + 16 * phys);
          s[st] = MK::run(kop, qop[kk], s[st]);
        }
      }
      // scale, causal mask, lazy running max
      const bool diag = key0 + kBN - 1 > past + tok0 + wave * TPW;   // may need masking
      float lm = -INFINITY;
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float v = s[st][r] * c2;
          if (diag) {
            const int key = key0 + 32 * st + 8 * (r >> 2) + 4 * eta + (r & 3);
            v = key <= row_lim ? v : -INFINITY;
          }
          s[st][r] = v;
          lm = fmaxf(lm, v);
        }
      if (__ballot(lm > m_run + kPfSlack)) {
        const float m_new = fmaxf(m_run, fmaxf(lm, __shfl_xor(lm, 32, 64)));
        const float alpha = fast_exp2(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < NDT; ++i) o[i] *= alpha;
      }
      // P (fp16, scaled) in the PV B-operand layout: chunk c = regs 8c..8c+7
      f16x8 p[4];
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pv = fast_exp2(s[st][r] - m_run);
          l_run += pv;
          p[2 * st + (r >> 3)][r & 7] = (f16)(pv * kPfPScale);
        }
      // O^T += V^T P^T
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const int d = 32 * dt + n;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int phys = (2 * c + eta) ^ (d & 7);
          const f16x8 vop = *reinterpret_cast<const f16x8*>(vl + d * Geo::VROW + 16 * phys);
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vop, p[c], o[dt], 0, 0, 0);
        }
      }
    }
    if (kt + 1 < ntiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: normalise, value scale, store the rows of this wave ----
  l_run += __shfl_xor(l_run, 32, 64);
  const int tok = tok0 + wave * TPW + n / G;
  if (tok < qlen) {
    const float inv = (l_run > 0.f) ? 1.f / (l_run * kPfPScale) : 0.f;
    TQ* orow = reinterpret_cast<TQ*>(a.out) + ((size_t)(q0 + tok) * H + hq) * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int d = 32 * dt + 8 * (r >> 2) + 4 * eta + (r & 3);
        const float vs = (SM == SCALE_CHANNEL) ? a.v_scale[h * D + d] : a.v_scale[h];
        orow[d] = from_f32<TQ>(o[dt][r] * inv * vs);
      }
  }
}

}  // namespace

bool prefill_mfma_supports(int head_size, int group, int block_size, int q_dtype) {
  const bool g_ok = group == 1 || group == 2 || group == 4 || group == 8 || group == 16 ||
                    group == 32;
  return (head_size == 64 || head_size == 128) && g_ok && block_size >= 16 &&
         (q_dtype == DT_F16 || q_dtype == DT_BF16);
}

template <int D, int KVF, int SM, typename TQ, typename TK>
static int launch_pf(const AttnArgs& a, hipStream_t st) {
  const int G = a.num_heads / a.hkv;
  const int TOK = kPfWaves * (32 / G);
  dim3 grid((a.max_query_len + TOK - 1) / TOK, a.hkv, a.batch);
  hipLaunchKernelGGL((prefill_mfma_kernel<D, KVF, SM, TQ, TK>), grid, dim3(kPfThreads), 0, st, a,
                     a.block_table);
  return 0;
}

template <int D, int KVF, int SM>
static int launch_pf_q(const AttnArgs& a, hipStream_t st) {
  if (a.q_dtype == DT_F16) return launch_pf<D, KVF, SM, f16, f16>(a, st);
  if (a.q_dtype == DT_BF16) {
    // bf16 QK only when both operands stay exact: per-head key scales
    if constexpr (SM == SCALE_HEAD) return launch_pf<D, KVF, SM, bf16, bf16>(a, st);
    return launch_pf<D, KVF, SM, bf16, f16>(a, st);
  }
  return -1;
}

template <int D>
static int launch_pf_d(const AttnArgs& a, hipStream_t st) {
  switch (a.kv_format * 2 + a.scale_mode) {
    case KV_INT8 * 2 + SCALE_CHANNEL: return launch_pf_q<D, KV_INT8, SCALE_CHANNEL>(a, st);
    case KV_INT8 * 2 + SCALE_HEAD: return launch_pf_q<D, KV_INT8, SCALE_HEAD>(a, st);
    case KV_INT4 * 2 + SCALE_CHANNEL: return launch_pf_q<D, KV_INT4, SCALE_CHANNEL>(a, st);
    case KV_INT4 * 2 + SCALE_HEAD: return launch_pf_q<D, KV_INT4, SCALE_HEAD>(a, st);
    case KV_FP8 * 2 + SCALE_CHANNEL: return launch_pf_q<D, KV_FP8, SCALE_CHANNEL>(a, st);
    case KV_FP8 * 2 + SCALE_HEAD: return launch_pf_q<D, KV_FP8, SCALE_HEAD>(a, st);
  }
  return -1;
}

int launch_prefill_mfma(const AttnArgs& a, hipStream_t st) {
  if (!prefill_mfma_supports(a.head_size, a.num_heads / a.hkv, a.block_size, a.q_dtype)) return -1;
  return a.head_size == 128 ? launch_pf_d<128>(a, st) : launch_pf_d<64>(a, st);
}

}  // namespace paq
