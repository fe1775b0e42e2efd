// decode_mfma.hip -- GQA paged decode over an INT8 / packed-INT4 / FP8 cache on
// gfx950 matrix cores (v_mfma_f32_16x16x32_f16), single pass or split-KV.
//
// Work unit: one workgroup per (kv head h, sequence b, KV chunk c); its waves
// take 32-key tiles of the chunk in turn, each with its own online softmax, and
// merge through LDS at the end.  Decode is HBM-bound (every K/V byte is read
// once -- "GQA GEMV decode", why-it-is-good item 1), so the design streams the
// cache straight from HBM into registers and never repacks it:
//
// * QK^T: A = a 16-key x 32-channel tile of K (lane l: key l%16, 8 channels of
//   its row), B = the folded query Q'^T (lane l: query column l%16).  The
//   per-channel key scale is folded into the query, normalised by the power of
//   two M_h >= max|k_scale| so the fp16 operand cannot overflow ("ONNX Runtime:
//   INT4 Paged KV Cache", section 3).  Q' = Q*s/M is split into fp16 hi + lo
//   parts (two MFMAs per tile) so the fold keeps ~22 bits, which the long-
//   context INT4 case with scales up to 6e4 needs.  Codes convert exactly to
//   fp16 in registers (INT8/INT4 by the 0x6400 mantissa construction, FP8 by
//   exponent rebias).
// * The 16x16 result puts keys 4q..4q+3 of column j in lane j+16q, which is
//   exactly the B-operand layout of the PV MFMA if its 32-key K dimension is
//   ordered as {4q..4q+3, 16+4q..16+4q+3} per lane group: no cross-lane moves.
// * PV: A = V^T (lane dd+16q: 8 keys x channel (D/16)*dd + nb), B = P^T in fp16
//   scaled by 2^15 (keeps small probabilities normal; "INT8-KV Tensor-Core
//   DynamicSparseAttention", why-it-is-good item 2), fp32 accumulation.
// * Online softmax in fp32 (exp2 with the log2(e) factor folded into the
//   score scale); the rescale of the accumulators is skipped when no lane's
//   running maximum moved.
// * Split-KV ("flash decoding", "GQA GEMV decode" section 2): chunk c covers
//   blocks [c*nb/S, (c+1)*nb/S) of the sequence and writes the normalised
//   partial output and its log-sum-exp for the combine kernel.
#include "device.hpp"
#include "launch.hpp"

namespace paq {

constexpr int kDecWaves = 8;
constexpr int kDecMaxGroup = 8;

template <int KVF, int D> struct KvGeom {
  static constexpr int C = (KVF == KV_INT4) ? D / 2 : D;      // bytes per row
  static constexpr int KBYTES = C / 4;                         // per lane per key (QK)
  static constexpr int KDW = KBYTES / 4;                       // dwords
  static constexpr int VBYTES = C / 16;                        // per lane per key (PV)
  static constexpr int NQK = D / 32;                           // QK MFMAs per 16 keys
  static constexpr int NPV = D / 16;                           // PV MFMAs per 32 keys
};

// Channel of slot e (0..7) of QK MFMA m for lane group grp.
template <int KVF, int D>
__device__ __forceinline__ int qk_channel(int grp, int m, int e) {
  if constexpr (KVF == KV_INT4) {
    const int p = (e & 1) ? 4 + (e >> 1) : (e >> 1);   // slots (c0,c4),(c1,c5),...
    return (D / 4) * grp + 8 * m + p;
  } else {
    return (D / 4) * grp + 8 * m + e;
  }
}

// K tile operand for QK MFMA m: 8 fp16 values from the lane's raw row bytes.
template <int KVF, int D>
__device__ __forceinline__ f16x8 k_operand(const uint32_t* kw, int m) {
  f16x8 r;
  if constexpr (KVF == KV_INT8) {
    const uint32_t w0 = kw[2 * m] ^ 0x80808080u, w1 = kw[2 * m + 1] ^ 0x80808080u;
    f16x2 a = i8pair_to_f16x2(w0, 0x04010400u), b = i8pair_to_f16x2(w0, 0x04030402u);
    f16x2 c = i8pair_to_f16x2(w1, 0x04010400u), d = i8pair_to_f16x2(w1, 0x04030402u);
    r = (f16x8){a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
  } else if constexpr (KVF == KV_INT4) {
    const uint32_t w = kw[m] ^ 0x88888888u;
    f16x2 a = nib_to_f16x2(w, 0), b = nib_to_f16x2(w, 4);
    f16x2 c = nib_to_f16x2(w, 8), d = nib_to_f16x2(w, 12);
    r = (f16x8){a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
  } else {
    const uint32_t w0 = kw[2 * m], w1 = kw[2 * m + 1];
    f16x2 a = e4m3_hi_bytes_to_f16x2(perm(w0, w0, 0x010C000Cu));
    f16x2 b = e4m3_hi_bytes_to_f16x2(perm(w0, w0, 0x030C020Cu));
    f16x2 c = e4m3_hi_bytes_to_f16x2(perm(w1, w1, 0x010C000Cu));
    f16x2 d = e4m3_hi_bytes_to_f16x2(perm(w1, w1, 0x030C020Cu));
    r = (f16x8){a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
  }
  return r;
}

// V^T operands for all NPV MFMAs from the lane's 8 keys (slot e = key e).
// vw[e][k]: dword k of key e's D/16 channels (channel (D/16)*dd + i is byte i,
// or nibble i for INT4).
template <int KVF, int D>
__device__ __forceinline__ void v_operands(const uint32_t (&vw)[8][2], f16x8 (&vop)[D / 16]) {
  constexpr int NPV = D / 16;
#pragma unroll
  for (int e = 0; e < 8; e += 2) {
    if constexpr (KVF == KV_INT8 || KVF == KV_FP8) {
#pragma unroll
      for (int nb = 0; nb < NPV; nb += 2) {
        const int dw = nb / 4, sh = nb % 4;
        const uint32_t lo = vw[e][dw], hi = vw[e + 1][dw];
        if constexpr (KVF == KV_INT8) {
          // bytes [e.nb, e+1.nb, e.nb+1, e+1.nb+1]
          const uint32_t sel = (uint32_t)sh | ((4u + sh) << 8) | ((uint32_t)(sh + 1) << 16) |
                               ((5u + sh) << 24);
          const uint32_t x = perm(hi, lo, sel) ^ 0x80808080u;
          const f16x2 p0 = i8pair_to_f16x2(x, 0x04010400u);
          const f16x2 p1 = i8pair_to_f16x2(x, 0x04030402u);
          vop[nb][e] = p0[0]; vop[nb][e + 1] = p0[1];
          vop[nb + 1][e] = p1[0]; vop[nb + 1][e + 1] = p1[1];
        } else {
          // [0, e.nb, 0, e+1.nb] and the same for nb+1
          const uint32_t s0 = 0x0Cu | ((uint32_t)sh << 8) | (0x0Cu << 16) | ((4u + sh) << 24);
          const uint32_t s1 = 0x0Cu | ((uint32_t)(sh + 1) << 8) | (0x0Cu << 16) | ((5u + sh) << 24);
          const f16x2 p0 = e4m3_hi_bytes_to_f16x2(perm(hi, lo, s0));
          const f16x2 p1 = e4m3_hi_bytes_to_f16x2(perm(hi, lo, s1));
          vop[nb][e] = p0[0]; vop[nb][e + 1] = p0[1];
          vop[nb + 1][e] = p1[0]; vop[nb + 1][e + 1] = p1[1];
        }
      }
    } else {  // INT4: key e's channels are the nibbles of one dword (D=128) or half of one (D=64)
#pragma unroll
      for (int j = 0; j < NPV / 2; j += 2) {
        // bytes [e.bj, e.bj+1, e+1.bj, e+1.bj+1]
        const uint32_t sel = (uint32_t)j | ((uint32_t)(j + 1) << 8) | ((uint32_t)(4 + j) << 16) |
                             ((uint32_t)(5 + j) << 24);
        const uint32_t x = perm(vw[e + 1][0], vw[e][0], sel) ^ 0x88888888u;
        const f16x2 c0 = nib_to_f16x2(x, 0), c1 = nib_to_f16x2(x, 4);
        const f16x2 c2 = nib_to_f16x2(x, 8), c3 = nib_to_f16x2(x, 12);
        vop[2 * j][e] = c0[0]; vop[2 * j][e + 1] = c0[1];
        vop[2 * j + 1][e] = c1[0]; vop[2 * j + 1][e + 1] = c1[1];
        vop[2 * j + 2][e] = c2[0]; vop[2 * j + 2][e + 1] = c2[1];
        vop[2 * j + 3][e] = c3[0]; vop[2 * j + 3][e + 1] = c3[1];
      }
    }
  }
}

template <int NB>
__device__ __forceinline__ void load_bytes(const uint8_t* p, uint32_t* w) {
  if constexpr (NB == 32) {
    u32x4 a = *reinterpret_cast<const u32x4*>(p);
    u32x4 b = *reinterpret_cast<const u32x4*>(p + 16);
    w[0] = a[0]; w[1] = a[1]; w[2] = a[2]; w[3] = a[3];
    w[4] = b[0]; w[5] = b[1]; w[6] = b[2]; w[7] = b[3];
  } else if constexpr (NB == 16) {
    u32x4 a = *reinterpret_cast<const u32x4*>(p);
    w[0] = a[0]; w[1] = a[1]; w[2] = a[2]; w[3] = a[3];
  } else if constexpr (NB == 8) {
    u32x2 a = *reinterpret_cast<const u32x2*>(p);
    w[0] = a[0]; w[1] = a[1];
  } else if constexpr (NB == 4) {
    w[0] = *reinterpret_cast<const uint32_t*>(p);
  } else {
    static_assert(NB == 2, "row chunk");
    w[0] = *reinterpret_cast<const uint16_t*>(p);
  }
}

template <int D, int KVF, int SM, typename TQ>
__global__ __launch_bounds__(kDecWaves * 64) void decode_mfma_kernel(AttnArgs a) {
  using Geo = KvGeom<KVF, D>;
  constexpr int C = Geo::C, NQK = Geo::NQK, NPV = Geo::NPV;
  const int h = blockIdx.x, b = blockIdx.y, chunk = blockIdx.z;
  const int q0 = a.cum_q[b];
  if (a.cum_q[b + 1] == q0) return;                       // no new token: no rows
  const int kv_len = a.past_lens[b] + 1;
  const int bs = a.block_size, hkv = a.hkv, H = a.num_heads;
  const int G = H / hkv;
  const int nb = (kv_len + bs - 1) / bs;
  const int S = a.num_splits;
  const int kbeg = (int)(((long)chunk * nb) / S) * bs;
  const int kend = min(kv_len, (int)(((long)(chunk + 1) * nb) / S) * bs);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int32_t* table = a.block_table + (size_t)b * a.max_blocks;

  // ---- fold the key scale into the query: Q' = Q * s / M, split hi + lo ----
  float smax = 0.f;
  if constexpr (SM == SCALE_CHANNEL) {
    for (int d = lane; d < D; d += 64) smax = fmaxf(smax, fabsf(a.k_scale[h * D + d]));
    smax = wave_max(smax);
  } else {
    smax = fabsf(a.k_scale[h]);
  }
  int ex;
  const float fr = frexpf(smax, &ex);                      // smax = fr * 2^ex, fr in [0.5,1)
  const float Mh = (smax == 0.f) ? 1.f : ldexpf(1.f, fr == 0.5f ? ex - 1 : ex);
  const float invM = 1.f / Mh;                             // exact (power of two)
  f16x8 qhi[NQK], qlo[NQK];
  {
    const TQ* q = reinterpret_cast<const TQ*>(a.query) + ((size_t)q0 * H + h * G + col) * D;
#pragma unroll
    for (int m = 0; m < NQK; ++m) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float x = 0.f;
        if (col < G) {
          const int ch = qk_channel<KVF, D>(grp, m, e);
          const float s = (SM == SCALE_CHANNEL) ? a.k_scale[h * D + ch] : a.k_scale[h];
          x = to_f32(q[ch]) * (s * invM);
        }
        const f16 hi = (f16)x;
        qhi[m][e] = hi;
        qlo[m][e] = (f16)(x - (float)hi);
      }
    }
  }
  const float c2 = a.softmax_scale * Mh * kLog2e;          // score -> log2 units

  // ---- per-wave online softmax over this wave's 32-key tiles ----
  float m_run = -INFINITY, l_run = 0.f;
  f32x4 o[NPV];
#pragma unroll
  for (int i = 0; i < NPV; ++i) o[i] = (f32x4){0.f, 0.f, 0.f, 0.f};

  const size_t row_stride = (size_t)hkv * C;               // bytes between tokens
  const uint8_t* kbase = a.key_cache + (size_t)h * C;
  const uint8_t* vbase = a.value_cache + (size_t)h * C;

  for (int k0 = kbeg + 32 * wave; k0 < kend; k0 += 32 * kDecWaves) {
    // physical blocks of the two 16-key halves (clamped into the chunk)
    const int kc0 = min(k0, kend - 1), kc1 = min(k0 + 16, kend - 1);
    const size_t blk0 = (size_t)table[kc0 / bs], blk1 = (size_t)table[kc1 / bs];
    // K rows: lane -> key (col) of each half, byte segment grp
    uint32_t kw[2][Geo::KDW];
    {
      const int key0 = min(k0 + col, kend - 1), key1 = min(k0 + 16 + col, kend - 1);
      const uint8_t* p0 = kbase + (blk0 * bs + key0 % bs) * row_stride + Geo::KBYTES * grp;
      const uint8_t* p1 = kbase + (blk1 * bs + key1 % bs) * row_stride + Geo::KBYTES * grp;
      load_bytes<Geo::KBYTES>(p0, kw[0]);
      load_bytes<Geo::KBYTES>(p1, kw[1]);
    }
    // V rows: lane (dd, grp) -> keys {4grp+r, 16+4grp+r}, channels (D/16)*dd..
    uint32_t vw[8][2];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int key = min(k0 + (e < 4 ? 4 * grp + e : 16 + 4 * grp + (e - 4)), kend - 1);
      const size_t blk = e < 4 ? blk0 : blk1;
      const uint8_t* p = vbase + (blk * bs + key % bs) * row_stride + Geo::VBYTES * col;
      vw[e][1] = 0;
      load_bytes<Geo::VBYTES>(p, vw[e]);
    }
    // S^T = K Q'^T (hi + lo)
    f32x4 s[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      f32x4 acc = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m = 0; m < NQK; ++m) {
        const f16x8 kop = k_operand<KVF, D>(kw[hh], m);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop, qhi[m], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop, qlo[m], acc, 0, 0, 0);
      }
      s[hh] = acc;
    }
    // scale, mask, tile maximum per query column
    float mt = -INFINITY;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = k0 + 16 * hh + 4 * grp + r;
        const float v = key < kend ? s[hh][r] * c2 : -INFINITY;
        s[hh][r] = v;
        mt = fmaxf(mt, v);
      }
    mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    const float m_new = fmaxf(m_run, mt);
    const float alpha = fast_exp2(m_run - m_new);          // 0 on the first tile
    m_run = m_new;
    f16x8 pop;
    float psum = 0.f;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = fast_exp2(s[hh][r] - m_new);
        psum += p;
        pop[4 * hh + r] = (f16)(p * 32768.0f);
      }
    l_run = l_run * alpha + psum;
    if (__ballot(alpha != 1.0f)) {
#pragma unroll
      for (int i = 0; i < NPV; ++i) o[i] *= alpha;
    }
    // O^T += V^T P^T
    f16x8 vop[NPV];
    v_operands<KVF, D>(vw, vop);
#pragma unroll
    for (int nbk = 0; nbk < NPV; ++nbk)
      o[nbk] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vop[nbk], pop, o[nbk], 0, 0, 0);
  }

  // ---- merge the waves through LDS ----
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  __shared__ float sm_m[kDecWaves][kDecMaxGroup], sm_l[kDecWaves][kDecMaxGroup];
  __shared__ float sm_o[kDecWaves][kDecMaxGroup][D];
  if (col < G) {
    if (grp == 0) { sm_m[wave][col] = m_run; sm_l[wave][col] = l_run; }
#pragma unroll
    for (int nbk = 0; nbk < NPV; ++nbk)
#pragma unroll
      for (int r = 0; r < 4; ++r) sm_o[wave][col][(D / 16) * (4 * grp + r) + nbk] = o[nbk][r];
  }
  __syncthreads();
  for (int t = threadIdx.x; t < G * D; t += kDecWaves * 64) {
    const int cq = t / D, d = t % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) M = fmaxf(M, sm_m[w][cq]);
    float L = 0.f, O = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kDecWaves; ++w) {
        const float f = fast_exp2(sm_m[w][cq] - M);
        L += f * sm_l[w][cq];
        O += f * sm_o[w][cq][d];
      }
    }
    const int hq = h * G + cq;
    const float vs = (SM == SCALE_CHANNEL) ? a.v_scale[h * D + d] : a.v_scale[h];
    const float val = (L > 0.f) ? O * (1.0f / 32768.0f) / L * vs : 0.f;
    if (S == 1) {
      reinterpret_cast<TQ*>(a.out)[((size_t)q0 * H + hq) * D + d] = from_f32<TQ>(val);
    } else {
      const size_t pi = ((size_t)q0 * H + hq) * S + chunk;
      a.part_o[pi * D + d] = val;
      if (d == 0) a.part_lse[pi] = (L > 0.f) ? (M + __log2f(L)) * kLn2 : -INFINITY;
    }
  }
}

bool decode_mfma_supports(int head_size, int group, int block_size, int q_dtype) {
  return (head_size == 64 || head_size == 128) && group >= 1 && group <= kDecMaxGroup &&
         block_size >= 16 && block_size % 16 == 0 && (q_dtype == DT_F16 || q_dtype == DT_BF16);
}

template <int D, int KVF, int SM>
static int launch_dq(const AttnArgs& a, hipStream_t st) {
  dim3 grid(a.hkv, a.batch, a.num_splits);
  if (a.q_dtype == DT_F16)
    hipLaunchKernelGGL((decode_mfma_kernel<D, KVF, SM, f16>), grid, dim3(kDecWaves * 64), 0, st, a);
  else if (a.q_dtype == DT_BF16)
    hipLaunchKernelGGL((decode_mfma_kernel<D, KVF, SM, bf16>), grid, dim3(kDecWaves * 64), 0, st, a);
  else
    return -1;
  return 0;
}

template <int D>
static int launch_d(const AttnArgs& a, hipStream_t st) {
  switch (a.kv_format * 2 + a.scale_mode) {
    case KV_INT8 * 2 + SCALE_CHANNEL: return launch_dq<D, KV_INT8, SCALE_CHANNEL>(a, st);
    case KV_INT8 * 2 + SCALE_HEAD: return launch_dq<D, KV_INT8, SCALE_HEAD>(a, st);
    case KV_INT4 * 2 + SCALE_CHANNEL: return launch_dq<D, KV_INT4, SCALE_CHANNEL>(a, st);
    case KV_INT4 * 2 + SCALE_HEAD: return launch_dq<D, KV_INT4, SCALE_HEAD>(a, st);
    case KV_FP8 * 2 + SCALE_CHANNEL: return launch_dq<D, KV_FP8, SCALE_CHANNEL>(a, st);
    case KV_FP8 * 2 + SCALE_HEAD: return launch_dq<D, KV_FP8, SCALE_HEAD>(a, st);
  }
  return -1;
}

int launch_decode_mfma(const AttnArgs& a, hipStream_t st) {
  if (!decode_mfma_supports(a.head_size, a.num_heads / a.hkv, a.block_size, a.q_dtype)) return -1;
  return a.head_size == 128 ? launch_d<128>(a, st) : launch_d<64>(a, st);
}

}  // namespace paq
