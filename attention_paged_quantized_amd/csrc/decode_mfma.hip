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

constexpr int kDecMaxGroup = 8;
constexpr float kMaxSlack = 8.0f;          // lazy running-max slack (log2 units)
constexpr float kPScaleLog2 = 7.0f;        // fp16 P = p * 2^7, p <= 2^8 -> <= 2^15

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

// ---------------------------------------------------------------------------
// Streaming through LDS.  Every wave owns a private ring of two tile slots.
// Tiles are copied HBM -> LDS with global_load_lds_dwordx4 (16 bytes per lane
// straight into LDS, no registers held while in flight), two tiles ahead of the
// one being computed.  A slot holds the 32 K rows then the 32 V rows of one
// tile, row-major; the 16-byte chunks of row r are stored XOR-swizzled by
// (r mod chunks-per-row) so that the operand reads below are free of bank
// conflicts.  The compiler does not track LDS-DMA completion, so the kernel
// waits on vmcnt itself (in-order completion of vector memory loads).
// ---------------------------------------------------------------------------
template <int KVF, int D> struct Ring {
  using Geo = KvGeom<KVF, D>;
  static constexpr int C = Geo::C;
  static constexpr int CH = C / 16;             // 16-byte chunks per row
  static constexpr int RPI = 64 / CH;           // rows per DMA instruction
  static constexpr int NI = 32 / RPI;           // DMA instructions per 32 rows
  static constexpr int SLOT = 64 * C;           // K rows + V rows
};

__device__ __forceinline__ void wait_vmcnt_le(int n) {
  // s_waitcnt with only the vector-memory counter limited (gfx9 encoding:
  // vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] at [15:14])
  switch (n) {
    case 0: __builtin_amdgcn_s_waitcnt(0x0F70); break;
    case 1: __builtin_amdgcn_s_waitcnt(0x0F71); break;
    case 2: __builtin_amdgcn_s_waitcnt(0x0F72); break;
    case 4: __builtin_amdgcn_s_waitcnt(0x0F74); break;
    case 8: __builtin_amdgcn_s_waitcnt(0x0F78); break;
    default: __builtin_amdgcn_s_waitcnt(0x0F70); break;
  }
}

// Queue the copy of the tile starting at key k0 into `slot` (wave-uniform).
// Keys past the chunk end are clamped to its last key (a valid row).
struct TileOffsets {
  size_t off0, off1;   // byte offsets of the physical blocks of the two 16-key halves
};

__device__ __forceinline__ TileOffsets tile_offsets(int k0, int kend, int lbs,
                                                    const int32_t* __restrict__ table,
                                                    uint32_t row_stride) {
  TileOffsets t;
  t.off0 = ((size_t)table[min(k0, kend - 1) >> lbs] << lbs) * row_stride;
  t.off1 = ((size_t)table[min(k0 + 16, kend - 1) >> lbs] << lbs) * row_stride;
  return t;
}

template <int KVF, int D>
__device__ __forceinline__ void issue_tile(uint8_t* slot, int k0, int kend, int lbs,
                                           TileOffsets to, const uint8_t* kbase,
                                           const uint8_t* vbase, uint32_t row_stride, int lane) {
  using R = Ring<KVF, D>;
  const int bmask = (1 << lbs) - 1;
  const size_t off0 = to.off0, off1 = to.off1;
  const int c = lane % R::CH;
#pragma unroll
  for (int i = 0; i < R::NI; ++i) {
    const int r = R::RPI * i + lane / R::CH;
    const uint32_t row = (uint32_t)(min(k0 + r, kend - 1) & bmask);
    const uint32_t lane_off = row * row_stride + 16u * (uint32_t)(c ^ (r % R::CH));
    const size_t off = (r < 16) ? off0 : off1;
    __builtin_amdgcn_global_load_lds(
        (const __attribute__((address_space(1))) void*)(kbase + off + lane_off),
        (__attribute__((address_space(3))) void*)(slot + i * 1024), 16, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < R::NI; ++i) {
    const int r = R::RPI * i + lane / R::CH;
    const uint32_t row = (uint32_t)(min(k0 + r, kend - 1) & bmask);
    const uint32_t lane_off = row * row_stride + 16u * (uint32_t)(c ^ (r % R::CH));
    const size_t off = (r < 16) ? off0 : off1;
    __builtin_amdgcn_global_load_lds(
        (const __attribute__((address_space(1))) void*)(vbase + off + lane_off),
        (__attribute__((address_space(3))) void*)(slot + 32 * R::C + i * 1024), 16, 0, 0);
  }
}

// Byte offset of byte b of row r inside a K or V block of a slot.
template <int KVF, int D>
__device__ __forceinline__ int slot_off(int r, int b) {
  using R = Ring<KVF, D>;
  return r * R::C + 16 * ((b >> 4) ^ (r % R::CH)) + (b & 15);
}

template <int NB>
__device__ __forceinline__ void lds_bytes(const uint8_t* p, uint32_t* w) {
  if constexpr (NB == 16) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(p);
    w[0] = a[0]; w[1] = a[1]; w[2] = a[2]; w[3] = a[3];
  } else if constexpr (NB == 8) {
    const u32x2 a = *reinterpret_cast<const u32x2*>(p);
    w[0] = a[0]; w[1] = a[1];
  } else if constexpr (NB == 4) {
    w[0] = *reinterpret_cast<const uint32_t*>(p);
  } else {
    static_assert(NB == 2, "row chunk");
    w[0] = *reinterpret_cast<const uint16_t*>(p);
  }
}

// One tile's operand bytes for this lane, read from a slot.
template <int KVF, int D> struct TileRaw {
  uint32_t kw[2][KvGeom<KVF, D>::KDW];   // K: key col of each 16-key half, segment grp
  uint32_t vw[8][2];                      // V: keys {4grp+r, 16+4grp+r}, channels (D/16)*col..
};

template <int KVF, int D>
__device__ __forceinline__ void read_tile(const uint8_t* slot, TileRaw<KVF, D>& t, int col,
                                          int grp) {
  using Geo = KvGeom<KVF, D>;
  using R = Ring<KVF, D>;
  constexpr int KB = Geo::KBYTES;
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int r = 16 * hh + col;
    if constexpr (KB >= 16) {
#pragma unroll
      for (int j = 0; j < KB / 16; ++j)
        lds_bytes<16>(slot + slot_off<KVF, D>(r, KB * grp + 16 * j), &t.kw[hh][4 * j]);
    } else {
      lds_bytes<KB>(slot + slot_off<KVF, D>(r, KB * grp), t.kw[hh]);
    }
  }
  const uint8_t* vs = slot + 32 * R::C;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int r = e < 4 ? 4 * grp + e : 16 + 4 * grp + (e - 4);
    t.vw[e][1] = 0;
    lds_bytes<Geo::VBYTES>(vs + slot_off<KVF, D>(r, Geo::VBYTES * col), t.vw[e]);
  }
}

// Per-wave online-softmax state: running max (log2 units), this lane's share of
// the running sum, and the O^T accumulators (lane j+16q: query column j,
// channels (D/16)*(4q+r) + nb).
template <int D> struct WaveState {
  float m = -INFINITY, l = 0.f;
  f32x4 o[D / 16];
};

template <int KVF, int D>
__device__ __forceinline__ void compute_tile(const TileRaw<KVF, D>& t, int k0, int kend,
                                             float c2, const f16x8 (&qhi)[D / 32],
                                             const f16x8 (&qlo)[D / 32], WaveState<D>& st,
                                             int grp) {
  constexpr int NQK = D / 32, NPV = D / 16;
  // S^T = K Q'^T (hi + lo); the two 16-key halves are independent chains
  f32x4 s0 = (f32x4){0.f, 0.f, 0.f, 0.f}, s1 = s0;
#pragma unroll
  for (int m = 0; m < NQK; ++m) {
    const f16x8 k0op = k_operand<KVF, D>(t.kw[0], m);
    const f16x8 k1op = k_operand<KVF, D>(t.kw[1], m);
    s0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(k0op, qhi[m], s0, 0, 0, 0);
    s1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(k1op, qhi[m], s1, 0, 0, 0);
    s0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(k0op, qlo[m], s0, 0, 0, 0);
    s1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(k1op, qlo[m], s1, 0, 0, 0);
  }
  // mask keys past the chunk (raw scores; c2 > 0 so maxima commute with it)
  float v[8];
  float lm = -INFINITY;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    v[r] = (k0 + 4 * grp + r < kend) ? s0[r] : -INFINITY;
    v[4 + r] = (k0 + 16 + 4 * grp + r < kend) ? s1[r] : -INFINITY;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) lm = fmaxf(lm, v[i]);
  lm *= c2;
  // The reference maximum of a column is shared by its four lane rows and only
  // moves when a score exceeds it by more than kMaxSlack (log2 units): then the
  // rows exchange their maxima and the accumulators are rescaled.  Otherwise
  // p = 2^(s - m) <= 2^kMaxSlack, which the 2^7-scaled fp16 P holds.
  if (__ballot(lm > st.m + kMaxSlack)) {
    const float m_new = fmaxf(st.m, rows_max(lm));
    const float alpha = fast_exp2(st.m - m_new);         // 0 on the first update
    st.m = m_new;
    st.l *= alpha;
#pragma unroll
    for (int i = 0; i < NPV; ++i) st.o[i] *= alpha;
  }
  // P' = 2^7 * 2^(s*c2 - m); the running sum carries the same factor
  const float bias = kPScaleLog2 - st.m;
  f16x8 pop;
  float psum = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float p = fast_exp2(fmaf(v[i], c2, bias));
    psum += p;
    pop[i] = (f16)p;
  }
  st.l += psum;
  // O^T += V^T P^T
  f16x8 vop[NPV];
  v_operands<KVF, D>(t.vw, vop);
#pragma unroll
  for (int nbk = 0; nbk < NPV; ++nbk)
    st.o[nbk] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vop[nbk], pop, st.o[nbk], 0, 0, 0);
}

// Fold the key scale into the query: Q' = Q * s / M_h with M_h the power of
// two >= max|s| of kv head h, split into fp16 hi + lo parts in the QK B-operand
// layout (lane col+16*grp: query column col, channels of segment grp).
template <int D, int KVF, int SM, typename TQ>
__device__ __forceinline__ void fold_query(const AttnArgs& a, int h, int q0, int G, int col,
                                           int grp, f16x8 (&qhi)[D / 32], f16x8 (&qlo)[D / 32],
                                           float& Mh) {
  constexpr int NQK = D / 32;
  const int H = a.num_heads;
  // ---- fold the key scale into the query: Q' = Q * s / M, split hi + lo ----
  // lane (col, grp) holds query column col, channels [(D/4)*grp, (D/4)*(grp+1))
  constexpr int SEG = D / 4;
  float sv[SEG];
  float smax;
  if constexpr (SM == SCALE_CHANNEL) {
    const f32x4* sp = reinterpret_cast<const f32x4*>(a.k_scale + h * D + SEG * grp);
#pragma unroll
    for (int i = 0; i < SEG / 4; ++i) {
      const f32x4 x = sp[i];
      sv[4 * i] = x[0]; sv[4 * i + 1] = x[1]; sv[4 * i + 2] = x[2]; sv[4 * i + 3] = x[3];
    }
    smax = 0.f;
#pragma unroll
    for (int i = 0; i < SEG; ++i) smax = fmaxf(smax, fabsf(sv[i]));
    smax = rows_max(smax);
  } else {
    smax = fabsf(a.k_scale[h]);
#pragma unroll
    for (int i = 0; i < SEG; ++i) sv[i] = a.k_scale[h];
  }
  int ex;
  const float fr = frexpf(smax, &ex);                      // smax = fr * 2^ex, fr in [0.5,1)
  Mh = (smax == 0.f) ? 1.f : ldexpf(1.f, fr == 0.5f ? ex - 1 : ex);
  const float invM = 1.f / Mh;                             // exact (power of two)
  {
    float qv[SEG];
#pragma unroll
    for (int i = 0; i < SEG; ++i) qv[i] = 0.f;
    if (col < G) {
      const TQ* q = reinterpret_cast<const TQ*>(a.query) + ((size_t)q0 * H + h * G + col) * D +
                    SEG * grp;
#pragma unroll
      for (int i = 0; i < SEG / 8; ++i) {
        const u32x4 x = reinterpret_cast<const u32x4*>(q)[i];
        const TQ* e = reinterpret_cast<const TQ*>(&x);
#pragma unroll
        for (int j = 0; j < 8; ++j) qv[8 * i + j] = to_f32(e[j]);
      }
    }
#pragma unroll
    for (int m = 0; m < NQK; ++m) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int c = qk_channel<KVF, D>(0, m, e);        // channel within the segment
        const float x = qv[c] * (sv[c] * invM);
        const f16 hi = (f16)x;
        qhi[m][e] = hi;
        qlo[m][e] = (f16)(x - (float)hi);
      }
    }
  }
}

template <int D, int KVF, int SM, typename TQ, int NW, int NS, int HP>
__global__ __launch_bounds__(NW * 64) void decode_mfma_kernel(AttnArgs a,
                                                             const int32_t* __restrict__ block_table) {
  using Geo = KvGeom<KVF, D>;
  using R = Ring<KVF, D>;
  constexpr int C = Geo::C, NQK = Geo::NQK, NPV = Geo::NPV;
  // HP kv heads per workgroup (2 when a head's cache row is shorter than a
  // 128-byte line: both heads' halves of every line are then read by the
  // same CU); NW / HP waves per head
  constexpr int NWH = NW / HP;
  const int wave_all = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = blockIdx.x * HP + wave_all / NWH, b = blockIdx.y, chunk = blockIdx.z;
  const int q0 = a.cum_q[b];
  if (a.cum_q[b + 1] == q0) return;                       // no new token: no rows
  const int kv_len = a.past_lens[b] + 1;
  const int bs = a.block_size, hkv = a.hkv, H = a.num_heads;
  const int G = H / hkv;
  const int nb = (kv_len + bs - 1) / bs;
  const int S = a.num_splits;
  const int kbeg = (int)(((long)chunk * nb) / S) * bs;
  const int kend = min(kv_len, (int)(((long)(chunk + 1) * nb) / S) * bs);
  const int lane = threadIdx.x & 63;
  const int wave = wave_all % NWH;                          // wave index within its head
  const int col = lane & 15, grp = lane >> 4;
  const int32_t* __restrict__ table = block_table + (size_t)b * a.max_blocks;
  const int lbs = a.block_size_log2;
  const uint32_t row_stride = (uint32_t)(hkv * C);         // bytes between tokens
  const uint8_t* kbase = a.key_cache + (size_t)h * C;
  const uint8_t* vbase = a.value_cache + (size_t)h * C;
  constexpr int stride = 32 * NWH;

  constexpr int WAVE_BYTES = NS * R::SLOT;                 // NS slots per wave
  __shared__ __attribute__((aligned(16))) uint8_t ring[NW][WAVE_BYTES];
  uint8_t* myring = ring[wave_all];

  // start streaming this wave's first NS tiles before the set-up work
  const int k_first = kbeg + 32 * wave;
  if (kbeg < kend) {
#pragma unroll
    for (int j = 0; j < NS; ++j)
      issue_tile<KVF, D>(myring + j * R::SLOT, k_first + j * stride, kend, lbs,
                         tile_offsets(k_first + j * stride, kend, lbs, table, row_stride), kbase,
                         vbase, row_stride, lane);
  }

  f16x8 qhi[NQK], qlo[NQK];
  float Mh;
  fold_query<D, KVF, SM, TQ>(a, h, q0, G, col, grp, qhi, qlo, Mh);
  const float c2 = a.softmax_scale * Mh * kLog2e;          // score -> log2 units

  // ---- per-wave online softmax over this wave's tiles ----
  WaveState<D> st;
#pragma unroll
  for (int i = 0; i < NPV; ++i) st.o[i] = (f32x4){0.f, 0.f, 0.f, 0.f};
  if (kbeg < kend) {
    int cur = 0;
    // block offsets of the tile issued next, fetched one iteration early
    TileOffsets nxt = tile_offsets(k_first + NS * stride, kend, lbs, table, row_stride);
    for (int k = k_first; k < kend; k += stride) {
      // this tile's copies are done once at most the later tiles' remain
      __builtin_amdgcn_sched_barrier(0);
      wait_vmcnt_le((NS - 1) * 2 * R::NI);
      __builtin_amdgcn_sched_barrier(0);
      uint8_t* slot = myring + cur * R::SLOT;
      TileRaw<KVF, D> t;
      read_tile<KVF, D>(slot, t, col, grp);
      // the slot is refilled (NS tiles ahead) once every lane has read it
      __builtin_amdgcn_s_waitcnt(0xC07F);                  // lgkmcnt(0)
      __builtin_amdgcn_sched_barrier(0);
      issue_tile<KVF, D>(slot, k + NS * stride, kend, lbs, nxt, kbase, vbase, row_stride, lane);
      nxt = tile_offsets(k + (NS + 1) * stride, kend, lbs, table, row_stride);
      __builtin_amdgcn_sched_barrier(0);
      compute_tile<KVF, D>(t, k, kend, c2, qhi, qlo, st, grp);
      cur = (cur + 1 == NS) ? 0 : cur + 1;
    }
  }
  // drain this wave's outstanding copies before its ring is reused below
  wait_vmcnt_le(0);
  __builtin_amdgcn_sched_barrier(0);

  // ---- merge the waves of each head through LDS (each wave writes its own ring) ----
  const float l_run = rows_sum(st.l);
  __shared__ float sm_ml[NW][2][kDecMaxGroup];             // running max, sum per wave
  float* wo = reinterpret_cast<float*>(myring);             // [kDecMaxGroup][D] per wave
  static_assert(kDecMaxGroup * D * 4 <= WAVE_BYTES, "merge area");
  if (col < G) {
    if (grp == 0) { sm_ml[wave_all][0][col] = st.m; sm_ml[wave_all][1][col] = l_run; }
#pragma unroll
    for (int nbk = 0; nbk < NPV; ++nbk)
#pragma unroll
      for (int r = 0; r < 4; ++r) wo[col * D + (D / 16) * (4 * grp + r) + nbk] = st.o[nbk][r];
  }
  __syncthreads();
  for (int t = threadIdx.x; t < HP * G * D; t += NW * 64) {
    const int hs = t / (G * D), cq = (t / D) % G, d = t % D;
    const int w0 = hs * NWH;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NWH; ++w) M = fmaxf(M, sm_ml[w0 + w][0][cq]);
    float L = 0.f, O = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < NWH; ++w) {
        const float f = fast_exp2(sm_ml[w0 + w][0][cq] - M);
        L += f * sm_ml[w0 + w][1][cq];
        O += f * reinterpret_cast<const float*>(ring[w0 + w])[cq * D + d];
      }
    }
    const int ho = blockIdx.x * HP + hs;
    const int hq = ho * G + cq;
    const float vs = (SM == SCALE_CHANNEL) ? a.v_scale[ho * D + d] : a.v_scale[ho];
    const float val = (L > 0.f) ? O / L * vs : 0.f;          // both carry 2^7
    if (S == 1) {
      reinterpret_cast<TQ*>(a.out)[((size_t)q0 * H + hq) * D + d] = from_f32<TQ>(val);
    } else {
      const size_t pi = ((size_t)q0 * H + hq) * S + chunk;
      a.part_o[pi * D + d] = val;
      if (d == 0) a.part_lse[pi] = (L > 0.f) ? (M + __log2f(L) - kPScaleLog2) * kLn2 : -INFINITY;
    }
  }
}

// ---------------------------------------------------------------------------
// Split-KV decode: one wave per (kv head, chunk).  A workgroup holds the (up
// to) 8 kv heads of one (sequence, chunk), so every token row of the chunk is
// read by one CU, and each wave streams its chunk through its own LDS ring with
// no cross-wave merge or barrier.  Each wave writes the normalised partial
// output and log-sum-exp of its G query heads for the combine kernel.
// ---------------------------------------------------------------------------
constexpr int kSplitWaves = 8;

template <int D, int KVF, int SM, typename TQ, int NS>
__global__ __launch_bounds__(kSplitWaves * 64) void decode_split_kernel(
    AttnArgs a, const int32_t* __restrict__ block_table) {
  using Geo = KvGeom<KVF, D>;
  using R = Ring<KVF, D>;
  constexpr int C = Geo::C, NQK = Geo::NQK, NPV = Geo::NPV;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = blockIdx.x * kSplitWaves + wave, b = blockIdx.y, chunk = blockIdx.z;
  if (h >= a.hkv) return;                                   // no barriers below
  const int q0 = a.cum_q[b];
  if (a.cum_q[b + 1] == q0) return;                         // no new token: no rows
  const int kv_len = a.past_lens[b] + 1;
  const int bs = a.block_size, hkv = a.hkv, H = a.num_heads;
  const int G = H / hkv;
  const int nb = (kv_len + bs - 1) / bs;
  const int S = a.num_splits;
  const int kbeg = (int)(((long)chunk * nb) / S) * bs;
  const int kend = min(kv_len, (int)(((long)(chunk + 1) * nb) / S) * bs);
  const int lane = threadIdx.x & 63;
  const int col = lane & 15, grp = lane >> 4;
  const int32_t* __restrict__ table = block_table + (size_t)b * a.max_blocks;
  const int lbs = a.block_size_log2;
  const uint32_t row_stride = (uint32_t)(hkv * C);
  const uint8_t* kbase = a.key_cache + (size_t)h * C;
  const uint8_t* vbase = a.value_cache + (size_t)h * C;

  __shared__ __attribute__((aligned(16))) uint8_t ring[kSplitWaves][NS * R::SLOT];
  uint8_t* myring = ring[wave];
  if (kbeg < kend) {
#pragma unroll
    for (int j = 0; j < NS; ++j)
      issue_tile<KVF, D>(myring + j * R::SLOT, kbeg + 32 * j, kend, lbs,
                         tile_offsets(kbeg + 32 * j, kend, lbs, table, row_stride), kbase, vbase,
                         row_stride, lane);
  }
  f16x8 qhi[NQK], qlo[NQK];
  float Mh;
  fold_query<D, KVF, SM, TQ>(a, h, q0, G, col, grp, qhi, qlo, Mh);
  const float c2 = a.softmax_scale * Mh * kLog2e;

  WaveState<D> st;
#pragma unroll
  for (int i = 0; i < NPV; ++i) st.o[i] = (f32x4){0.f, 0.f, 0.f, 0.f};
  if (kbeg < kend) {
    int cur = 0;
    TileOffsets nxt = tile_offsets(kbeg + 32 * NS, kend, lbs, table, row_stride);
    for (int k = kbeg; k < kend; k += 32) {
      __builtin_amdgcn_sched_barrier(0);
      wait_vmcnt_le((NS - 1) * 2 * R::NI);
      __builtin_amdgcn_sched_barrier(0);
      uint8_t* slot = myring + cur * R::SLOT;
      TileRaw<KVF, D> t;
      read_tile<KVF, D>(slot, t, col, grp);
      __builtin_amdgcn_s_waitcnt(0xC07F);                  // lgkmcnt(0)
      __builtin_amdgcn_sched_barrier(0);
      issue_tile<KVF, D>(slot, k + 32 * NS, kend, lbs, nxt, kbase, vbase, row_stride, lane);
      nxt = tile_offsets(k + 32 * (NS + 1), kend, lbs, table, row_stride);
      __builtin_amdgcn_sched_barrier(0);
      compute_tile<KVF, D>(t, k, kend, c2, qhi, qlo, st, grp);
      cur = (cur + 1 == NS) ? 0 : cur + 1;
    }
  }
  wait_vmcnt_le(0);

  // normalised partial output and log-sum-exp of this wave's G query heads
  const float L = rows_sum(st.l);
  if (col < G) {
    const int hq = h * G + col;
    const size_t pi = ((size_t)q0 * H + hq) * S + chunk;
    const float inv = (L > 0.f) ? 1.f / L : 0.f;            // both carry 2^7
    float* po = a.part_o + pi * D;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int d0 = (D / 16) * (4 * grp + r);
#pragma unroll
      for (int nbk = 0; nbk < NPV; ++nbk) {
        const int d = d0 + nbk;
        const float vs = (SM == SCALE_CHANNEL) ? a.v_scale[h * D + d] : a.v_scale[h];
        po[d] = st.o[nbk][r] * inv * vs;
      }
    }
    if (grp == 0)
      a.part_lse[pi] = (L > 0.f) ? (st.m + __log2f(L) - kPScaleLog2) * kLn2 : -INFINITY;
  }
}

bool decode_mfma_supports(int head_size, int group, int block_size, int q_dtype) {
  return (head_size == 64 || head_size == 128) && group >= 1 && group <= kDecMaxGroup &&
         block_size >= 16 && block_size % 16 == 0 && (q_dtype == DT_F16 || q_dtype == DT_BF16);
}

template <int D, int KVF, int SM, int NW, int NS, int HP>
static int launch_dqw(const AttnArgs& a, hipStream_t st) {
  dim3 grid(a.hkv / HP, a.batch, a.num_splits);
  if (a.q_dtype == DT_F16)
    hipLaunchKernelGGL((decode_mfma_kernel<D, KVF, SM, f16, NW, NS, HP>), grid, dim3(NW * 64), 0,
                       st, a, a.block_table);
  else if (a.q_dtype == DT_BF16)
    hipLaunchKernelGGL((decode_mfma_kernel<D, KVF, SM, bf16, NW, NS, HP>), grid, dim3(NW * 64), 0,
                       st, a, a.block_table);
  else
    return -1;
  return 0;
}

// Waves per workgroup: enough tiles per wave to amortise the set-up, and at
// most one tile per wave per 256-key chunk of split decode.  Rows shorter than
// a 128-byte line (packed INT4 with D=128, any format with D=64) pair two kv
// heads per workgroup when the head count allows.
template <int D, int KVF, int SM>
static int launch_split(const AttnArgs& a, hipStream_t st) {
  dim3 grid((a.hkv + kSplitWaves - 1) / kSplitWaves, a.batch, a.num_splits);
  if (a.q_dtype == DT_F16)
    hipLaunchKernelGGL((decode_split_kernel<D, KVF, SM, f16, 2>), grid, dim3(kSplitWaves * 64), 0,
                       st, a, a.block_table);
  else if (a.q_dtype == DT_BF16)
    hipLaunchKernelGGL((decode_split_kernel<D, KVF, SM, bf16, 2>), grid, dim3(kSplitWaves * 64),
                       0, st, a, a.block_table);
  else
    return -1;
  return 0;
}

// Single pass: one workgroup per (sequence, kv head) whose waves take the
// tiles in turn and merge at the end; rows shorter than a 128-byte line
// (packed INT4 with D=128, any format with D=64) pair two kv heads per
// workgroup so both halves of every line are read by the same CU.  Split-KV:
// one wave per (kv head, chunk).
template <int D, int KVF, int SM>
static int launch_dq(const AttnArgs& a, hipStream_t st) {
  if (a.num_splits > 1) return launch_split<D, KVF, SM>(a, st);
  constexpr bool short_rows = KvGeom<KVF, D>::C < 128;
  if constexpr (short_rows) {
    if (a.hkv % 2 == 0) return launch_dqw<D, KVF, SM, 12, 2, 2>(a, st);
  }
  return launch_dqw<D, KVF, SM, 12, 1, 1>(a, st);
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
