// decode_mfma.hip -- GQA paged decode over an INT8 / packed-INT4 / FP8 cache on
// gfx950 matrix cores (v_mfma_f32_16x16x32_f16), single pass or split-KV.
//
// Work unit: a wave streams 32-key tiles of a key range for HW adjacent kv
// heads (HW = min(2, 128 / row bytes): whole 128-byte lines per copied row
// segment for 64-byte rows; the 32-byte rows of INT4 at head size 64 are
// copied as 64-byte segments, since four heads per wave need more registers
// than a wave has) with its own online softmax; the 8 waves of a workgroup
// take the tiles of a key range in turn and merge through LDS at its end.
// Decode is HBM-bound (every K/V byte is read once -- "GQA GEMV decode",
// why-it-is-good item 1), so the design streams the raw codes HBM -> LDS with
// whole-line non-temporal DMA copies, reads each lane's operand bytes from
// there and converts them in registers; nothing is written back or repacked:
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
//   scaled by 2^7 (keeps small probabilities normal; "INT8-KV Tensor-Core
//   DynamicSparseAttention", why-it-is-good item 2), fp32 accumulation.
// * Online softmax in fp32 (exp2 with the log2(e) factor folded into the
//   score scale).  The running maximum is refreshed lazily: only when a score
//   exceeds it by more than 2^8 are the maxima exchanged and the accumulators
//   rescaled, so P stays <= 2^15, inside fp16 range.
// * Split-KV ("flash decoding", "GQA GEMV decode" section 2), in two forms:
//   block-aligned chunks per sequence, or an equal share of all tiles per
//   workgroup (see the partition below); partial results are merged by the
//   last workgroup of a sequence to finish, inside the same launch.
#include <type_traits>

#include "append.hpp"
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
    f16x2 p[4];
    int4x8_to_f16x2x4(kw[m], p);
    r = (f16x8){p[0][0], p[0][1], p[1][0], p[1][1], p[2][0], p[2][1], p[3][0], p[3][1]};
  } else {
    // FP8 keys enter as value / 256 (exact); the factor is in the score scale
    const uint32_t w0 = kw[2 * m], w1 = kw[2 * m + 1];
    f16x2 a = e4m3_hi_bytes_to_f16x2_raw(perm(w0, w0, 0x010C000Cu));
    f16x2 b = e4m3_hi_bytes_to_f16x2_raw(perm(w0, w0, 0x030C020Cu));
    f16x2 c = e4m3_hi_bytes_to_f16x2_raw(perm(w1, w1, 0x010C000Cu));
    f16x2 d = e4m3_hi_bytes_to_f16x2_raw(perm(w1, w1, 0x030C020Cu));
    r = (f16x8){a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
  }
  return r;
}

// Scale of the fp16 key operand relative to the key codes (FP8: value / 256).
template <int KVF> constexpr float kKeyOperandScale = (KVF == KV_FP8) ? 1.f / 256.f : 1.f;

// The V^T operands are affine images of the value codes, v' = a_c + b_c * v:
//   INT8: 1152 + v (the 0x6400 construction without its bias subtraction);
//   INT4: 1032 + v for even channels (low nibbles), 1152 + 16 v for odd ones;
//   FP8:  v / 256.
// Since the fp16 probabilities P that multiply them sum to l exactly as
// accumulated (l is the sum of those same fp16 values), the output
// O = sum_j P_j v_j is recovered from O' = sum_j P_j v'_j as
// (O'/l - a_c) / b_c.  This saves the per-value bias arithmetic; the
// subtraction costs ~10 of fp32's 24 bits, far inside the output tolerance.
template <int KVF>
__device__ __forceinline__ float v_unbias(float o_over_l, int d) {
  if constexpr (KVF == KV_INT8) {
    return o_over_l - 1152.f;
  } else if constexpr (KVF == KV_INT4) {
    return (d & 1) ? (o_over_l - 1152.f) * 0.0625f : o_over_l - 1032.f;
  } else {
    return o_over_l * 256.f;
  }
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
          const f16x2 p0 = bitcast<f16x2>(perm(0x64646464u, x, 0x04010400u));   // 1152 + v
          const f16x2 p1 = bitcast<f16x2>(perm(0x64646464u, x, 0x04030402u));
          vop[nb][e] = p0[0]; vop[nb][e + 1] = p0[1];
          vop[nb + 1][e] = p1[0]; vop[nb + 1][e + 1] = p1[1];
        } else {
          // [0, e.nb, 0, e+1.nb] and the same for nb+1
          const uint32_t s0 = 0x0Cu | ((uint32_t)sh << 8) | (0x0Cu << 16) | ((4u + sh) << 24);
          const uint32_t s1 = 0x0Cu | ((uint32_t)(sh + 1) << 8) | (0x0Cu << 16) | ((5u + sh) << 24);
          const f16x2 p0 = e4m3_hi_bytes_to_f16x2_raw(perm(hi, lo, s0));      // v / 256
          const f16x2 p1 = e4m3_hi_bytes_to_f16x2_raw(perm(hi, lo, s1));
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
        f16x2 c[4];
        int4x8_to_f16x2x4_raw(perm(vw[e + 1][0], vw[e][0], sel), c);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          vop[2 * j + i][e] = c[i][0];
          vop[2 * j + i][e + 1] = c[i][1];
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Streaming through LDS.  Every wave owns a private ring of NS tile slots and
// streams its own key range, so no wave ever waits for another while keys are
// being read.  A wave serves HW adjacent kv heads: their HW * C bytes of a
// token row are adjacent in the cache, and HW = 128 / C makes that a whole
// 128-byte line.  Tiles of 32 tokens are copied HBM -> LDS with
// global_load_lds_dwordx4 (16 bytes per lane straight into LDS, no registers
// held while in flight): each copy instruction moves 1 KB, i.e. RPI whole row
// segments of RB bytes, CH lanes per segment.  A slot holds the 32 K row
// segments then the 32 V row segments of a tile; the 16-byte chunks of row r
// are stored XOR-swizzled by (r mod chunks-per-row) so that the operand reads
// are free of bank conflicts.  The compiler does not track LDS-DMA completion,
// so the kernel waits on vmcnt itself (vector memory loads complete in order).
// ---------------------------------------------------------------------------
template <int KVF, int D, int HW> struct StreamGeo {
  static constexpr int C = KvGeom<KVF, D>::C;   // bytes of one head's row
  static constexpr int RB = HW * C;             // bytes of the wave's row segment
  static constexpr int CH = RB / 16;            // 16-byte chunks per segment
  static constexpr int RPI = 64 / CH;           // segments per copy instruction
  static constexpr int NI = 32 / RPI;           // copy instructions per 32 rows
  static constexpr int SLOT = 64 * RB;          // K rows + V rows of one tile
  static_assert(CH >= 2 && CH <= 8 && (CH & (CH - 1)) == 0, "row segment");
};

// Cache policy of the streaming copies: non-temporal.  Every K/V byte is read
// exactly once per call, and with whole-line copies the hint measurably raises
// the achieved HBM rate.
constexpr int kNonTemporal = 2;

template <int N>
__device__ __forceinline__ void wait_vmcnt_le() {
  // s_waitcnt with only the vector-memory counter limited (gfx9 encoding:
  // vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] at [15:14])
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// LDS offset of byte b of row r's segment inside the K (or V) half of a slot.
template <int KVF, int D, int HW>
__device__ __forceinline__ int stream_off(int r, int b) {
  using SG = StreamGeo<KVF, D, HW>;
  return r * SG::RB + 16 * ((b >> 4) ^ (r % SG::CH)) + (b & 15);
}

// One wave's copies of its tiles.  Copy instruction i of a half-tile (K or V)
// fills slot bytes [1024 i, 1024 i + 1024); lane l of it loads the global
// chunk that belongs at chunk position l % CH of tile row RPI*i + l / CH.
template <int KVF, int D, int HW> struct WaveCopy {
  using SG = StreamGeo<KVF, D, HW>;
  uint32_t lane_off[SG::NI];   // row * row_stride + 16 * global chunk, per instruction
  int row[SG::NI];             // tile row of this lane's chunk, per instruction

  __device__ __forceinline__ void init(int lane, uint32_t row_stride) {
#pragma unroll
    for (int i = 0; i < SG::NI; ++i) {
      const int r = SG::RPI * i + lane / SG::CH;
      row[i] = r;
      lane_off[i] = (uint32_t)r * row_stride + 16u * (uint32_t)((lane % SG::CH) ^ (r % SG::CH));
    }
  }

  // Queue the copy of the tile at key k0 (a multiple of 32) of a key range
  // ending at kend into `slot`.  Rows at or past kend repeat row kend - 1 (a
  // valid row; their scores are masked).  Each 16-key half of the tile lies in
  // one physical block (block_size is a multiple of 16, and of 32 when a block
  // holds both halves).
  struct Blocks { int32_t b0, b1; };
  // table entry of 16-key half `half` of the tile at k0 (clamped into
  // [0, kend - 1]: an empty range reads entry 0, never used)
  __device__ __forceinline__ static int entry(int k0, int kend, int lbs, int half) {
    return max(0, min(k0 + 16 * half, kend - 1)) >> lbs;
  }
  __device__ __forceinline__ static Blocks blocks(int k0, int kend, int lbs,
                                                 const int32_t* __restrict__ table) {
    return Blocks{table[entry(k0, kend, lbs, 0)], table[entry(k0, kend, lbs, 1)]};
  }
  __device__ __forceinline__ void issue(uint8_t* slot, int k0, int kend, int lbs,
                                        const int32_t* __restrict__ table, const uint8_t* kbase,
                                        const uint8_t* vbase, uint32_t row_stride) const {
    issue(slot, k0, kend, lbs, blocks(k0, kend, lbs, table), kbase, vbase, row_stride);
  }
  __device__ __forceinline__ void issue(uint8_t* slot, int k0, int kend, int lbs, Blocks bb,
                                        const uint8_t* kbase, const uint8_t* vbase,
                                        uint32_t row_stride) const {
    const int bmask = (1 << lbs) - 1;
    const size_t blk0 = (size_t)bb.b0 << lbs;
    const size_t blk1 = (size_t)bb.b1 << lbs;
    // key k0 + r sits in row (k0 & bmask) + r of block blk0 for r < 16 and in
    // row ((k0 + 16) & bmask) + r - 16 of block blk1 otherwise
    const size_t base0 = (blk0 + (size_t)(k0 & bmask)) * row_stride;
    const size_t base1 = (blk1 + (size_t)((k0 + 16) & bmask)) * row_stride - 16 * (size_t)row_stride;
    const bool full = k0 + 32 <= kend;
#pragma unroll
    for (int i = 0; i < SG::NI; ++i) {
      size_t off;
      if (full) {
        off = (row[i] < 16 ? base0 : base1) + lane_off[i];
      } else {
        const int r = row[i];
        const uint32_t rr = (uint32_t)(min(k0 + r, kend - 1) & bmask);
        off = ((r < 16 ? blk0 : blk1) + rr) * row_stride +
              (lane_off[i] - (uint32_t)r * row_stride);
      }
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)(kbase + off),
          (__attribute__((address_space(3))) void*)(slot + i * 1024), 16, 0, kNonTemporal);
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)(vbase + off),
          (__attribute__((address_space(3))) void*)(slot + 32 * SG::RB + i * 1024), 16, 0,
          kNonTemporal);
    }
  }
};

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

// One tile's operand bytes of head hh (0..HW-1) of the wave's segment, for
// this lane, read from a slot.
template <int KVF, int D> struct TileRaw {
  uint32_t kw[2][KvGeom<KVF, D>::KDW];   // K: key col of each 16-key half, segment grp
  uint32_t vw[8][2];                      // V: keys {4grp+r, 16+4grp+r}, channels (D/16)*col..
};

template <int KVF, int D, int HW>
__device__ __forceinline__ void read_tile(const uint8_t* slot, TileRaw<KVF, D>& t, int col,
                                          int grp, int hh) {
  using Geo = KvGeom<KVF, D>;
  using SG = StreamGeo<KVF, D, HW>;
  constexpr int KB = Geo::KBYTES;
  const int hb = hh * Geo::C;                              // head's first byte in the segment
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int r = 16 * half + col;
    if constexpr (KB >= 16) {
#pragma unroll
      for (int j = 0; j < KB / 16; ++j)
        lds_bytes<16>(slot + stream_off<KVF, D, HW>(r, hb + KB * grp + 16 * j),
                      &t.kw[half][4 * j]);
    } else {
      lds_bytes<KB>(slot + stream_off<KVF, D, HW>(r, hb + KB * grp), t.kw[half]);
    }
  }
  const uint8_t* vs = slot + 32 * SG::RB;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int r = e < 4 ? 4 * grp + e : 16 + 4 * grp + (e - 4);
    t.vw[e][1] = 0;
    lds_bytes<Geo::VBYTES>(vs + stream_off<KVF, D, HW>(r, hb + Geo::VBYTES * col), t.vw[e]);
  }
}

// Per-wave online-softmax state: running maximum of the raw scores (the
// MFMA outputs, before the score factor), this lane's share of the running
// sum, and the O^T accumulators (lane j+16q: query column j, channels
// (D/16)*(4q+r) + nb).
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
  // mask keys past the range (raw scores; c2 > 0 so maxima commute with it)
  float v[8];
  float lm = -INFINITY;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    v[r] = s0[r];
    v[4 + r] = s1[r];
  }
  if (k0 + 32 > kend) {                                    // tile cut by the end (uniform)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (k0 + 4 * grp + r >= kend) v[r] = -INFINITY;
      if (k0 + 16 + 4 * grp + r >= kend) v[4 + r] = -INFINITY;
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) lm = fmaxf(lm, v[i]);
  // The reference maximum of a column is shared by its four lane rows and only
  // moves when a score exceeds it by more than kMaxSlack (log2 units): then the
  // rows exchange their maxima and the accumulators are rescaled.  Otherwise
  // p = 2^(c2 (s - m)) <= 2^kMaxSlack, which the 2^7-scaled fp16 P holds.  The
  // gap is formed on the raw scores and scaled afterwards, so it cannot
  // overflow whatever the factor.
  if (__ballot((lm - st.m) * c2 > kMaxSlack)) {
    const float m_new = fmaxf(st.m, rows_max(lm));
    const float alpha = fast_exp2((st.m - m_new) * c2);  // 0 on the first update
    st.m = m_new;
    st.l *= alpha;
#pragma unroll
    for (int i = 0; i < NPV; ++i) st.o[i] *= alpha;
  }
  // P' = 2^7 * 2^(c2 (s - m)) in fp16; the running sum adds exactly those fp16
  // values (two per dot), which the value unbiasing in the epilogue relies on
  const float mlog = st.m * c2;
  f16x8 pop;
  if (__builtin_expect(__ballot(!(fabsf(mlog) <= kHugeScoreLog2)) == 0, 1)) {
    const float bias = kPScaleLog2 - mlog;
#pragma unroll
    for (int i = 0; i < 8; ++i) pop[i] = (f16)fast_exp2(fmaf(v[i], c2, bias));
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) pop[i] = (f16)fast_exp2(safe_score_arg(v[i], st.m, c2, kPScaleLog2));
  }
  const f16x2 ones = (f16x2){(f16)1.0f, (f16)1.0f};
  float l0 = __builtin_amdgcn_fdot2((f16x2){pop[0], pop[1]}, ones, st.l, false);
  float l1 = __builtin_amdgcn_fdot2((f16x2){pop[2], pop[3]}, ones, 0.f, false);
  l0 = __builtin_amdgcn_fdot2((f16x2){pop[4], pop[5]}, ones, l0, false);
  l1 = __builtin_amdgcn_fdot2((f16x2){pop[6], pop[7]}, ones, l1, false);
  st.l = l0 + l1;
  // O^T += V^T P^T
  f16x8 vop[NPV];
  v_operands<KVF, D>(t.vw, vop);
#pragma unroll
  for (int nbk = 0; nbk < NPV; ++nbk)
    st.o[nbk] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vop[nbk], pop, st.o[nbk], 0, 0, 0);
}

// The raw inputs of the query fold for one lane (col, grp): query column col,
// channels [(D/4)*grp, (D/4)*(grp+1)), as loaded from memory.  Loading them is
// kept apart from the arithmetic so that the loads can be issued before the
// first tile copies (vector-memory results return in order).
template <int D, int SM> struct QueryRaw {
  static constexpr int SEG = D / 4;
  u32x4 q[SEG / 8];                                  // SEG 16-bit query values
  f32x4 s[SM == SCALE_CHANNEL ? SEG / 4 : 1];         // key scales (or the head's one)
};

template <int D, int SM, typename TQ>
__device__ __forceinline__ void load_query(const AttnArgs& a, int h, int q0, int G, int col,
                                           int grp, QueryRaw<D, SM>& r) {
  constexpr int SEG = D / 4;
  if constexpr (SM == SCALE_CHANNEL) {
    const f32x4* sp = reinterpret_cast<const f32x4*>(a.k_scale + h * D + SEG * grp);
#pragma unroll
    for (int i = 0; i < SEG / 4; ++i) r.s[i] = sp[i];
  } else {
    const float x = a.k_scale[h];
    r.s[0] = (f32x4){x, x, x, x};
  }
#pragma unroll
  for (int i = 0; i < SEG / 8; ++i) r.q[i] = (u32x4){0u, 0u, 0u, 0u};
  if (col < G) {
    const TQ* q = reinterpret_cast<const TQ*>(a.query) +
                  ((size_t)q0 * a.num_heads + h * G + col) * D + SEG * grp;
#pragma unroll
    for (int i = 0; i < SEG / 8; ++i) r.q[i] = reinterpret_cast<const u32x4*>(q)[i];
  }
}

// Fold the key scale into the query: Q' = Q * s / M_h with M_h = 2^e the power
// of two >= max|s| of kv head h (scale_exponent: finite for every finite
// scale), split into fp16 hi + lo parts in the QK B-operand layout (lane
// col+16*grp: query column col, channels of segment grp).  s / M_h is formed
// as ldexp(s, -e), exact also for subnormal scales.  Returns e.
template <int D, int KVF, int SM, typename TQ>
__device__ __forceinline__ int fold_loaded_query(const QueryRaw<D, SM>& r, f16x8 (&qhi)[D / 32],
                                                 f16x8 (&qlo)[D / 32]) {
  constexpr int NQK = D / 32;
  constexpr int SEG = D / 4;
  float sv[SEG];
  float smax;
  if constexpr (SM == SCALE_CHANNEL) {
#pragma unroll
    for (int i = 0; i < SEG / 4; ++i) {
      sv[4 * i] = r.s[i][0]; sv[4 * i + 1] = r.s[i][1];
      sv[4 * i + 2] = r.s[i][2]; sv[4 * i + 3] = r.s[i][3];
    }
    smax = 0.f;
#pragma unroll
    for (int i = 0; i < SEG; ++i) smax = fmaxf(smax, fabsf(sv[i]));
    smax = rows_max(smax);
  } else {
    smax = fabsf(r.s[0][0]);
#pragma unroll
    for (int i = 0; i < SEG; ++i) sv[i] = r.s[0][0];
  }
  const int e = scale_exponent(smax);
  float qv[SEG];
#pragma unroll
  for (int i = 0; i < SEG / 8; ++i) {
    const TQ* x = reinterpret_cast<const TQ*>(&r.q[i]);
#pragma unroll
    for (int j = 0; j < 8; ++j) qv[8 * i + j] = to_f32(x[j]);
  }
#pragma unroll
  for (int m = 0; m < NQK; ++m) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int c = qk_channel<KVF, D>(0, m, k);          // channel within the segment
      const float x = qv[c] * ldexpf(sv[c], -e);
      const f16 hi = (f16)x;
      qhi[m][k] = hi;
      qlo[m][k] = (f16)(x - (float)hi);
    }
  }
  return e;
}

// ---------------------------------------------------------------------------
// Partition of the keys over workgroups.  A segment is the key range of one
// (sequence, head group) pair; a piece is a contiguous run of a segment's
// 32-key tiles that one workgroup streams, its NW waves taking the tiles in
// turn.  Three partitions (the host plan picks one):
//   DEC_SINGLE  one workgroup per segment (single pass);
//   DEC_CHUNKS  S block-aligned chunks per sequence (chunk c = blocks
//               [c*nb/S, (c+1)*nb/S), "GQA GEMV decode", section 2), CPW
//               consecutive chunks per workgroup;
//   DEC_STREAM  the tiles of all segments, concatenated (sequence-major, head
//               group next), cut into N equal runs, one per workgroup: every
//               workgroup streams the same bytes whatever the lengths, and a
//               long sequence is spread over as many compute units as it
//               needs.  A workgroup's run covers whole segments (written
//               directly) and at most two partial pieces, its first and its
//               last.
// A piece that is a whole segment writes its output directly.  Otherwise it
// writes a normalised partial (raw maximum, sum, output) and counts its
// arrival; the last piece of the segment to arrive merges them all by their
// maxima and writes the output -- in the same launch.
// ---------------------------------------------------------------------------

// Where a stream-partition workgroup starts: the sequence holding global tile
// g (a wave-wide prefix sum of HG * tiles_b over the sequences with a new row,
// 64 sequences at a time), with its offsets.  Not inlined: it runs once per
// workgroup and, kept apart, leaves the streaming loop's registers alone.
struct StreamPos {
  int b;        // sequence (-1: past the last tile)
  int off;      // g - first global tile of sequence b
  int tiles;    // 32-key tiles of sequence b
  int q0, past;
};
__device__ __attribute__((noinline)) StreamPos stream_find(const int32_t* __restrict__ cum_q,
                                                          const int32_t* __restrict__ past,
                                                          int batch, int hgs, long long g) {
  const int lane = (int)(threadIdx.x & 63);
  long long before = 0;
  for (int b0 = 0; b0 < batch; b0 += 64) {
    const int b = b0 + lane;
    int tiles = 0, q0 = 0, ps = 0;
    if (b < batch) {
      q0 = cum_q[b];
      ps = past[b];
      if (cum_q[b + 1] > q0) tiles = (ps + 32) >> 5;       // ceil((past + 1) / 32)
    }
    long long incl = (long long)tiles * hgs;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const long long t = __shfl_up(incl, o, 64);
      if (lane >= o) incl += t;
    }
    const unsigned long long hit = __ballot(before + incl > g);
    if (hit) {
      const int l = (int)__builtin_ctzll(hit);
      const long long incl_l = __shfl(incl, l, 64);
      const int tiles_l = __shfl(tiles, l, 64);
      return StreamPos{b0 + l, (int)(g - (before + incl_l - (long long)tiles_l * hgs)), tiles_l,
                       __shfl(q0, l, 64), __shfl(ps, l, 64)};
    }
    before += __shfl(incl, 63, 64);
  }
  return StreamPos{-1, 0, 0, 0, 0};
}

// The stream-partition workgroup whose run holds global tile g: the largest
// w with floor(w * T / N) <= g.
__device__ __forceinline__ int stream_owner(long long g, long long T, int N) {
  return (int)(((g + 1) * (long long)N - 1) / T);
}

// Key range [k0, k1) of part j of a sequence of kv_len keys, chunk partition.
__device__ __forceinline__ void chunk_part_keys(const AttnArgs& a, int j, int kv_len, int& k0,
                                                int& k1) {
  const uint64_t nb = (uint64_t)((kv_len + a.block_size - 1) >> a.block_size_log2);
  const uint64_t S = (uint64_t)a.num_splits;
  const uint64_t c0 = (uint64_t)j * a.dec_chunks_per_part;
  const uint64_t c1 = min(S, c0 + (uint64_t)a.dec_chunks_per_part);
  k0 = (int)((c0 * nb / S) << a.block_size_log2);
  k1 = min(kv_len, (int)((c1 * nb / S) << a.block_size_log2));
}

// Decode: every workgroup streams one piece (single, chunks) or a run of
// pieces (stream) for one head group of HW adjacent kv heads; the NW waves
// take the 32-key tiles of a piece in turn, each with its own online softmax,
// and merge through LDS at the end of the piece.
// APPEND: 0 plain decode; 1 the step's new rows fused in, in the query's
// dtype; 2 the same, new rows in fp32.
template <int D, int KVF, int SM, typename TQ, int NW, int NS, int HW, int MODE, int APPEND>
__global__ __launch_bounds__(NW * 64) void decode_stream_kernel(
    AttnArgs a, const int32_t* __restrict__ block_table) {
  using Geo = KvGeom<KVF, D>;
  using SG = StreamGeo<KVF, D, HW>;
  using WC = WaveCopy<KVF, D, HW>;
  constexpr int NQK = Geo::NQK, NPV = Geo::NPV;
  constexpr int stride = 32 * NW;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int col = lane & 15, grp = lane >> 4;
  const int hgs = a.dec_head_groups;
  const int lbs = a.block_size_log2;
  const int hkv = a.hkv, H = a.num_heads;
  const int G = H / hkv;
  const uint32_t row_stride = (uint32_t)(hkv * Geo::C);   // bytes between tokens

  __shared__ __attribute__((aligned(16))) uint8_t ring[NW][NS * SG::SLOT];
  __shared__ float sm_ml[NW][HW][2][kDecMaxGroup];        // running max, sum per wave
  __shared__ float sm_c2[HW];
  __shared__ int sm_last;
  __shared__ int progress[NW];                            // tiles each wave has computed
  uint8_t* myring = ring[wave];
  WC cp;
  cp.init(lane, row_stride);
  if (lane == 0) progress[wave] = 0;
  int done = 0;

  // One piece: keys [k0, k1) of segment (b, hg), whose sequence starts at row
  // q0 and holds past + 1 keys.  nparts == 1: the piece is the whole segment.
  // Otherwise its partial goes to slot `slot`, and the last of the segment's
  // nparts pieces to arrive merges the slots part_slot(0 .. nparts-1).
  // spec: the block ids of this wave's first tile read early for the range
  // [spec_kb, spec_ke) (used if the true range names the same entries), or
  // {-1, -1}.
  auto run_piece = [&](int b, int hg, int k0, int k1, int q0, int past,
                       typename WC::Blocks spec, int spec_kb, int spec_ke, int nparts, int slot,
                       auto part_slot) {
    const int32_t* __restrict__ table = block_table + (size_t)b * a.max_blocks;
    const uint8_t* kbase = a.key_cache + (size_t)hg * SG::RB;
    const uint8_t* vbase = a.value_cache + (size_t)hg * SG::RB;
    const int kb = k0 + 32 * wave, ke = k1;
    const bool spec_ok = spec.b0 >= 0 &&
                         WC::entry(kb, ke, lbs, 0) == WC::entry(spec_kb, spec_ke, lbs, 0) &&
                         WC::entry(kb, ke, lbs, 1) == WC::entry(spec_kb, spec_ke, lbs, 1);
    // query and key-scale loads go out first, then this wave's first NS tiles
    QueryRaw<D, SM> qraw[HW];
#pragma unroll
    for (int hh = 0; hh < HW; ++hh)
      load_query<D, SM, TQ>(a, hg * HW + hh, q0, G, col, grp, qraw[hh]);
    // Fused append: the step's new token sits at key `past` (the last key).
    // The wave whose tile holds it quantizes the new key and value rows of
    // its HW heads -- lane l < RB / 4 forms 4 bytes of the key row segment,
    // the next RB / 4 lanes 4 bytes of the value row, so no lane does more
    // than 8 channels -- stores them into the caches, and writes the same
    // bytes over that row of the tile (and the rows after it, copies of it)
    // once the tile is in LDS (the copy may have read the slot before the
    // store), so no wait on the store is needed.  (Forming the codes before
    // the first copies measured faster than after them.)
    const int kt_app = k0 + 32 * ((past - k0) >> 5);       // tile holding the new key
    const bool app = APPEND && k0 <= past && past < k1 &&
                     (((past - k0) >> 5) % NW) == wave;
    constexpr int kAppLanes = SG::RB / 4;                  // lanes per row segment
    const bool app_lane = app && lane < 2 * kAppLanes;
    const bool app_v = lane >= kAppLanes;
    const int app_b = 4 * (app_v ? lane - kAppLanes : lane);   // byte in the segment
    uint32_t app_codes = 0;
    if constexpr (APPEND != 0) {
      if (app_lane) {
        const int hh = app_b / SG::C, bo = app_b % SG::C;
        const int h = hg * HW + hh;
        using TI = typename std::conditional<APPEND == 2, float, TQ>::type;
        const TI* x_row = reinterpret_cast<const TI*>(app_v ? a.new_value : a.new_key) +
                          ((size_t)q0 * hkv + h) * D;
        Raw4 raw;
        load_raw4<KVF, SM, TI>(x_row, app_v ? a.v_scale : a.k_scale, h, D, bo, raw);
        app_codes = codes4_from<KVF, TI>(raw);
        const int32_t blk = table[past >> lbs];
        uint8_t* dst = const_cast<uint8_t*>(app_v ? a.value_cache : a.key_cache) +
                       (((size_t)blk << lbs) + (size_t)(past & ((1 << lbs) - 1))) * row_stride +
                       (size_t)hg * SG::RB + app_b;
        *reinterpret_cast<uint32_t*>(dst) = app_codes;
      }
    }
    if (kb < ke)
      cp.issue(myring, kb, ke, lbs, spec_ok ? spec : WC::blocks(kb, ke, lbs, table), kbase,
               vbase, row_stride);
#pragma unroll
    for (int j = 1; j < NS; ++j)
      if (kb + j * stride < ke)
        cp.issue(myring + j * SG::SLOT, kb + j * stride, ke, lbs, table, kbase, vbase, row_stride);
    // The waits below count NS - 1 tiles in flight behind the current one;
    // with fewer tiles than that, wait for everything instead.
    if (kb + (NS - 1) * stride >= ke) wait_vmcnt_le<0>();

    f16x8 qhi[HW][NQK], qlo[HW][NQK];
    float c2[HW];
#pragma unroll
    for (int hh = 0; hh < HW; ++hh) {
      const int e = fold_loaded_query<D, KVF, SM, TQ>(qraw[hh], qhi[hh], qlo[hh]);
      c2[hh] = score_factor_log2(a.softmax_scale, e, kKeyOperandScale<KVF>);   // raw -> log2 units
    }

    WaveState<D> st[HW];
#pragma unroll
    for (int hh = 0; hh < HW; ++hh)
#pragma unroll
      for (int i = 0; i < NPV; ++i) st[hh].o[i] = (f32x4){0.f, 0.f, 0.f, 0.f};
    int cur = 0;
    // block ids of the next tile to issue, fetched one iteration ahead
    typename WC::Blocks nb_next = WC::blocks(kb + NS * stride, ke, lbs, table);
    for (int k = kb; k < ke; k += stride) {
      // this tile's copies are done once at most the later tiles' remain
      __builtin_amdgcn_sched_barrier(0);
      wait_vmcnt_le<(NS - 1) * 2 * SG::NI>();
      __builtin_amdgcn_sched_barrier(0);
      // Waves w and w ^ 4 share a SIMD, whose issue arbitration favours the
      // older wave: left alone, the younger one falls behind through every
      // tile's computation, and the piece ends when its slowest wave does.
      // A wave behind its partner in tiles computed raises its priority.
      if constexpr (NW == 8) {
        const int other = __builtin_amdgcn_readfirstlane(progress[wave ^ 4]);
        if (done < other) __builtin_amdgcn_s_setprio(2);
        else __builtin_amdgcn_s_setprio(0);
      }
      uint8_t* slotp = myring + cur * SG::SLOT;
      if constexpr (APPEND != 0) {
        // the new key's row and the rows after it, which the copy fills with
        // the last key's row again (masked, but their value bytes still meet
        // a zero probability: a stale FP8 NaN there would survive it)
        if (app_lane && k == kt_app) {
          uint8_t* half = slotp + (app_v ? 32 * SG::RB : 0);
          for (int r = past - kt_app; r < 32; ++r)
            *reinterpret_cast<uint32_t*>(half + stream_off<KVF, D, HW>(r, app_b)) = app_codes;
        }
      }
      TileRaw<KVF, D> t[HW];
#pragma unroll
      for (int hh = 0; hh < HW; ++hh) read_tile<KVF, D, HW>(slotp, t[hh], col, grp, hh);
      // the slot is refilled (NS tiles ahead) once every lane has read it
      __builtin_amdgcn_s_waitcnt(0xC07F);                 // lgkmcnt(0)
      __builtin_amdgcn_sched_barrier(0);
      const int kn = k + NS * stride;
      if (kn < ke) cp.issue(slotp, kn, ke, lbs, nb_next, kbase, vbase, row_stride);
      else wait_vmcnt_le<0>();                            // nothing more to issue: keep vmcnt exact
      nb_next = WC::blocks(kn + stride, ke, lbs, table);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int hh = 0; hh < HW; ++hh)
        compute_tile<KVF, D>(t[hh], k, ke, c2[hh], qhi[hh], qlo[hh], st[hh], grp);
      ++done;
      if (lane == 0) progress[wave] = done;
      cur = (cur + 1 == NS) ? 0 : cur + 1;
    }
    __builtin_amdgcn_s_setprio(0);
    wait_vmcnt_le<0>();
    __builtin_amdgcn_sched_barrier(0);

    // ---- merge the waves of each head through LDS (each wave writes its own ring) ----
    float* wo = reinterpret_cast<float*>(myring);          // [HW][kDecMaxGroup][D] per wave
    static_assert(HW * kDecMaxGroup * D * 4 <= NS * SG::SLOT, "merge area");
#pragma unroll
    for (int hh = 0; hh < HW; ++hh) {
      const float l_run = rows_sum(st[hh].l);
      if (col < G) {
        if (grp == 0) { sm_ml[wave][hh][0][col] = st[hh].m; sm_ml[wave][hh][1][col] = l_run; }
#pragma unroll
        for (int nbk = 0; nbk < NPV; ++nbk)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            wo[(hh * kDecMaxGroup + col) * D + (D / 16) * (4 * grp + r) + nbk] = st[hh].o[nbk][r];
      }
      if (wave == 0 && lane == 0) sm_c2[hh] = c2[hh];
    }
    __syncthreads();
    const bool direct = nparts == 1;
    for (int t = threadIdx.x; t < HW * G * D; t += NW * 64) {
      const int hh = t / (G * D), cq = (t / D) % G, d = t % D;
      const float cf = sm_c2[hh];
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < NW; ++w) M = fmaxf(M, sm_ml[w][hh][0][cq]);
      float L = 0.f, O = 0.f;
      if (M != -INFINITY) {
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          const float f = fast_exp2((sm_ml[w][hh][0][cq] - M) * cf);
          L += f * sm_ml[w][hh][1][cq];
          O += f * reinterpret_cast<const float*>(ring[w])[(hh * kDecMaxGroup + cq) * D + d];
        }
      }
      const int ho = hg * HW + hh;
      const int hq = ho * G + cq;
      if (direct) {
        const float vs = (SM == SCALE_CHANNEL) ? a.v_scale[ho * D + d] : a.v_scale[ho];
        const float val = (L > 0.f) ? v_unbias<KVF>(O / L, d) * vs : 0.f;   // both carry 2^7
        reinterpret_cast<TQ*>(a.out)[((size_t)q0 * H + hq) * D + d] = from_f32<TQ>(val);
      } else {
        // this piece's partial: normalised output (value scale not applied),
        // its raw maximum and its sum (which carries 2^7, like every piece's)
        const size_t pi = (size_t)slot * HW * G + hh * G + cq;
        store_agent(&a.part_o[pi * D + d], (L > 0.f) ? v_unbias<KVF>(O / L, d) : 0.f);
        if (d == 0) {
          store_agent(&a.part_ml[2 * pi], M);
          store_agent(&a.part_ml[2 * pi + 1], L);
        }
      }
    }
    if (direct) {
      __syncthreads();                                     // the rings are reused next
      return;
    }

    // ---- arrival: the last piece of this segment merges ----
    // Every thread's partial stores are device-coherent and complete before
    // the barrier, so they precede the counter increment; the last piece to
    // arrive reads the others' partials with device-coherent loads.
    wait_stores();
    __syncthreads();
    int32_t* ctr = a.dec_counters + (size_t)b * hgs + hg;
    if (threadIdx.x == 0)
      sm_last = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                nparts - 1;
    __syncthreads();
    if (!sm_last) return;
    // Merge: every thread takes two output elements and runs a merge over
    // the pieces by their raw maxima, U pieces at a time with all their loads
    // (maximum, sum and the two outputs) issued together, so the merge costs
    // one memory round trip per U pieces.
    // (8 pieces per round where the merge sits inside the stream partition's
    // piece loop with two heads per wave: 16 would not fit the registers)
    constexpr int NT = NW * 64, U = (MODE == DEC_STREAM && HW > 1) ? 8 : 16;
    for (int t0 = threadIdx.x; t0 < HW * G * D; t0 += 2 * NT) {
      int pr[2], dd[2];
      bool on[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int t = t0 + e * NT;
        on[e] = t < HW * G * D;
        pr[e] = on[e] ? t / D : 0;
        dd[e] = on[e] ? t % D : 0;
      }
      float M[2] = {-INFINITY, -INFINITY}, L[2] = {0.f, 0.f}, O[2] = {0.f, 0.f};
      for (int p0 = 0; p0 < nparts; p0 += U) {
        float pm[2][U], pl[2][U], po[2][U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const bool ok = p0 + u < nparts;
          const size_t sl = ok ? (size_t)part_slot(p0 + u) * HW * G : 0;
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const size_t pi = sl + pr[e];
            pm[e][u] = (ok && on[e]) ? load_agent(&a.part_ml[2 * pi]) : -INFINITY;
            pl[e][u] = (ok && on[e]) ? load_agent(&a.part_ml[2 * pi + 1]) : 0.f;
            po[e][u] = (ok && on[e]) ? load_agent(&a.part_o[pi * D + dd[e]]) : 0.f;
          }
        }
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const float cf = sm_c2[pr[e] / G];
          float mn = M[e];
#pragma unroll
          for (int u = 0; u < U; ++u) mn = fmaxf(mn, pm[e][u]);
          if (mn == -INFINITY) continue;                   // only empty pieces so far
          const float sc = fast_exp2((M[e] - mn) * cf);    // 0 while M is -inf
          L[e] *= sc;
          O[e] *= sc;
#pragma unroll
          for (int u = 0; u < U; ++u) {
            const float wgt = fast_exp2((pm[e][u] - mn) * cf) * pl[e][u];   // empty: 0
            L[e] += wgt;
            O[e] = fmaf(wgt, po[e][u], O[e]);
          }
          M[e] = mn;
        }
      }
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        if (!on[e]) continue;
        const int ho = hg * HW + pr[e] / G;
        const int hq = ho * G + pr[e] % G;
        const float vs = (SM == SCALE_CHANNEL) ? a.v_scale[ho * D + dd[e]] : a.v_scale[ho];
        reinterpret_cast<TQ*>(a.out)[((size_t)q0 * H + hq) * D + dd[e]] =
            from_f32<TQ>((L[e] > 0.f) ? O[e] / L[e] * vs : 0.f);
      }
    }
    // every counter is zero again when the launch ends
    if (threadIdx.x == 0) __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();                                       // the rings are reused next
  };

  if constexpr (MODE == DEC_SINGLE || MODE == DEC_CHUNKS) {
    const int hg = (int)(blockIdx.x % (unsigned)hgs);     // consecutive workgroups: other XCDs
    const int item = (int)(blockIdx.x / (unsigned)hgs);
    const int P = MODE == DEC_SINGLE ? 1 : a.dec_parts_per_seq;
    const int b = item / P, j = item % P;
    const int32_t* __restrict__ table = block_table + (size_t)b * a.max_blocks;
    // The first tile's block ids are read before this sequence's length
    // arrives, for the batch's longest length (inside the table row either
    // way); they serve whenever the true range names the same table entries,
    // which saves the table round trip before the first copy.
    int k0s = 0, k1s = a.max_kv_len;
    if constexpr (MODE == DEC_CHUNKS) chunk_part_keys(a, j, a.max_kv_len, k0s, k1s);
    const typename WC::Blocks spec = WC::blocks(k0s + 32 * wave, k1s, lbs, table);
    const int q0 = a.cum_q[b];
    const int past = a.past_lens[b];
    // no new token: no rows.  The test also reads the past and the speculative
    // entries (a negative past never occurs), so all these loads go out
    // together instead of one behind the other.
    if ((a.cum_q[b + 1] == q0) | ((past < 0) & (spec.b0 == spec.b1))) return;
    const int kv_len = past + 1;
    int k0 = 0, k1 = kv_len;
    if constexpr (MODE == DEC_CHUNKS) chunk_part_keys(a, j, kv_len, k0, k1);
    run_piece(b, hg, k0, k1, q0, past, spec, k0s + 32 * wave, k1s, P, (int)blockIdx.x,
              [&](int p) { return (b * P + p) * hgs + hg; });
  } else {
    // Stream partition: this workgroup's run of the concatenated tiles.
    const long long T = a.dec_total_tiles;
    const int N = (int)gridDim.x;
    const int w = (int)blockIdx.x;
    long long g = (long long)w * T / N;
    const long long g1 = (long long)(w + 1) * T / N;
    if (g >= g1) return;
    StreamPos pos = stream_find(a.cum_q, a.past_lens, a.batch, hgs, g);
    int b = __builtin_amdgcn_readfirstlane(pos.b);
    if (b < 0) return;
    int tiles = __builtin_amdgcn_readfirstlane(pos.tiles);
    int off = __builtin_amdgcn_readfirstlane(pos.off);
    int q0 = __builtin_amdgcn_readfirstlane(pos.q0);
    int past = __builtin_amdgcn_readfirstlane(pos.past);
    long long seq_first = g - off;                         // first global tile of sequence b
    int hg = off / tiles, t = off % tiles;
    bool first = true;
    for (;;) {
      const int n = (int)min((long long)(tiles - t), g1 - g);
      const long long seg = seq_first + (long long)hg * tiles;   // the segment's first tile
      const int kv_len = past + 1;
      int nparts = 1, slot = 0, wfirst = 0, before = 0;
      if (!(t == 0 && n == tiles)) {
        wfirst = stream_owner(seg, T, N);
        nparts = stream_owner(seg + tiles - 1, T, N) - wfirst + 1;
        slot = 2 * w + (first ? 0 : 1);
        // only the first owner can start before the segment
        before = (long long)wfirst * T / N < seg ? 1 : 0;
      }
      run_piece(b, hg, 32 * t, min(kv_len, 32 * (t + n)), q0, past,
                typename WC::Blocks{-1, -1}, 0, 0, nparts, slot, [&](int p) {
                  // a piece is its workgroup's first unless that workgroup
                  // started before the segment (then it is its last)
                  return 2 * (wfirst + p) + (p == 0 ? before : 0);
                });
      g += n;
      if (g >= g1) break;
      first = false;
      t = 0;
      if (++hg == hgs) {
        // next sequence with a new row
        hg = 0;
        seq_first += (long long)hgs * tiles;
        do {
          ++b;
          if (b >= a.batch) return;
          q0 = a.cum_q[b];
          past = a.past_lens[b];
          tiles = a.cum_q[b + 1] > q0 ? (past + 32) >> 5 : 0;
        } while (tiles == 0);
      }
    }
  }
}

bool decode_mfma_supports(int head_size, int group, int block_size, int q_dtype) {
  return (head_size == 64 || head_size == 128) && group >= 1 && group <= kDecMaxGroup &&
         block_size >= 16 && block_size % 16 == 0 && (q_dtype == DT_F16 || q_dtype == DT_BF16);
}

// Launch: a 1-D grid of (parts x head groups) workgroups of NW waves, NS = 1
// tile in flight per wave besides the one being read (the copies of 8 waves
// then keep ~64 KB per CU in flight, where measured HBM efficiency peaks).
// The partition, the part count and the waves per workgroup come from the
// host plan.
template <int D, int KVF, int SM, typename TQ, int HW, int NW, int APPEND>
static int launch_nw(const AttnArgs& a, hipStream_t st) {
  const dim3 grid(a.grid_x), block(NW * 64);
  switch (a.dec_mode) {
    case DEC_SINGLE:
      hipLaunchKernelGGL((decode_stream_kernel<D, KVF, SM, TQ, NW, 1, HW, DEC_SINGLE, APPEND>),
                         grid, block, 0, st, a, a.block_table);
      return 0;
    case DEC_CHUNKS:
      hipLaunchKernelGGL((decode_stream_kernel<D, KVF, SM, TQ, NW, 1, HW, DEC_CHUNKS, APPEND>),
                         grid, block, 0, st, a, a.block_table);
      return 0;
    case DEC_STREAM:
      hipLaunchKernelGGL((decode_stream_kernel<D, KVF, SM, TQ, NW, 1, HW, DEC_STREAM, APPEND>),
                         grid, block, 0, st, a, a.block_table);
      return 0;
  }
  return -1;
}

template <int D, int KVF, int SM, typename TQ, int HW>
static int launch_hw_q(const AttnArgs& a, hipStream_t st) {
  if (a.dec_waves != 8) return -1;
  if (a.new_key && a.new_rows_f32) return launch_nw<D, KVF, SM, TQ, HW, 8, 2>(a, st);
  if (a.new_key) return launch_nw<D, KVF, SM, TQ, HW, 8, 1>(a, st);
  return launch_nw<D, KVF, SM, TQ, HW, 8, 0>(a, st);
}

template <int D, int KVF, int SM, int HW>
static int launch_hw(const AttnArgs& a, hipStream_t st) {
  if (a.q_dtype == DT_F16) return launch_hw_q<D, KVF, SM, f16, HW>(a, st);
  if (a.q_dtype == DT_BF16) return launch_hw_q<D, KVF, SM, bf16, HW>(a, st);
  return -1;
}

// HW = min(2, 128 / C) heads per wave when the kv head count allows, else
// the largest power of two dividing it (decode_heads_per_wave).
template <int D, int KVF, int SM>
static int launch_dq(const AttnArgs& a, hipStream_t st) {
  constexpr int C = KvGeom<KVF, D>::C;
  static_assert(C == 32 || C == 64 || C == 128, "row bytes");
  const int hw = decode_heads_per_wave(KVF, D, a.hkv);
  if (a.hkv / hw != a.dec_head_groups) return -1;
  switch (hw) {
    case 1: return launch_hw<D, KVF, SM, 1>(a, st);
    case 2: if constexpr (C <= 64) return launch_hw<D, KVF, SM, 2>(a, st); break;
  }
  return -1;
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
  if (a.dec_mode != DEC_SINGLE && (!a.part_o || !a.part_ml || !a.dec_counters)) return -1;
  return a.head_size == 128 ? launch_d<128>(a, st) : launch_d<64>(a, st);
}

}  // namespace paq
