// prefill_mfma.hip -- ragged, causal, chunked prefill over an INT8 / packed-INT4
// / FP8 paged cache on gfx950 matrix cores (v_mfma_f32_32x32x16).
//
// Work units (query tile, kv head, sequence), as many query tiles as the exact
// max_query_len of the host cum_q needs ("PagedAttention FA path: exact
// max_query_len", section 1); a tile past its sequence's q_len exits at once,
// so zero-token sequences cost one early exit.  The 1-D grid is ordered for
// the 8 XCDs: workgroup i runs on XCD i % 8, and XCD x takes every 8th
// (sequence, kv head) pair, so the query tiles of a pair re-read its keys and
// values from one L2 and ragged sequences spread evenly over the XCDs; within
// a pair the heaviest tiles (the last ones, which see the most keys) run
// first.
//
// Workgroup = 4 waves = 32/G tokens per wave x the G query heads of one kv head:
// the GQA group is packed into the 32 MFMA query columns of every wave.
//
// Per 64-key KV tile ("FlashInfer FP8 KV-cache prefill", repack section: convert
// once into shared memory instead of per use):
//   * all 256 threads load the codes of tile kt+2 while tile kt is computed,
//     and convert the codes of tile kt+1 exactly to 16-bit values in the other
//     LDS buffer beside tile kt's products (K rows beside the QK MFMAs, V^T rows
//     beside the PV MFMAs), so the conversion's VALU and LDS work overlaps the
//     matrix cores: K row-major, V transposed (channel-major) with keys in the
//     order the PV operand wants; rows are padded by 16 bytes against bank
//     conflicts;
//   * two 4-wave workgroups share a compute unit, so each SIMD interleaves
//     waves of two independent workgroups;
//   * S^T = K Q'^T: A = 32 keys x 16 channels of K, B = Q'^T (lane: query column
//     l%32), so every lane owns one query column and reduces its softmax row
//     with a single cross-lane exchange (lanes l and l^32);
//   * the 16 scores a lane holds per 32-key block are exactly the B operand of
//     two PV MFMAs (keys {8(r/4)+4(l/32)+r%4}), so P never moves between lanes;
//   * O^T += V^T P^T with fp16 P scaled by 2^7 under a lazily refreshed running
//     maximum (rescale only when a score exceeds it by more than 2^8);
//   * causal mask (row i sees keys <= past + i) only where a tile crosses the
//     diagonal.
// Key scales: per-channel scales are folded into the query (power-of-two
// normaliser M_h >= max|s|, "ONNX Runtime: INT4 Paged KV Cache", section 3);
// per-head scales go into the score factor.  Value scales are applied in the
// epilogue.  QK runs in fp16, or in bf16 for bf16 queries with per-head scales
// (then both operands are exact); PV always runs in fp16 (codes are exact).
#include <type_traits>

#include "device.hpp"
#include "launch.hpp"

namespace paq {

namespace {

constexpr int kBN = 64;                      // keys per KV tile
constexpr int kPfWavesPerGroup = kPrefillWaves;   // waves per workgroup (32/G tokens each)
constexpr float kPfSlack = 8.0f;             // lazy running-max slack (log2 units)
constexpr float kPfPScaleLog2 = 7.0f;        // fp16 P = p * 2^7

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

template <int KVF, int D, int NT = 256> struct PfGeo {
  static constexpr int C = (KVF == KV_INT4) ? D / 2 : D;     // bytes per cache row
  static constexpr int CPU = (KVF == KV_INT4) ? 32 : 16;     // channels per 16-byte unit
  static constexpr int UPR = C / 16;                         // 16-byte units per row
  // LDS rows: K rows are padded by 16 bytes, so 16 lanes reading the same
  // 16-byte column of 16 consecutive rows hit 16 different 4-bank groups; V
  // rows by 64 bytes, so the 32 lanes of a transposing 8-byte operand read
  // (4 rows x 8 blocks of 4 channels) hit 64 different banks.  Every address
  // is a per-lane base plus an immediate offset.
  static constexpr int KROW = D * 2 + 16;                    // bytes of a K row in LDS
  static constexpr int VROW = D * 2 + 64;                    // bytes of a V row in LDS
  static constexpr int TILE = kBN * KROW + kBN * VROW;       // one LDS buffer
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
// FP8 E4M3 -> fp16 / bf16 (exact: every E4M3 value, subnormals included, is
// representable in both): gfx950's scaled packed conversion takes the two codes
// of one 16-bit half of a word, with a unit scale
template <>
__device__ __forceinline__ void decode_unit<KV_FP8, f16>(const u32x4& w, uint32_t (&out)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[i], 1.0f, false));
    out[2 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[i], 1.0f, true));
  }
}
template <>
__device__ __forceinline__ void decode_unit<KV_FP8, bf16>(const u32x4& w, uint32_t (&out)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i], 1.0f, false));
    out[2 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i], 1.0f, true));
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

// 16 raw value codes -> the PV operand: the exact fp16 values for FP8, and
// for the integer formats their affine images 1152 + v (INT8) and 1032 + v
// (INT4), the 0x6400 constructions without their bias subtraction.  The
// epilogue removes the bias once: O/l - bias, with l the sum of the same fp16
// probabilities the products use.
template <int KVF> constexpr float kPfVBias = KVF == KV_INT8 ? 1152.f : KVF == KV_INT4 ? 1032.f : 0.f;
template <int KVF>
__device__ __forceinline__ void decode_unit_v(const u32x4& w, uint32_t (&out)[PfGeo<KVF, 128>::CPU / 2]) {
  if constexpr (KVF == KV_INT8) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t x = w[i] ^ 0x80808080u;
      out[2 * i] = perm(0x64646464u, x, 0x04010400u);
      out[2 * i + 1] = perm(0x64646464u, x, 0x04030402u);
    }
  } else if constexpr (KVF == KV_INT4) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t x = w[i] ^ 0x88888888u;
      out[4 * i] = ((x & 0xFu) | ((x << 12) & 0xF0000u)) | 0x64006400u;
      out[4 * i + 1] = (((x >> 8) & 0xFu) | ((x << 4) & 0xF0000u)) | 0x64006400u;
      out[4 * i + 2] = (((x >> 16) & 0xFu) | ((x >> 4) & 0xF0000u)) | 0x64006400u;
      out[4 * i + 3] = (((x >> 24) & 0xFu) | ((x >> 12) & 0xF0000u)) | 0x64006400u;
    }
  } else {
    decode_unit<KVF, f16>(w, out);
  }
}

// a if c else b, computed on the values
__device__ __forceinline__ int32_t choose(bool c, int32_t a, int32_t b) {
  return b ^ ((a ^ b) & -(int32_t)c);
}

// The (pair, query tile) item of prefill workgroup i as pair << 32 | tile, or
// -1 past its XCD's items (see the kernel for the order).  Not inlined: the
// search runs once per workgroup, and kept apart it leaves the register
// allocation of the kernel's main loop as it is.
__device__ __attribute__((noinline)) long long prefill_find_item(const int32_t* __restrict__ cum_q,
                                                           int P, int hkv, int TOK, int i) {
  const int x = i % 8, k = i / 8;
  const int lane = (int)(threadIdx.x & 63);
  int before = 0;
  for (int j0 = 0; x + 8 * j0 < P; j0 += 64) {
    const int pr = x + 8 * (j0 + lane);
    int cnt = 0;
    if (pr < P) {
      const int sb = pr / hkv;
      cnt = (cum_q[sb + 1] - cum_q[sb] + TOK - 1) / TOK;
    }
    int incl = cnt;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int t = __shfl_up(incl, off, 64);
      if (lane >= off) incl += t;
    }
    const unsigned long long hit = __ballot(before + incl > k);
    if (hit) {
      const int l = (int)__builtin_ctzll(hit);
      const int incl_l = __shfl(incl, l, 64), cnt_l = __shfl(cnt, l, 64);
      return ((long long)(x + 8 * (j0 + l)) << 32) |
             (long long)(cnt_l - 1 - (k - (before + incl_l - cnt_l)));
    }
    before += __shfl(incl, 63, 64);
  }
  return -1;
}

template <int D, int KVF, int SM, typename TQ, typename TK, int NW, bool KPU>
__global__ __launch_bounds__(NW * 64, 2) void prefill_mfma_kernel(
    AttnArgs a, const int32_t* __restrict__ block_table) {
  constexpr int kPfThreads = NW * 64;
  constexpr int kPfWaves = NW;
  using Geo = PfGeo<KVF, D, NW * 64>;
  // KPU (the comparison variant of "INT8-KV Tensor-Core DynamicSparseAttention",
  // section 1): K tiles are kept in LDS as raw 1-byte codes and every wave
  // converts the operands it reads, instead of converting each tile once
  // ("FlashInfer FP8 KV-cache prefill", repack section).  V is staged the
  // same way in both (its operand takes 8 keys of one channel per lane, which
  // the transposing 16-bit LDS read provides only from converted rows).
  static_assert(!KPU || KVF != KV_INT4, "per-use K conversion: 1-byte formats only");
  constexpr int KROW = KPU ? D + 16 : Geo::KROW;   // bytes of a K row in LDS
  constexpr int KB = KPU ? 1 : 2;                  // bytes per K channel in LDS
  using MK = mfma32<TK>;
  typedef typename MK::vec kvec;
  constexpr int C = Geo::C;
  constexpr int NKK = D / 16;                   // QK MFMAs per 32-key block
  constexpr int NDT = D / 32;                   // output channel tiles
  const int G = a.num_heads / a.hkv;
  const int TPW = 32 / G;                       // tokens per wave
  const int TOK = kPfWaves * TPW;               // tokens per workgroup
  // Workgroup i is dispatched to XCD i % 8.  XCD x takes the (sequence, kv
  // head) pairs x, x + 8, x + 16, ... (with 8 kv heads: one head of every
  // sequence, which balances ragged batches across XCDs); all query tiles of a
  // pair run on its XCD and re-read the pair's keys and values from that L2,
  // the pair's heaviest tiles first.  Workgroup i is item i / 8 of XCD i % 8's
  // list of (pair, tile) items, pairs in order, each with ceil(q_len / TOK)
  // tiles: found by a wave-wide prefix sum over the tile counts of the XCD's
  // pairs, 64 pairs at a time.
  // When every sequence has the same tile count (pf_ntq > 0) the item is
  // plain arithmetic.
  int pair, qt;
  if (a.pf_ntq > 0) {
    const int k = (int)(blockIdx.x / 8);
    pair = (int)(blockIdx.x % 8) + 8 * (k / a.pf_ntq);
    qt = a.pf_ntq - 1 - k % a.pf_ntq;
    if (pair >= a.hkv * a.batch) pair = -1;
  } else {
    const long long item =
        prefill_find_item(a.cum_q, a.hkv * a.batch, a.hkv, TOK, (int)blockIdx.x);
    pair = item < 0 ? -1 : (int)(item >> 32);
    qt = (int)(item & 0xFFFFFFFFll);
  }
  pair = __builtin_amdgcn_readfirstlane(pair);        // uniform: keep it (and all
  qt = __builtin_amdgcn_readfirstlane(qt);            // derived from it) scalar
  if (pair < 0) return;                               // past this XCD's items
  const int h = pair % a.hkv, b = pair / a.hkv;
  const int q0 = a.cum_q[b];
  const int qlen = a.cum_q[b + 1] - q0;
  const int tok0 = qt * TOK;
  if (tok0 >= qlen) return;            // a padded grid's tile past the new rows
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

  __shared__ __attribute__((aligned(16))) uint8_t lds[2][Geo::TILE];

  // ---- staging: codes of a tile -> registers -> converted LDS tile ----
  // The physical blocks of a 64-key tile (at most 4 with 16-token blocks) are
  // wave-uniform, so they are fetched with scalar loads one tile ahead.
  // Blocks past the sequence's last one are clamped to it and rows are taken
  // within their block, so every load stays inside an allocated block; keys
  // past kv_end read whatever the block holds there: their scores are masked
  // and their value codes are zeroed before conversion.
  static_assert(kBN == 16 * kPfWaves, "each wave stages 16 keys of a tile");
  const int nbt = (kBN >> lbs) > 0 ? (kBN >> lbs) : 1;       // blocks per tile (<= 4)
  const int last_blk = (kv_end - 1) >> lbs;
  const uint32_t blk_bytes = (uint32_t)bs * row_stride;
  // (the choices below are made on values with choose(): a conditional
  // expression on the fields lets the compiler pick a field address instead,
  // which keeps the struct in scratch memory)
  struct TileBlocks { int32_t b0, b1, b2, b3; };
  auto tile_blocks = [&](int kt) {
    const int first = (kt * kBN) >> lbs;
    return TileBlocks{table[min(first, last_blk)], table[min(first + min(1, nbt - 1), last_blk)],
                      table[min(first + min(2, nbt - 1), last_blk)],
                      table[min(first + min(3, nbt - 1), last_blk)]};
  };
  // K and V alike: wave w stages keys [16w, 16w + 16) of a tile, which lie in
  // one block for every supported block size: the block is wave-uniform and
  // a lane's offset into it is constant.  KL loads per lane, KPL keys per
  // load, lane l taking key l % KPL and 16-byte unit l / KPL of it: the row
  // writes of such a load to LDS are free of bank conflicts (with the unit
  // index running fastest over the lanes they are not).
  constexpr int KL = Geo::UPR >= 4 ? Geo::UPR / 4 : 1;
  constexpr int KPL = Geo::UPR >= 4 ? 64 / Geo::UPR : 16;      // keys per load
  const bool k_active = Geo::UPR >= 4 || lane < 16 * Geo::UPR;
  const int kx = lane % KPL, kc = lane / KPL;                  // key, unit
  // (V rows are 320 bytes apart for D = 128, where rows kx and kx+4 share
  // banks: the second four rows of a load take their units in swapped pairs)
  const int vc = kc ^ ((kx >> 2) & 1);
  uint32_t koff[KL], voff[KL];
#pragma unroll
  for (int i = 0; i < KL; ++i) {
    koff[i] = (uint32_t)(i * KPL + kx) * row_stride + 16 * kc;
    voff[i] = (uint32_t)(i * KPL + kx) * row_stride + 16 * vc;
  }
  auto row_base = [&](const uint8_t* base, const TileBlocks& tb, int kt) -> const uint8_t* {
    const int key = kt * kBN + 16 * wave;
    const int j = (key >> lbs) - ((kt * kBN) >> lbs);         // 0..3, uniform
    const int32_t blk =
        choose(j >= 3, tb.b3, choose(j >= 2, tb.b2, choose(j >= 1, tb.b1, tb.b0)));
    return base + ((size_t)blk * bs + (key & (bs - 1))) * row_stride;
  };
  // Raw codes of a tile, held by this thread between their load and their
  // conversion into LDS one step later (K codes of tile t+3 and V codes of
  // tile t+2 are loaded at the end of step t).  The V load address stays live
  // until its set is converted: otherwise the compiler may hand its registers
  // to MFMA accumulators and then drain the loads to avoid overwriting a
  // vector-memory source operand.
  struct RawK { u32x4 k[KL]; };
  auto load_k = [&](RawK& r, const TileBlocks& tb, int kt) {
    const uint8_t* rb = row_base(kbase, tb, kt);
    if (k_active) {
#pragma unroll
      for (int i = 0; i < KL; ++i) r.k[i] = *reinterpret_cast<const u32x4*>(rb + koff[i]);
    }
  };
  auto load_v = [&](RawK& r, const TileBlocks& tb, int kt) {
    const uint8_t* rb = row_base(vbase, tb, kt);
    if (k_active) {
#pragma unroll
      for (int i = 0; i < KL; ++i) r.k[i] = *reinterpret_cast<const u32x4*>(rb + voff[i]);
    }
  };
  // Conversions into LDS buffer `buf`: the K and V rows of a tile, row-major,
  // in pieces that phase B spreads over its matrix products.
  typedef uint32_t KWords[Geo::CPU / 2];
  auto stage_write = [&](int buf, int vpart, int i, const KWords& w) {   // unit i of this lane
    if (!k_active) return;
    const int rowb = vpart ? Geo::VROW : KROW;
    const int c = vpart ? vc : kc;
    uint8_t* rl = lds[buf] + (vpart ? kBN * KROW : 0) + (16 * wave + i * KPL + kx) * rowb;
    // channels [CPU*c, CPU*c + CPU) = 16-byte chunks CPU*c/8 ...
#pragma unroll
    for (int j = 0; j < Geo::CPU / 8; ++j)
      *reinterpret_cast<u32x4*>(rl + 2 * Geo::CPU * c + 16 * j) =
          (u32x4){w[4 * j], w[4 * j + 1], w[4 * j + 2], w[4 * j + 3]};
  };
  auto stage_raw_k = [&](int buf, int i, const u32x4& w) {   // KPU: unit i as raw codes
    if (!k_active) return;
    *reinterpret_cast<u32x4*>(lds[buf] + (16 * wave + i * KPL + kx) * KROW + 16 * kc) = w;
  };
  // V codes of unit i of tile t as the PV operand
  auto v_decode = [&](const RawK& r, int t, int i, KWords& w) { decode_unit_v<KVF>(r.k[i], w); };
  // Keys past kv_end hold whatever their block holds: E4M3 NaN codes there
  // would survive the zero P (0 * NaN).  For FP8, once the V rows of a tile
  // that reaches past kv_end are written, this lane's rows of such keys are
  // overwritten with zeros (same lane, same addresses: the writes stay in
  // order).
  auto v_zero_tail = [&](int t, int buf) {
    if constexpr (KVF == KV_FP8) {
      if ((t + 1) * kBN > kv_end) {
        const KWords z = {};
#pragma unroll
        for (int i = 0; i < KL; ++i)
          if (t * kBN + 16 * wave + i * KPL + kx >= kv_end) stage_write(buf, 1, i, z);
      }
    }
  };
  auto store_k = [&](const RawK& r, int buf) {
#pragma unroll
    for (int i = 0; i < KL; ++i) {
      if constexpr (KPU) {
        stage_raw_k(buf, i, r.k[i]);
      } else {
        KWords w;
        decode_unit<KVF, TK>(r.k[i], w);
        stage_write(buf, 0, i, w);
      }
    }
  };
  auto store_v = [&](const RawK& r, int t, int buf) {
#pragma unroll
    for (int i = 0; i < KL; ++i) {
      KWords w;
      v_decode(r, t, i, w);
      stage_write(buf, 1, i, w);
    }
    v_zero_tail(t, buf);
  };

  // tiles 0 and 1 are converted before the first step; tile 2's K codes and
  // tile 1's V codes are in registers when it starts
  TileBlocks tbA = tile_blocks(0), tbB = tile_blocks(1);
  RawK rk, rk1, rv;
  load_k(rk, tbA, 0);
  load_v(rv, tbA, 0);
  load_k(rk1, tbB, 1);
  const TileBlocks tb2 = tile_blocks(2);

  // ---- query operand: Q'^T columns, fold of the key scale ----
  const int my_tok = min(tok0 + wave * TPW + n / G, qlen - 1);      // clamp padded rows
  const int hq = h * G + (n % G);
  const TQ* qrow = reinterpret_cast<const TQ*>(a.query) + ((size_t)(q0 + my_tok) * H + hq) * D;
  // per-channel scales: M_h = 2^e >= max|s| (finite for every finite scale),
  // q' = q * s / M_h with s / M_h = ldexp(s, -e) exact; the score factor
  // keeps softmax_scale * M_h (per-head scales: softmax_scale * s) and is
  // clamped finite (score_factor_log2)
  int e_h = 0;
  if constexpr (SM == SCALE_CHANNEL) {
    float smax = 0.f;
#pragma unroll
    for (int i = 0; i < D / 64; ++i) smax = fmaxf(smax, fabsf(a.k_scale[h * D + lane + 64 * i]));
    e_h = scale_exponent(wave_max(smax));
  }
  kvec qop[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    const u32x4 x = *reinterpret_cast<const u32x4*>(qrow + 16 * kk + 8 * eta);
    const TQ* e = reinterpret_cast<const TQ*>(&x);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float v = to_f32(e[j]);
      if constexpr (SM == SCALE_CHANNEL) v *= ldexpf(a.k_scale[h * D + 16 * kk + 8 * eta + j], -e_h);
      qop[kk][j] = (TK)v;
    }
  }
  const float c2 = (SM == SCALE_CHANNEL)
                       ? score_factor_log2(a.softmax_scale, e_h, 1.f)
                       : fminf(fmaxf(a.softmax_scale * a.k_scale[h] * kLog2e, 0x1p-126f),
                               0x1.fffffep127f);
  const int row_lim = past + my_tok;              // last key this query column sees

  // running maximum of the raw scores (lazily refreshed), the same in log2
  // units for the fast exponent form, and the running sum
  float m_run = -INFINITY, m_log = -INFINITY, l_run = 0.f;
  f32x16 o[NDT];
#pragma unroll
  for (int i = 0; i < NDT; ++i) o[i] = (f32x16){};

  // K operand of one QK product: 8 channels of one key row, read from LDS
  // as 16-bit values, or (KPU) as 8 raw codes converted here
  using KOp = std::conditional_t<KPU, u32x2, kvec>;
  auto kread = [&](const uint8_t* p) -> KOp { return *reinterpret_cast<const KOp*>(p); };
  auto kop = [&](const KOp& x) -> kvec {
    if constexpr (KPU) {
      uint32_t w[8];
      decode_unit<KVF, TK>((u32x4){x[0], x[1], 0u, 0u}, w);
      return __builtin_bit_cast(kvec, (u32x4){w[0], w[1], w[2], w[3]});
    } else {
      return x;
    }
  };
  // (sched_group_barrier masks: 0x002 VALU, 0x008 MFMA, 0x100 LDS read,
  // 0x200 LDS write, 0x400 transcendental)
  // S^T = K Q'^T of tile t (keys 0-31 in s[0], 32-63 in s[1]), from LDS
  // buffer t & 1; the two accumulations alternate.
  auto qk = [&](int t, f32x16 (&s)[2]) {
    const uint8_t* k0p = lds[t & 1] + n * KROW + 8 * KB * eta;
    const uint8_t* k1p = k0p + 32 * KROW;
    s[0] = (f32x16){};
    s[1] = (f32x16){};
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const kvec a0 = kop(kread(k0p + 16 * KB * kk));
      const kvec a1 = kop(kread(k1p + 16 * KB * kk));
      s[0] = MK::run(a0, qop[kk], s[0]);
      s[1] = MK::run(a1, qop[kk], s[1]);
    }
  };
  // Causal mask of tile t (only where it crosses this wave's diagonal; the
  // first row is clamped like the rows themselves, so a wave of padded rows
  // masks the keys past the end too), then the lazy running maximum of the
  // raw scores: the accumulators are rescaled only when a score exceeds it by
  // more than kPfSlack in log2 units.  The gap is formed on the raw scores
  // and scaled afterwards (exact near the maximum, and it cannot overflow).
  auto mask_and_max = [&](int t, f32x16 (&s)[2]) {
    const int key0 = t * kBN;
    if (key0 + kBN - 1 > past + min(tok0 + wave * TPW, qlen - 1)) {
      const int lim = row_lim - key0 - 4 * eta;     // last visible key offset (eta = 0)
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          s[st][r] = 32 * st + 8 * (r >> 2) + (r & 3) <= lim ? s[st][r] : -INFINITY;
    }
    float lm = -INFINITY;
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int r = 0; r < 16; ++r) lm = fmaxf(lm, s[st][r]);
    if (__ballot((lm - m_run) * c2 > kPfSlack)) {
      const float m_new = fmaxf(m_run, fmaxf(lm, __shfl_xor(lm, 32, 64)));
      const float alpha = fast_exp2((m_run - m_new) * c2);
      m_run = m_new;
      m_log = m_new * c2;
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < NDT; ++i) o[i] *= alpha;
    }
  };
  // P' = 2^7 * 2^(s*c2 - m) in fp16, in the PV B-operand layout (chunk c =
  // regs 8c..8c+7), and partial sums of the same fp16 values, two per dot.
  auto exps = [&](const f32x16 (&s)[2], f16x8 (&p)[4], float (&lp)[4], bool huge) {
    const float bias = kPfPScaleLog2 - m_log;
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        p[2 * st + (r >> 3)][r & 7] =
            huge ? (f16)fast_exp2(safe_score_arg(s[st][r], m_run, c2, kPfPScaleLog2))
                 : (f16)fast_exp2(fmaf(s[st][r], c2, bias));
    const f16x2 ones = (f16x2){(f16)1.0f, (f16)1.0f};
#pragma unroll
    for (int i = 0; i < 4; ++i) lp[i] = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        lp[i] = __builtin_amdgcn_fdot2((f16x2){p[c][2 * i], p[c][2 * i + 1]}, ones, lp[i], false);
  };
  // The phases below are written as 16 bundles, each one matrix product plus
  // the operand reads and vector work placed beside it; sched_barrier fences
  // keep the bundles in order, so every product finds its operands already
  // read (up to four LDS reads in flight) and the vector ALUs work while the
  // matrix cores run.
  //
  // Phase A of step t: the QK product of tile t+1 (operand i: rows
  // 32*(i%2)..+31, channels 16*(i/2)..+15; the two accumulations alternate)
  // beside the exponentials of tile t, two scores per bundle.
  auto phase_a = [&](auto do_qk, int t, const f32x16 (&s_cur)[2], f32x16 (&s_next)[2],
                     f16x8 (&p)[4], float (&lp)[4]) {
    constexpr bool QK = decltype(do_qk)::value;
    constexpr int NM = 2 * NKK;                     // products (16 for D = 128)
    const float bias = kPfPScaleLog2 - m_log;
    const f16x2 ones = (f16x2){(f16)1.0f, (f16)1.0f};
    const uint8_t* k0p = lds[(t + 1) & 1] + n * KROW + 8 * KB * eta;
    auto kaddr = [&](int i) { return k0p + (i & 1) * 32 * KROW + 16 * KB * (i >> 1); };
    KOp ka[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) lp[i] = 0.f;
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (QK) {
      s_next[0] = (f32x16){};
      s_next[1] = (f32x16){};
#pragma unroll
      for (int i = 0; i < 4 && i < NM; ++i) ka[i] = kread(kaddr(i));
    }
    // score pair j = scores 2j, 2j+1 of this lane (block j/8, registers
    // 2j%16, +1); bundle i forms the exponent of pair i+1, the powers of pair
    // i and the fp16 values and sums of pair i-1, so no result is used in the
    // bundle that makes it
    auto arg = [&](int j, int e) { return fmaf(s_cur[j >> 3][(2 * j + e) & 15], c2, bias); };
    float x0 = arg(0, 0), x1 = arg(0, 1), y0 = 0.f, y1 = 0.f;
    auto finish = [&](int j, float a0, float a1) {
      const f16 e0 = (f16)a0, e1 = (f16)a1;
      const int st = j >> 3, r = (2 * j) & 15;
      p[2 * st + (r >> 3)][r & 7] = e0;
      p[2 * st + (r >> 3)][(r & 7) + 1] = e1;
      lp[j & 3] = __builtin_amdgcn_fdot2((f16x2){e0, e1}, ones, lp[j & 3], false);
    };
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (QK) {
        if (i < NM) {
          s_next[i & 1] = MK::run(kop(ka[i & 3]), qop[i >> 1], s_next[i & 1]);
          if (i + 4 < NM) ka[i & 3] = kread(kaddr(i + 4));
        }
      }
      if (i > 0) finish(i - 1, y0, y1);
      y0 = fast_exp2(x0);
      y1 = fast_exp2(x1);
      if (i + 1 < 16) {
        x0 = arg(i + 1, 0);
        x1 = arg(i + 1, 1);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    finish(15, y0, y1);
    __builtin_amdgcn_sched_barrier(0);
  };
  // Phase B of step t: O^T += V^T P^T for tile t (product i: channel tile
  // i/4, key chunk i%4) beside the conversion of the K codes of tile t+2
  // (into buffer t & 1) and the V codes of tile t+1 (into buffer (t+1) & 1),
  // and then the loads of the codes of K(t+3) and V(t+2) into the same
  // registers.
  // The V^T operand comes from the row-major V tile through transposing
  // reads (ds_read_b64_tr_b16): in each 16-lane group, lane s gives the
  // address of 4 channels (block s%4 of the group's 16) of one key (s/4 of a
  // run of 4), and lane j receives channel j of those 4 keys.  Two reads give
  // a lane the 8 keys its operand slots hold in the layout of P (keys
  // 16c + 4*eta + {0..3, 8..11} of chunk c).
  const int vg = lane >> 4, vs = lane & 15;
  const uint32_t v_lane = (uint32_t)((4 * (vg >> 1) + (vs >> 2)) * Geo::VROW +
                                     2 * (16 * (vg & 1) + 4 * (vs & 3)));
  auto phase_b = [&](int t, const f16x8 (&p)[4], RawK& rk, RawK& rv, const TileBlocks& tbk,
                     const TileBlocks& tbv) {
    constexpr int NM = 4 * NDT;                     // products (16 for D = 128)
    typedef short i16x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    const uint8_t* vb = lds[t & 1] + kBN * KROW + v_lane;
    auto vread = [&](int i) -> f16x8 {
      const uint8_t* q = vb + 16 * (i & 3) * Geo::VROW + 64 * (i >> 2);
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(q));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(q + 8 * Geo::VROW));
      return __builtin_bit_cast(f16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    f16x8 va[4];
    KWords kw[2], vw[2];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 4; ++i) va[i] = vread(i);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      __builtin_amdgcn_sched_barrier(0);
      if (i < NM) {
        o[i >> 2] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va[i & 3], p[i & 3], o[i >> 2], 0, 0, 0);
        if (i + 4 < NM) va[i & 3] = vread(i + 4);
      }
      // unit u: K decoded in bundle u and written in bundle u+1, V decoded in
      // bundle KL+1+u and written in bundle KL+2+u
      if constexpr (KPU) {
        if (i < KL) stage_raw_k(t & 1, i, rk.k[i]);
      } else {
        if (i >= 1 && i <= KL) stage_write(t & 1, 0, i - 1, kw[(i - 1) & 1]);
        if (i < KL) decode_unit<KVF, TK>(rk.k[i], kw[i & 1]);
      }
      if (i >= KL + 2 && i <= 2 * KL + 1) stage_write((t + 1) & 1, 1, i - KL - 2, vw[(i - KL - 2) & 1]);
      if (i >= KL + 1 && i <= 2 * KL) v_decode(rv, t + 1, i - KL - 1, vw[(i - KL - 1) & 1]);
      if (i == 15) {
        load_k(rk, tbk, t + 3);
        load_v(rv, tbv, t + 2);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  // Step t: mask/max/rescale of tile t, phase A, phase B (which also issues
  // the loads of K(t+3) and V(t+2) once the codes it converts are read),
  // barrier.  The conversions of step t write LDS regions no wave reads
  // during step t (K(t) and V(t-1) were last read before the previous
  // barrier), and what they write is read after this step's barrier.
  auto step = [&](int t, f32x16 (&s_cur)[2], f32x16 (&s_next)[2]) {
    mask_and_max(t, s_cur);
    const TileBlocks tbC = tile_blocks(t + 4);
    f16x8 p[4];
    float lp[4];
    if (t + 1 < ntiles)
      phase_a(std::true_type{}, t, s_cur, s_next, p, lp);
    else
      phase_a(std::false_type{}, t, s_cur, s_next, p, lp);
    if (__builtin_expect(__ballot(!(fabsf(m_log) <= kHugeScoreLog2)) != 0, 0))
      exps(s_cur, p, lp, true);
    l_run += (lp[0] + lp[1]) + (lp[2] + lp[3]);
    phase_b(t, p, rk, rv, tbB, tbA);
    v_zero_tail(t + 1, (t + 1) & 1);
    __syncthreads();
    tbA = tbB;
    tbB = tbC;
  };

  store_k(rk, 0);
  store_v(rv, 0, 0);
  store_k(rk1, 1);
  load_k(rk, tb2, 2);
  load_v(rv, tbB, 1);
  tbA = tb2;
  tbB = tile_blocks(3);
  __syncthreads();
  f32x16 sa[2], sb[2];
  qk(0, sa);
  __syncthreads();                 // buffer 0's K rows are rewritten in step 0
  for (int kt = 0; kt < ntiles; kt += 2) {
    step(kt, sa, sb);
    if (kt + 1 >= ntiles) break;
    step(kt + 1, sb, sa);
  }

  // ---- epilogue: normalise, value scale, store the rows of this wave ----
  l_run += __shfl_xor(l_run, 32, 64);
  const int tok = tok0 + wave * TPW + n / G;
  if (tok < qlen) {
    const float inv = (l_run > 0.f) ? 1.f / l_run : 0.f;       // both carry 2^7
    const float bias = (l_run > 0.f) ? kPfVBias<KVF> : 0.f;
    TQ* orow = reinterpret_cast<TQ*>(a.out) + ((size_t)(q0 + tok) * H + hq) * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int d = 32 * dt + 8 * (r >> 2) + 4 * eta + (r & 3);
        const float vs = (SM == SCALE_CHANNEL) ? a.v_scale[h * D + d] : a.v_scale[h];
        orow[d] = from_f32<TQ>((o[dt][r] * inv - bias) * vs);
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
  constexpr int NW = kPfWavesPerGroup;
  static_assert(NW == kPrefillWaves, "prefill geometry");
  dim3 grid(a.grid_x, 1, 1);                  // from the host plan (exact tile counts)
  if (a.pf_k_per_use) {
    // the per-use conversion variant: 1-byte formats at head size 128
    if constexpr (KVF != KV_INT4 && D == 128) {
      hipLaunchKernelGGL((prefill_mfma_kernel<D, KVF, SM, TQ, TK, NW, true>), grid,
                         dim3(NW * 64), 0, st, a, a.block_table);
      return 0;
    }
    return -1;
  }
  hipLaunchKernelGGL((prefill_mfma_kernel<D, KVF, SM, TQ, TK, NW, false>), grid, dim3(NW * 64),
                     0, st, a, a.block_table);
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
