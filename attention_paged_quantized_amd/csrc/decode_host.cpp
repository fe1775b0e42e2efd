// decode_host.cpp -- GQA decode on the host CPU over host-resident paged,
// quantized caches ("GQA GEMV decode", sections 2-3): a dedicated M = 1 kernel
// that streams each key row straight into dot products and each value row
// into a weighted sum, with no matrix packing; when batch x kv heads leaves
// threads idle, every sequence's keys are split into chunks (flash decoding)
// whose partial results are merged by their log-sum-exps.
//
// Per work unit (sequence b, key chunk [k0, k1)) every kv head g and its G
// query heads are handled together, so each key and value row is dequantized
// once and the cache is read in address order:
//   q'[h][d] = softmax_scale * q[h][d] * k_scale[g][d]      (fp32)
//   s[h][t]  = sum_d q'[h][d] * kcode[t][d]                 (8 partial sums)
//   a tile of 256 keys at a time: running max m, sum l, acc += p * vcode,
//   out[h][d] = acc[h][d] * v_scale[g][d] / l.
// fp32 throughout; the codes are exact in fp32.
#include "decode_host.hpp"

#include <math.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <thread>
#include <vector>

namespace paq {
namespace {

constexpr int kTile = 256;           // keys per softmax tile

// OCP E4M3 value of every code (bias 7, subnormals below exponent 1, S.1111.111 NaN)
struct Fp8Table {
  float v[256];
  Fp8Table() {
    for (int c = 0; c < 256; ++c) {
      const int e = (c >> 3) & 15, m = c & 7;
      float x;
      if (e == 15 && m == 7) x = NAN;
      else if (e == 0) x = ldexpf((float)m, -9);
      else x = ldexpf((float)(8 + m), e - 10);
      v[c] = (c & 128) ? -x : x;
    }
  }
};
const Fp8Table& fp8_table() {
  static const Fp8Table t;
  return t;
}

// 8-wide float vectors (two SSE registers on any x86-64, one AVX register
// where the AVX2 copy of the unit runs)
typedef float f8 __attribute__((ext_vector_type(8)));
typedef int8_t i8x8 __attribute__((ext_vector_type(8)));
typedef uint8_t u8x4 __attribute__((ext_vector_type(4)));
typedef int8_t s8x4 __attribute__((ext_vector_type(4)));

inline f8 load8(const float* p) {
  f8 v;
  memcpy(&v, p, sizeof v);
  return v;
}

// codes of one cache row (kv head g of a token) as D / 8 float vectors
template <int D, int KVF>
inline void row_codes(const uint8_t* row, f8* out) {
  if constexpr (KVF == 0) {                                // INT8
    for (int i = 0; i < D / 8; ++i) {
      i8x8 c;
      memcpy(&c, row + 8 * i, 8);
      out[i] = __builtin_convertvector(c, f8);
    }
  } else if constexpr (KVF == 1) {                         // INT4, low nibble first
    for (int i = 0; i < D / 8; ++i) {
      u8x4 b;
      memcpy(&b, row + 4 * i, 4);
      const s8x4 lo = __builtin_convertvector((b & (uint8_t)15) ^ (uint8_t)8, s8x4) - (int8_t)8;
      const s8x4 hi = __builtin_convertvector((b >> 4) ^ (uint8_t)8, s8x4) - (int8_t)8;
      const i8x8 c = __builtin_shufflevector(lo, hi, 0, 4, 1, 5, 2, 6, 3, 7);
      out[i] = __builtin_convertvector(c, f8);
    }
  } else {                                                 // FP8 E4M3
    const float* t = fp8_table().v;
    alignas(32) float f[D];
    for (int d = 0; d < D; ++d) f[d] = t[row[d]];
    for (int i = 0; i < D / 8; ++i) out[i] = load8(f + 8 * i);
  }
}

typedef int32_t i32x8 __attribute__((ext_vector_type(8)));

inline float hsum(f8 s) { return ((s[0] + s[1]) + (s[2] + s[3])) + ((s[4] + s[5]) + (s[6] + s[7])); }

// e^x for the softmax's arguments x <= 0, 8 at a time, and exactly 0 below
// -87 (where e^x leaves the normal fp32 range): x = n ln2 + r with n the
// nearest integer to x / ln2 (ln2 split into a 24-bit head and a tail, so r is
// exact to rounding), e^r from its Taylor series to r^8 / 8! (|r| <= ln2 / 2,
// truncation below 1e-8 relative), times 2^n built in the exponent field.
inline f8 exp8(f8 x) {
  x = __builtin_elementwise_max(x, (f8)(-88.f));
  const f8 t = x * 1.44269504088896341f;
  const f8 n = (t + 12582912.f) - 12582912.f;              // round to nearest (|t| < 2^22)
  const f8 r = (x - n * 0.693145751953125f) - n * 1.42860682030941723e-6f;
  f8 p = 1.f / 40320.f;
  p = p * r + 1.f / 5040.f;
  p = p * r + 1.f / 720.f;
  p = p * r + 1.f / 120.f;
  p = p * r + 1.f / 24.f;
  p = p * r + 1.f / 6.f;
  p = p * r + 0.5f;
  p = p * r + 1.f;
  p = p * r + 1.f;
  const i32x8 bits = (__builtin_convertvector(n, i32x8) + 127) << 23;
  const f8 e = p * __builtin_bit_cast(f8, bits);
  const i32x8 keep = x >= (f8)(-87.f);                     // all ones where kept
  return __builtin_bit_cast(f8, __builtin_bit_cast(i32x8, e) & keep);
}

// dot product of D / 8 vector pairs, one vector of partial sums
template <int D>
inline float dot(const f8* a, const f8* b) {
  f8 s = a[0] * b[0];
  for (int i = 1; i < D / 8; ++i) s += a[i] * b[i];
  return hsum(s);
}

struct Partial {
  std::vector<float> m, l;           // [H]
  std::vector<f8> acc;               // [H][D / 8]
};

// One work unit: sequence b, keys [k0, k1), every kv head at once -- a
// token's key (value) rows of all kv heads are one contiguous run of
// hkv * C bytes, so the unit streams the cache in address order.
template <int D, int KVF>
__attribute__((always_inline)) inline void run_unit_t(const HostDecodeArgs& a, int b, int k0,
                                                      int k1, Partial& p) {
  const int H = a.num_heads, hkv = a.hkv, G = H / hkv;
  constexpr int C = KVF == 1 ? D / 2 : D;
  const int row = a.cum_q[b];
  f8 kc[D / 8], vc[D / 8];
  std::vector<f8> q((size_t)H * D / 8);
  std::vector<float> s((size_t)H * kTile);
  p.m.assign(H, -INFINITY);
  p.l.assign(H, 0.f);
  p.acc.assign((size_t)H * D / 8, f8{});
  for (int h = 0; h < H; ++h) {
    const int g = h / G;
    const float* qs = a.query + ((size_t)row * H + h) * D;
    for (int d = 0; d < D; ++d) {
      const float ks = a.scale_mode == 0 ? a.k_scale[g * D + d] : a.k_scale[g];
      q[(size_t)h * D / 8 + d / 8][d % 8] = a.softmax_scale * qs[d] * ks;
    }
  }
  const int32_t* table = a.block_table + (size_t)b * a.max_blocks;
  const size_t tok_bytes = (size_t)hkv * C;
  auto token_rows = [&](const uint8_t* cache, int t) {
    const int blk = table[t / a.block_size];
    return cache + ((size_t)blk * a.block_size + t % a.block_size) * tok_bytes;
  };
  for (int t0 = k0; t0 < k1; t0 += kTile) {
    const int n = std::min(kTile, k1 - t0);
    for (int j = 0; j < n; ++j) {                          // scores of the tile
      const uint8_t* kr = token_rows(a.key_cache, t0 + j);
      for (int g = 0; g < hkv; ++g) {
        row_codes<D, KVF>(kr + (size_t)g * C, kc);
        for (int hh = 0; hh < G; ++hh) {
          const int h = g * G + hh;
          s[(size_t)h * kTile + j] = dot<D>(&q[(size_t)h * D / 8], kc);
        }
      }
    }
    for (int h = 0; h < H; ++h) {                          // online softmax update
      float* sh = &s[(size_t)h * kTile];
      float mt = p.m[h];
      for (int j = 0; j < n; ++j) mt = std::max(mt, sh[j]);
      const float alpha = (p.m[h] == -INFINITY) ? 0.f : expf(p.m[h] - mt);
      p.l[h] *= alpha;
      for (int i = 0; i < D / 8; ++i) p.acc[(size_t)h * D / 8 + i] *= alpha;
      p.m[h] = mt;
      const int n8 = (n + 7) & ~7;                       // (kTile is a multiple of 8)
      for (int j = n; j < n8; ++j) sh[j] = -INFINITY;
      f8 l = {};
      for (int j = 0; j < n8; j += 8) {
        const f8 e = exp8(load8(sh + j) - mt);
        memcpy(sh + j, &e, sizeof e);
        l += e;
      }
      p.l[h] += hsum(l);
    }
    for (int j = 0; j < n; ++j) {                          // weighted value rows
      const uint8_t* vr = token_rows(a.value_cache, t0 + j);
      for (int g = 0; g < hkv; ++g) {
        row_codes<D, KVF>(vr + (size_t)g * C, vc);
        for (int hh = 0; hh < G; ++hh) {
          const int h = g * G + hh;
          const float w = s[(size_t)h * kTile + j];
          f8* acc = &p.acc[(size_t)h * D / 8];
          for (int i = 0; i < D / 8; ++i) acc[i] += w * vc[i];
        }
      }
    }
  }
}

// The same unit compiled twice: for any x86-64, and with AVX2 + FMA (taken
// when the CPU has them; the code is identical, the vector width differs).
template <int D, int KVF>
void run_unit_base(const HostDecodeArgs& a, int b, int k0, int k1, Partial& p) {
  run_unit_t<D, KVF>(a, b, k0, k1, p);
}
template <int D, int KVF>
__attribute__((target("avx2,fma"))) void run_unit_avx2(const HostDecodeArgs& a, int b, int k0,
                                                         int k1, Partial& p) {
  run_unit_t<D, KVF>(a, b, k0, k1, p);
}

typedef void (*UnitFn)(const HostDecodeArgs&, int, int, int, Partial&);

template <int D>
UnitFn pick_fmt(int kv_format, bool avx2) {
  switch (kv_format) {
    case 0: return avx2 ? run_unit_avx2<D, 0> : run_unit_base<D, 0>;
    case 1: return avx2 ? run_unit_avx2<D, 1> : run_unit_base<D, 1>;
    case 2: return avx2 ? run_unit_avx2<D, 2> : run_unit_base<D, 2>;
  }
  return nullptr;
}

UnitFn pick_unit(int head_size, int kv_format) {
  static const bool avx2 = __builtin_cpu_supports("avx2") && __builtin_cpu_supports("fma");
  if (head_size == 64) return pick_fmt<64>(kv_format, avx2);
  if (head_size == 128) return pick_fmt<128>(kv_format, avx2);
  return nullptr;
}

}  // namespace

int host_decode(const HostDecodeArgs& a) {
  const int H = a.num_heads, D = a.head_size;
  const UnitFn run_unit = pick_unit(D, a.kv_format);
  if (!run_unit) return -1;
  // work units: (active sequence, key chunk of whole blocks); with fewer
  // than four units per thread every sequence is cut into S chunks
  // (flash decoding), merged below by their log-sum-exps
  std::vector<int> seqs;
  for (int b = 0; b < a.batch; ++b)
    if (a.cum_q[b + 1] > a.cum_q[b]) seqs.push_back(b);
  if (seqs.empty()) return 0;
  const int threads = std::max(1, a.threads);
  const long nseq = (long)seqs.size();
  int S = 1;
  if (a.splits > 0) S = a.splits;
  else if (nseq < 4L * threads) S = (int)((4L * threads + nseq - 1) / nseq);
  struct Item { int b, c; };
  std::vector<Item> items;
  for (int b : seqs)
    for (int c = 0; c < S; ++c) items.push_back({b, c});
  std::vector<Partial> parts(items.size());
  std::atomic<size_t> next(0);
  auto worker = [&]() {
    for (size_t i; (i = next.fetch_add(1)) < items.size();) {
      const Item& it = items[i];
      const int L = a.past_lens[it.b] + 1;
      const int nb = (L + a.block_size - 1) / a.block_size;
      const int k0 = (int)((long)it.c * nb / S) * a.block_size;
      const int k1 = std::min(L, (int)((long)(it.c + 1) * nb / S) * a.block_size);
      if (k0 >= k1) {
        parts[i].m.assign(H, -INFINITY);
        parts[i].l.assign(H, 0.f);
        parts[i].acc.assign((size_t)H * D / 8, f8{});
        continue;
      }
      run_unit(a, it.b, k0, k1, parts[i]);
    }
  };
  const int nthr = (int)std::min<size_t>(threads, items.size());
  std::vector<std::thread> pool;
  for (int t = 1; t < nthr; ++t) pool.emplace_back(worker);
  worker();
  for (auto& t : pool) t.join();
  // merge the S chunks of each sequence by their log-sum-exps
  const int G = H / a.hkv;
  for (size_t u = 0; u < items.size(); u += S) {
    const int b = items[u].b, row = a.cum_q[b];
    for (int h = 0; h < H; ++h) {
      const int g = h / G;
      float M = -INFINITY;
      for (int c = 0; c < S; ++c) M = std::max(M, parts[u + c].m[h]);
      float L = 0.f;
      float* o = a.out + ((size_t)row * H + h) * D;
      for (int d = 0; d < D; ++d) o[d] = 0.f;
      if (M == -INFINITY) continue;
      for (int c = 0; c < S; ++c) {
        const Partial& p = parts[u + c];
        if (p.m[h] == -INFINITY) continue;
        const float f = expf(p.m[h] - M);
        L += f * p.l[h];
        for (int d = 0; d < D; ++d) o[d] += f * p.acc[((size_t)h * D + d) / 8][d % 8];
      }
      for (int d = 0; d < D; ++d) {
        const float vs = a.scale_mode == 0 ? a.v_scale[g * D + d] : a.v_scale[g];
        o[d] = o[d] / L * vs;
      }
    }
  }
  return 0;
}

}  // namespace paq
