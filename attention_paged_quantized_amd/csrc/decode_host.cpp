// decode_host.cpp -- GQA decode on the host CPU over host-resident paged,
// quantized caches ("GQA GEMV decode", sections 2-3): a dedicated M = 1 kernel
// that streams each key row straight into dot products and each value row
// into a weighted sum, with no matrix packing; when batch x kv heads leaves
// threads idle, every sequence's keys are split into chunks (flash decoding)
// whose partial results are merged by their log-sum-exps.
//
// Per work unit (sequence b, kv head g, key chunk [k0, k1)) the G query heads
// of g are handled together, so each key and value row is dequantized once:
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
constexpr int kMaxG = 64;            // query heads per kv head handled at once

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

// codes of one cache row (kv head g of a token) as floats
void row_codes(const uint8_t* row, int kv_format, int D, float* out) {
  if (kv_format == 0) {                                    // INT8
    const int8_t* r = reinterpret_cast<const int8_t*>(row);
    for (int d = 0; d < D; ++d) out[d] = (float)r[d];
  } else if (kv_format == 1) {                             // INT4, low nibble first
    for (int j = 0; j < D / 2; ++j) {
      const int b = row[j];
      out[2 * j] = (float)((b & 15) ^ 8) - 8.f;
      out[2 * j + 1] = (float)((b >> 4) ^ 8) - 8.f;
    }
  } else {                                                 // FP8 E4M3
    const float* t = fp8_table().v;
    for (int d = 0; d < D; ++d) out[d] = t[row[d]];
  }
}

// dot product with 8 partial sums (vectorizes without reassociation flags)
inline float dot8(const float* a, const float* b, int D) {
  float s[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int d = 0; d < D; d += 8)
    for (int i = 0; i < 8; ++i) s[i] += a[d + i] * b[d + i];
  return ((s[0] + s[1]) + (s[2] + s[3])) + ((s[4] + s[5]) + (s[6] + s[7]));
}

struct Partial {
  float m[kMaxG], l[kMaxG];
  std::vector<float> acc;            // [G][D]
};

void run_unit(const HostDecodeArgs& a, int b, int g, int k0, int k1, Partial& p) {
  const int D = a.head_size, G = a.num_heads / a.hkv, hkv = a.hkv;
  const int C = a.kv_format == 1 ? D / 2 : D;
  const int row = a.cum_q[b];
  std::vector<float> q(G * D), kc(D), vc(D), s(G * kTile);
  for (int h = 0; h < G; ++h) {
    const float* qs = a.query + ((size_t)row * a.num_heads + g * G + h) * D;
    for (int d = 0; d < D; ++d) {
      const float ks = a.scale_mode == 0 ? a.k_scale[g * D + d] : a.k_scale[g];
      q[h * D + d] = a.softmax_scale * qs[d] * ks;
    }
    p.m[h] = -INFINITY;
    p.l[h] = 0.f;
  }
  p.acc.assign((size_t)G * D, 0.f);
  const int32_t* table = a.block_table + (size_t)b * a.max_blocks;
  auto cache_row = [&](const uint8_t* cache, int t) {
    const int blk = table[t / a.block_size];
    return cache + (((size_t)blk * a.block_size + t % a.block_size) * hkv + g) * C;
  };
  for (int t0 = k0; t0 < k1; t0 += kTile) {
    const int n = std::min(kTile, k1 - t0);
    for (int j = 0; j < n; ++j) {                          // scores of the tile
      row_codes(cache_row(a.key_cache, t0 + j), a.kv_format, D, kc.data());
      for (int h = 0; h < G; ++h) s[h * kTile + j] = dot8(&q[h * D], kc.data(), D);
    }
    for (int h = 0; h < G; ++h) {                          // online softmax update
      float mt = p.m[h];
      for (int j = 0; j < n; ++j) mt = std::max(mt, s[h * kTile + j]);
      const float alpha = (p.m[h] == -INFINITY) ? 0.f : expf(p.m[h] - mt);
      p.l[h] *= alpha;
      for (int d = 0; d < D; ++d) p.acc[h * D + d] *= alpha;
      p.m[h] = mt;
      for (int j = 0; j < n; ++j) {
        const float e = expf(s[h * kTile + j] - mt);
        s[h * kTile + j] = e;
        p.l[h] += e;
      }
    }
    for (int j = 0; j < n; ++j) {                          // weighted value rows
      row_codes(cache_row(a.value_cache, t0 + j), a.kv_format, D, vc.data());
      for (int h = 0; h < G; ++h) {
        const float w = s[h * kTile + j];
        float* acc = &p.acc[h * D];
        for (int d = 0; d < D; ++d) acc[d] += w * vc[d];
      }
    }
  }
}

}  // namespace

int host_decode(const HostDecodeArgs& a) {
  const int G = a.num_heads / a.hkv, D = a.head_size;
  if (G > kMaxG) return -1;
  // work units: (active sequence, kv head), split into S key chunks of whole
  // blocks when they would leave threads idle
  std::vector<int> seqs;
  for (int b = 0; b < a.batch; ++b)
    if (a.cum_q[b + 1] > a.cum_q[b]) seqs.push_back(b);
  if (seqs.empty()) return 0;
  const int threads = std::max(1, a.threads);
  const long units = (long)seqs.size() * a.hkv;
  int S = 1;
  if (a.splits > 0) S = a.splits;
  else if (units < threads) S = (int)((threads + units - 1) / units);
  struct Item { int b, g, c; };
  std::vector<Item> items;
  for (int b : seqs)
    for (int g = 0; g < a.hkv; ++g)
      for (int c = 0; c < S; ++c) items.push_back({b, g, c});
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
        for (int h = 0; h < G; ++h) { parts[i].m[h] = -INFINITY; parts[i].l[h] = 0.f; }
        parts[i].acc.assign((size_t)G * D, 0.f);
        continue;
      }
      run_unit(a, it.b, it.g, k0, k1, parts[i]);
    }
  };
  const int nthr = (int)std::min<size_t>(threads, items.size());
  std::vector<std::thread> pool;
  for (int t = 1; t < nthr; ++t) pool.emplace_back(worker);
  worker();
  for (auto& t : pool) t.join();
  // merge the S chunks of each (sequence, kv head) by their log-sum-exps
  for (size_t u = 0; u < items.size(); u += S) {
    const int b = items[u].b, g = items[u].g, row = a.cum_q[b];
    for (int h = 0; h < G; ++h) {
      float M = -INFINITY;
      for (int c = 0; c < S; ++c) M = std::max(M, parts[u + c].m[h]);
      float L = 0.f;
      float* o = a.out + ((size_t)row * a.num_heads + g * G + h) * D;
      for (int d = 0; d < D; ++d) o[d] = 0.f;
      if (M == -INFINITY) continue;
      for (int c = 0; c < S; ++c) {
        const Partial& p = parts[u + c];
        if (p.m[h] == -INFINITY) continue;
        const float f = expf(p.m[h] - M);
        L += f * p.l[h];
        for (int d = 0; d < D; ++d) o[d] += f * p.acc[h * D + d];
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
