// attn_f32.hip -- portable fp32 paged attention over the quantized cache.
//
// Plays the role of the "safe FP32" kernel of "ONNX Runtime: INT4 Paged KV
// Cache" (reviewer-feedback section): every product and sum is fp32, no fold of
// the key scale into a 16-bit query, so it takes fp32 queries and any case the
// 16-bit MFMA kernels do not cover.  One workgroup per (query row, kv head,
// KV chunk); it handles the whole GQA group of that kv head.  Any q_len (the
// causal cut is per row), so it serves decode and prefill; with num_splits > 1
// it writes normalised partials (o, lse) for the combine kernel instead of the
// output ("GQA GEMV decode", section 2: flash decoding partials).
//
// Keys are processed 256 at a time, one per thread for the scores (online
// softmax across chunks; the thread loads its key's key and value rows at
// once and leaves the value row in LDS), then every thread owns one channel of
// one key slice for the probability-weighted value sum over those LDS rows.  Scores stay in raw units (query
// times key scale over its power-of-two normaliser, dotted with the codes);
// exponents are formed as (raw - raw max) * factor, so key scales anywhere in
// the finite fp32 range neither overflow nor produce a NaN.
#include "append.hpp"
#include "device.hpp"
#include "launch.hpp"

namespace paq {

constexpr int kF32Threads = 256;
constexpr int kF32MaxGroup = kF32KernelMaxGroup;
constexpr int kF32MaxD = 128;

constexpr int kF32Units = kF32MaxD / 16;      // 16-byte units of the longest row

// 16 channel values from channel d0 (a multiple of 16) of a cache row held as
// its raw 16-byte units (the index is a compile-time constant wherever the
// callers' loops are unrolled).
template <int KVF>
__device__ __forceinline__ void codes16(const u32x4 (&w)[kF32Units], int d0, float (&k)[16]) {
  if constexpr (KVF == KV_INT4) {
    const u32x4 u = w[d0 / 32];                 // bytes d0/2 .. d0/2 + 7
    const uint32_t x0 = (d0 & 16) ? u[2] : u[0], x1 = (d0 & 16) ? u[3] : u[1];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t nib = ((i < 8 ? x0 : x1) >> (4 * (i % 8))) & 0xF;
      k[i] = (float)((int)(nib ^ 8u) - 8);
    }
  } else {
    const u32x4 u = w[d0 / 16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t byte = (u[i / 4] >> (8 * (i % 4))) & 0xFF;
      if constexpr (KVF == KV_INT8) {
        k[i] = (float)(int8_t)byte;
      } else {
        k[i] = e4m3_to_f32(byte);
      }
    }
  }
}

// the value of channel d of a cache row in LDS
template <int KVF>
__device__ __forceinline__ float code_at(const uint8_t* row, int d) {
  if constexpr (KVF == KV_INT4) {
    const uint32_t nib = (row[d / 2] >> (4 * (d & 1))) & 0xF;
    return (float)((int)(nib ^ 8u) - 8);
  } else if constexpr (KVF == KV_INT8) {
    return (float)(int8_t)row[d];
  } else {
    return e4m3_to_f32((uint32_t)row[d]);
  }
}

// MG: the largest GQA group the instance serves (4 or 16): loops over the
// group and the LDS arrays are sized by it, so small groups run short code.
// APPEND: the decode step's new key and value rows (a.new_key / a.new_value,
// in the query's dtype) are quantized here by the workgroup whose chunk holds
// the new key -- threads [0, 2 D / 8) form 8 channels' codes each with the
// append's arithmetic, store them into the caches and into LDS -- and the
// thread of that key takes its codes from LDS, so the cache store needs no
// wait.
template <int KVF, int SM, typename TQ, int MG, bool APPEND>
__global__ __launch_bounds__(kF32Threads) void attn_f32_kernel(AttnArgs a) {
  const int r = blockIdx.x;
  const int g = blockIdx.y;
  const int chunk = blockIdx.z;
  const int H = a.num_heads, hkv = a.hkv, D = a.head_size, bs = a.block_size;
  const int G = H / hkv;
  const int C = (KVF == KV_INT4) ? D / 2 : D;
  const int tid = threadIdx.x;

  // Loads that do not depend on the row's sequence go first, so that they
  // share one memory latency with the sequence search: this thread's key
  // scale (for the normaliser) and its query elements with their scales.
  const float ks_mine = (SM == SCALE_CHANNEL) ? (tid < D ? fabsf(a.k_scale[g * D + tid]) : 0.f)
                                              : fabsf(a.k_scale[g]);
  constexpr int kQPer = MG * kF32MaxD / kF32Threads;
  const TQ* q = reinterpret_cast<const TQ*>(a.query);
  float qv[kQPer], sv[kQPer];
#pragma unroll
  for (int u = 0; u < kQPer; ++u) {
    const int i = tid + u * kF32Threads;
    qv[u] = 0.f;
    sv[u] = 0.f;
    if (i < G * D) {
      const int hh = i / D, d = i % D;
      qv[u] = to_f32(q[((size_t)r * H + g * G + hh) * D + d]);
      sv[u] = (SM == SCALE_CHANNEL) ? a.k_scale[g * D + d] : a.k_scale[g];
    }
  }

  // the new rows' elements of this thread's 8 channels (loads go out now)
  const int app_units = 2 * D / 8;                      // 8-channel groups of K and V
  const bool app_thread = APPEND && tid < app_units;
  const bool app_v = tid >= D / 8;
  const int app_d0 = 8 * (app_v ? tid - D / 8 : tid);
  float app_x[8], app_s[8];
  if constexpr (APPEND) {
    if (app_thread) {
      load8(reinterpret_cast<const TQ*>(app_v ? a.new_value : a.new_key) +
                ((size_t)r * hkv + g) * D + app_d0,
            app_x);
      load_scales8<SM>(app_v ? a.v_scale : a.k_scale, g, D, app_d0, app_s);
    }
  }

  // sequence of this row: the largest b with cum_q[b] <= r, i.e. the number
  // of entries cum_q[1..batch] that are <= r (cum_q never decreases), counted
  // by every wave 64 entries per round trip
  const int wave = tid / 64, lane = tid % 64;
  int b = 0;
  for (int base = 1; base <= a.batch; base += 64) {
    const int idx = base + lane;
    const unsigned long long le = __ballot(idx <= a.batch && a.cum_q[idx] <= r);
    b += __builtin_popcountll(le);
    if (le != ~0ull) break;
  }
  const int i = r - a.cum_q[b];
  const int qlen = a.cum_q[b + 1] - a.cum_q[b];
  const int past = a.past_lens[b];
  const int kv_len = past + qlen;
  const int visible = past + i + 1;                    // keys 0..past+i
  const int nb = (kv_len + bs - 1) / bs;
  const int S = a.num_splits;                 // one partial per chunk (part_count == S)
  const int kbeg = (int)(((long)chunk * nb) / S) * bs;
  const int kend = min(visible, (int)(((long)(chunk + 1) * nb) / S) * bs);
  const int32_t* table = a.block_table + (size_t)b * a.max_blocks;

  __shared__ float qs[MG][kF32MaxD];
  __shared__ float sc[MG][kF32Threads];
  __shared__ float m_sh[MG], l_sh[MG], alpha_sh[MG];
  __shared__ int e_sh;
  __shared__ __attribute__((aligned(16))) uint8_t vrows[kF32Threads * (kF32MaxD + 16)];
  __shared__ __attribute__((aligned(16))) uint8_t new_rows[2][kF32MaxD];   // fused append

  // fused append: this chunk holds the new key (decode: row r is the
  // sequence's one new token, at key `past`)
  const bool app_here = APPEND && qlen == 1 && kbeg <= past && past < kend;
  if constexpr (APPEND) {
    if (app_here && app_thread) {
      const u32x2 w = codes8<KVF>(app_x, app_s);
      const int ob = (KVF == KV_INT4) ? app_d0 / 2 : app_d0;   // byte offset in the row
      const int blk = table[past / bs];
      uint8_t* dst = const_cast<uint8_t*>(app_v ? a.value_cache : a.key_cache) +
                     (((size_t)blk * bs + past % bs) * hkv + g) * C + ob;
      if constexpr (KVF == KV_INT4) {
        *reinterpret_cast<uint32_t*>(dst) = w[0];
        *reinterpret_cast<uint32_t*>(&new_rows[app_v][ob]) = w[0];
      } else {
        *reinterpret_cast<u32x2*>(dst) = w;
        *reinterpret_cast<u32x2*>(&new_rows[app_v][ob]) = w;
      }
    }
  }

  // q' = q * s / M with M = 2^e >= max|s| of this kv head (exact scaling; M
  // finite for every finite scale): raw scores q'.codes never overflow, and
  // the score factor c2 = softmax_scale * M * log2(e) is kept finite
  const int e = key_scale_exponent_of<SM>(ks_mine, &e_sh);
  const float c2 = score_factor_log2(a.softmax_scale, e, 1.f);
#pragma unroll
  for (int u = 0; u < kQPer; ++u) {
    const int i2 = tid + u * kF32Threads;
    if (i2 < G * D) qs[i2 / D][i2 % D] = qv[u] * ldexpf(sv[u], -e);
  }
  if (tid < G) { m_sh[tid] = -INFINITY; l_sh[tid] = 0.f; }

  const int nslice = kF32Threads / D;
  const int my_d = tid % D;
  const int my_slice = tid / D;
  float acc[MG];
#pragma unroll
  for (int hh = 0; hh < MG; ++hh) acc[hh] = 0.f;
  __syncthreads();

  const int vst = C + 16;                 // LDS value row stride (16-byte aligned, padded)
  for (int base = kbeg; base < kend; base += kF32Threads) {
    // one key per thread: its key and value rows are loaded together (every
    // unit in flight at once), the value row goes to LDS for the weighted sum
    const int j = base + tid;
    float dot[MG];
#pragma unroll
    for (int hh = 0; hh < MG; ++hh) dot[hh] = 0.f;
    if (j < kend) {
      u32x4 kw[kF32Units], vw[kF32Units];
      if (APPEND && app_here && j == past) {
        // the new key's codes, formed above (the cache store may not have landed)
#pragma unroll
        for (int u = 0; u < kF32Units; ++u) {
          if (16 * u >= C) break;
          kw[u] = *reinterpret_cast<const u32x4*>(&new_rows[0][16 * u]);
          vw[u] = *reinterpret_cast<const u32x4*>(&new_rows[1][16 * u]);
        }
      } else {
        const int blk = table[j / bs];
        const size_t off = (((size_t)blk * bs + j % bs) * hkv + g) * C;
#pragma unroll
        for (int u = 0; u < kF32Units; ++u) {
          if (16 * u >= C) break;
          kw[u] = *reinterpret_cast<const u32x4*>(a.key_cache + off + 16 * u);
          vw[u] = *reinterpret_cast<const u32x4*>(a.value_cache + off + 16 * u);
        }
      }
#pragma unroll
      for (int u = 0; u < kF32Units; ++u) {
        if (16 * u >= C) break;
        *reinterpret_cast<u32x4*>(vrows + tid * vst + 16 * u) = vw[u];
      }
#pragma unroll
      for (int u = 0; u < kF32Units; ++u) {
        if (16 * u >= D) break;
        float k[16];
        codes16<KVF>(kw, 16 * u, k);
#pragma unroll
        for (int hh = 0; hh < MG; ++hh) {
          if (hh < G) {
            float s = dot[hh];
#pragma unroll
            for (int e = 0; e < 16; ++e) s = fmaf(qs[hh][16 * u + e], k[e], s);
            dot[hh] = s;
          }
        }
      }
    }
#pragma unroll
    for (int hh = 0; hh < MG; ++hh)
      if (hh < G) sc[hh][tid] = (j < kend) ? dot[hh] : -INFINITY;   // raw scores
    __syncthreads();
    // per-head chunk maximum -> new running max and rescale factor
    for (int hh = wave; hh < G; hh += kF32Threads / 64) {
      float mx = -INFINITY;
      for (int t = lane; t < kF32Threads; t += 64) mx = fmaxf(mx, sc[hh][t]);
      mx = wave_max(mx);
      if (lane == 0) {
        const float m_old = m_sh[hh];
        const float m_new = fmaxf(m_old, mx);
        alpha_sh[hh] = (m_old == -INFINITY) ? 0.f : exp2f((m_old - m_new) * c2);
        m_sh[hh] = m_new;
      }
    }
    __syncthreads();
    for (int hh = 0; hh < G; ++hh) {
      const float v = sc[hh][tid];
      sc[hh][tid] = (v == -INFINITY) ? 0.f : exp2f((v - m_sh[hh]) * c2);
    }
    __syncthreads();
    for (int hh = wave; hh < G; hh += kF32Threads / 64) {
      float s = 0.f;
      for (int t = lane; t < kF32Threads; t += 64) s += sc[hh][t];
      s = wave_sum(s);
      if (lane == 0) l_sh[hh] = l_sh[hh] * alpha_sh[hh] + s;
    }
    // probability-weighted values: thread (slice, channel)
    if (my_slice < nslice) {
#pragma unroll
      for (int hh = 0; hh < MG; ++hh)
        if (hh < G) acc[hh] *= alpha_sh[hh];
      const int jn = min(kend - base, kF32Threads);
      // four keys per step with all their LDS reads issued first (the stride
      // is a run-time value, so the compiler does not unroll this itself),
      // then the rest one at a time; the sums run in key order either way
      int t = my_slice;
      for (; t + 3 * nslice < jn; t += 4 * nslice) {
        float v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = code_at<KVF>(vrows + (t + u * nslice) * vst, my_d);
#pragma unroll
        for (int hh = 0; hh < MG; ++hh) {
          if (hh < G) {
            float w[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) w[u] = sc[hh][t + u * nslice];
            float s = acc[hh];
#pragma unroll
            for (int u = 0; u < 4; ++u) s = fmaf(w[u], v[u], s);
            acc[hh] = s;
          }
        }
      }
      for (; t < jn; t += nslice) {
        const float v = code_at<KVF>(vrows + t * vst, my_d);
#pragma unroll
        for (int hh = 0; hh < MG; ++hh)
          if (hh < G) acc[hh] = fmaf(sc[hh][t], v, acc[hh]);
      }
    }
    __syncthreads();
  }

  // merge the key slices in one exchange: slices 1.. write their sums to sc
  // reused as [slice - 1][G][D] scratch ((nslice - 1) * G * D <= MG * 256
  // floats, since nslice * D = 256), then slice 0 adds them in slice order
  float* scratch = &sc[0][0];
  if (my_slice > 0 && my_slice < nslice) {
#pragma unroll
    for (int hh = 0; hh < MG; ++hh)
      if (hh < G) scratch[((my_slice - 1) * G + hh) * D + my_d] = acc[hh];
  }
  __syncthreads();
  if (my_slice != 0) return;
  for (int sl = 1; sl < nslice; ++sl) {
#pragma unroll
    for (int hh = 0; hh < MG; ++hh)
      if (hh < G) acc[hh] += scratch[((sl - 1) * G + hh) * D + my_d];
  }
  const float vs = (SM == SCALE_CHANNEL) ? a.v_scale[g * D + my_d] : a.v_scale[g];
#pragma unroll
  for (int hh = 0; hh < MG; ++hh) {
    if (hh >= G) break;
    const int h = g * G + hh;
    const float l = l_sh[hh];
    const float o = (l > 0.f) ? acc[hh] / l : 0.f;
    if (S == 1) {
      TQ* out = reinterpret_cast<TQ*>(a.out);
      out[((size_t)r * H + h) * D + my_d] = from_f32<TQ>(o * vs);
    } else {
      // split-KV partials leave the value scale to the combine; the chunk's
      // log-sum-exp is kept as the pair (raw maximum, log2 of the sum), which
      // cannot overflow at any score factor (the combine scales differences
      // of raw maxima by c2)
      const size_t pi = ((size_t)r * H + h) * S + chunk;
      a.part_o[pi * D + my_d] = o;
      if (my_d == 0) {
        a.part_lse[2 * pi] = (l > 0.f) ? m_sh[hh] : -INFINITY;
        a.part_lse[2 * pi + 1] = (l > 0.f) ? log2f(l) : -INFINITY;
      }
    }
  }
}

template <int KVF, int SM, int MG, bool APPEND>
static int launch_qa(const AttnArgs& a, dim3 grid, hipStream_t st) {
  switch (a.q_dtype) {
    case DT_F32: hipLaunchKernelGGL((attn_f32_kernel<KVF, SM, float, MG, APPEND>), grid, dim3(kF32Threads), 0, st, a); return 0;
    case DT_F16: hipLaunchKernelGGL((attn_f32_kernel<KVF, SM, f16, MG, APPEND>), grid, dim3(kF32Threads), 0, st, a); return 0;
    case DT_BF16: hipLaunchKernelGGL((attn_f32_kernel<KVF, SM, bf16, MG, APPEND>), grid, dim3(kF32Threads), 0, st, a); return 0;
  }
  return -1;
}

template <int KVF, int SM, int MG>
static int launch_q(const AttnArgs& a, dim3 grid, hipStream_t st) {
  return a.new_key ? launch_qa<KVF, SM, MG, true>(a, grid, st)
                   : launch_qa<KVF, SM, MG, false>(a, grid, st);
}

template <int KVF, int SM>
static int launch_g(const AttnArgs& a, dim3 grid, hipStream_t st) {
  return a.num_heads / a.hkv <= 4 ? launch_q<KVF, SM, 4>(a, grid, st)
                                  : launch_q<KVF, SM, kF32MaxGroup>(a, grid, st);
}

int launch_decode_f32(const AttnArgs& a, hipStream_t st) {
  if (a.num_heads / a.hkv > kF32MaxGroup || a.head_size > kF32MaxD || a.token_count == 0) return -1;
  dim3 grid(a.token_count, a.hkv, a.num_splits);
  switch (a.kv_format * 2 + a.scale_mode) {
    case KV_INT8 * 2 + SCALE_CHANNEL: return launch_g<KV_INT8, SCALE_CHANNEL>(a, grid, st);
    case KV_INT8 * 2 + SCALE_HEAD: return launch_g<KV_INT8, SCALE_HEAD>(a, grid, st);
    case KV_INT4 * 2 + SCALE_CHANNEL: return launch_g<KV_INT4, SCALE_CHANNEL>(a, grid, st);
    case KV_INT4 * 2 + SCALE_HEAD: return launch_g<KV_INT4, SCALE_HEAD>(a, grid, st);
    case KV_FP8 * 2 + SCALE_CHANNEL: return launch_g<KV_FP8, SCALE_CHANNEL>(a, grid, st);
    case KV_FP8 * 2 + SCALE_HEAD: return launch_g<KV_FP8, SCALE_HEAD>(a, grid, st);
  }
  return -1;
}

}  // namespace paq
