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
// softmax across chunks, exact exp), then every thread owns one channel of one
// key slice for the probability-weighted value sum.
#include "device.hpp"
#include "launch.hpp"

namespace paq {

constexpr int kF32Threads = 256;
constexpr int kF32MaxGroup = 16;
constexpr int kF32MaxD = 128;

template <int KVF>
__device__ __forceinline__ void load_codes16(const uint8_t* row, int d0, float (&k)[16]) {
  if constexpr (KVF == KV_INT4) {
    u32x2 w = *reinterpret_cast<const u32x2*>(row + d0 / 2);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      uint32_t nib = (w[i / 8] >> (4 * (i % 8))) & 0xF;
      k[i] = (float)((int)(nib ^ 8u) - 8);
    }
  } else {
    u32x4 w = *reinterpret_cast<const u32x4*>(row + d0);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      uint32_t byte = (w[i / 4] >> (8 * (i % 4))) & 0xFF;
      if constexpr (KVF == KV_INT8) {
        k[i] = (float)(int8_t)byte;
      } else {
        k[i] = e4m3_to_f32(byte);
      }
    }
  }
}

template <int KVF>
__device__ __forceinline__ float load_code1(const uint8_t* row, int d) {
  if constexpr (KVF == KV_INT4) {
    uint32_t nib = (row[d / 2] >> (4 * (d & 1))) & 0xF;
    return (float)((int)(nib ^ 8u) - 8);
  } else if constexpr (KVF == KV_INT8) {
    return (float)(int8_t)row[d];
  } else {
    return e4m3_to_f32((uint32_t)row[d]);
  }
}

template <int KVF, int SM, typename TQ>
__global__ __launch_bounds__(kF32Threads) void attn_f32_kernel(AttnArgs a) {
  const int r = blockIdx.x;
  const int g = blockIdx.y;
  const int chunk = blockIdx.z;
  const int H = a.num_heads, hkv = a.hkv, D = a.head_size, bs = a.block_size;
  const int G = H / hkv;
  const int C = (KVF == KV_INT4) ? D / 2 : D;
  const int tid = threadIdx.x;

  // sequence of this row: the largest b with cum_q[b] <= r
  int lo = 0, hi = a.batch;
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (a.cum_q[mid] <= r) lo = mid; else hi = mid;
  }
  const int b = lo;
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

  __shared__ float qs[kF32MaxGroup][kF32MaxD];
  __shared__ float sc[kF32MaxGroup][kF32Threads];
  __shared__ float m_sh[kF32MaxGroup], l_sh[kF32MaxGroup], alpha_sh[kF32MaxGroup];

  const TQ* q = reinterpret_cast<const TQ*>(a.query);
  for (int e = tid; e < G * D; e += kF32Threads) {
    const int hh = e / D, d = e % D;
    const float s = (SM == SCALE_CHANNEL) ? a.k_scale[g * D + d] : a.k_scale[g];
    qs[hh][d] = to_f32(q[((size_t)r * H + g * G + hh) * D + d]) * s;
  }
  if (tid < G) { m_sh[tid] = -INFINITY; l_sh[tid] = 0.f; }

  const int nslice = kF32Threads / D;
  const int my_d = tid % D;
  const int my_slice = tid / D;
  float acc[kF32MaxGroup];
#pragma unroll
  for (int hh = 0; hh < kF32MaxGroup; ++hh) acc[hh] = 0.f;
  __syncthreads();

  const int wave = tid / 64, lane = tid % 64;
  for (int base = kbeg; base < kend; base += kF32Threads) {
    // scores: one key per thread
    const int j = base + tid;
    float dot[kF32MaxGroup];
#pragma unroll
    for (int hh = 0; hh < kF32MaxGroup; ++hh) dot[hh] = 0.f;
    if (j < kend) {
      const int blk = table[j / bs];
      const uint8_t* row = a.key_cache + (((size_t)blk * bs + j % bs) * hkv + g) * C;
      for (int d0 = 0; d0 < D; d0 += 16) {
        float k[16];
        load_codes16<KVF>(row, d0, k);
#pragma unroll
        for (int hh = 0; hh < kF32MaxGroup; ++hh) {
          if (hh < G) {
            float s = dot[hh];
#pragma unroll
            for (int e = 0; e < 16; ++e) s = fmaf(qs[hh][d0 + e], k[e], s);
            dot[hh] = s;
          }
        }
      }
    }
#pragma unroll
    for (int hh = 0; hh < kF32MaxGroup; ++hh)
      if (hh < G) sc[hh][tid] = (j < kend) ? dot[hh] * a.softmax_scale : -INFINITY;
    __syncthreads();
    // per-head chunk maximum -> new running max and rescale factor
    for (int hh = wave; hh < G; hh += kF32Threads / 64) {
      float mx = -INFINITY;
      for (int t = lane; t < kF32Threads; t += 64) mx = fmaxf(mx, sc[hh][t]);
      mx = wave_max(mx);
      if (lane == 0) {
        const float m_old = m_sh[hh];
        const float m_new = fmaxf(m_old, mx);
        alpha_sh[hh] = (m_old == -INFINITY) ? 0.f : expf(m_old - m_new);
        m_sh[hh] = m_new;
      }
    }
    __syncthreads();
    for (int hh = 0; hh < G; ++hh) {
      const float v = sc[hh][tid];
      sc[hh][tid] = (v == -INFINITY) ? 0.f : expf(v - m_sh[hh]);
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
      for (int hh = 0; hh < kF32MaxGroup; ++hh)
        if (hh < G) acc[hh] *= alpha_sh[hh];
      const int jn = min(kend - base, kF32Threads);
      for (int t = my_slice; t < jn; t += nslice) {
        const int jj = base + t;
        const int blk = table[jj / bs];
        const uint8_t* row = a.value_cache + (((size_t)blk * bs + jj % bs) * hkv + g) * C;
        const float v = load_code1<KVF>(row, my_d);
#pragma unroll
        for (int hh = 0; hh < kF32MaxGroup; ++hh)
          if (hh < G) acc[hh] = fmaf(sc[hh][t], v, acc[hh]);
      }
    }
    __syncthreads();
  }

  // merge the key slices (reuse sc as [slice][G][D] scratch; G*D <= 16*128)
  float* scratch = &sc[0][0];
  for (int s = 1; s < nslice; ++s) {
    if (my_slice == s) {
#pragma unroll
      for (int hh = 0; hh < kF32MaxGroup; ++hh)
        if (hh < G) scratch[hh * D + my_d] = acc[hh];
    }
    __syncthreads();
    if (my_slice == 0) {
#pragma unroll
      for (int hh = 0; hh < kF32MaxGroup; ++hh)
        if (hh < G) acc[hh] += scratch[hh * D + my_d];
    }
    __syncthreads();
  }
  if (my_slice != 0) return;
  const float vs = (SM == SCALE_CHANNEL) ? a.v_scale[g * D + my_d] : a.v_scale[g];
#pragma unroll
  for (int hh = 0; hh < kF32MaxGroup; ++hh) {
    if (hh >= G) break;
    const int h = g * G + hh;
    const float l = l_sh[hh];
    const float o = (l > 0.f) ? acc[hh] / l : 0.f;
    if (S == 1) {
      TQ* out = reinterpret_cast<TQ*>(a.out);
      out[((size_t)r * H + h) * D + my_d] = from_f32<TQ>(o * vs);
    } else {
      // split-KV partials leave the value scale to the combine
      const size_t pi = ((size_t)r * H + h) * S + chunk;
      a.part_o[pi * D + my_d] = o;
      if (my_d == 0) a.part_lse[pi] = (l > 0.f) ? m_sh[hh] + logf(l) : -INFINITY;
    }
  }
}

template <int KVF, int SM>
static int launch_q(const AttnArgs& a, dim3 grid, hipStream_t st) {
  switch (a.q_dtype) {
    case DT_F32: hipLaunchKernelGGL((attn_f32_kernel<KVF, SM, float>), grid, dim3(kF32Threads), 0, st, a); return 0;
    case DT_F16: hipLaunchKernelGGL((attn_f32_kernel<KVF, SM, f16>), grid, dim3(kF32Threads), 0, st, a); return 0;
    case DT_BF16: hipLaunchKernelGGL((attn_f32_kernel<KVF, SM, bf16>), grid, dim3(kF32Threads), 0, st, a); return 0;
  }
  return -1;
}

int launch_decode_f32(const AttnArgs& a, hipStream_t st) {
  if (a.num_heads / a.hkv > kF32MaxGroup || a.head_size > kF32MaxD || a.token_count == 0) return -1;
  dim3 grid(a.token_count, a.hkv, a.num_splits);
  switch (a.kv_format * 2 + a.scale_mode) {
    case KV_INT8 * 2 + SCALE_CHANNEL: return launch_q<KV_INT8, SCALE_CHANNEL>(a, grid, st);
    case KV_INT8 * 2 + SCALE_HEAD: return launch_q<KV_INT8, SCALE_HEAD>(a, grid, st);
    case KV_INT4 * 2 + SCALE_CHANNEL: return launch_q<KV_INT4, SCALE_CHANNEL>(a, grid, st);
    case KV_INT4 * 2 + SCALE_HEAD: return launch_q<KV_INT4, SCALE_HEAD>(a, grid, st);
    case KV_FP8 * 2 + SCALE_CHANNEL: return launch_q<KV_FP8, SCALE_CHANNEL>(a, grid, st);
    case KV_FP8 * 2 + SCALE_HEAD: return launch_q<KV_FP8, SCALE_HEAD>(a, grid, st);
  }
  return -1;
}

}  // namespace paq
