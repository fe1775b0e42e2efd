// combine.hip -- log-sum-exp merge of the fp32 kernel's split-KV partials
// (flash decoding, "GQA GEMV decode", section 2): for every (row, head), with
// chunk partials (o_c, lse_c), L = log sum_c exp(lse_c) and
// out = sum_c exp(lse_c - L) o_c.  Each log-sum-exp arrives as the pair
// (raw maximum m_c, log2 of the chunk's sum lg_c) -- see attn_f32.hip -- so a
// chunk's weight against the running raw maximum M is 2^((m_c - M) c2 + lg_c)
// with the kv head's score factor c2: never an overflow, whatever the key
// scales.  (The MFMA decode merges its parts inside its own launch.)
// Empty chunks carry lse = -inf and contribute nothing.  The partial outputs
// are sums of probability-weighted value codes; the per-channel (or per-head)
// value scale, the same for every chunk, is applied here once.
//
// One workgroup of 4 waves per (row, head).  The waves take every 4th chunk,
// four chunks per round: each lane loads their log-sum-exps and its D/64
// consecutive channels of their partials together, so one memory round trip
// serves the whole merge.  Each wave keeps a running maximum and rescales its
// sums when it grows (the merge is exact in any order up to rounding); the
// four wave results meet in LDS.
#include "device.hpp"
#include "launch.hpp"

namespace paq {

constexpr int kCombineWaves = 4;
constexpr int kCombineThreads = kCombineWaves * 64;
constexpr int kCombineMaxSplits = 4096;

template <typename TO, int D, int SM>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_lse, TO* __restrict__ out,
    const float* __restrict__ v_scale, const float* __restrict__ k_scale, float softmax_scale,
    int num_heads, int group, int S) {
  constexpr int PER_LANE = D / 64;                 // 2 for D=128, 1 for D=64
  const int r = blockIdx.x / num_heads;
  const int h = blockIdx.x % num_heads;
  const size_t base = ((size_t)r * num_heads + h) * S;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ float red_m[kCombineWaves], red_w[kCombineWaves];
  __shared__ float acc_sh[kCombineWaves][D];
  __shared__ int e_sh;
  // the partials' log-sum-exps are in raw score units: their differences
  // scale by the kv head's score factor (the same one the partials used)
  const int hk = h / group;                                   // kv head of query head h
  const float c2 = score_factor_log2(softmax_scale, key_scale_exponent<SM>(k_scale, hk, D, &e_sh),
                                     1.f);
  constexpr int U = 4;                              // chunks per round and wave
  float m = -INFINITY, wsum = 0.f;
  float acc[PER_LANE];
#pragma unroll
  for (int i = 0; i < PER_LANE; ++i) acc[i] = 0.f;
  for (int c0 = wave; c0 < S; c0 += U * kCombineWaves) {
    float l[U], lg[U], v[U][PER_LANE];
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int c = c0 + j * kCombineWaves;
      l[j] = -INFINITY;
      lg[j] = -INFINITY;
#pragma unroll
      for (int i = 0; i < PER_LANE; ++i) v[j][i] = 0.f;
      if (c < S) {
        l[j] = part_lse[2 * (base + c)];
        lg[j] = part_lse[2 * (base + c) + 1];
        const float* po = part_o + (base + c) * D + PER_LANE * lane;
        if constexpr (PER_LANE == 2) {
          const float2 t = *reinterpret_cast<const float2*>(po);
          v[j][0] = t.x;
          v[j][1] = t.y;
        } else {
          v[j][0] = po[0];
        }
      }
    }
    float mn = m;
#pragma unroll
    for (int j = 0; j < U; ++j) mn = fmaxf(mn, l[j]);
    if (mn == -INFINITY) continue;                  // only empty chunks so far
    const float sc = exp2f((m - mn) * c2);          // 0 while m is -inf
    wsum *= sc;
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i) acc[i] *= sc;
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const float w = exp2f((l[j] - mn) * c2 + lg[j]);   // 0 for empty chunks (o = 0 there)
      wsum += w;
#pragma unroll
      for (int i = 0; i < PER_LANE; ++i) acc[i] = fmaf(w, v[j][i], acc[i]);
    }
    m = mn;
  }
#pragma unroll
  for (int i = 0; i < PER_LANE; ++i) acc_sh[wave][PER_LANE * lane + i] = acc[i];
  if (lane == 0) {
    red_m[wave] = m;
    red_w[wave] = wsum;
  }
  __syncthreads();
  if (wave == 0) {
    float M = red_m[0];
#pragma unroll
    for (int i = 1; i < kCombineWaves; ++i) M = fmaxf(M, red_m[i]);
    float f[kCombineWaves], tot = 0.f;
#pragma unroll
    for (int i = 0; i < kCombineWaves; ++i) {
      f[i] = (red_m[i] == -INFINITY) ? 0.f : exp2f((red_m[i] - M) * c2);
      tot = fmaf(f[i], red_w[i], tot);
    }
    const float inv = tot > 0.f ? 1.0f / tot : 0.f;
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i) {
      const int d = PER_LANE * lane + i;
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < kCombineWaves; ++w) v = fmaf(f[w], acc_sh[w][d], v);
      const float vs = (SM == SCALE_CHANNEL) ? v_scale[hk * D + d] : v_scale[hk];
      out[((size_t)r * num_heads + h) * D + d] = from_f32<TO>(v * inv * vs);
    }
  }
}

template <int D, int SM>
static int launch_combine_ds(const AttnArgs& a, hipStream_t st) {
  dim3 grid(a.token_count * a.num_heads);
  switch (a.q_dtype) {
#define PAQ_COMBINE_CASE(DTV, TYPE)                                                           \
  case DTV:                                                                                 \
    hipLaunchKernelGGL((combine_kernel<TYPE, D, SM>), grid, dim3(kCombineThreads), 0, st,      \
                       a.part_o, a.part_lse, (TYPE*)a.out, a.v_scale, a.k_scale,              \
                       a.softmax_scale, a.num_heads, a.num_heads / a.hkv, a.part_count);      \
    return 0;
    PAQ_COMBINE_CASE(DT_F32, float)
    PAQ_COMBINE_CASE(DT_F16, f16)
    PAQ_COMBINE_CASE(DT_BF16, bf16)
#undef PAQ_COMBINE_CASE
  }
  return -1;
}

template <int D>
static int launch_combine_d(const AttnArgs& a, hipStream_t st) {
  return a.scale_mode == SCALE_CHANNEL ? launch_combine_ds<D, SCALE_CHANNEL>(a, st)
                                       : launch_combine_ds<D, SCALE_HEAD>(a, st);
}

int launch_combine(const AttnArgs& a, hipStream_t st) {
  if (a.part_count > kCombineMaxSplits || a.token_count == 0) return -1;
  if (a.head_size == 128) return launch_combine_d<128>(a, st);
  if (a.head_size == 64) return launch_combine_d<64>(a, st);
  return -1;
}

}  // namespace paq
