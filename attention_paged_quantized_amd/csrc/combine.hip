// combine.hip -- log-sum-exp merge of split-KV partials (flash decoding,
// "GQA GEMV decode", section 2): for every (row, head), with chunk partials
// (o_c, lse_c), L = log sum_c exp(lse_c) and out = sum_c exp(lse_c - L) o_c.
// Empty chunks carry lse = -inf and contribute nothing.  The partial outputs
// are sums of probability-weighted value codes; the per-channel (or per-head)
// value scale, the same for every chunk, is applied here once.
//
// One workgroup of 4 waves per (row, head): the waves take every 4th chunk,
// each lane owns D/64 consecutive channels (one vector load per chunk), and
// the four partial sums meet in LDS.  The loads of a wave are independent, so
// many are in flight at once.
#include "device.hpp"
#include "launch.hpp"

namespace paq {

constexpr int kCombineWaves = 4;
constexpr int kCombineThreads = kCombineWaves * 64;
constexpr int kCombineMaxSplits = 4096;

template <typename TO, int D>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_lse, TO* __restrict__ out,
    const float* __restrict__ v_scale, int num_heads, int group, int per_channel, int S) {
  constexpr int PER_LANE = D / 64;                 // 2 for D=128, 1 for D=64
  const int r = blockIdx.x / num_heads;
  const int h = blockIdx.x % num_heads;
  const size_t base = ((size_t)r * num_heads + h) * S;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ float red[kCombineWaves];
  __shared__ float acc_sh[kCombineWaves][D];
  // global maximum of the chunk log-sum-exps
  float mx = -INFINITY;
  for (int c = tid; c < S; c += kCombineThreads) mx = fmaxf(mx, part_lse[base + c]);
  mx = wave_max(mx);
  if (lane == 0) red[wave] = mx;
  __syncthreads();
  mx = red[0];
#pragma unroll
  for (int i = 1; i < kCombineWaves; ++i) mx = fmaxf(mx, red[i]);
  // weighted sum of the partial outputs; weights sum to 1 after division
  float acc[PER_LANE];
#pragma unroll
  for (int i = 0; i < PER_LANE; ++i) acc[i] = 0.f;
  float wsum = 0.f;
  if (mx != -INFINITY) {
#pragma unroll 4
    for (int c = wave; c < S; c += kCombineWaves) {
      const float l = part_lse[base + c];
      const float w = (l == -INFINITY) ? 0.f : __expf(l - mx);
      wsum += w;
      const float* po = part_o + (base + c) * D + PER_LANE * lane;
      if constexpr (PER_LANE == 2) {
        const float2 v = *reinterpret_cast<const float2*>(po);
        acc[0] = fmaf(w, v.x, acc[0]);
        acc[1] = fmaf(w, v.y, acc[1]);
      } else {
        acc[0] = fmaf(w, po[0], acc[0]);
      }
    }
  }
  __syncthreads();                                  // red[] reads done
#pragma unroll
  for (int i = 0; i < PER_LANE; ++i) acc_sh[wave][PER_LANE * lane + i] = acc[i];
  if (lane == 0) red[wave] = wsum;
  __syncthreads();
  if (wave == 0) {
    const int hk = h / group;                                 // kv head of query head h
    float tot = 0.f;
#pragma unroll
    for (int i = 0; i < kCombineWaves; ++i) tot += red[i];
    const float inv = tot > 0.f ? 1.0f / tot : 0.f;
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i) {
      const int d = PER_LANE * lane + i;
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < kCombineWaves; ++w) v += acc_sh[w][d];
      const float vs = per_channel ? v_scale[hk * D + d] : v_scale[hk];
      out[((size_t)r * num_heads + h) * D + d] = from_f32<TO>(v * inv * vs);
    }
  }
}

template <int D>
static int launch_combine_d(const AttnArgs& a, hipStream_t st) {
  dim3 grid(a.token_count * a.num_heads);
  switch (a.q_dtype) {
#define PAQ_COMBINE_CASE(DTV, TYPE)                                                           \
  case DTV:                                                                                 \
    hipLaunchKernelGGL((combine_kernel<TYPE, D>), grid, dim3(kCombineThreads), 0, st, a.part_o, \
                       a.part_lse, (TYPE*)a.out, a.v_scale, a.num_heads, a.num_heads / a.hkv,   \
                       a.scale_mode == SCALE_CHANNEL ? 1 : 0, a.part_count);                  \
    return 0;
    PAQ_COMBINE_CASE(DT_F32, float)
    PAQ_COMBINE_CASE(DT_F16, f16)
    PAQ_COMBINE_CASE(DT_BF16, bf16)
#undef PAQ_COMBINE_CASE
  }
  return -1;
}

int launch_combine(const AttnArgs& a, hipStream_t st) {
  if (a.part_count > kCombineMaxSplits || a.token_count == 0) return -1;
  if (a.head_size == 128) return launch_combine_d<128>(a, st);
  if (a.head_size == 64) return launch_combine_d<64>(a, st);
  return -1;
}

}  // namespace paq
