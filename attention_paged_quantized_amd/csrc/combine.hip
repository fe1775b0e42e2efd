// combine.hip -- log-sum-exp merge of split-KV partials (flash decoding,
// "GQA GEMV decode", section 2): for every (row, head), with chunk partials
// (o_c, lse_c), L = log sum_c exp(lse_c) and out = sum_c exp(lse_c - L) o_c.
// Empty chunks carry lse = -inf and contribute nothing.
#include "device.hpp"
#include "launch.hpp"

namespace paq {

constexpr int kCombineThreads = 128;

// One workgroup per (row, head); thread t owns channels t, t+128, ...
template <typename TO>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_lse, TO* __restrict__ out,
    const int32_t* __restrict__ cum_q, int batch, int num_heads, int head_size, int S) {
  const int r = blockIdx.x / num_heads;
  const int h = blockIdx.x % num_heads;
  const size_t base = ((size_t)r * num_heads + h) * S;
  __shared__ float w[4096];
  __shared__ float red[kCombineThreads / 64];
  // maximum lse
  float mx = -INFINITY;
  for (int c = threadIdx.x; c < S; c += kCombineThreads) mx = fmaxf(mx, part_lse[base + c]);
  mx = wave_max(mx);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
  __syncthreads();
  mx = red[0];
  for (int i = 1; i < kCombineThreads / 64; ++i) mx = fmaxf(mx, red[i]);
  __syncthreads();
  float sum = 0.f;
  for (int c = threadIdx.x; c < S; c += kCombineThreads) {
    const float l = part_lse[base + c];
    const float e = (l == -INFINITY) ? 0.f : expf(l - mx);
    w[c] = e;
    sum += e;
  }
  sum = wave_sum(sum);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = sum;
  __syncthreads();
  sum = 0.f;
  for (int i = 0; i < kCombineThreads / 64; ++i) sum += red[i];
  const float inv = sum > 0.f ? 1.0f / sum : 0.f;
  for (int d = threadIdx.x; d < head_size; d += kCombineThreads) {
    float acc = 0.f;
    for (int c = 0; c < S; ++c) acc = fmaf(w[c], part_o[(base + c) * head_size + d], acc);
    out[((size_t)r * num_heads + h) * head_size + d] = from_f32<TO>(acc * inv);
  }
}

int launch_combine(const AttnArgs& a, hipStream_t st) {
  if (a.num_splits > 4096 || a.token_count == 0) return -1;
  dim3 grid(a.token_count * a.num_heads);
  switch (a.q_dtype) {
#define PAQ_COMBINE_CASE(DTV, TYPE)                                                         \
  case DTV:                                                                               \
    hipLaunchKernelGGL((combine_kernel<TYPE>), grid, dim3(kCombineThreads), 0, st, a.part_o, \
                       a.part_lse, (TYPE*)a.out, a.cum_q, a.batch, a.num_heads,             \
                       a.head_size, a.num_splits);                                         \
    return 0;
    PAQ_COMBINE_CASE(DT_F32, float)
    PAQ_COMBINE_CASE(DT_F16, f16)
    PAQ_COMBINE_CASE(DT_BF16, bf16)
#undef PAQ_COMBINE_CASE
  }
  return -1;
}

}  // namespace paq
