// sparse_select.hip -- block-sparse attention ("INT8-KV Tensor-Core
// DynamicSparseAttention", section 1): the selected logical blocks of every
// sequence become a compact block table, and the sequence's effective past
// length, so that the ordinary kernels attend to exactly the selected keys.
// Decode: softmax does not depend on the order of the keys; the selection is
// ascending, so a selected partial last block stays last and its tail past
// kv_len stays masked.
// Prefill: the compact table is the selected earlier blocks (each wholly
// before past) followed by every block that holds a new token; the chunk then
// starts at n * block_size + past % block_size, and the dense causal rule
// (key j visible to row i iff j <= past' + i) over the compact table is the
// causal rule over the original positions, since every selected key lies
// before the first new token and the local blocks keep their order.
#include "device.hpp"
#include "launch.hpp"

namespace paq {

__global__ __launch_bounds__(256) void sparse_compact_kernel(
    const int32_t* __restrict__ block_table, int max_blocks, const int32_t* __restrict__ sel,
    const int32_t* __restrict__ num_sel, int max_sel, const int32_t* __restrict__ cum_q,
    const int32_t* __restrict__ past_lens, int block_size, int32_t* __restrict__ compact,
    int32_t* __restrict__ eff_past) {
  const int b = blockIdx.x;
  if (cum_q[b + 1] == cum_q[b]) {                 // no new row: never read
    if (threadIdx.x == 0) eff_past[b] = 0;
    return;
  }
  const int n = num_sel[b];
  const int32_t* s = sel + (size_t)b * max_sel;
  for (int i = threadIdx.x; i < n; i += blockDim.x)
    compact[(size_t)b * max_sel + i] = block_table[(size_t)b * max_blocks + s[i]];
  if (threadIdx.x == 0) {
    const int kv_len = past_lens[b] + 1;
    const int last = s[n - 1];
    eff_past[b] = (n - 1) * block_size + min(block_size, kv_len - last * block_size) - 1;
  }
}

__global__ __launch_bounds__(256) void sparse_prefill_compact_kernel(
    const int32_t* __restrict__ block_table, int max_blocks, const int32_t* __restrict__ sel,
    const int32_t* __restrict__ num_sel, int max_sel, const int32_t* __restrict__ cum_q,
    const int32_t* __restrict__ past_lens, int block_size, int stride,
    int32_t* __restrict__ compact, int32_t* __restrict__ eff_past) {
  const int b = blockIdx.x;
  const int q = cum_q[b + 1] - cum_q[b];
  if (q == 0) {                                   // no new row: never read
    if (threadIdx.x == 0) eff_past[b] = 0;
    return;
  }
  const int n = max_sel > 0 ? num_sel[b] : 0;
  const int past = past_lens[b];
  const int first = past / block_size;                          // first local block
  const int nloc = (past + q + block_size - 1) / block_size - first;
  const int32_t* row = block_table + (size_t)b * max_blocks;
  int32_t* c = compact + (size_t)b * stride;
  for (int i = threadIdx.x; i < n + nloc; i += blockDim.x)
    c[i] = row[i < n ? sel[(size_t)b * max_sel + i] : first + (i - n)];
  if (threadIdx.x == 0) eff_past[b] = n * block_size + past % block_size;
}

int launch_sparse_prefill_compact(const int32_t* block_table, int max_blocks, const int32_t* sel,
                                  const int32_t* num_sel, int max_sel, const int32_t* cum_q,
                                  const int32_t* past_lens, int block_size, int batch,
                                  int stride, int32_t* compact, int32_t* eff_past,
                                  hipStream_t st) {
  if (batch <= 0) return 0;
  hipLaunchKernelGGL(sparse_prefill_compact_kernel, dim3(batch), dim3(256), 0, st, block_table,
                     max_blocks, sel, num_sel, max_sel, cum_q, past_lens, block_size, stride,
                     compact, eff_past);
  return 0;
}

int launch_sparse_compact(const int32_t* block_table, int max_blocks, const int32_t* sel,
                          const int32_t* num_sel, int max_sel, const int32_t* cum_q,
                          const int32_t* past_lens, int block_size, int batch, int32_t* compact,
                          int32_t* eff_past, hipStream_t st) {
  if (batch <= 0) return 0;
  hipLaunchKernelGGL(sparse_compact_kernel, dim3(batch), dim3(256), 0, st, block_table,
                     max_blocks, sel, num_sel, max_sel, cum_q, past_lens, block_size, compact,
                     eff_past);
  return 0;
}

}  // namespace paq
