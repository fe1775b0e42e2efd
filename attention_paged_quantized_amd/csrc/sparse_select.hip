// sparse_select.hip -- block-sparse decode ("INT8-KV Tensor-Core
// DynamicSparseAttention", section 1): the selected logical blocks of every
// sequence become a compact block table, and the sequence's effective key
// count, so that the ordinary decode kernels (single pass or split-KV)
// attend to exactly the selected keys.  Softmax does not depend on the order
// of the keys; the selection is ascending, so a selected partial last block
// stays last and its tail past kv_len stays masked.
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
