// decode_host.hpp -- interface of the host-CPU decode (decode_host.cpp) for
// the library's host code; arguments validated by the caller.
#pragma once

#include <stdint.h>

namespace paq {

struct HostDecodeArgs {
  const float* query;          // (token_count, num_heads, head_size) fp32, host
  float* out;                  // same shape, host
  const uint8_t* key_cache;    // (num_blocks, block_size, hkv, C), host
  const uint8_t* value_cache;
  const float* k_scale;        // (hkv, head_size) or (hkv)
  const float* v_scale;
  const int32_t* block_table;  // (batch, max_blocks)
  const int32_t* cum_q;        // (batch + 1), host
  const int32_t* past_lens;    // (batch), host
  int batch, num_heads, hkv, head_size, block_size, max_blocks;
  int kv_format, scale_mode;
  float softmax_scale;
  int splits;                  // key chunks per sequence, 0 = as many as idle threads ask for
  int threads;
};

// Returns 0, or -1 for a shape it does not handle (a head size other than
// 64 or 128).
int host_decode(const HostDecodeArgs& a);

}  // namespace paq
