// entry.hpp -- host entry logic shared between the C-ABI translation units.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/paq.h"

namespace paq {

// The body of paged_attn_decode: validate, plan, check the workspace, launch.
int decode_entry(const paq_desc* d, const void* query, void* out, const void* key_cache,
                 const void* value_cache, const float* k_scale, const float* v_scale,
                 const int32_t* block_table, const int32_t* cum_q, const int32_t* past_lens,
                 const int32_t* cum_q_host, const int32_t* past_lens_host, float softmax_scale,
                 int32_t num_splits, void* workspace, size_t workspace_bytes, void* stream);

// Record a failure for paq_last_error(); returns code.
int set_error(int code, const char* msg);

}  // namespace paq
