// decode_noalloc.hip -- paged_attn_decode without a caller workspace, for
// callers that cannot allocate device memory (code under graph capture, tight
// serving loops, harnesses that forbid allocation).
//
// The workspace -- arrival counters, then the partials of a split or
// length-balanced decode -- lives in a file-scope device array of
// kNoAllocScratchBytes.  Its address on a device is taken once per device,
// with that device current, by hipGetSymbolAddress (the array's name in host
// code is not a device address), and kept per device.  Each GPU holds its own
// copy until the process ends.  The counters at its head are zero when the
// code object loads, and every call's kernels return each counter they use to
// zero before they end, so every call starts from zero counters; the partials
// are overwritten by each call.  Calls that overlap on one GPU share the
// array and race: order them (one stream, or events).
#include <hip/hip_runtime.h>
#include <stdio.h>

#include <mutex>

#include "../../include/paq.h"
#include "entry.hpp"

namespace {

constexpr size_t kNoAllocScratchBytes = 16u << 20;   // 16 MiB per device

__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// The current device's address of `scratch` (taken on its first use there).
int scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0)
    return paq::set_error(PAQ_ERR_HIP, "hipGetDevice failed (no GPU?)");
  if (dev >= kMaxDevices)
    return paq::set_error(PAQ_ERR_UNSUPPORTED, "device index beyond the scratch table");
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      char msg[160];
      snprintf(msg, sizeof msg, "hipGetSymbolAddress of the decode scratch failed: %s",
               hipGetErrorString(e));
      return paq::set_error(PAQ_ERR_HIP, msg);
    }
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return PAQ_OK;
}

}  // namespace

extern "C" int32_t paged_attn_decode_noalloc(const paq_desc* d, const void* query, void* out,
                                             const void* key_cache, const void* value_cache,
                                             const float* k_scale, const float* v_scale,
                                             const int32_t* block_table, const int32_t* cum_q,
                                             const int32_t* past_lens, const int32_t* cum_q_host,
                                             const int32_t* past_lens_host, float softmax_scale,
                                             int32_t num_splits, void* stream) {
  paq_plan p;
  int32_t rc = paq_plan_decode(d, cum_q_host, past_lens_host, num_splits, 0, &p);
  if (rc) return rc;
  if (p.workspace_bytes > kNoAllocScratchBytes) {
    char msg[200];
    snprintf(msg, sizeof msg,
             "this decode needs %llu workspace bytes; the allocation-free decode holds %llu "
             "(use paged_attn_decode with a workspace, or fewer splits)",
             (unsigned long long)p.workspace_bytes, (unsigned long long)kNoAllocScratchBytes);
    return paq::set_error(PAQ_ERR_WORKSPACE, msg);
  }
  void* ws = nullptr;
  if (p.workspace_bytes > 0) {
    rc = scratch_address(&ws);
    if (rc) return rc;
  }
  return paq::decode_entry(d, query, out, key_cache, value_cache, k_scale, v_scale, block_table,
                           cum_q, past_lens, cum_q_host, past_lens_host, softmax_scale,
                           num_splits, ws, ws ? kNoAllocScratchBytes : 0, stream);
}
