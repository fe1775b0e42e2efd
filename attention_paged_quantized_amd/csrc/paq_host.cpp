// paq_host.cpp -- the C ABI (include/paq.h): argument validation, host-side
// planning and kernel dispatch.
//
// Every check runs before anything is launched, so a failed call writes
// nothing (the pages ask for explicit checks on values that cross the host /
// device boundary: "PagedAttention FA path: exact max_query_len", lessons).
// The grid of every kernel is sized from the exact maximum query length read
// from the host copy of cum_q (same page, section 1), never from
// token_count - batch + 1, which undercounts (or goes negative) as soon as a
// sequence has no new token.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <vector>
#include <thread>
#include <string>

#include "../../include/paq.h"
#include "decode_host.hpp"
#include "entry.hpp"
#include "launch.hpp"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

struct SeqStats {
  int max_q = 0;       // exact max_query_len
  int max_kv = 0;      // over sequences with new rows
  int active = 0;      // sequences with new rows
};

bool valid_block_size(int bs) { return bs == 16 || bs == 32 || bs == 64 || bs == 128; }

// Shape/enum/host-array checks shared by all calls.
int validate(const paq_desc* d, const int32_t* cum_q_host, const int32_t* past_host,
             SeqStats* st) {
  if (!d) return fail(PAQ_ERR_INVALID_ARG, "desc is NULL");
  if (d->batch < 0) return fail(PAQ_ERR_INVALID_ARG, "batch %d < 0", d->batch);
  if (d->token_count < 0) return fail(PAQ_ERR_INVALID_ARG, "token_count %d < 0", d->token_count);
  if (d->num_heads < 1 || d->kv_num_heads < 1)
    return fail(PAQ_ERR_INVALID_ARG, "num_heads %d / kv_num_heads %d must be >= 1",
                d->num_heads, d->kv_num_heads);
  if (d->num_heads % d->kv_num_heads)
    return fail(PAQ_ERR_INVALID_ARG, "num_heads %d is not a multiple of kv_num_heads %d",
                d->num_heads, d->kv_num_heads);
  if (d->q_dtype < PAQ_DT_F32 || d->q_dtype > PAQ_DT_BF16)
    return fail(PAQ_ERR_INVALID_ARG, "q_dtype %d unknown", d->q_dtype);
  if (d->kv_format < PAQ_KV_INT8 || d->kv_format > PAQ_KV_FP8_E4M3)
    return fail(PAQ_ERR_INVALID_ARG, "kv_format %d unknown", d->kv_format);
  if (d->scale_mode < PAQ_SCALE_PER_CHANNEL || d->scale_mode > PAQ_SCALE_PER_HEAD)
    return fail(PAQ_ERR_INVALID_ARG, "scale_mode %d unknown", d->scale_mode);
  if (d->head_size != 64 && d->head_size != 128)
    return fail(PAQ_ERR_UNSUPPORTED, "head_size %d not built (64, 128)", d->head_size);
  if (!valid_block_size(d->block_size))
    return fail(PAQ_ERR_UNSUPPORTED, "block_size %d not built (16, 32, 64, 128)", d->block_size);
  if (d->num_blocks < 0 || d->max_blocks_per_seq < 0)
    return fail(PAQ_ERR_INVALID_ARG, "num_blocks %d / max_blocks_per_seq %d < 0",
                d->num_blocks, d->max_blocks_per_seq);
  if (d->batch > 0 && (!cum_q_host || !past_host))
    return fail(PAQ_ERR_INVALID_ARG, "cum_q_host / past_lens_host is NULL");
  if (d->batch == 0) {
    if (d->token_count != 0)
      return fail(PAQ_ERR_INVALID_ARG, "batch 0 with token_count %d", d->token_count);
    if (cum_q_host && cum_q_host[0] != 0)
      return fail(PAQ_ERR_INVALID_ARG, "cum_q[0] = %d, expected 0", cum_q_host[0]);
    return PAQ_OK;
  }
  if (cum_q_host[0] != 0) return fail(PAQ_ERR_INVALID_ARG, "cum_q[0] = %d, expected 0", cum_q_host[0]);
  const long cap = (long)d->max_blocks_per_seq * d->block_size;
  for (int b = 0; b < d->batch; ++b) {
    const long q = (long)cum_q_host[b + 1] - cum_q_host[b];
    if (q < 0)
      return fail(PAQ_ERR_INVALID_ARG, "cum_q decreases at sequence %d (%d -> %d)", b,
                  cum_q_host[b], cum_q_host[b + 1]);
    if (past_host[b] < 0) return fail(PAQ_ERR_INVALID_ARG, "past_lens[%d] = %d < 0", b, past_host[b]);
    const long kv = (long)past_host[b] + q;
    if (kv > 0x7fffffffL) return fail(PAQ_ERR_INVALID_ARG, "sequence %d length overflows", b);
    if (q > 0) {
      if (kv > cap)
        return fail(PAQ_ERR_INVALID_ARG,
                    "sequence %d needs %ld blocks of %d tokens, block_table has %d", b,
                    (kv + d->block_size - 1) / d->block_size, d->block_size,
                    d->max_blocks_per_seq);
      st->active++;
      st->max_q = std::max<long>(st->max_q, q);
      st->max_kv = std::max<long>(st->max_kv, kv);
    }
  }
  if (cum_q_host[d->batch] != d->token_count)
    return fail(PAQ_ERR_INVALID_ARG, "cum_q[batch] = %d but token_count = %d",
                cum_q_host[d->batch], d->token_count);
  if (st->active > 0 && d->num_blocks < 1)
    return fail(PAQ_ERR_INVALID_ARG, "num_blocks is 0 but sequences have tokens");
  return PAQ_OK;
}

int device_cu_count(int* out) {
  static std::mutex mu;
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0)
    return fail(PAQ_ERR_HIP, "hipGetDevice failed (no GPU?)");
  std::lock_guard<std::mutex> lock(mu);
  if (dev < 64 && cache[dev] > 0) { *out = cache[dev]; return PAQ_OK; }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return fail(PAQ_ERR_HIP, "cannot query the compute-unit count of device %d", dev);
  if (dev < 64) cache[dev] = n;
  *out = n;
  return PAQ_OK;
}

// Compute units to plan for: the caller's count, else the current device's,
// else (no device visible: sizing on a host without a GPU) 256.
int resolve_cus(int num_cus) {
  if (num_cus > 0) return num_cus;
  int n = 0;
  if (device_cu_count(&n) == PAQ_OK) return n;
  return 256;
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Length-balanced (stream) decode: about one workgroup per compute unit, each
// streaming at least kStreamMinTiles 32-key tiles (two per wave).
constexpr int kStreamMinTiles = 16;

// lengths_exact: the device lengths equal the host ones (false for the
// block-sparse decode, whose host lengths are upper bounds): the
// length-balanced partitions cut the tiles by the host lengths and need them
// exact, so without it only the single pass and the chunk partition (cut on
// the device) are planned.
int plan_decode(const paq_desc* d, const int32_t* cum_q_host, const int32_t* past_host,
                int num_splits, int num_cus, paq_plan* p, bool lengths_exact = true) {
  memset(p, 0, sizeof *p);
  SeqStats st;
  int rc = validate(d, cum_q_host, past_host, &st);
  if (rc) return rc;
  for (int b = 0; b < d->batch; ++b) {
    const int q = cum_q_host[b + 1] - cum_q_host[b];
    if (q > 1)
      return fail(PAQ_ERR_INVALID_ARG,
                  "decode needs q_len in {0,1}; sequence %d has %d new tokens", b, q);
  }
  if (num_splits > 4096) return fail(PAQ_ERR_INVALID_ARG, "num_splits %d > 4096", num_splits);
  p->max_query_len = st.max_q;
  p->max_kv_len = st.max_kv;
  p->active_seqs = st.active;
  p->work_units = st.active * d->kv_num_heads;
  if (st.active == 0) {
    p->path = PAQ_PATH_NONE;
    return PAQ_OK;
  }
  const int group = d->num_heads / d->kv_num_heads;
  const bool mfma = d->q_dtype != PAQ_DT_F32 &&
                    paq::decode_mfma_supports(d->head_size, group, d->block_size, d->q_dtype);
  const int max_nb = (st.max_kv + d->block_size - 1) / d->block_size;
  const int cus = resolve_cus(num_cus);
  const size_t head = paq::kDecCounterBytes;
  if (!mfma) {
    if (group > paq::kF32KernelMaxGroup)
      return fail(PAQ_ERR_UNSUPPORTED,
                  "no decode kernel for %s queries with %d query heads per kv head "
                  "(the fp32 kernel takes at most %d)",
                  d->q_dtype == PAQ_DT_F32 ? "fp32" : "16-bit", group, paq::kF32KernelMaxGroup);
    // Flash-decoding rule ("GQA GEMV decode", section 2): split the KV of a
    // sequence only when the (sequence, kv head) units under-fill the device
    // and a sequence has more than one KV chunk.  Aim at two workgroups per CU
    // with chunks of at least 256 keys.  (A length-balanced request takes the
    // same rule.)
    int S = num_splits;
    if (S <= 0) {
      S = 1;
      if (p->work_units < cus && max_nb > 1) {
        const int want = (2 * cus + p->work_units - 1) / p->work_units;
        const int by_len = std::max(1, st.max_kv / 256);
        S = std::max(1, std::min(std::min(want, by_len), max_nb));
      }
    }
    if (S > 1 && (unsigned long long)(S + 1) * (unsigned long long)d->max_blocks_per_seq >=
                     (1ull << 32))
      return fail(PAQ_ERR_UNSUPPORTED, "num_splits %d x max_blocks_per_seq %d too large", S,
                  d->max_blocks_per_seq);
    p->num_splits = S;
    p->path = S > 1 ? PAQ_PATH_F32_SPLIT : PAQ_PATH_F32_SINGLE;
    p->grid_x = d->token_count;
    p->grid_y = d->kv_num_heads;
    p->grid_z = S;
    p->waves_per_group = 4;
    if (S > 1) {
      const size_t rows = (size_t)d->token_count * d->num_heads * S;
      p->workspace_bytes = head + align_up(rows * d->head_size * sizeof(float)) +
                           align_up(rows * 2 * sizeof(float));
    }
    return PAQ_OK;
  }

  // MFMA decode: workgroups of 8 waves over one head group (HW adjacent kv
  // heads) and one part of one sequence.
  const int hw = paq::decode_heads_per_wave(d->kv_format, d->head_size, d->kv_num_heads);
  const int hg = d->kv_num_heads / hw;
  const long units = (long)st.active * hg;
  const bool counters_fit = (long)d->batch * hg <= paq::kDecCounters;
  int mode = paq::DEC_SINGLE, S = 1;
  long groups = 0;                    // stream partition: workgroups
  long total = 0;                     // stream partition: tiles of all segments
  for (int b = 0; b < d->batch; ++b)
    if (cum_q_host[b + 1] > cum_q_host[b]) total += ((long)past_host[b] + 32) / 32;
  total *= hg;
  if (num_splits > 1) {
    if (!counters_fit)
      return fail(PAQ_ERR_UNSUPPORTED, "split decode of %d sequences x %d head groups: at most %d",
                  d->batch, hg, paq::kDecCounters);
    if ((unsigned long long)(num_splits + 1) * (unsigned long long)d->max_blocks_per_seq >=
        (1ull << 32))
      return fail(PAQ_ERR_UNSUPPORTED, "num_splits %d x max_blocks_per_seq %d too large",
                  num_splits, d->max_blocks_per_seq);
    mode = paq::DEC_CHUNKS;
    S = num_splits;
  } else if (num_splits < 0) {
    if (!lengths_exact)
      return fail(PAQ_ERR_UNSUPPORTED,
                  "a length-balanced partition needs exact key counts (block-sparse decode: "
                  "num_splits >= 0)");
    if (!counters_fit)
      return fail(PAQ_ERR_UNSUPPORTED, "split decode of %d sequences x %d head groups: at most %d",
                  d->batch, hg, paq::kDecCounters);
    groups = -(long)num_splits;
    if (groups > paq::kDecMaxPartsPerSeq)
      return fail(PAQ_ERR_UNSUPPORTED, "a length-balanced decode over %ld workgroups: at most %d",
                  groups, paq::kDecMaxPartsPerSeq);
    mode = paq::DEC_STREAM;
  } else if (num_splits == 0 && counters_fit && units < cus && max_nb > 1) {
    // Automatic: the flash-decoding rule of "GQA GEMV decode" (section 2):
    // split the KV of the sequences only when the (sequence, kv head) units
    // under-fill the device.  With near-uniform lengths, block-aligned chunks
    // of every sequence (about two workgroups per compute unit, chunks of at
    // least 256 keys); with skewed lengths the length-balanced partition,
    // which deals every compute unit the same share of all tiles.
    long sum_kv = 0;
    for (int b = 0; b < d->batch; ++b)
      if (cum_q_host[b + 1] > cum_q_host[b]) sum_kv += (long)past_host[b] + 1;
    // (max > 1.5 x mean, and long enough for a split to pay: 512 keys)
    const bool skewed =
        lengths_exact && 2L * st.max_kv * st.active > 3L * sum_kv && st.max_kv >= 512;
    if (skewed) {
      groups = std::min<long>(std::min<long>(cus, paq::kDecMaxPartsPerSeq),
                              std::max<long>(1, total / kStreamMinTiles));
      mode = paq::DEC_STREAM;
    } else {
      const long want = (2L * cus + units - 1) / units;
      const long by_len = std::max(1, st.max_kv / 256);
      S = (int)std::max<long>(1, std::min<long>(std::min<long>(want, by_len), max_nb));
      if (S > 1) mode = paq::DEC_CHUNKS;
    }
  }
  p->path = mode == paq::DEC_SINGLE ? PAQ_PATH_SINGLE
            : mode == paq::DEC_CHUNKS ? PAQ_PATH_SPLIT : PAQ_PATH_BALANCED;
  p->waves_per_group = 8;
  long parts, slots;
  if (mode == paq::DEC_SINGLE) {
    parts = d->batch;
    slots = 0;
    p->num_splits = 1;
  } else if (mode == paq::DEC_CHUNKS) {
    // about one workgroup per compute unit: parts of ceil(S / P) chunks each
    long P = std::max<long>(1, std::min<long>(std::min<long>(S, paq::kDecMaxPartsPerSeq),
                                              (cus + units - 1) / units));
    const long cpw = (S + P - 1) / P;
    P = (S + cpw - 1) / cpw;
    p->num_splits = S;
    p->parts_per_seq = (int)P;
    p->chunks_per_part = (int)cpw;
    parts = (long)d->batch * P;
    slots = parts * hg;                 // one partial per workgroup
  } else {
    groups = std::min<long>(groups, std::max<long>(1, total));
    p->num_splits = 0;
    p->keys_per_group = (int)std::min<long>(32 * ((total + groups - 1) / groups), 1L << 30);
    p->total_tiles = total;
    parts = groups;
    slots = 2 * groups;                 // a first and a last piece per workgroup
  }
  const long grid = mode == paq::DEC_STREAM ? parts : parts * hg;
  if (grid > 0x7fffffffL) return fail(PAQ_ERR_UNSUPPORTED, "decode grid too large");
  p->parts = (int)parts;
  p->grid_x = (int)grid;
  p->grid_y = 1;
  p->grid_z = 1;
  if (mode != paq::DEC_SINGLE) {
    // per partial slot: (raw maximum, sum) and the output of the HW * G query
    // heads of one head group
    const size_t rows = (size_t)slots * (d->num_heads / hg);
    p->workspace_bytes = head + align_up(rows * d->head_size * sizeof(float)) +
                         align_up(rows * 2 * sizeof(float));
  }
  return PAQ_OK;
}

int plan_prefill(const paq_desc* d, const int32_t* cum_q_host, const int32_t* past_host,
                 paq_plan* p) {
  memset(p, 0, sizeof *p);
  SeqStats st;
  int rc = validate(d, cum_q_host, past_host, &st);
  if (rc) return rc;
  p->max_query_len = st.max_q;
  p->max_kv_len = st.max_kv;
  p->active_seqs = st.active;
  p->work_units = st.active * d->kv_num_heads;
  p->num_splits = 1;
  if (st.max_q == 0) {
    p->path = PAQ_PATH_NONE;          // nothing to launch (and no invalid grid)
    return PAQ_OK;
  }
  const int group = d->num_heads / d->kv_num_heads;
  if (d->q_dtype != PAQ_DT_F32 &&
      paq::prefill_mfma_supports(d->head_size, group, d->block_size, d->q_dtype)) {
    p->path = PAQ_PATH_PREFILL;
    p->grid_x = paq::prefill_grid(cum_q_host, d->batch, group, d->kv_num_heads);
    p->grid_y = 1;
    p->grid_z = 1;
  } else {
    if (group > paq::kF32KernelMaxGroup)
      return fail(PAQ_ERR_UNSUPPORTED,
                  "no prefill kernel for %s queries with %d query heads per kv head",
                  d->q_dtype == PAQ_DT_F32 ? "fp32" : "16-bit", group);
    p->path = PAQ_PATH_F32_PREFILL;
    p->grid_x = d->token_count;
    p->grid_y = d->kv_num_heads;
    p->grid_z = 1;
  }
  return PAQ_OK;
}

paq::AttnArgs attn_args(const paq_desc* d, const void* query, void* out, const void* kc,
                        const void* vc, const float* ks, const float* vs, const int32_t* bt,
                        const int32_t* cum_q, const int32_t* past, float softmax_scale,
                        const paq_plan& p) {
  paq::AttnArgs a;
  memset(&a, 0, sizeof a);
  a.query = query;
  a.out = out;
  a.key_cache = (const uint8_t*)kc;
  a.value_cache = (const uint8_t*)vc;
  a.k_scale = ks;
  a.v_scale = vs;
  a.block_table = bt;
  a.cum_q = cum_q;
  a.past_lens = past;
  a.batch = d->batch;
  a.token_count = d->token_count;
  a.num_heads = d->num_heads;
  a.hkv = d->kv_num_heads;
  a.head_size = d->head_size;
  a.block_size = d->block_size;
  a.max_blocks = d->max_blocks_per_seq;
  a.q_dtype = d->q_dtype;
  a.kv_format = d->kv_format;
  a.scale_mode = d->scale_mode;
  a.num_splits = p.num_splits > 0 ? p.num_splits : 1;
  a.max_query_len = p.max_query_len;
  a.max_kv_len = p.max_kv_len;
  a.grid_x = p.grid_x;
  a.block_size_log2 = __builtin_ctz((unsigned)d->block_size);
  a.softmax_scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)d->head_size);
  return a;
}

int check_attn_pointers(const void* query, void* out, const void* kc, const void* vc,
                        const float* ks, const float* vs, const int32_t* bt,
                        const int32_t* cum_q, const int32_t* past) {
  if (!query || !out || !kc || !vc || !ks || !vs || !bt || !cum_q || !past)
    return fail(PAQ_ERR_INVALID_ARG, "a device pointer argument is NULL");
  return PAQ_OK;
}

int launched(int launcher_rc, const char* what) {
  if (launcher_rc != 0)
    return fail(PAQ_ERR_UNSUPPORTED, "%s: no kernel built for this combination", what);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PAQ_ERR_HIP, "%s launch: %s", what, hipGetErrorString(e));
  return PAQ_OK;
}

// Decode launch shared by the dense and the block-sparse entry points: the
// kernels and launch shape the plan describes (the launchers recompute
// nothing), and the fp32 kernel's combine after a split.  Workspace layout:
// the arrival counters (kDecCounterBytes, zero before and after every call),
// then the partials.
int run_decode(const paq_desc* d, const paq_plan& p, paq::AttnArgs& a, void* workspace,
               hipStream_t st) {
  int rc;
  char* ws = (char*)workspace;
  const size_t head = paq::kDecCounterBytes;
  if (p.path == PAQ_PATH_SINGLE || p.path == PAQ_PATH_SPLIT || p.path == PAQ_PATH_BALANCED) {
    a.dec_mode = p.path == PAQ_PATH_SINGLE ? paq::DEC_SINGLE
                 : p.path == PAQ_PATH_SPLIT ? paq::DEC_CHUNKS : paq::DEC_STREAM;
    a.dec_waves = p.waves_per_group;
    a.dec_head_groups =
        d->kv_num_heads / paq::decode_heads_per_wave(d->kv_format, d->head_size, d->kv_num_heads);
    a.dec_parts_per_seq = p.parts_per_seq;
    a.dec_chunks_per_part = p.chunks_per_part;
    a.dec_total_tiles = p.total_tiles;
    if (a.dec_mode != paq::DEC_SINGLE) {
      const size_t slots = a.dec_mode == paq::DEC_STREAM ? 2 * (size_t)p.parts
                                                          : (size_t)p.parts * a.dec_head_groups;
      const size_t rows = slots * (d->num_heads / a.dec_head_groups);
      a.dec_counters = (int32_t*)ws;
      a.part_o = (float*)(ws + head);
      a.part_ml = (float*)(ws + head + align_up(rows * d->head_size * sizeof(float)));
    }
    return launched(paq::launch_decode_mfma(a, st), "decode (MFMA)");
  }
  if (p.num_splits > 1) {
    a.part_count = p.num_splits;
    const size_t rows = (size_t)d->token_count * d->num_heads * a.part_count;
    a.part_o = (float*)(ws + head);
    a.part_lse = (float*)(ws + head + align_up(rows * d->head_size * sizeof(float)));
  }
  rc = launched(paq::launch_decode_f32(a, st), "decode (fp32)");
  if (rc) return rc;
  if (p.num_splits > 1) rc = launched(paq::launch_combine(a, st), "split-KV combine");
  return rc;
}

// Block-sparse decode plan: the decode over the compact table of selected
// blocks (max_sel columns), with every active sequence's key count bounded by
// num_sel * block_size (the exact count, known on the device, can be smaller
// only by the unused tail of a selected last block).
int plan_sparse(const paq_desc* d, const int32_t* cum_q_host, const int32_t* past_host,
                const int32_t* num_sel_host, int max_sel, int num_splits, paq_desc* dc,
                std::vector<int32_t>* past_c, paq_plan* p) {
  SeqStats st;
  int rc = validate(d, cum_q_host, past_host, &st);
  if (rc) return rc;
  if (max_sel < 1) return fail(PAQ_ERR_INVALID_ARG, "max_sel %d < 1", max_sel);
  if (d->batch > 0 && !num_sel_host) return fail(PAQ_ERR_INVALID_ARG, "num_sel_host is NULL");
  *dc = *d;
  dc->max_blocks_per_seq = max_sel;
  past_c->assign(d->batch, 0);
  for (int b = 0; b < d->batch; ++b) {
    if (cum_q_host[b + 1] == cum_q_host[b]) continue;
    const int nb = (past_host[b] + 1 + d->block_size - 1) / d->block_size;
    const int n = num_sel_host[b];
    if (n < 1 || n > max_sel || n > nb)
      return fail(PAQ_ERR_INVALID_ARG,
                  "sequence %d selects %d blocks (needs 1..min(max_sel %d, its %d blocks))", b,
                  n, max_sel, nb);
    (*past_c)[b] = n * d->block_size - 1;
  }
  return plan_decode(dc, cum_q_host, past_c->data(), num_splits, 0, p, false);
}

size_t sparse_head_bytes(int batch, int max_sel) {
  return align_up((size_t)batch * max_sel * 4) + align_up((size_t)batch * 4);
}

// Block-sparse prefill plan: the dense prefill over the compact table of the
// selected earlier blocks followed by the blocks holding new tokens, whose
// chunk starts at num_sel * block_size + past % block_size.  *stride gets the
// compact table's row length (max_sel + the most local blocks of a sequence).
int plan_sparse_prefill(const paq_desc* d, const int32_t* cum_q_host, const int32_t* past_host,
                        const int32_t* num_sel_host, int max_sel, paq_desc* dc,
                        std::vector<int32_t>* past_c, int* stride, paq_plan* p) {
  SeqStats st;
  int rc = validate(d, cum_q_host, past_host, &st);
  if (rc) return rc;
  if (max_sel < 0) return fail(PAQ_ERR_INVALID_ARG, "max_sel %d < 0", max_sel);
  if (d->batch > 0 && max_sel > 0 && !num_sel_host)
    return fail(PAQ_ERR_INVALID_ARG, "num_sel_host is NULL");
  int max_local = 0;
  past_c->assign(d->batch, 0);
  for (int b = 0; b < d->batch; ++b) {
    const int q = cum_q_host[b + 1] - cum_q_host[b];
    if (q == 0) continue;
    const int past = past_host[b], bs = d->block_size;
    const int n = max_sel > 0 ? num_sel_host[b] : 0;
    if (n < 0 || n > max_sel || n > past / bs)
      return fail(PAQ_ERR_INVALID_ARG,
                  "sequence %d selects %d blocks (needs 0..min(max_sel %d, its %d blocks "
                  "before the first new token))", b, n, max_sel, past / bs);
    const int local = (int)(((long)past + q + bs - 1) / bs) - past / bs;
    max_local = std::max(max_local, local);
    (*past_c)[b] = n * bs + past % bs;
  }
  *dc = *d;
  *stride = max_sel + max_local;
  dc->max_blocks_per_seq = *stride;
  return plan_prefill(dc, cum_q_host, past_c->data(), p);
}

}  // namespace

namespace paq {

int set_error(int code, const char* msg) { return fail(code, "%s", msg); }

int decode_entry(const paq_desc* d, const void* query, void* out, const void* key_cache,
                 const void* value_cache, const float* k_scale, const float* v_scale,
                 const int32_t* block_table, const int32_t* cum_q, const int32_t* past_lens,
                 const int32_t* cum_q_host, const int32_t* past_lens_host, float softmax_scale,
                 int32_t num_splits, void* workspace, size_t workspace_bytes, void* stream) {
  paq_plan p;
  int rc = plan_decode(d, cum_q_host, past_lens_host, num_splits, 0, &p);
  if (rc) return rc;
  if (p.path == PAQ_PATH_NONE) return PAQ_OK;
  rc = check_attn_pointers(query, out, key_cache, value_cache, k_scale, v_scale, block_table,
                           cum_q, past_lens);
  if (rc) return rc;
  if (p.workspace_bytes > 0) {
    if (!workspace || workspace_bytes < p.workspace_bytes)
      return fail(PAQ_ERR_WORKSPACE, "split decode needs %llu workspace bytes, got %llu",
                  (unsigned long long)p.workspace_bytes, (unsigned long long)workspace_bytes);
    if (((uintptr_t)workspace) % 16)
      return fail(PAQ_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  }
  paq::AttnArgs a = attn_args(d, query, out, key_cache, value_cache, k_scale, v_scale,
                              block_table, cum_q, past_lens, softmax_scale, p);
  return run_decode(d, p, a, workspace, (hipStream_t)stream);
}

}  // namespace paq

extern "C" {

int32_t paq_abi_version(void) { return PAQ_ABI_VERSION; }

const char* paq_status_string(int32_t s) {
  switch (s) {
    case PAQ_OK: return "ok";
    case PAQ_ERR_INVALID_ARG: return "invalid argument";
    case PAQ_ERR_UNSUPPORTED: return "unsupported configuration";
    case PAQ_ERR_WORKSPACE: return "workspace missing or too small";
    case PAQ_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* paq_last_error(void) { return g_last_error.c_str(); }

int32_t paq_plan_decode(const paq_desc* d, const int32_t* cum_q_host,
                        const int32_t* past_lens_host, int32_t num_splits, int32_t num_cus,
                        paq_plan* plan) {
  if (!plan) return fail(PAQ_ERR_INVALID_ARG, "plan is NULL");
  return plan_decode(d, cum_q_host, past_lens_host, num_splits, num_cus, plan);
}

int32_t paq_plan_prefill(const paq_desc* d, const int32_t* cum_q_host,
                         const int32_t* past_lens_host, paq_plan* plan) {
  if (!plan) return fail(PAQ_ERR_INVALID_ARG, "plan is NULL");
  return plan_prefill(d, cum_q_host, past_lens_host, plan);
}

size_t paged_attn_decode_workspace_size(const paq_desc* d, const int32_t* cum_q_host,
                                        const int32_t* past_lens_host, int32_t num_splits) {
  paq_plan p;
  if (plan_decode(d, cum_q_host, past_lens_host, num_splits, 0, &p) != PAQ_OK) return 0;
  return (size_t)p.workspace_bytes;
}

int32_t paged_attn_decode(const paq_desc* d, const void* query, void* out,
                          const void* key_cache, const void* value_cache,
                          const float* k_scale, const float* v_scale,
                          const int32_t* block_table, const int32_t* cum_q,
                          const int32_t* past_lens, const int32_t* cum_q_host,
                          const int32_t* past_lens_host, float softmax_scale,
                          int32_t num_splits, void* workspace, size_t workspace_bytes,
                          void* stream) {
  return paq::decode_entry(d, query, out, key_cache, value_cache, k_scale, v_scale, block_table,
                           cum_q, past_lens, cum_q_host, past_lens_host, softmax_scale,
                           num_splits, workspace, workspace_bytes, stream);
}

// ---- block-sparse decode ----

int32_t paged_attn_decode_sparse(const paq_desc* d, const void* query, void* out,
                                 const void* key_cache, const void* value_cache,
                                 const float* k_scale, const float* v_scale,
                                 const int32_t* block_table, const int32_t* cum_q,
                                 const int32_t* past_lens, const int32_t* cum_q_host,
                                 const int32_t* past_lens_host, const int32_t* sel_blocks,
                                 const int32_t* num_sel, const int32_t* num_sel_host,
                                 int32_t max_sel, float softmax_scale, int32_t num_splits,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  paq_desc dc;
  std::vector<int32_t> past_c;
  paq_plan p;
  int rc = plan_sparse(d, cum_q_host, past_lens_host, num_sel_host, max_sel, num_splits, &dc,
                       &past_c, &p);
  if (rc) return rc;
  if (p.path == PAQ_PATH_NONE) return PAQ_OK;
  rc = check_attn_pointers(query, out, key_cache, value_cache, k_scale, v_scale, block_table,
                           cum_q, past_lens);
  if (rc) return rc;
  if (!sel_blocks || !num_sel) return fail(PAQ_ERR_INVALID_ARG, "sel_blocks / num_sel is NULL");
  const size_t head = sparse_head_bytes(d->batch, max_sel);
  if (!workspace || workspace_bytes < head + p.workspace_bytes)
    return fail(PAQ_ERR_WORKSPACE, "sparse decode needs %llu workspace bytes, got %llu",
                (unsigned long long)(head + p.workspace_bytes),
                (unsigned long long)workspace_bytes);
  if (((uintptr_t)workspace) % 16)
    return fail(PAQ_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  int32_t* compact = (int32_t*)workspace;
  int32_t* eff_past = (int32_t*)((char*)workspace + align_up((size_t)d->batch * max_sel * 4));
  hipStream_t st = (hipStream_t)stream;
  rc = launched(paq::launch_sparse_compact(block_table, d->max_blocks_per_seq, sel_blocks,
                                           num_sel, max_sel, cum_q, past_lens, d->block_size,
                                           d->batch, compact, eff_past, st),
                "sparse block selection");
  if (rc) return rc;
  paq::AttnArgs a = attn_args(&dc, query, out, key_cache, value_cache, k_scale, v_scale,
                              compact, cum_q, eff_past, softmax_scale, p);
  return run_decode(&dc, p, a, (char*)workspace + head, st);
}

size_t paged_attn_decode_sparse_workspace_size(const paq_desc* d, const int32_t* cum_q_host,
                                               const int32_t* past_lens_host,
                                               const int32_t* num_sel_host, int32_t max_sel,
                                               int32_t num_splits) {
  paq_desc dc;
  std::vector<int32_t> past_c;
  paq_plan p;
  if (plan_sparse(d, cum_q_host, past_lens_host, num_sel_host, max_sel, num_splits, &dc,
                  &past_c, &p))
    return 0;
  if (p.path == PAQ_PATH_NONE) return 0;
  return sparse_head_bytes(d->batch, max_sel) + p.workspace_bytes;
}

}  // extern "C"

namespace {

// Prefill launch.  padded_mql > 0 sizes the grid from that max_query_len
// (every pair gets the same tile count; tiles past a sequence's rows exit at
// once) instead of the exact per-pair tile counts.
int run_prefill(const paq_desc* d, const void* query, void* out, const void* key_cache,
                const void* value_cache, const float* k_scale, const float* v_scale,
                const int32_t* block_table, const int32_t* cum_q, const int32_t* past_lens,
                const int32_t* cum_q_host, const int32_t* past_lens_host, float softmax_scale,
                int padded_mql, void* stream, bool k_per_use = false) {
  paq_plan p;
  int rc = plan_prefill(d, cum_q_host, past_lens_host, &p);
  if (rc) return rc;
  if (k_per_use && (p.path == PAQ_PATH_F32_PREFILL || d->kv_format == PAQ_KV_INT4 ||
                    d->head_size != 128))
    return fail(PAQ_ERR_UNSUPPORTED,
                "the per-use K conversion variant covers 16-bit queries over 1-byte codes at "
                "head size 128");
  if (p.path == PAQ_PATH_NONE) return PAQ_OK;
  if (padded_mql > 0 && padded_mql < p.max_query_len)
    return fail(PAQ_ERR_INVALID_ARG,
                "max_query_len %d is below the exact maximum %d: rows would be left unwritten",
                padded_mql, p.max_query_len);
  rc = check_attn_pointers(query, out, key_cache, value_cache, k_scale, v_scale, block_table,
                           cum_q, past_lens);
  if (rc) return rc;
  paq::AttnArgs a = attn_args(d, query, out, key_cache, value_cache, k_scale, v_scale,
                              block_table, cum_q, past_lens, softmax_scale, p);
  a.pf_k_per_use = k_per_use ? 1 : 0;
  hipStream_t st = (hipStream_t)stream;
  if (p.path == PAQ_PATH_PREFILL) {
    const int group = d->num_heads / d->kv_num_heads;
    if (padded_mql > 0) {
      const int tok = paq::prefill_tokens_per_workgroup(group);
      const long ntq = ((long)padded_mql + tok - 1) / tok;
      const long pairs = (long)d->kv_num_heads * d->batch;
      const long grid = 8 * ((pairs + 7) / 8) * ntq;
      if (grid > 0x7fffffffL) return fail(PAQ_ERR_UNSUPPORTED, "padded prefill grid too large");
      a.pf_ntq = (int)ntq;
      a.grid_x = (int)grid;
    } else {
      a.pf_ntq = paq::prefill_uniform_tiles(cum_q_host, d->batch, group);
    }
    return launched(paq::launch_prefill_mfma(a, st), "prefill (MFMA)");
  }
  return launched(paq::launch_decode_f32(a, st), "prefill (fp32)");
}

}  // namespace

extern "C" {

int32_t paged_attn_prefill(const paq_desc* d, const void* query, void* out,
                           const void* key_cache, const void* value_cache,
                           const float* k_scale, const float* v_scale,
                           const int32_t* block_table, const int32_t* cum_q,
                           const int32_t* past_lens, const int32_t* cum_q_host,
                           const int32_t* past_lens_host, float softmax_scale,
                           void* stream) {
  return run_prefill(d, query, out, key_cache, value_cache, k_scale, v_scale, block_table, cum_q,
                     past_lens, cum_q_host, past_lens_host, softmax_scale, 0, stream);
}

int32_t paged_attn_prefill_padded(const paq_desc* d, const void* query, void* out,
                                  const void* key_cache, const void* value_cache,
                                  const float* k_scale, const float* v_scale,
                                  const int32_t* block_table, const int32_t* cum_q,
                                  const int32_t* past_lens, const int32_t* cum_q_host,
                                  const int32_t* past_lens_host, float softmax_scale,
                                  int32_t max_query_len, void* stream) {
  if (max_query_len < 1) return fail(PAQ_ERR_INVALID_ARG, "max_query_len %d < 1", max_query_len);
  return run_prefill(d, query, out, key_cache, value_cache, k_scale, v_scale, block_table, cum_q,
                     past_lens, cum_q_host, past_lens_host, softmax_scale, max_query_len, stream);
}

int32_t paged_attn_prefill_k_per_use(const paq_desc* d, const void* query, void* out,
                                     const void* key_cache, const void* value_cache,
                                     const float* k_scale, const float* v_scale,
                                     const int32_t* block_table, const int32_t* cum_q,
                                     const int32_t* past_lens, const int32_t* cum_q_host,
                                     const int32_t* past_lens_host, float softmax_scale,
                                     void* stream) {
  return run_prefill(d, query, out, key_cache, value_cache, k_scale, v_scale, block_table, cum_q,
                     past_lens, cum_q_host, past_lens_host, softmax_scale, 0, stream, true);
}

// ---- block-sparse prefill ----

int32_t paged_attn_prefill_sparse(const paq_desc* d, const void* query, void* out,
                                  const void* key_cache, const void* value_cache,
                                  const float* k_scale, const float* v_scale,
                                  const int32_t* block_table, const int32_t* cum_q,
                                  const int32_t* past_lens, const int32_t* cum_q_host,
                                  const int32_t* past_lens_host, const int32_t* sel_blocks,
                                  const int32_t* num_sel, const int32_t* num_sel_host,
                                  int32_t max_sel, float softmax_scale, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  paq_desc dc;
  std::vector<int32_t> past_c;
  paq_plan p;
  int stride = 0;
  int rc = plan_sparse_prefill(d, cum_q_host, past_lens_host, num_sel_host, max_sel, &dc,
                               &past_c, &stride, &p);
  if (rc) return rc;
  if (p.path == PAQ_PATH_NONE) return PAQ_OK;
  rc = check_attn_pointers(query, out, key_cache, value_cache, k_scale, v_scale, block_table,
                           cum_q, past_lens);
  if (rc) return rc;
  if (max_sel > 0 && (!sel_blocks || !num_sel))
    return fail(PAQ_ERR_INVALID_ARG, "sel_blocks / num_sel is NULL");
  const size_t need = sparse_head_bytes(d->batch, stride);
  if (!workspace || workspace_bytes < need)
    return fail(PAQ_ERR_WORKSPACE, "sparse prefill needs %llu workspace bytes, got %llu",
                (unsigned long long)need, (unsigned long long)workspace_bytes);
  if (((uintptr_t)workspace) % 16)
    return fail(PAQ_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  int32_t* compact = (int32_t*)workspace;
  int32_t* eff_past = (int32_t*)((char*)workspace + align_up((size_t)d->batch * stride * 4));
  rc = launched(paq::launch_sparse_prefill_compact(block_table, d->max_blocks_per_seq,
                                                   sel_blocks, num_sel, max_sel, cum_q,
                                                   past_lens, d->block_size, d->batch, stride,
                                                   compact, eff_past, (hipStream_t)stream),
                "sparse prefill block selection");
  if (rc) return rc;
  return run_prefill(&dc, query, out, key_cache, value_cache, k_scale, v_scale, compact, cum_q,
                     eff_past, cum_q_host, past_c.data(), softmax_scale, 0, stream);
}

size_t paged_attn_prefill_sparse_workspace_size(const paq_desc* d, const int32_t* cum_q_host,
                                                const int32_t* past_lens_host,
                                                const int32_t* num_sel_host, int32_t max_sel) {
  paq_desc dc;
  std::vector<int32_t> past_c;
  paq_plan p;
  int stride = 0;
  if (plan_sparse_prefill(d, cum_q_host, past_lens_host, num_sel_host, max_sel, &dc, &past_c,
                          &stride, &p))
    return 0;
  if (p.path == PAQ_PATH_NONE) return 0;
  return sparse_head_bytes(d->batch, stride);
}

int32_t kv_quant_append(const paq_desc* d, int32_t kv_in_dtype, const void* key,
                        const void* value, void* key_cache, void* value_cache,
                        const float* k_scale, const float* v_scale,
                        const int32_t* block_table, const int32_t* cum_q,
                        const int32_t* past_lens, const int32_t* cum_q_host,
                        const int32_t* past_lens_host, void* stream) {
  SeqStats st;
  int rc = validate(d, cum_q_host, past_lens_host, &st);
  if (rc) return rc;
  if (kv_in_dtype < PAQ_DT_F32 || kv_in_dtype > PAQ_DT_BF16)
    return fail(PAQ_ERR_INVALID_ARG, "kv_in_dtype %d unknown", kv_in_dtype);
  if (st.max_q == 0) return PAQ_OK;
  if (!key || !value || !key_cache || !value_cache || !k_scale || !v_scale || !block_table ||
      !cum_q || !past_lens)
    return fail(PAQ_ERR_INVALID_ARG, "a device pointer argument is NULL");
  paq::AppendArgs a;
  memset(&a, 0, sizeof a);
  a.key = key;
  a.value = value;
  a.key_cache = key_cache;
  a.value_cache = value_cache;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.block_table = block_table;
  a.cum_q = cum_q;
  a.past_lens = past_lens;
  a.batch = d->batch;
  a.hkv = d->kv_num_heads;
  a.head_size = d->head_size;
  a.block_size = d->block_size;
  a.max_blocks = d->max_blocks_per_seq;
  a.kv_format = d->kv_format;
  a.scale_mode = d->scale_mode;
  a.in_dtype = kv_in_dtype;
  a.max_query_len = st.max_q;
  const int chunks_per_tok = 2 * d->kv_num_heads * d->head_size / 8;
  a.tokens_per_wg = std::max(1, 2048 / chunks_per_tok);
  return launched(paq::launch_quant_append(a, (hipStream_t)stream), "kv_quant_append");
}

int32_t paged_attn_decode_append(const paq_desc* d, int32_t kv_in_dtype, const void* key,
                                 const void* value, const void* query, void* out,
                                 void* key_cache, void* value_cache, const float* k_scale,
                                 const float* v_scale, const int32_t* block_table,
                                 const int32_t* cum_q, const int32_t* past_lens,
                                 const int32_t* cum_q_host, const int32_t* past_lens_host,
                                 float softmax_scale, int32_t num_splits, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  // Every check of both operations runs before anything is launched.
  paq_plan p;
  int rc = plan_decode(d, cum_q_host, past_lens_host, num_splits, 0, &p);
  if (rc) return rc;
  if (kv_in_dtype < PAQ_DT_F32 || kv_in_dtype > PAQ_DT_BF16)
    return fail(PAQ_ERR_INVALID_ARG, "kv_in_dtype %d unknown", kv_in_dtype);
  if (p.path == PAQ_PATH_NONE) return PAQ_OK;             // no new token: nothing to append
  rc = check_attn_pointers(query, out, key_cache, value_cache, k_scale, v_scale, block_table,
                           cum_q, past_lens);
  if (rc) return rc;
  if (!key || !value) return fail(PAQ_ERR_INVALID_ARG, "key / value is NULL");
  if (p.workspace_bytes > 0) {
    if (!workspace || workspace_bytes < p.workspace_bytes)
      return fail(PAQ_ERR_WORKSPACE, "split decode needs %llu workspace bytes, got %llu",
                  (unsigned long long)p.workspace_bytes, (unsigned long long)workspace_bytes);
    if (((uintptr_t)workspace) % 16)
      return fail(PAQ_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  }
  // The decode kernels quantize the new rows themselves when everything is
  // 16-byte aligned (16-byte code stores and row loads) and the rows come in
  // the query's dtype (or in fp32, for the MFMA decode); otherwise the two
  // operations run one after the other on the stream.
  const bool aligned = ((uintptr_t)key_cache | (uintptr_t)value_cache) % 16 == 0 &&
                       ((uintptr_t)key | (uintptr_t)value) % 16 == 0;
  const bool mfma = p.path == PAQ_PATH_SINGLE || p.path == PAQ_PATH_SPLIT ||
                    p.path == PAQ_PATH_BALANCED;
  const bool rows_ok = kv_in_dtype == d->q_dtype || (mfma && kv_in_dtype == PAQ_DT_F32);
  if (!rows_ok || !aligned) {
    rc = kv_quant_append(d, kv_in_dtype, key, value, key_cache, value_cache, k_scale, v_scale,
                         block_table, cum_q, past_lens, cum_q_host, past_lens_host, stream);
    if (rc) return rc;
    return paq::decode_entry(d, query, out, key_cache, value_cache, k_scale, v_scale,
                             block_table, cum_q, past_lens, cum_q_host, past_lens_host,
                             softmax_scale, num_splits, workspace, workspace_bytes, stream);
  }
  paq::AttnArgs a = attn_args(d, query, out, key_cache, value_cache, k_scale, v_scale,
                              block_table, cum_q, past_lens, softmax_scale, p);
  a.new_key = key;
  a.new_value = value;
  a.new_rows_f32 = kv_in_dtype == PAQ_DT_F32 && d->q_dtype != PAQ_DT_F32;
  return run_decode(d, p, a, workspace, (hipStream_t)stream);
}

int32_t paged_attn_decode_host(const paq_desc* d, const float* query, float* out,
                               const void* key_cache, const void* value_cache,
                               const float* k_scale, const float* v_scale,
                               const int32_t* block_table, const int32_t* cum_q,
                               const int32_t* past_lens, float softmax_scale,
                               int32_t num_splits, int32_t num_threads) {
  SeqStats st;
  int rc = validate(d, cum_q, past_lens, &st);
  if (rc) return rc;
  if (d->q_dtype != PAQ_DT_F32)
    return fail(PAQ_ERR_UNSUPPORTED, "the host decode takes fp32 queries (q_dtype %d)",
                d->q_dtype);
  for (int b = 0; b < d->batch; ++b)
    if (cum_q[b + 1] - cum_q[b] > 1)
      return fail(PAQ_ERR_INVALID_ARG, "decode needs q_len 0 or 1 (sequence %d has %d)", b,
                  cum_q[b + 1] - cum_q[b]);
  if (num_splits < 0) return fail(PAQ_ERR_INVALID_ARG, "num_splits %d < 0", num_splits);
  if (d->num_heads / d->kv_num_heads > 64)
    return fail(PAQ_ERR_UNSUPPORTED, "more than 64 query heads per kv head");
  if (st.active == 0) return PAQ_OK;
  if (!query || !out || !key_cache || !value_cache || !k_scale || !v_scale || !block_table)
    return fail(PAQ_ERR_INVALID_ARG, "a host pointer argument is NULL");
  paq::HostDecodeArgs a;
  a.query = query;
  a.out = out;
  a.key_cache = (const uint8_t*)key_cache;
  a.value_cache = (const uint8_t*)value_cache;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.block_table = block_table;
  a.cum_q = cum_q;
  a.past_lens = past_lens;
  a.batch = d->batch;
  a.num_heads = d->num_heads;
  a.hkv = d->kv_num_heads;
  a.head_size = d->head_size;
  a.block_size = d->block_size;
  a.max_blocks = d->max_blocks_per_seq;
  a.kv_format = d->kv_format;
  a.scale_mode = d->scale_mode;
  a.softmax_scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)d->head_size);
  a.splits = num_splits;
  a.threads = num_threads > 0 ? num_threads : (int)std::max(1u, std::thread::hardware_concurrency());
  if (paq::host_decode(a)) return fail(PAQ_ERR_UNSUPPORTED, "host decode shape not handled");
  return PAQ_OK;
}

int32_t kv_quant_append_rotary(const paq_desc* d, int32_t kv_in_dtype, void* query,
                               const void* key, const void* value, void* key_cache,
                               void* value_cache, const float* k_scale, const float* v_scale,
                               const int32_t* block_table, const int32_t* cum_q,
                               const int32_t* past_lens, const int32_t* cum_q_host,
                               const int32_t* past_lens_host, const float* cos_cache,
                               const float* sin_cache, int32_t max_position,
                               int32_t rotary_dim, int32_t interleaved, void* stream) {
  SeqStats st;
  int rc = validate(d, cum_q_host, past_lens_host, &st);
  if (rc) return rc;
  if (kv_in_dtype < PAQ_DT_F32 || kv_in_dtype > PAQ_DT_BF16)
    return fail(PAQ_ERR_INVALID_ARG, "kv_in_dtype %d unknown", kv_in_dtype);
  if (rotary_dim <= 0 || rotary_dim % 2 || rotary_dim > d->head_size)
    return fail(PAQ_ERR_INVALID_ARG, "rotary_dim %d must be even and in [2, head_size %d]",
                rotary_dim, d->head_size);
  if (rotary_dim % 16)
    return fail(PAQ_ERR_UNSUPPORTED, "rotary_dim %d is not a multiple of 16", rotary_dim);
  if (interleaved != 0 && interleaved != 1)
    return fail(PAQ_ERR_INVALID_ARG, "interleaved %d must be 0 or 1", interleaved);
  if (max_position < 1) return fail(PAQ_ERR_INVALID_ARG, "max_position %d < 1", max_position);
  for (int b = 0; b < d->batch; ++b) {
    const int64_t last = (int64_t)past_lens_host[b] + cum_q_host[b + 1] - cum_q_host[b] - 1;
    if (cum_q_host[b + 1] > cum_q_host[b] && last >= max_position)
      return fail(PAQ_ERR_INVALID_ARG, "sequence %d reaches position %lld >= max_position %d", b,
                  (long long)last, max_position);
  }
  if (st.max_q == 0) return PAQ_OK;
  if (!key || !value || !key_cache || !value_cache || !k_scale || !v_scale || !block_table ||
      !cum_q || !past_lens || !cos_cache || !sin_cache)
    return fail(PAQ_ERR_INVALID_ARG, "a device pointer argument is NULL");
  if (((uintptr_t)cos_cache | (uintptr_t)sin_cache) & 15)
    return fail(PAQ_ERR_INVALID_ARG, "cos_cache and sin_cache must be 16-byte aligned");
  paq::AppendArgs a;
  memset(&a, 0, sizeof a);
  a.key = key;
  a.value = value;
  a.key_cache = key_cache;
  a.value_cache = value_cache;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.block_table = block_table;
  a.cum_q = cum_q;
  a.past_lens = past_lens;
  a.batch = d->batch;
  a.hkv = d->kv_num_heads;
  a.head_size = d->head_size;
  a.block_size = d->block_size;
  a.max_blocks = d->max_blocks_per_seq;
  a.kv_format = d->kv_format;
  a.scale_mode = d->scale_mode;
  a.in_dtype = kv_in_dtype;
  a.max_query_len = st.max_q;
  a.query = query;
  a.cos_cache = cos_cache;
  a.sin_cache = sin_cache;
  a.num_heads = d->num_heads;
  a.q_dtype = d->q_dtype;
  a.rotary_dim = rotary_dim;
  a.interleaved = interleaved;
  // work units of one token: query pairs, key units, value chunks
  const int ur = interleaved ? rotary_dim / 8 : rotary_dim / 16;
  const int per_tok = (query ? d->num_heads * ur : 0) +
                      d->kv_num_heads * (ur + (d->head_size - rotary_dim) / 8) +
                      d->kv_num_heads * d->head_size / 8;
  a.tokens_per_wg = std::max(1, 2048 / per_tok);
  return launched(paq::launch_rotary_append(a, (hipStream_t)stream), "kv_quant_append_rotary");
}

}  // extern "C"
