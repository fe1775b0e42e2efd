"""Exact attention over a block-paged, quantized KV cache, in float64.

Test infrastructure only (see the package docstring).

What is computed (the plain definition every kernel is a faster route to):
the pages compare tensor-core results against an fp64 reference (P2,
"INT8-KV Tensor-Core DynamicSparseAttention", why-it-is-good item 2) and the
flash/GEMV decode against the naive one (P4, "GQA GEMV decode", parity-test
section).  Our reading of the pieces the pages leave open:

* Shapes (P1, section 2; P3, section 1): query (token_count, num_heads,
  head_size); caches (num_blocks, block_size, kv_num_heads, cache_head_size);
  block_table (batch, max_blocks_per_seq); cum_q (batch+1) with
  q_len_b = cum_q[b+1] - cum_q[b]; past_lens (batch).
* The step's new keys/values are already in the cache, so sequence b holds
  kv_len_b = past_b + q_len_b tokens.  Query row i of sequence b sees cache
  positions 0 .. past_b + i (causal, aligned to the end).
* GQA: query head h reads kv head h // (num_heads // kv_num_heads).
* Scores use softmax_scale, 1/sqrt(head_size) by default; no bias, window or
  soft-cap.
* Dequantization is code * scale, exact in fp64.
* Sequences with q_len 0 produce no rows (P3, why-it-is-good: zero-token
  batches).
"""

import math

import numpy as np

from . import quant


def max_query_len(cum_q):
    """Exact maximum of q_len_b over the batch, from the host copy of cum_q
    (P3, section 1).  0 for an empty batch."""
    c = [int(v) for v in cum_q]
    best = 0
    for b in range(len(c) - 1):
        best = max(best, c[b + 1] - c[b])
    return best


def heuristic_max_query_len(token_count, batch):
    """The formula P3 replaced (section 1, "Before"); kept only for tests that
    show where it is wrong."""
    return token_count - batch + 1


def gather_rows(cache, table_row, kv_len):
    """Stored rows of positions 0..kv_len-1 of one sequence, shape
    (kv_len, Hkv, C): position t lives in block table_row[t // bs], row t % bs."""
    bs = cache.shape[1]
    out = np.empty((kv_len,) + cache.shape[2:], dtype=cache.dtype)
    for t in range(kv_len):
        out[t] = cache[int(table_row[t // bs]), t % bs]
    return out


def sequence_kv(cache, kv_format, scale, table_row, kv_len, head_size):
    """Dequantized keys or values of one sequence, float64 (kv_len, Hkv, D)."""
    return quant.dequantize(gather_rows(cache, table_row, kv_len), kv_format,
                            scale, head_size)


def default_scale(head_size, softmax_scale=None):
    if softmax_scale is None or softmax_scale == 0.0:
        return 1.0 / math.sqrt(head_size)
    return float(softmax_scale)


def attend_rows(q_rows, k, v, past, sigma, lo=0, hi=None):
    """Exact causal attention for consecutive query rows of one head.

    q_rows (n, D); k, v (L, D); row i sees keys j <= past + i, restricted to
    j in [lo, hi).  Returns (o, lse): o (n, D) normalised over the visible
    keys of the range, lse (n,) the natural-log sum of exp(scores); a row
    with no visible key gets o = 0 and lse = -inf.
    """
    n = q_rows.shape[0]
    L = k.shape[0]
    hi = L if hi is None else hi
    o = np.zeros((n, v.shape[1]))
    lse = np.full(n, -np.inf)
    if hi <= lo or n == 0:
        return o, lse
    s = sigma * (q_rows @ k[lo:hi].T)                     # (n, hi-lo)
    j = np.arange(lo, hi)[None, :]
    i = np.arange(n)[:, None]
    visible = j <= past + i
    s = np.where(visible, s, -np.inf)
    m = s.max(axis=1)
    has = np.isfinite(m)
    msafe = np.where(has, m, 0.0)
    p = np.exp(s - msafe[:, None])                        # masked -> 0
    l = p.sum(axis=1)
    with np.errstate(invalid="ignore", divide="ignore"):
        o = np.where(has[:, None], (p @ v[lo:hi]) / np.where(has, l, 1.0)[:, None], 0.0)
        lse = np.where(has, msafe + np.log(np.where(has, l, 1.0)), -np.inf)
    return o, lse


def combine_partials(os_, lses):
    """Merge per-chunk (o_c, lse_c): L = logsumexp_c lse_c,
    o = sum_c exp(lse_c - L) o_c (P4, section 2: flash decoding partials)."""
    lses = np.stack(lses)                                  # (S, n)
    os_ = np.stack(os_)                                    # (S, n, D)
    L = lses.max(axis=0)
    has = np.isfinite(L)
    Ls = np.where(has, L, 0.0)
    w = np.exp(lses - Ls[None])                            # -inf -> 0
    tot = w.sum(axis=0)
    L = np.where(has, Ls + np.log(np.where(has, tot, 1.0)), -np.inf)
    w = w / np.where(has, tot, 1.0)[None]
    return (w[..., None] * os_).sum(axis=0), L


def chunk_block_ranges(num_seq_blocks, num_splits):
    """Block-aligned balanced partition: chunk c owns blocks
    [floor(c*nb/S), floor((c+1)*nb/S)).  (P4 leaves kv_chunk_count open.)"""
    return [((c * num_seq_blocks) // num_splits,
             ((c + 1) * num_seq_blocks) // num_splits) for c in range(num_splits)]


def paged_attention(query, key_cache, value_cache, k_scale, v_scale,
                    block_table, cum_q, past_lens, kv_format,
                    softmax_scale=None, num_splits=1):
    """Attention of every new query row over its sequence's cached keys.

    query: (T, H, D) values (any float dtype; widened exactly to fp64).
    Returns float64 (T, H, D).  With num_splits > 1 each sequence's keys are
    cut into block-aligned chunks, each chunk is attended separately and the
    partials are merged with combine_partials (the split-KV form; equal to the
    single pass up to rounding).
    """
    q = np.asarray(query, dtype=np.float64)
    T, H, D = q.shape
    hkv = key_cache.shape[2]
    if H % hkv:
        raise ValueError("num_heads must be a multiple of kv_num_heads")
    G = H // hkv
    bs = key_cache.shape[1]
    sigma = default_scale(D, softmax_scale)
    out = np.zeros((T, H, D))
    for b in range(len(past_lens)):
        r0, r1 = int(cum_q[b]), int(cum_q[b + 1])
        n = r1 - r0
        if n == 0:
            continue
        past = int(past_lens[b])
        L = past + n
        K = sequence_kv(key_cache, kv_format, k_scale, block_table[b], L, D)
        V = sequence_kv(value_cache, kv_format, v_scale, block_table[b], L, D)
        nb = -(-L // bs)
        for h in range(H):
            g = h // G
            if num_splits <= 1:
                o, _ = attend_rows(q[r0:r1, h], K[:, g], V[:, g], past, sigma)
            else:
                parts = [attend_rows(q[r0:r1, h], K[:, g], V[:, g], past, sigma,
                                     lo=b0 * bs, hi=min(b1 * bs, L))
                         for b0, b1 in chunk_block_ranges(nb, num_splits)]
                o, _ = combine_partials([p[0] for p in parts], [p[1] for p in parts])
            out[r0:r1, h] = o
    return out


def attention_row(query, key_cache, value_cache, k_scale, v_scale,
                  block_table, cum_q, past_lens, kv_format, row, head,
                  softmax_scale=None):
    """One output row (D,) of paged_attention, for sampled checks at sizes
    where the whole tensor is too slow on the CPU."""
    q = np.asarray(query[row, head], dtype=np.float64)
    H, D = query.shape[1], query.shape[2]
    hkv = key_cache.shape[2]
    g = head // (H // hkv)
    c = [int(x) for x in cum_q]
    b = max(i for i in range(len(c) - 1) if c[i] <= row < c[i + 1])
    i = row - c[b]
    past = int(past_lens[b])
    L = past + i + 1
    K = sequence_kv(key_cache, kv_format, k_scale, block_table[b], L, D)[:, g]
    V = sequence_kv(value_cache, kv_format, v_scale, block_table[b], L, D)[:, g]
    o, _ = attend_rows(q[None], K, V, L - 1, default_scale(D, softmax_scale))
    return o[0]
