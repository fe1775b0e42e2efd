"""Block-sparse decode: each new query row attends only to the keys of the
KV blocks selected for its sequence.  Test infrastructure only (see the
package docstring).

Source.  "INT8-KV Tensor-Core DynamicSparseAttention" (P2), section 1: a
decode (and prefill) attention over a dynamically selected subset of an INT8
KV cache, with a split-K variant.  The page does not give the selection
rule.  Reading (the plainest): the caller passes, for sequence b, num_sel[b]
ascending logical block indices sel[b, :num_sel[b]] (each < ceil(kv_len/bs));
the query row attends to exactly the keys t < kv_len whose block t // bs is
selected, with the ordinary scaled-dot-product softmax over them.

Prefill (the same section names prefill beside decode).  Reading: a chunk of
new tokens attends causally, as in dense prefill, to (a) every key of the
blocks that hold one of its new tokens -- blocks past // bs .. (kv_len-1) //
bs, including the cached keys that share the first of them -- and (b) every
key of the earlier blocks the caller selects, sel[b, :num_sel[b]], ascending
indices each below past // bs (blocks holding cached keys only).  The local
blocks are always attended, so no row is left without keys.
"""

import numpy as np

from . import attention


def block_sparse_decode(query, key_cache, value_cache, k_scale, v_scale, block_table, cum_q,
                        past_lens, kv_format, sel, num_sel, softmax_scale=None):
    """query (T, H, D), one row per sequence with a new token; returns float64 (T, H, D)."""
    q = np.asarray(query, dtype=np.float64)
    T, H, D = q.shape
    hkv = key_cache.shape[2]
    G = H // hkv
    bs = key_cache.shape[1]
    sigma = attention.default_scale(D, softmax_scale)
    out = np.zeros((T, H, D))
    for b in range(len(past_lens)):
        r0, r1 = int(cum_q[b]), int(cum_q[b + 1])
        if r1 == r0:
            continue
        if r1 - r0 != 1:
            raise ValueError("decode: one new row per sequence")
        L = int(past_lens[b]) + 1
        K = attention.sequence_kv(key_cache, kv_format, k_scale, block_table[b], L, D)
        V = attention.sequence_kv(value_cache, kv_format, v_scale, block_table[b], L, D)
        chosen = set(int(x) for x in sel[b][: int(num_sel[b])])
        keep = np.array([t // bs in chosen for t in range(L)])
        for h in range(H):
            g = h // G
            s = sigma * (K[keep, g] @ q[r0, h])
            p = np.exp(s - s.max())
            out[r0, h] = (p @ V[keep, g]) / p.sum()
    return out


def block_sparse_prefill(query, key_cache, value_cache, k_scale, v_scale, block_table, cum_q,
                         past_lens, kv_format, sel, num_sel, softmax_scale=None):
    """query (T, H, D), q_len_b rows per sequence; returns float64 (T, H, D).

    Row i of sequence b (position past_b + i) sees key t iff t <= past_b + i
    and block t // bs is selected or holds a new token (t // bs >= past_b // bs).
    """
    q = np.asarray(query, dtype=np.float64)
    T, H, D = q.shape
    hkv = key_cache.shape[2]
    G = H // hkv
    bs = key_cache.shape[1]
    sigma = attention.default_scale(D, softmax_scale)
    out = np.zeros((T, H, D))
    for b in range(len(past_lens)):
        r0, r1 = int(cum_q[b]), int(cum_q[b + 1])
        if r1 == r0:
            continue
        past = int(past_lens[b])
        L = past + (r1 - r0)
        K = attention.sequence_kv(key_cache, kv_format, k_scale, block_table[b], L, D)
        V = attention.sequence_kv(value_cache, kv_format, v_scale, block_table[b], L, D)
        chosen = set(int(x) for x in sel[b][: int(num_sel[b])])
        if any(x >= past // bs or x < 0 for x in chosen):
            raise ValueError("sparse prefill: selected blocks must lie before past // block_size")
        blk = np.arange(L) // bs
        attended = np.array([x in chosen or x >= past // bs for x in blk])
        for i in range(r1 - r0):
            keep = attended & (np.arange(L) <= past + i)
            for h in range(H):
                g = h // G
                sc = sigma * (K[keep, g] @ q[r0 + i, h])
                pr = np.exp(sc - sc.max())
                out[r0 + i, h] = (pr @ V[keep, g]) / pr.sum()
    return out
