"""Test-side helpers: fill an oracle cache from a seeded workload.

The cache pool starts poisoned (0x7F: INT8 127, FP8 NaN, INT4 nibbles 7/-1)
so that any read of an unused slot shows up, then the past tokens and the
step's new tokens are appended with the oracle's quantizer -- the same two
appends the HIP path performs on its side.
"""

import numpy as np

from oracle import quant

POISON = 0x7F


def f32(t):
    return t.to(dtype=__import__("torch").float32).numpy()


def oracle_caches(w):
    """(key_cache, value_cache) uint8 after appending past and new tokens."""
    shape = (w.num_blocks, w.block_size, w.kv_num_heads, w.cache_head_size)
    kc = np.full(shape, POISON, np.uint8)
    vc = np.full(shape, POISON, np.uint8)
    zeros = np.zeros(w.batch, np.int32)
    if w.past_key.shape[0]:
        kc, vc = quant.quant_append(kc, vc, f32(w.past_key), f32(w.past_value),
                                    w.k_scale, w.v_scale, w.block_table, w.cum_past,
                                    zeros, w.kv_format)
    if w.new_key.shape[0]:
        kc, vc = quant.quant_append(kc, vc, f32(w.new_key), f32(w.new_value),
                                    w.k_scale, w.v_scale, w.block_table, w.cum_q,
                                    w.past_lens, w.kv_format)
    return kc, vc


def oracle_attention(w, kc, vc, num_splits=1, softmax_scale=None):
    from oracle import attention
    return attention.paged_attention(f32(w.query), kc, vc, w.k_scale, w.v_scale,
                                     w.block_table, w.cum_q, w.past_lens, w.kv_format,
                                     softmax_scale=softmax_scale, num_splits=num_splits)
