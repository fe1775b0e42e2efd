"""Pure-Python scalar-loop attention over the paged cache, for tiny inputs.

Test infrastructure only (see the package docstring).  It restates the same
definition as ``attention.paged_attention`` with plain Python numbers and
loops -- no NumPy -- so that the vectorised oracle can be checked against it
on small shapes.  Inputs are nested lists (or anything indexable) of Python
numbers; cache entries are byte values 0..255.
"""

import math


def _byte_code(byte, kv_format, half):
    """Value of one stored byte: the whole byte for int8/fp8, one nibble of it
    for int4 (half 0 = low nibble, half 1 = high nibble)."""
    byte = int(byte)
    if kv_format == "int8":
        return byte - 256 if byte >= 128 else byte
    if kv_format == "int4":
        nib = (byte >> (4 * half)) & 0xF
        return nib - 16 if nib >= 8 else nib
    if kv_format == "fp8":
        sign = -1.0 if byte & 0x80 else 1.0
        e = (byte >> 3) & 0xF
        m = byte & 7
        if e == 15 and m == 7:
            return math.nan
        if e == 0:
            return sign * math.ldexp(m, -9)
        return sign * math.ldexp(8 + m, e - 10)
    raise ValueError(kv_format)


def _value(cache, blk, row, h, d, kv_format, scale):
    if kv_format == "int4":
        code = _byte_code(cache[blk][row][h][d // 2], kv_format, d % 2)
    else:
        code = _byte_code(cache[blk][row][h][d], kv_format, 0)
    s = scale[h][d] if isinstance(scale[h], (list, tuple)) else scale[h]
    return code * float(s)


def paged_attention(query, key_cache, value_cache, k_scale, v_scale, block_table,
                    cum_q, past_lens, kv_format, num_heads, kv_num_heads, head_size,
                    block_size, softmax_scale=None):
    """Returns a dict {(row, head): [D floats]} for every new query row."""
    sigma = (1.0 / math.sqrt(head_size)) if not softmax_scale else softmax_scale
    group = num_heads // kv_num_heads
    out = {}
    for b in range(len(past_lens)):
        for i in range(cum_q[b + 1] - cum_q[b]):
            row = cum_q[b] + i
            last = past_lens[b] + i          # highest visible position
            for h in range(num_heads):
                g = h // group
                scores = []
                for j in range(last + 1):
                    blk = block_table[b][j // block_size]
                    acc = 0.0
                    for d in range(head_size):
                        acc += float(query[row][h][d]) * _value(
                            key_cache, blk, j % block_size, g, d, kv_format, k_scale)
                    scores.append(sigma * acc)
                mx = max(scores)
                w = [math.exp(s - mx) for s in scores]
                tot = sum(w)
                o = []
                for d in range(head_size):
                    acc = 0.0
                    for j in range(last + 1):
                        blk = block_table[b][j // block_size]
                        acc += w[j] * _value(value_cache, blk, j % block_size, g, d,
                                             kv_format, v_scale)
                    o.append(acc / tot)
                out[(row, h)] = o
    return out
