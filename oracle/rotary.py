"""Rotary position embedding (RoPE) of a step's new rows, and the fused
rotate-then-quantize append, written plainly.

Test infrastructure only (see the package docstring).

Source.  "PagedAttention FA path: exact max_query_len" (P3), sections 1-2 and
"why it is better": a rotary-embedding kernel runs over the step's new rows
(laid out by the cumulative query lengths), and with its grid sized by the
heuristic max_query_len = token_count - batch + 1 it dropped rows whenever a
sequence had zero new tokens; the exact host maximum fixes it.  The pages do
not spell out the rotation itself.  Readings (the plainest, standard RoPE):

* Row i of sequence b (row cum_q[b] + i) has position past_b + i, the position
  its key is stored at by the append.
* Channels 0 .. rotary_dim-1 rotate in pairs, the rest pass through.  Pair k
  is (k, k + rotary_dim/2) in the non-interleaved layout and (2k, 2k+1) in the
  interleaved one.
* The angle of pair k at position p comes from the caller as fp32 tables
  cos_cache[p, k] and sin_cache[p, k].  A pair (x, y) becomes
  (x cos - y sin, y cos + x sin), i.e. x + iy times cos + i sin.
* Precision.  `rotate` is exact in fp64.  The cache codes, integers decided by
  floating point, are decided in the kernel's precision: `rotate_fp32` rounds
  each product to fp32 and then the difference or sum to fp32 (no fused
  multiply-add).  Rotated queries are rounded half-even to the query dtype.
"""

import numpy as np

from . import quant


def pair_channels(rotary_dim, interleaved):
    """(first, second) channel index arrays of the rotary_dim/2 pairs."""
    half = rotary_dim // 2
    if interleaved:
        first = [2 * k for k in range(half)]
        second = [2 * k + 1 for k in range(half)]
    else:
        first = [k for k in range(half)]
        second = [k + half for k in range(half)]
    return np.array(first, dtype=np.int64), np.array(second, dtype=np.int64)


def positions(cum_q, past_lens):
    """Position of every new row: row cum_q[b] + i sits at past_b + i."""
    pos = np.zeros(int(cum_q[-1]), dtype=np.int64)
    for b in range(len(past_lens)):
        for i in range(int(cum_q[b + 1]) - int(cum_q[b])):
            pos[int(cum_q[b]) + i] = int(past_lens[b]) + i
    return pos


def rotate(x, pos, cos_cache, sin_cache, rotary_dim, interleaved):
    """Exact fp64 rotation of rows x (rows, heads, D); row r uses position pos[r]."""
    x = np.asarray(x, dtype=np.float64)
    out = x.copy()
    first, second = pair_channels(rotary_dim, interleaved)
    c = np.asarray(cos_cache, dtype=np.float64)[pos][:, None, :]      # (rows, 1, half)
    s = np.asarray(sin_cache, dtype=np.float64)[pos][:, None, :]
    a = x[..., first]
    b = x[..., second]
    out[..., first] = a * c - b * s
    out[..., second] = b * c + a * s
    return out


def _fl32(v):
    """Round fp64 values to fp32.  Applied to the exact-or-double-rounded fp64
    result of one operation on fp32 operands it gives the correctly rounded
    fp32 result (53 >= 2*24 + 2, Figueroa's theorem)."""
    with np.errstate(over="ignore"):
        return np.asarray(v, dtype=np.float64).astype(np.float32).astype(np.float64)


def rotate_fp32(x, pos, cos_cache, sin_cache, rotary_dim, interleaved):
    """The same rotation with fp32 rounding after every operation:
    x' = fl32(fl32(x c) - fl32(y s)), y' = fl32(fl32(y c) + fl32(x s)).
    x must hold fp32 values; returns float32."""
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    out = x.copy()
    first, second = pair_channels(rotary_dim, interleaved)
    c = np.asarray(cos_cache, dtype=np.float32).astype(np.float64)[pos][:, None, :]
    s = np.asarray(sin_cache, dtype=np.float32).astype(np.float64)[pos][:, None, :]
    a = x[..., first]
    b = x[..., second]
    out[..., first] = _fl32(_fl32(a * c) - _fl32(b * s))
    out[..., second] = _fl32(_fl32(b * c) + _fl32(a * s))
    return out.astype(np.float32)


def round_to_dtype(x, dtype):
    """Round fp32 values half-even to "f32", "f16" or "bf16"; returned as
    float32 holding the rounded values (finite inputs)."""
    x = np.asarray(x, dtype=np.float32)
    if dtype == "f32":
        return x.copy()
    if dtype == "f16":
        with np.errstate(over="ignore"):
            return x.astype(np.float16).astype(np.float32)
    # bf16: keep the top 16 bits of the fp32 pattern, rounding half to even
    u = x.view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return (r << 16).astype(np.uint32).view(np.float32)


def rotary_append(key_cache, value_cache, query, key, value, k_scale, v_scale,
                  block_table, cum_q, past_lens, kv_format, cos_cache, sin_cache,
                  rotary_dim, interleaved, q_dtype):
    """Rotate the new query and key rows at their positions, then quantize and
    append keys and values.

    query (T, H, D) and key/value (T, Hkv, D) hold fp32-exact values.  Returns
    (key_cache, value_cache, rotated query rounded to q_dtype, as float32).
    """
    pos = positions(cum_q, past_lens)
    k_rot = rotate_fp32(key, pos, cos_cache, sin_cache, rotary_dim, interleaved)
    q_rot = rotate_fp32(query, pos, cos_cache, sin_cache, rotary_dim, interleaved)
    kc, vc = quant.quant_append(key_cache, value_cache, k_rot, value, k_scale, v_scale,
                                block_table, cum_q, past_lens, kv_format)
    return kc, vc, round_to_dtype(q_rot, q_dtype)
