"""Symmetric quantizers and the quantize-and-append step, written plainly.

Test infrastructure only (see the package docstring).

Definitions and readings (the pages name the formats but not the rounding):
* Scales are fp32 inputs (static calibration), per channel with shape
  (kv_num_heads, head_size) -- the PER_CHANNEL mode of P1 ("INT4 Paged KV
  Cache", section 3) -- or per kv head with shape (kv_num_heads,).
* The quotient is the correctly rounded fp32 value fl32(x / s), where x is the
  input widened to fp32 (exact from fp16 and bf16).  We emulate it as
  float32(float64(x) / float64(s)); double rounding is innocuous for division
  because 53 >= 2*24 + 2 (Figueroa's theorem).
* INT8 code = clamp(round_half_even(q), -127, 127); INT4 the same with +-7
  (symmetric ranges, -128 and -8 unused); FP8 code = E4M3 round-half-even with
  saturation to +-448.
* Appending: token i of sequence b sits at position t = past_b + i, in
  physical block block_table[b, t // block_size] at row t % block_size
  (cache shape (num_blocks, block_size, kv_num_heads, cache_head_size), P1
  section 2).  New rows of the query/key/value tensors are laid out by the
  cumulative query lengths cum_q (P3, section 1).  Nothing else in the cache
  changes.
"""

import numpy as np

from . import codecs

QMAX = {"int8": 127, "int4": 7}


def fl32_quotient(x, s):
    """Correctly rounded fp32 quotient x/s of fp32 operands."""
    x64 = np.asarray(x, dtype=np.float32).astype(np.float64)
    s64 = np.asarray(s, dtype=np.float32).astype(np.float64)
    with np.errstate(over="ignore", divide="ignore"):
        return (x64 / s64).astype(np.float32)


def quantize(x, s, kv_format):
    """Quantize fp32 values x with (broadcastable) fp32 scales s.

    Returns int64 codes for "int8"/"int4" and uint8 E4M3 codes for "fp8".
    """
    q = fl32_quotient(x, s)
    if kv_format in QMAX:
        m = QMAX[kv_format]
        return np.clip(np.rint(q.astype(np.float64)), -m, m).astype(np.int64)
    if kv_format == "fp8":
        return codecs.e4m3_encode(q)
    raise ValueError(kv_format)


def encode_rows(codes, kv_format):
    """Codes (..., D) -> stored bytes (..., cache_head_size) as uint8."""
    if kv_format == "int8":
        return np.asarray(codes, dtype=np.int64).astype(np.int8).view(np.uint8)
    if kv_format == "int4":
        return codecs.int4_pack(codes)
    if kv_format == "fp8":
        return np.asarray(codes, dtype=np.uint8)
    raise ValueError(kv_format)


def decode_rows(stored, kv_format, head_size):
    """Stored bytes (..., C) -> exact code values (..., D) as float64."""
    b = np.asarray(stored, dtype=np.uint8)
    if kv_format == "int8":
        return b.view(np.int8).astype(np.float64)
    if kv_format == "int4":
        return codecs.int4_unpack(b, head_size).astype(np.float64)
    if kv_format == "fp8":
        return codecs.e4m3_decode(b)
    raise ValueError(kv_format)


def expand_scale(scale, kv_num_heads, head_size):
    """Per-channel (Hkv, D) or per-head (Hkv,) fp32 scales -> (Hkv, D) float64."""
    s = np.asarray(scale, dtype=np.float32).astype(np.float64)
    if s.shape == (kv_num_heads,):
        return np.repeat(s[:, None], head_size, axis=1)
    if s.shape == (kv_num_heads, head_size):
        return s
    raise ValueError("scale shape %r" % (s.shape,))


def dequantize(stored, kv_format, scale, head_size):
    """Stored rows (..., Hkv, C) -> real values (..., Hkv, D) in float64:
    code * scale, exact in fp64."""
    hkv = stored.shape[-2]
    return decode_rows(stored, kv_format, head_size) * expand_scale(scale, hkv, head_size)


def quant_append(key_cache, value_cache, key, value, k_scale, v_scale,
                 block_table, cum_q, past_lens, kv_format):
    """Return copies of the caches with the new tokens quantized and stored.

    key, value: (token_count, Hkv, D) real inputs (fp32-exact values).
    caches: uint8 (num_blocks, block_size, Hkv, C).
    """
    kc = np.array(key_cache, dtype=np.uint8, copy=True)
    vc = np.array(value_cache, dtype=np.uint8, copy=True)
    bs = kc.shape[1]
    hkv = kc.shape[2]
    d = np.asarray(key).shape[-1]
    ks = expand_scale(k_scale, hkv, d).astype(np.float32)
    vs = expand_scale(v_scale, hkv, d).astype(np.float32)
    key = np.asarray(key, dtype=np.float32)
    value = np.asarray(value, dtype=np.float32)
    kcode = encode_rows(quantize(key, ks[None], kv_format), kv_format)
    vcode = encode_rows(quantize(value, vs[None], kv_format), kv_format)
    for b in range(len(past_lens)):
        for i in range(int(cum_q[b + 1]) - int(cum_q[b])):
            r = int(cum_q[b]) + i
            t = int(past_lens[b]) + i
            blk = int(block_table[b][t // bs])
            kc[blk, t % bs] = kcode[r]
            vc[blk, t % bs] = vcode[r]
    return kc, vc
