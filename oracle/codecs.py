"""Storage codecs of the quantized KV cache, written from their definitions.

Test infrastructure only (see the package docstring).

* FP8 E4M3 -- the cache format of the FP8 KV page (P5, "FlashInfer FP8
  KV-cache prefill", section 1: one-byte KV that is not FP4).  The pages do
  not name the variant; we read it as the OCP "E4M3" format (OCP 8-bit
  Floating Point Specification v1.0): sign, 4 exponent bits with bias 7,
  3 mantissa bits, no infinities, S.1111.111 is NaN, largest finite 448.
  Encoding rounds to nearest, ties to even, and saturates to +-448.
* Packed INT4 -- P1 ("INT4 Paged KV Cache", section 2): two 4-bit values share
  one uint8 and cache_head_size = (head_size + 1) // 2.  The nibble order is
  not stated; we read channel 2j as the low nibble and channel 2j+1 as the
  high nibble, each a two's-complement 4-bit integer.  For odd head sizes the
  last high nibble is zero and ignored.
"""

import numpy as np

E4M3_BIAS = 7
E4M3_MAX = 448.0


def e4m3_decode(codes):
    """Decode uint8 E4M3 codes to float64 (exact).  NaN codes give NaN.

    value = (-1)^s * 2^(e-7) * (1 + m/8)  for exponent field e >= 1,
            (-1)^s * 2^(-6)  * (m/8)      for e == 0 (subnormal),
    with S.1111.111 reserved for NaN.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 0xF
    m = c & 0x7
    normal = np.ldexp(1.0 + m / 8.0, (e - E4M3_BIAS).astype(np.int64))
    sub = np.ldexp(m / 8.0, np.full_like(e, 1 - E4M3_BIAS))
    mag = np.where(e == 0, sub, normal)
    mag = np.where((e == 0xF) & (m == 0x7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


def e4m3_encode(y):
    """Encode float32 values to E4M3 with round-to-nearest-even and
    saturation to +-448 (the sign of zero is kept).

    The grid spacing inside the binade [2^k, 2^(k+1)) is 2^(k-3); below the
    smallest normal 2^-6 the spacing is the subnormal step 2^-9.  Dividing by
    a power-of-two spacing is exact in fp64, so rint() (ties to even) gives
    the nearest grid point; an even integer multiple of the spacing is an even
    mantissa, so this is IEEE round-half-even.
    """
    y = np.asarray(y, dtype=np.float32).astype(np.float64)
    if np.isnan(y).any():
        raise ValueError("NaN inputs are outside the quantizer's contract")
    neg = np.signbit(y)
    a = np.abs(y)
    with np.errstate(invalid="ignore", over="ignore"):
        _, ex = np.frexp(a)                   # a in [2^(ex-1), 2^ex)
        k = np.maximum(ex.astype(np.int64) - 1, 1 - E4M3_BIAS)
        step = np.ldexp(1.0, k - 3)
        r = np.rint(a / step) * step
    r = np.where(np.isinf(a), E4M3_MAX, r)
    r = np.minimum(r, E4M3_MAX)
    # value -> fields
    out = np.zeros(a.shape, dtype=np.int64)
    nz = r > 0
    rr = np.where(nz, r, 1.0)
    _, ex2 = np.frexp(rr)
    kk = ex2.astype(np.int64) - 1             # rr in [2^kk, 2^(kk+1))
    is_sub = rr < 2.0 ** (1 - E4M3_BIAS)
    mant_sub = np.rint(rr / 2.0 ** (1 - E4M3_BIAS - 3)).astype(np.int64)
    efield = kk + E4M3_BIAS
    mant_norm = np.rint((rr / np.ldexp(1.0, kk) - 1.0) * 8.0).astype(np.int64)
    bits = np.where(is_sub, mant_sub, (efield << 3) | mant_norm)
    out = np.where(nz, bits, 0)
    out = out | (neg.astype(np.int64) << 7)
    return out.astype(np.uint8)


def int4_pack(codes):
    """Pack signed 4-bit codes (..., D) in [-8, 7] into uint8 (..., (D+1)//2).

    byte j = (code[2j] mod 16) + 16 * (code[2j+1] mod 16); a missing odd
    channel counts as 0.
    """
    c = np.asarray(codes, dtype=np.int64)
    if c.size and (c.min() < -8 or c.max() > 7):
        raise ValueError("INT4 codes must lie in [-8, 7]")
    d = c.shape[-1]
    if d % 2:
        c = np.concatenate([c, np.zeros(c.shape[:-1] + (1,), np.int64)], axis=-1)
    lo = np.mod(c[..., 0::2], 16)
    hi = np.mod(c[..., 1::2], 16)
    return (lo + 16 * hi).astype(np.uint8)


def int4_unpack(packed, head_size):
    """Inverse of int4_pack: uint8 (..., C) -> int64 codes (..., head_size)."""
    b = np.asarray(packed, dtype=np.uint8).astype(np.int64)
    lo = b % 16
    hi = b // 16
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), dtype=np.int64)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out[..., :head_size]


def cache_head_size(head_size, kv_format):
    """Bytes per (token, kv head) row: (head_size+1)//2 for INT4, else head_size
    (P1, section 2)."""
    return (head_size + 1) // 2 if kv_format == "int4" else head_size
