"""Pins for oracle.quant: the quantizers against closed forms (exact for
power-of-two scales), exact rational arithmetic (Fractions) for the fp32
quotient, exhaustive sweeps over every finite fp16 and bf16 input, and the
append step's slot mapping against a contiguous layout."""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import codecs, quant, attention


def _all_finite(dtype):
    bits = torch.arange(0, 1 << 16, dtype=torch.int32).to(torch.int16)
    v = bits.view(dtype).to(torch.float32).numpy()
    return v[np.isfinite(v)]


ALL_F16 = _all_finite(torch.float16)
ALL_BF16 = _all_finite(torch.bfloat16)


@pytest.mark.parametrize("fmt,qmax", [("int8", 127), ("int4", 7)])
@pytest.mark.parametrize("src", ["f16", "bf16"])
def test_integer_quantizer_power_of_two_scales_exhaustive(fmt, qmax, src):
    xs = ALL_F16 if src == "f16" else ALL_BF16
    if src == "bf16":
        xs = xs[np.abs(xs) < 1e30]      # keep x / 2^k inside fp32 for k < 0
    for k in (-3, 0, 2, 5):
        s = np.float32(2.0 ** k)
        got = quant.quantize(xs, s, fmt)
        # closed form: x / 2^k is exact, Python's round() is half-to-even
        expect = [max(-qmax, min(qmax, round(float(x) / 2.0 ** k))) for x in xs]
        assert np.array_equal(got, np.array(expect)), (fmt, src, k)


def _correctly_rounded_f32(num, den):
    """Check helper: the float32 nearest to num/den (ties to even), by exact
    rational comparison of the two neighbouring float32 candidates."""
    q = Fraction(num) / Fraction(den)
    c = np.float32(float(q))
    cands = {c, np.nextafter(c, np.float32(np.inf)), np.nextafter(c, np.float32(-np.inf))}
    best = sorted(cands, key=lambda f: (abs(Fraction(float(f)) - q),
                                       int(np.array(f).view(np.int32)) & 1))
    return best[0]


def test_fp32_quotient_is_correctly_rounded():
    rng = np.random.default_rng(3)
    x = rng.choice(ALL_F16, 4000).astype(np.float32)
    s = np.exp(rng.uniform(np.log(1e-3), np.log(6e4), 4000)).astype(np.float32)
    got = quant.fl32_quotient(x, s)
    for xi, si, gi in zip(x, s, got):
        assert gi == _correctly_rounded_f32(float(xi), float(si)), (xi, si, gi)


@pytest.mark.parametrize("fmt,qmax", [("int8", 127), ("int4", 7)])
def test_integer_quantizer_properties_general_scales(fmt, qmax):
    xs = np.sort(ALL_F16)
    for s in (np.float32(1e-3), np.float32(6e4), np.float32(0.0173), np.float32(3.7)):
        c = quant.quantize(xs, s, fmt)
        assert np.all(np.diff(c) >= 0)                                 # monotone
        neg = quant.quantize(-xs, s, fmt)
        assert np.array_equal(neg, -c)                                 # odd symmetry
        y = xs.astype(np.float64) / float(s)
        inside = np.abs(y) <= qmax
        # nearest code to the fp32 quotient: within 1/2 plus one fp32 rounding of y
        assert np.all(np.abs(y[inside] - c[inside]) <= 0.5 + np.abs(y[inside]) * 2.0 ** -23)
        assert np.all(np.abs(c) <= qmax)
        assert np.all(c[y > qmax + 0.5] == qmax) and np.all(c[y < -qmax - 0.5] == -qmax)


def test_fp8_quantizer_exhaustive_f16():
    for k in (-4, 0, 3):
        s = np.float32(2.0 ** k)
        got = quant.quantize(ALL_F16, s, "fp8")
        y = (ALL_F16.astype(np.float64) / 2.0 ** k).astype(np.float32)    # exact
        ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        inr = np.abs(y) <= 464.0
        assert np.array_equal(got[inr], ref[inr])
        big = ~inr
        assert np.all(got[big] == np.where(y[big] > 0, 0x7E, 0xFE))


def test_dequantize_per_channel_and_per_head():
    rng = np.random.default_rng(5)
    codes = rng.integers(-127, 128, (3, 2, 4))
    stored = quant.encode_rows(codes, "int8")
    sc = np.array([[1, 2, 3, 4], [5, 6, 7, 8]], np.float32)
    deq = quant.dequantize(stored, "int8", sc, 4)
    for t in range(3):
        for h in range(2):
            for d in range(4):
                assert deq[t, h, d] == codes[t, h, d] * sc[h, d]
    sh = np.array([0.5, 4.0], np.float32)
    deq = quant.dequantize(stored, "int8", sh, 4)
    assert np.array_equal(deq, codes * np.array([0.5, 4.0])[None, :, None])


def _poisoned(nb, bs, hkv, c):
    return np.full((nb, bs, hkv, c), 0x7F, dtype=np.uint8)


@pytest.mark.parametrize("fmt", ["int8", "int4", "fp8"])
def test_append_matches_contiguous_layout_and_touches_nothing_else(fmt):
    rng = np.random.default_rng(11)
    B, hkv, D, bs = 3, 2, 6, 4
    lens = [5, 0, 9]
    nb = sum(-(-L // bs) for L in lens) + 3
    perm = rng.permutation(nb)
    table = np.full((B, 4), -1, np.int64)
    pos = 0
    for b, L in enumerate(lens):
        n = -(-L // bs)
        table[b, :n] = perm[pos:pos + n]
        pos += n
    C = codecs.cache_head_size(D, fmt)
    cum = np.concatenate([[0], np.cumsum(lens)])
    x = (rng.standard_normal((cum[-1], hkv, D)) * 3).astype(np.float32)
    sc = np.full((hkv, D), 0.05, np.float32)
    k0 = _poisoned(nb, bs, hkv, C)
    kc, vc = quant.quant_append(k0, k0, x, -x, sc, sc, table, cum, [0, 0, 0], fmt)
    rows = quant.encode_rows(quant.quantize(x, sc[None], fmt), fmt)
    touched = np.zeros(kc.shape[:2], bool)
    for b, L in enumerate(lens):
        got = attention.gather_rows(kc, table[b], L)
        assert np.array_equal(got, rows[cum[b]:cum[b + 1]])
        for t in range(L):
            touched[table[b, t // bs], t % bs] = True
    assert np.all(kc[~touched] == 0x7F) and np.all(vc[~touched] == 0x7F)


def test_append_in_two_steps_equals_one_step():
    rng = np.random.default_rng(12)
    hkv, D, bs = 2, 8, 4
    table = np.array([[3, 0, 5, -1], [1, 4, 2, -1]])
    x = rng.standard_normal((7 + 6, hkv, D)).astype(np.float32)
    sc = np.full((hkv,), 0.02, np.float32)
    z = _poisoned(6, bs, hkv, D)
    one, _ = quant.quant_append(z, z, x, x, sc, sc, table, [0, 7, 13], [0, 0], "fp8")
    # first 4 + 2 tokens, then the remaining 3 + 4
    a = np.concatenate([x[0:4], x[7:9]])
    b_ = np.concatenate([x[4:7], x[9:13]])
    s1, _ = quant.quant_append(z, z, a, a, sc, sc, table, [0, 4, 6], [0, 0], "fp8")
    s2, _ = quant.quant_append(s1, s1, b_, b_, sc, sc, table, [0, 3, 7], [4, 2], "fp8")
    assert np.array_equal(one, s2)
