"""Pins for oracle.codecs: E4M3 and packed INT4, checked against the OCP
specification's listed values, torch's float8_e4m3fn casts (a library special
case), exhaustive enumeration and closed forms."""

import math
import os

import numpy as np
import pytest
import torch

from oracle import codecs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_e4m3():
    rows = []
    with open(os.path.join(GOLDEN, "e4m3_spec_values.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            c, v = line.split()
            rows.append((int(c, 16), float(v)))
    return rows


def test_e4m3_spec_values():
    for code, val in _golden_e4m3():
        got = codecs.e4m3_decode(np.uint8(code))
        if math.isnan(val):
            assert np.isnan(got)
        else:
            assert got == val and math.copysign(1, got) == math.copysign(1, val), (code, got)


def test_e4m3_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = codecs.e4m3_decode(codes)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])
    assert np.array_equal(np.signbit(ref[ok]), np.signbit(got[ok]))


def test_e4m3_positive_codes_strictly_increase():
    v = codecs.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    assert np.all(np.diff(v) > 0)
    assert v[-1] == 448.0


def test_e4m3_roundtrip_every_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = codecs.e4m3_decode(codes).astype(np.float32)
    assert np.array_equal(codecs.e4m3_encode(vals), codes)


def test_e4m3_midpoints_round_to_even():
    v = codecs.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = ((v[:-1] + v[1:]) / 2).astype(np.float32)
    assert np.array_equal(mids.astype(np.float64), (v[:-1] + v[1:]) / 2)  # exact in fp32
    enc = codecs.e4m3_encode(mids).astype(np.int64)
    lo = np.arange(0x7E)
    expect = np.where(lo % 2 == 0, lo, lo + 1)
    assert np.array_equal(enc, expect)
    assert np.array_equal(codecs.e4m3_encode(-mids).astype(np.int64), expect | 0x80)


def test_e4m3_encode_matches_torch_in_range():
    rng = np.random.default_rng(7)
    mags = np.exp(rng.uniform(np.log(1e-5), np.log(464.0), 200000))
    y = (mags * rng.choice([-1.0, 1.0], mags.size)).astype(np.float32)
    y = y[np.abs(y) <= 464.0]
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codecs.e4m3_encode(y), ref)


def test_e4m3_saturates_and_keeps_sign_of_zero():
    y = np.array([465.0, 1e6, np.inf, -500.0, -np.inf, 0.0, -0.0, -1e-30, 1e-30],
                 dtype=np.float32)
    got = codecs.e4m3_encode(y)
    assert list(got) == [0x7E, 0x7E, 0x7E, 0xFE, 0xFE, 0x00, 0x80, 0x80, 0x00]


def test_int4_roundtrip_all_pairs():
    lo, hi = np.meshgrid(np.arange(-8, 8), np.arange(-8, 8), indexing="ij")
    codes = np.stack([lo.ravel(), hi.ravel()], axis=1)
    packed = codecs.int4_pack(codes)
    assert packed.shape == (256, 1)
    assert np.array_equal(codecs.int4_unpack(packed, 2), codes)
    assert sorted(packed.ravel().tolist()) == list(range(256))


def test_int4_byte_layout_closed_form():
    b = np.arange(256, dtype=np.uint8).reshape(256, 1)
    codes = codecs.int4_unpack(b, 2)
    for byte, (lo, hi) in zip(range(256), codes):
        assert -8 <= lo <= 7 and -8 <= hi <= 7
        assert (lo % 16) + 16 * (hi % 16) == byte          # low nibble = channel 0
        assert lo == (byte & 0xF) - (16 if byte & 0x8 else 0)


def test_int4_odd_head_size_and_cache_head_size():
    codes = np.array([[1, -2, 3, -4, 5]])
    p = codecs.int4_pack(codes)
    assert p.shape == (1, 3) and p[0, 2] == 5            # high nibble of the last byte is 0
    assert np.array_equal(codecs.int4_unpack(p, 5), codes)
    assert codecs.cache_head_size(5, "int4") == 3
    assert codecs.cache_head_size(128, "int4") == 64
    assert codecs.cache_head_size(128, "int8") == 128
    assert codecs.cache_head_size(128, "fp8") == 128


def test_int4_rejects_out_of_range():
    with pytest.raises(ValueError):
        codecs.int4_pack(np.array([[8, 0]]))
