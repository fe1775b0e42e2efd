"""Pins for oracle.rotary: the fp64 rotation against complex multiplication
(numpy's complex arithmetic), its invariants (pair norms, dependence of
rotated dot products on relative position only, the group law of angles),
the interleaved and half layouts against each other under a channel
permutation, and the fp32 rounding contract against exact rational
arithmetic and hand-computed worked values; the position map and the fused
append against brute-force enumeration and the pinned quantize-append step;
the bf16 rounding against PyTorch's conversion."""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import attention, quant, rotary


def _tables(max_pos, rotary_dim, base=10000.0):
    """Standard RoPE angle tables in fp64: angle(p, k) = p * base^(-2k/rd)."""
    k = np.arange(rotary_dim // 2)
    theta = base ** (-2.0 * k / rotary_dim)
    ang = np.arange(max_pos)[:, None] * theta[None, :]
    return np.cos(ang), np.sin(ang)


@pytest.mark.parametrize("interleaved", [False, True])
@pytest.mark.parametrize("rd", [16, 64, 128])
def test_rotation_is_complex_multiplication(interleaved, rd):
    rng = np.random.default_rng(rd + interleaved)
    D, T, heads = 128, 7, 3
    x = rng.standard_normal((T, heads, D))
    cos, sin = _tables(50, rd)
    pos = rng.integers(0, 50, T)
    got = rotary.rotate(x, pos, cos, sin, rd, interleaved)
    half = rd // 2
    for r in range(T):
        for k in range(half):
            i, j = (2 * k, 2 * k + 1) if interleaved else (k, k + half)
            z = (x[r, :, i] + 1j * x[r, :, j]) * np.exp(1j * np.arctan2(sin[pos[r], k],
                                                                          cos[pos[r], k]))
            np.testing.assert_allclose(got[r, :, i], z.real, rtol=0, atol=1e-13)
            np.testing.assert_allclose(got[r, :, j], z.imag, rtol=0, atol=1e-13)
    # channels past rotary_dim pass through untouched
    assert np.array_equal(got[..., rd:], x[..., rd:])


def test_direction_on_unit_vectors():
    """e_x rotated by a quarter turn is e_y; e_y goes to -e_x."""
    x = np.zeros((1, 1, 2))
    x[0, 0, 0] = 1.0
    c, s = np.array([[0.0]]), np.array([[1.0]])
    got = rotary.rotate(x, np.array([0]), c, s, 2, False)
    assert got[0, 0].tolist() == [0.0, 1.0]
    x = np.zeros((1, 1, 2))
    x[0, 0, 1] = 1.0
    got = rotary.rotate(x, np.array([0]), c, s, 2, True)
    assert got[0, 0].tolist() == [-1.0, 0.0]


@pytest.mark.parametrize("interleaved", [False, True])
def test_pair_norms_preserved(interleaved):
    rng = np.random.default_rng(5)
    x = rng.standard_normal((9, 4, 64))
    cos, sin = _tables(100, 64)
    pos = rng.integers(0, 100, 9)
    y = rotary.rotate(x, pos, cos, sin, 64, interleaved)
    f, s = rotary.pair_channels(64, interleaved)
    np.testing.assert_allclose(x[..., f] ** 2 + x[..., s] ** 2, y[..., f] ** 2 + y[..., s] ** 2,
                               rtol=1e-13)


@pytest.mark.parametrize("interleaved", [False, True])
def test_dot_products_depend_on_relative_position_only(interleaved):
    rng = np.random.default_rng(6)
    q = rng.standard_normal((1, 1, 128))
    k = rng.standard_normal((1, 1, 128))
    cos, sin = _tables(4096, 128)
    rot = lambda v, p: rotary.rotate(v, np.array([p]), cos, sin, 128, interleaved)[0, 0]
    for m, n in [(5, 2), (100, 37), (7, 7)]:
        ref = rot(q, m) @ rot(k, n)
        for shift in (1, 13, 2000):
            np.testing.assert_allclose(rot(q, m + shift) @ rot(k, n + shift), ref, rtol=1e-10,
                                       atol=1e-10)


def test_angles_compose():
    """Rotating by the angles of position a, then of position b, equals
    rotating by those of a + b (standard tables are linear in the position)."""
    rng = np.random.default_rng(7)
    x = rng.standard_normal((1, 2, 64))
    cos, sin = _tables(64, 64)
    a = rotary.rotate(x, np.array([11]), cos, sin, 64, False)
    ab = rotary.rotate(a, np.array([20]), cos, sin, 64, False)
    np.testing.assert_allclose(ab, rotary.rotate(x, np.array([31]), cos, sin, 64, False),
                               atol=1e-12)


def test_interleaved_and_half_layouts_agree_under_permutation():
    rng = np.random.default_rng(8)
    rd, D = 32, 64
    xh = rng.standard_normal((3, 2, D))
    perm = np.arange(D)                           # interleaved channel -> half channel
    perm[0:rd:2] = np.arange(rd // 2)
    perm[1:rd:2] = np.arange(rd // 2) + rd // 2
    xi = xh[..., perm]
    cos, sin = _tables(10, rd)
    pos = np.array([0, 3, 9])
    np.testing.assert_array_equal(rotary.rotate(xi, pos, cos, sin, rd, True),
                                  rotary.rotate(xh, pos, cos, sin, rd, False)[..., perm])
    np.testing.assert_array_equal(
        rotary.rotate_fp32(xi.astype(np.float32), pos, cos, sin, rd, True),
        rotary.rotate_fp32(xh.astype(np.float32), pos, cos, sin, rd, False)[..., perm])


def _rn32(q):
    """The float32 nearest to the rational q (ties to even)."""
    c = np.float32(float(q))
    cands = {c, np.nextafter(c, np.float32(np.inf)), np.nextafter(c, np.float32(-np.inf))}
    return sorted(cands, key=lambda f: (abs(Fraction(float(f)) - q),
                                        int(np.array(f).view(np.int32)) & 1))[0]


@pytest.mark.parametrize("interleaved", [False, True])
def test_fp32_contract_against_exact_rationals(interleaved):
    rng = np.random.default_rng(9)
    rd = 16
    x = (rng.standard_normal((6, 2, rd)) * np.exp2(rng.integers(-20, 20, (6, 2, rd)))
         ).astype(np.float32)
    cos, sin = _tables(40, rd)
    cos, sin = cos.astype(np.float32), sin.astype(np.float32)
    pos = rng.integers(0, 40, 6)
    got = rotary.rotate_fp32(x, pos, cos, sin, rd, interleaved)
    f, s = rotary.pair_channels(rd, interleaved)
    for r in range(6):
        for h in range(2):
            for k in range(rd // 2):
                a, b = Fraction(float(x[r, h, f[k]])), Fraction(float(x[r, h, s[k]]))
                c, sn = Fraction(float(cos[pos[r], k])), Fraction(float(sin[pos[r], k]))
                ac, bs = Fraction(float(_rn32(a * c))), Fraction(float(_rn32(b * sn)))
                bc, as_ = Fraction(float(_rn32(b * c))), Fraction(float(_rn32(a * sn)))
                assert got[r, h, f[k]] == _rn32(ac - bs)
                assert got[r, h, s[k]] == _rn32(bc + as_)


def test_fp32_contract_worked_values_and_no_fused_rounding():
    # exactly representable: (3, 5) at cos 0.5, sin 0.25 -> (0.25, 3.25)
    x = np.array([[[3.0, 5.0]]], np.float32)
    got = rotary.rotate_fp32(x, np.array([0]), np.array([[0.5]]), np.array([[0.25]]), 2, False)
    assert got[0, 0].tolist() == [0.25, 3.25]
    # a case where a fused multiply-add would differ: x c rounds, y s = x c
    # exactly in fp32 after rounding, so the two-rounding result is exactly 0
    a = np.float32(1.0 + 2.0 ** -12)
    c = np.float32(1.0 + 2.0 ** -12)           # a*c = 1 + 2^-11 + 2^-24: rounds to 1 + 2^-11
    y = np.float32(1.0 + 2.0 ** -11)
    sn = np.float32(1.0)
    x = np.array([[[a, y]]], np.float32)
    got = rotary.rotate_fp32(x, np.array([0]), np.array([[c]]), np.array([[sn]]), 2, False)
    assert got[0, 0, 0] == 0.0                 # fma(a, c, -y) would give 2^-24
    assert got[0, 0, 0] == np.float32(a * c) - np.float32(y * sn)   # numpy's own fp32 ops


def test_fp32_within_rounding_bound_of_fp64():
    rng = np.random.default_rng(10)
    x = rng.standard_normal((20, 4, 128)).astype(np.float32)
    cos, sin = _tables(3000, 128)
    cos32, sin32 = cos.astype(np.float32), sin.astype(np.float32)
    pos = rng.integers(0, 3000, 20)
    y32 = rotary.rotate_fp32(x, pos, cos32, sin32, 128, False).astype(np.float64)
    y64 = rotary.rotate(x, pos, cos32, sin32, 128, False)
    f, s = rotary.pair_channels(128, False)
    c = cos32.astype(np.float64)[pos][:, None, :]
    sn = sin32.astype(np.float64)[pos][:, None, :]
    mag = np.abs(x[..., f] * c) + np.abs(x[..., s] * sn)
    bound = 2.0 ** -23 * mag * 1.5
    assert np.all(np.abs(y32[..., f] - y64[..., f]) <= bound)
    mag = np.abs(x[..., s] * c) + np.abs(x[..., f] * sn)
    assert np.all(np.abs(y32[..., s] - y64[..., s]) <= 2.0 ** -23 * mag * 1.5)


def test_zero_position_identity_and_passthrough_fp32():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((4, 2, 64)).astype(np.float32)
    cos, sin = np.ones((1, 16), np.float32), np.zeros((1, 16), np.float32)
    got = rotary.rotate_fp32(x, np.zeros(4, np.int64), cos, sin, 32, False)
    assert np.array_equal(got, x)


def test_positions_brute_force_with_zero_token_sequences():
    cum_q = np.array([0, 3, 3, 4, 4, 9], np.int32)          # sequences 1 and 3 empty
    past = np.array([10, 99, 0, 7, 2], np.int32)
    pos = rotary.positions(cum_q, past)
    expect = []
    for b in range(5):
        expect += [int(past[b]) + i for i in range(int(cum_q[b + 1] - cum_q[b]))]
    assert pos.tolist() == expect == [10, 11, 12, 0, 2, 3, 4, 5, 6]
    # with zero-token sequences the heuristic token_count - batch + 1 falls
    # below the longest sequence: a grid sized by it would drop rows
    cum_q2 = np.array([0, 0, 0, 6], np.int32)
    assert attention.heuristic_max_query_len(6, 3) < attention.max_query_len(cum_q2)


@pytest.mark.parametrize("fmt", ["int8", "int4", "fp8"])
def test_fused_append_is_rotation_then_append(fmt):
    rng = np.random.default_rng(12)
    H, Hkv, D, bs, rd = 4, 2, 64, 16, 32
    cum_q = np.array([0, 5, 5, 8], np.int32)
    past = np.array([3, 40, 0], np.int32)
    bt = np.array([[0, 1, 2, 3], [4, 5, 6, 7], [8, 9, 10, 11]], np.int32)
    C = (D + 1) // 2 if fmt == "int4" else D
    kc0 = np.full((12, bs, Hkv, C), 0x7F, np.uint8)
    vc0 = kc0.copy()
    q = rng.standard_normal((8, H, D)).astype(np.float32)
    k = rng.standard_normal((8, Hkv, D)).astype(np.float32)
    v = rng.standard_normal((8, Hkv, D)).astype(np.float32)
    ks = np.full((Hkv, D), 0.02, np.float32)
    vs = np.full((Hkv, D), 0.03, np.float32)
    cos, sin = _tables(64, rd)
    kc, vc, qr = rotary.rotary_append(kc0, vc0, q, k, v, ks, vs, bt, cum_q, past, fmt, cos, sin,
                                      rd, False, "f16")
    # brute force: rotate each row at its own position, then the pinned append
    kr = np.empty_like(k)
    qq = np.empty_like(q)
    # sequence 0: rows 0..4 at positions 3..7; sequence 1 empty; sequence 2:
    # rows 5..7 at positions 0..2
    for r, p in [(0, 3), (1, 4), (2, 5), (3, 6), (4, 7), (5, 0), (6, 1), (7, 2)]:
        kr[r] = rotary.rotate_fp32(k[r:r + 1], np.array([p]), cos, sin, rd, False)[0]
        qq[r] = rotary.rotate_fp32(q[r:r + 1], np.array([p]), cos, sin, rd, False)[0]
    ekc, evc = quant.quant_append(kc0, vc0, kr, v, ks, vs, bt, cum_q, past, fmt)
    assert np.array_equal(kc, ekc) and np.array_equal(vc, evc)
    assert np.array_equal(qr, qq.astype(np.float16).astype(np.float32))


def test_bf16_rounding_matches_pytorch():
    rng = np.random.default_rng(13)
    x = np.concatenate([rng.standard_normal(20000).astype(np.float32) *
                        np.exp2(rng.integers(-60, 60, 20000)).astype(np.float32),
                        np.array([0.0, -0.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8,
                                  3.0e38, -1.0e-40], np.float32)])
    got = rotary.round_to_dtype(x, "bf16")
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
