"""Key scales far outside the 16-bit ranges, on the GPU vs the fp64 oracle.

The MFMA kernels fold the per-channel key scale into the fp16 query after
dividing by the power of two M_h >= max|k_scale| of the kv head ("ONNX Runtime:
INT4 Paged KV Cache", section 3), so no fp16 operand can overflow whatever the
scales; the score factor softmax_scale * M_h stays in fp32.  These cases put
per-channel scales log-uniformly over [2^-60, 2^100] (and per-head scales at
the same extremes, and at the intermediate magnitudes where the running
maximum's own rounding reaches whole powers of two), with keys drawn as codes
times scales in fp32, and require
the usual tolerance and finite outputs.  Value scales stay ordinary so that the
outputs fit the query dtype.
"""

import zlib

import numpy as np
import pytest

import workloads
from tests import compare
from tests.gpu_cases import Device
from tests.oracle_cases import oracle_attention, oracle_caches

pytestmark = pytest.mark.gpu

SIGMA = {"int8": 40.0, "int4": 2.0, "fp8": 100.0}


def _scales(rng, hkv, D, mode):
    if mode == "channel":
        return np.exp2(rng.uniform(-60.0, 100.0, (hkv, D))).astype(np.float32)
    if mode == "mid":
        # maxima of the log2 scores between ~2^22 and ~2^40: where an fp32
        # running maximum has an ulp of 1 to 2^17, so the exponent of an fp16
        # P must be formed from exact differences to it
        return np.array([2.0 ** 14, 2.0 ** 20, 2.0 ** 26, 2.0 ** 32][:hkv], np.float32)
    return np.array([2.0 ** 100, 2.0 ** -60, 1.0, 6e4][:hkv], np.float32)


def _scale_mode(mode):
    return "channel" if mode == "channel" else "head"


def _near_ties(w, kc, vc, rel=2.0 ** -17):
    """For every (query row, head): the keys whose fp64 logit lies within
    rel * |max logit| of the maximum.  With logits this large (|s| up to
    ~1e31) the softmax is a hard argmax, and two keys closer than the fp32
    resolution of the scores are equally valid answers for a kernel that
    computes them in fp32."""
    from oracle import attention as oatt
    q = w.query.to(dtype=__import__("torch").float64).numpy()
    H, D = w.num_heads, w.head_size
    G = H // w.kv_num_heads
    sigma = oatt.default_scale(D)
    ties = {}
    for b in range(w.batch):
        r0, r1 = int(w.cum_q[b]), int(w.cum_q[b + 1])
        if r1 == r0:
            continue
        past = int(w.past_lens[b])
        L = past + (r1 - r0)
        k = oatt.sequence_kv(kc, w.kv_format, w.k_scale, w.block_table[b], L, D)
        v = oatt.sequence_kv(vc, w.kv_format, w.v_scale, w.block_table[b], L, D)
        for i in range(r1 - r0):
            for h in range(H):
                s = sigma * (k[: past + i + 1, h // G] @ q[r0 + i, h])
                m = s.max()
                cand = np.nonzero(s >= m - rel * abs(m))[0]
                ties[(r0 + i, h)] = v[cand, h // G]
    return ties


def _run(w, splits=None):
    g = Device(w).fill()
    out = g.attend(num_splits=splits)
    kc, vc = oracle_caches(w)
    assert (g.kc.cpu().numpy() == kc).all(), "key cache differs from the oracle"
    ref = oracle_attention(w, kc, vc)
    got = out.float().cpu().numpy()
    assert np.isfinite(got).all()
    # rows whose top logits tie within fp32 resolution: the output must be a
    # convex combination of the tied keys' values (elementwise within their
    # range, up to the usual tolerance); elsewhere the element-wise rule holds
    tol = compare.TOL[w.q_dtype] * np.abs(ref).max()
    for (r, h), cand in _near_ties(w, kc, vc).items():
        if len(cand) > 1:
            lo = cand.min(axis=0) - tol - compare.ulp(cand.min(axis=0), w.q_dtype)
            hi = cand.max(axis=0) + tol + compare.ulp(cand.max(axis=0), w.q_dtype)
            assert ((got[r, h] >= lo) & (got[r, h] <= hi)).all(), (w.name, r, h)
            got[r, h] = ref[r, h]                       # checked above
    return compare.check(got, ref, w.q_dtype, w.name)


@pytest.mark.parametrize("fmt", ["int8", "int4", "fp8"])
@pytest.mark.parametrize("qdt", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("mode", ["channel", "head", "mid"])
@pytest.mark.parametrize("splits", [1, 4])
def test_decode_extreme_key_scales(fmt, qdt, mode, splits):
    name = "ext_dec_%s_%s_%s_s%d" % (fmt, qdt, mode, splits)
    print("case", name, flush=True)
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    w = workloads.custom(name, 41, batch=3, num_heads=16, kv_num_heads=4, head_size=128,
                         block_size=16, past=np.array([90, 0, 33]),
                         q_lens=np.ones(3, np.int32), q_dtype=qdt, kv_format=fmt,
                         scale_mode=_scale_mode(mode), kv_in_dtype="f32", num_splits=splits,
                         key_scale=_scales(rng, 4, 128, mode), key_code_sigma=SIGMA[fmt])
    _run(w)


@pytest.mark.parametrize("fmt", ["int8", "int4", "fp8"])
@pytest.mark.parametrize("qdt", ["f16", "bf16"])
@pytest.mark.parametrize("mode", ["channel", "head", "mid"])
def test_prefill_extreme_key_scales(fmt, qdt, mode):
    name = "ext_pf_%s_%s_%s" % (fmt, qdt, mode)
    print("case", name, flush=True)
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    w = workloads.custom(name, 43, batch=3, num_heads=16, kv_num_heads=4, head_size=128,
                         block_size=16, past=np.array([0, 40, 7]), q_lens=np.array([70, 9, 0]),
                         q_dtype=qdt, kv_format=fmt, scale_mode=_scale_mode(mode), kv_in_dtype="f32",
                         kind="prefill", key_scale=_scales(rng, 4, 128, mode),
                         key_code_sigma=SIGMA[fmt])
    _run(w)
