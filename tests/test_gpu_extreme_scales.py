"""Key scales far outside the 16-bit ranges, on the GPU vs the fp64 oracle.

The kernels fold the per-channel key scale into the query after dividing by
the power of two M_h = 2^e >= max|k_scale| of the kv head ("ONNX Runtime: INT4
Paged KV Cache", section 3), with e capped at 127 so M_h is finite for every
finite scale, and keep raw scores (query' . codes) apart from the score factor
softmax_scale * M_h, which they clamp into the finite fp32 range.  Every
exponent is formed from a raw-score difference to the running maximum, so
nothing overflows: this is the kernels' own automatic switch to safe
arithmetic for scales the 16-bit path cannot take directly (the same page,
reviewer-feedback section, asks for a safe fallback and for stability tests
at FLT_MAX-like scales).  The cases:

* "channel": per-channel scales log-uniform over [2^-60, 2^100];
* "head": per-head scales 2^100, 2^-60, 1, 6e4;
* "mid": per-head scales that put the maxima of the log2 scores between
  ~2^22 and ~2^40, where the fast exponent form hands over to the safe one;
* "fltmax": per-channel scales log-uniform over the whole positive fp32
  range, subnormals included, with one channel of every kv head at FLT_MAX;
* "fltmax_head": per-head scales FLT_MAX, 2^-149 (the smallest subnormal),
  2^-126 and 3e38.

The first three append keys drawn as codes times scales (fp32 inputs); the
FLT_MAX cases write uniformly drawn codes straight into both caches (keys of
|code| * FLT_MAX do not exist in fp32, and the append is tested elsewhere).
Value scales stay ordinary so that the outputs fit the query dtype.

Near ties.  With logits this large the softmax is a hard argmax, and two keys
whose logits differ by less than the kernel's own rounding error are equally
valid answers.  The error of a computed score is bounded, key by key, by
    delta_j = eps * A_j + eta * softmax_scale * M_h * sum_d |c_jd|,
with A_j = softmax_scale * sum_d |q_d k_jd| (the sum of the magnitudes of
the score's terms) and c the codes.  eps collects every relative rounding on
the way (see EPS below); eta the absolute floor of a subnormal fp16 fold.
A row's candidate keys are those within delta_top + delta_j + T of the
top logit, T = ln(keys * max|v| / (tol * max|ref|)) (past that, a key's
weight stays below the tolerance's share even if every score is off by its
full bound).  If a row has several candidates and their bounds exceed 1e-4,
its output must be a convex combination of their values (elementwise within
their range, up to the usual tolerance); every other row meets the
element-wise rule.
"""

import dataclasses
import math
import zlib

import numpy as np
import pytest
import torch

import attention_paged_quantized_amd as paq
import workloads
from oracle import attention as oatt
from oracle import quant
from tests import compare
from tests.gpu_cases import Device, desc_for
from tests.oracle_cases import oracle_attention, oracle_caches

pytestmark = pytest.mark.gpu

SIGMA = {"int8": 40.0, "int4": 2.0, "fp8": 100.0}
FLT_MAX = float(np.finfo(np.float32).max)
U = 2.0 ** -24                       # unit roundoff of fp32

# Relative error bounds of a computed score, per kernel path:
# * MFMA decode: the fold q * s / M split into fp16 hi + lo keeps 22 bits
#   (2^-22); the score is one chain of 2 * D/32 = 8 16x16x32 products, each
#   counted as at most log2(32) + 1 = 6 fp32 roundings of a sum of its terms'
#   magnitudes; the score factor, the running maximum and the exponent's
#   fused multiply-add add 3 more.
# * MFMA prefill: one fp16 rounding of the fold (2^-11) for per-channel
#   scales, none for per-head scales (f16/bf16 queries and codes are exact
#   operands); D/16 = 8 32x32x16 products of at most log2(16) + 1 = 5
#   roundings; 3 more as above.
# * fp32 kernel: the fold's fp32 rounding, D sequential fused multiply-adds,
#   3 more.
EPS = {
    "mfma_decode": 2.0 ** -22 + (8 * 6 + 3) * U,
    "mfma_prefill_channel": 2.0 ** -11 + (8 * 5 + 3) * U,
    "mfma_prefill_head": (8 * 5 + 3) * U,
    "f32": (1 + 128 + 3) * U,
}
ETA = {"mfma_decode": 2.0 ** -25, "mfma_prefill_channel": 2.0 ** -25, "mfma_prefill_head": 0.0,
       "f32": 2.0 ** -150}


def _scales(rng, hkv, D, mode):
    if mode == "channel":
        return np.exp2(rng.uniform(-60.0, 100.0, (hkv, D))).astype(np.float32)
    if mode == "mid":
        # maxima of the log2 scores between ~2^22 and ~2^40: where an fp32
        # running maximum has an ulp of 1 to 2^17, so the exponent of an fp16
        # P must be formed from exact differences to it
        return np.array([2.0 ** 14, 2.0 ** 20, 2.0 ** 26, 2.0 ** 32][:hkv], np.float32)
    if mode == "head":
        return np.array([2.0 ** 100, 2.0 ** -60, 1.0, 6e4][:hkv], np.float32)
    if mode == "fltmax":
        s = np.exp2(rng.uniform(-149.0, 128.0, (hkv, D)))
        s = np.minimum(s, FLT_MAX).astype(np.float32)
        s[:, int(rng.integers(0, D))] = FLT_MAX
        return np.maximum(s, np.float32(2.0 ** -149))
    if mode == "fltmax_head":
        return np.array([FLT_MAX, 2.0 ** -149, 2.0 ** -126, 3e38][:hkv], np.float32)
    raise ValueError(mode)


def _scale_mode(mode):
    return "channel" if mode in ("channel", "fltmax") else "head"


def _kernel_path(w):
    if w.q_dtype == "f32":
        return "f32"
    if w.kind == "decode":
        return "mfma_decode"
    return "mfma_prefill_channel" if w.scale_mode == "channel" else "mfma_prefill_head"


def _direct_caches(w, rng):
    """Pools (poisoned like the oracle's) holding uniformly drawn codes at
    every position the workload's sequences use."""
    shape = (w.num_blocks, w.block_size, w.kv_num_heads, w.cache_head_size)
    kc = np.full(shape, 0x7F, np.uint8)
    vc = np.full(shape, 0x7F, np.uint8)

    def codes(n):
        if w.kv_format == "fp8":
            c = rng.integers(0, 256, (n, w.kv_num_heads, w.head_size))
            c[(c & 0x7F) == 0x7F] = 0x38                 # no NaN codes (0x38 = 1.0)
            return c.astype(np.uint8)
        m = 127 if w.kv_format == "int8" else 7
        return quant.encode_rows(rng.integers(-m, m + 1, (n, w.kv_num_heads, w.head_size)),
                                 w.kv_format)

    bs = w.block_size
    for b in range(w.batch):
        L = int(w.past_lens[b] + w.q_lens[b])
        t = np.arange(L)
        blk = w.block_table[b][t // bs]
        kc[blk, t % bs] = codes(L)
        vc[blk, t % bs] = codes(L)
    return kc, vc


def _candidates(w, kc, vc, ref):
    """(row, head) -> values of the row's candidate keys when the row is a
    near tie within the kernel's error bound (see the module docstring)."""
    q = w.query.to(dtype=torch.float64).numpy()
    H, D = w.num_heads, w.head_size
    G = H // w.kv_num_heads
    sigma = oatt.default_scale(D)
    path = _kernel_path(w)
    eps, eta = EPS[path], ETA[path]
    tol = compare.TOL[w.q_dtype]
    ref_max = np.abs(ref).max()
    ks = quant.expand_scale(w.k_scale, w.kv_num_heads, D)
    Mh = np.exp2(np.minimum(np.ceil(np.log2(np.abs(ks).max(axis=1))), 127.0))
    out = {}
    for b in range(w.batch):
        r0, r1 = int(w.cum_q[b]), int(w.cum_q[b + 1])
        if r1 == r0:
            continue
        past = int(w.past_lens[b])
        L = past + (r1 - r0)
        rows = oatt.gather_rows(kc, w.block_table[b], L)
        c = quant.decode_rows(rows, w.kv_format, D)                     # codes (L, Hkv, D)
        k = c * ks[None]
        v = oatt.sequence_kv(vc, w.kv_format, w.v_scale, w.block_table[b], L, D)
        for i in range(r1 - r0):
            n = past + i + 1
            for h in range(H):
                g = h // G
                terms = k[:n, g] * q[r0 + i, h][None]
                s = sigma * terms.sum(axis=1)
                A = sigma * np.abs(terms).sum(axis=1)
                delta = eps * A + eta * sigma * Mh[g] * np.abs(c[:n, g]).sum(axis=1)
                top = int(np.argmax(s))
                vmax = np.abs(v[:n, g]).max()
                T = math.log(n / tol) + max(0.0, math.log(max(vmax, 1e-300) / ref_max))
                cand = np.nonzero(s[top] - s <= delta[top] + delta + T)[0]
                if len(cand) > 1 and delta[cand].max() > 1e-4:
                    out[(r0 + i, h)] = v[cand, g]
    return out


def _check(w, got, kc, vc, ref):
    assert np.isfinite(got).all(), "non-finite outputs"
    tol = compare.TOL[w.q_dtype] * np.abs(ref).max()
    got = got.copy()
    n_ties = 0
    for (r, h), cand in _candidates(w, kc, vc, ref).items():
        lo = cand.min(axis=0) - tol - compare.ulp(cand.min(axis=0), w.q_dtype)
        hi = cand.max(axis=0) + tol + compare.ulp(cand.max(axis=0), w.q_dtype)
        assert ((got[r, h] >= lo) & (got[r, h] <= hi)).all(), (w.name, r, h)
        got[r, h] = ref[r, h]                       # checked above
        n_ties += 1
    print("  %s: %d near-tie rows checked as convex combinations" % (w.name, n_ties), flush=True)
    return compare.check(got, ref, w.q_dtype, w.name)


def _run(w, splits=None):
    if w.notes.get("direct"):
        rng = np.random.default_rng(zlib.crc32(w.name.encode()) + 1)
        kc, vc = _direct_caches(w, rng)
        g = Device(w)
        g.kc.copy_(torch.from_numpy(kc))
        g.vc.copy_(torch.from_numpy(vc))
    else:
        g = Device(w).fill()
        kc, vc = oracle_caches(w)
        assert (g.kc.cpu().numpy() == kc).all(), "key cache differs from the oracle"
    out = g.attend(num_splits=splits)
    ref = oracle_attention(w, kc, vc)
    return _check(w, out.float().cpu().numpy(), kc, vc, ref)


def _workload(name, fmt, qdt, mode, kind, splits, past, qlen):
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    ks = _scales(rng, 4, 128, mode)
    direct = mode.startswith("fltmax")
    w = workloads.custom(name, 41 if kind == "decode" else 43, batch=3, num_heads=16,
                         kv_num_heads=4, head_size=128, block_size=16, past=past, q_lens=qlen,
                         q_dtype=qdt, kv_format=fmt, scale_mode=_scale_mode(mode),
                         kv_in_dtype="f32", num_splits=splits, kind=kind,
                         key_scale=None if direct else ks, key_code_sigma=SIGMA[fmt])
    if direct:
        w = dataclasses.replace(w, k_scale=ks, notes={"direct": True})
    return w


MODES = ["channel", "head", "mid", "fltmax", "fltmax_head"]


@pytest.mark.parametrize("fmt", ["int8", "int4", "fp8"])
@pytest.mark.parametrize("qdt", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("splits", [1, 4, -5])
def test_decode_extreme_key_scales(fmt, qdt, mode, splits):
    name = "ext_dec_%s_%s_%s_s%d" % (fmt, qdt, mode, splits)
    print("case", name, flush=True)
    w = _workload(name, fmt, qdt, mode, "decode", splits, np.array([90, 0, 33]),
                  np.ones(3, np.int32))
    _run(w)


@pytest.mark.parametrize("fmt", ["int8", "int4", "fp8"])
@pytest.mark.parametrize("qdt", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("mode", MODES)
def test_prefill_extreme_key_scales(fmt, qdt, mode):
    name = "ext_pf_%s_%s_%s" % (fmt, qdt, mode)
    print("case", name, flush=True)
    w = _workload(name, fmt, qdt, mode, "prefill", 1, np.array([0, 40, 7]),
                  np.array([70, 9, 0]))
    _run(w)
