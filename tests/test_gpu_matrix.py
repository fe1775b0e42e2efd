"""Decode and prefill on the GPU vs the fp64 oracle across the format space:
KV format (INT8, packed INT4, FP8 E4M3) x query dtype (fp16, bf16) x head size
(64, 128) x scale mode (per channel, per kv head), plus GQA group sizes, kv
head counts that change how many heads one decode wave serves, block sizes and
the length edge cases (empty sequences, a single key, block boundaries).

Every case is small enough for the oracle to finish in well under a second,
and long enough to span several key tiles with a ragged tail.
"""

import itertools

import numpy as np
import pytest

import workloads
from tests import compare
from tests.gpu_cases import Device
from tests.oracle_cases import oracle_attention, oracle_caches

pytestmark = pytest.mark.gpu

FORMATS = ["int8", "int4", "fp8"]
QDT = ["f16", "bf16"]
HEADS = [64, 128]
MODES = ["channel", "head"]


def _run(w, splits=None):
    g = Device(w).fill()
    out = g.attend(num_splits=splits)
    kc, vc = oracle_caches(w)
    # the cache the GPU wrote must be the oracle's, byte for byte
    assert (g.kc.cpu().numpy() == kc).all(), "key cache differs from the oracle"
    assert (g.vc.cpu().numpy() == vc).all(), "value cache differs from the oracle"
    ref = oracle_attention(w, kc, vc)
    return compare.check(out.float().cpu().numpy(), ref, w.q_dtype, w.name)


@pytest.mark.parametrize("fmt,qdt,D,mode",
                         list(itertools.product(FORMATS, QDT, HEADS, MODES)))
@pytest.mark.parametrize("splits", [1, 5, -7])
def test_decode_formats(fmt, qdt, D, mode, splits):
    name = "dec_%s_%s_d%d_%s_s%d" % (fmt, qdt, D, mode, splits)
    print("case", name, flush=True)
    # lengths: one key only, a block boundary either side, a q_len-0 sequence,
    # and a longer ragged one
    past = np.array([0, 15, 16, 200, 90, 47])
    qlen = np.array([1, 1, 1, 1, 0, 1])
    seed = 11 + 7 * FORMATS.index(fmt) + 3 * QDT.index(qdt) + D + MODES.index(mode) + \
        (splits < 0)
    w = workloads.custom(name, seed, batch=6, num_heads=16, kv_num_heads=4, head_size=D,
                         block_size=16, past=past, q_lens=qlen, q_dtype=qdt, kv_format=fmt,
                         scale_mode=mode, num_splits=splits)
    _run(w)


@pytest.mark.parametrize("fmt,qdt,D,mode",
                         list(itertools.product(FORMATS, QDT, HEADS, MODES)))
def test_prefill_formats(fmt, qdt, D, mode):
    name = "pf_%s_%s_d%d_%s" % (fmt, qdt, D, mode)
    print("case", name, flush=True)
    # ragged new-token counts (one empty), pasts from 0 across block edges
    past = np.array([0, 37, 16, 5, 0])
    qlen = np.array([70, 1, 0, 33, 3])
    seed = 101 + 7 * FORMATS.index(fmt) + 3 * QDT.index(qdt) + D + MODES.index(mode)
    w = workloads.custom(name, seed, batch=5, num_heads=8, kv_num_heads=2, head_size=D,
                         block_size=16, past=past, q_lens=qlen, q_dtype=qdt, kv_format=fmt,
                         scale_mode=mode, kind="prefill")
    _run(w)


@pytest.mark.parametrize("H,Hkv", [(4, 4), (16, 2), (12, 3), (8, 1)])
@pytest.mark.parametrize("fmt,D", [("int8", 128), ("int4", 128), ("int4", 64), ("int8", 64)])
@pytest.mark.parametrize("splits", [1, 3])
def test_decode_head_layouts(H, Hkv, fmt, D, splits):
    """GQA groups 1..8 and kv head counts 1..4: one decode wave serves 128/row
    bytes adjacent kv heads when the count allows, fewer otherwise."""
    name = "dec_heads_%d_%d_%s_d%d_s%d" % (H, Hkv, fmt, D, splits)
    print("case", name, flush=True)
    past = np.array([100, 33, 64])
    w = workloads.custom(name, 5 + H + Hkv + D, batch=3, num_heads=H, kv_num_heads=Hkv,
                         head_size=D, block_size=32, past=past, q_lens=np.ones(3, np.int32),
                         q_dtype="f16", kv_format=fmt, num_splits=splits)
    _run(w)


@pytest.mark.parametrize("bs", [16, 32, 64, 128])
@pytest.mark.parametrize("kind", ["decode", "prefill"])
def test_block_sizes(bs, kind):
    name = "bs%d_%s" % (bs, kind)
    print("case", name, flush=True)
    if kind == "decode":
        past, qlen = np.array([300, 127, 128, 0]), np.ones(4, np.int32)
    else:
        past, qlen = np.array([0, 129, 64, 7]), np.array([100, 20, 0, 64])
    w = workloads.custom(name, 900 + bs, batch=4, num_heads=8, kv_num_heads=2, head_size=128,
                         block_size=bs, past=past, q_lens=qlen, q_dtype="f16",
                         kv_format="int8", kind=kind)
    _run(w)


@pytest.mark.parametrize("G", [1, 2, 8, 16])
def test_prefill_groups(G):
    name = "pf_group%d" % G
    print("case", name, flush=True)
    hkv = 2
    w = workloads.custom(name, 300 + G, batch=3, num_heads=G * hkv, kv_num_heads=hkv,
                         head_size=128, block_size=16, past=np.array([10, 0, 65]),
                         q_lens=np.array([40, 17, 9]), q_dtype="f16", kv_format="int8",
                         kind="prefill")
    _run(w)


def test_decode_many_splits_empty_chunks():
    """More chunks than blocks: most chunks are empty (lse = -inf)."""
    print("case many splits", flush=True)
    w = workloads.custom("dec_empty_chunks", 77, batch=3, num_heads=8, kv_num_heads=2,
                         head_size=128, block_size=16, past=np.array([20, 0, 70]),
                         q_lens=np.ones(3, np.int32), q_dtype="f16", kv_format="int4",
                         num_splits=40)
    _run(w)
