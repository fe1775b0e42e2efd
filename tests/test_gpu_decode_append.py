"""paged_attn_decode_append: the decode step's append and attention in one
call, on the GPU, against the two operations one after the other and the
fp64 oracle.

Two devices start from the same poisoned pools with the past tokens
appended.  One runs kv_quant_append of the step's new rows and then
paged_attn_decode; the other runs paged_attn_decode_append.  The caches must
be byte-equal (the fused quantizer is the append's arithmetic) and the
outputs bit-identical (the fused kernel reads the same code bytes: the wave
holding the new token's tile places its codes in the tile), and both match
the oracle.  The cases cover the three formats, both scale modes, head sizes
64 and 128 (one and two kv heads per wave), the single pass, block-aligned
chunks and the balanced partition, sequences without a new token, new tokens
at the first, middle and last row of a tile, the fp32 kernel's own fused
append (fp32 queries, groups beyond the MFMA decode's), the path that runs the
two operations separately (key rows in another dtype), and the whole
tiny_decode and int8_decode steps.
"""

import itertools

import numpy as np
import pytest
import torch

import attention_paged_quantized_amd as paq
import workloads
from tests import compare
from tests.gpu_cases import COUNTERS, TORCH_DT, Device, desc_for
from tests.oracle_cases import oracle_attention, oracle_caches

pytestmark = pytest.mark.gpu


def _both(w, splits):
    ref = Device(w)
    ref.append_past()
    fused = Device(w)
    fused.append_past()
    d = desc_for(w, w.token_count)
    nbytes = paq.paged_attn_decode_workspace_size(d, w.cum_q, w.past_lens, splits)
    outs = []
    for g, is_fused in ((ref, False), (fused, True)):
        ws = torch.zeros(max(1, nbytes // 4), dtype=torch.float32, device="cuda") \
            if nbytes else None
        out = torch.full((w.token_count, w.num_heads, w.head_size), float("nan"),
                         dtype=TORCH_DT[w.q_dtype], device="cuda")
        nk, nv = w.new_key.cuda(), w.new_value.cuda()
        if is_fused:
            paq.paged_attn_decode_append(d, w.kv_in_dtype, nk, nv, g.query, out, g.kc, g.vc,
                                         g.k_scale, g.v_scale, g.block_table, g.cum_q, g.past,
                                         w.cum_q, w.past_lens, 0.0, splits, ws)
        else:
            paq.kv_quant_append(d, w.kv_in_dtype, nk, nv, g.kc, g.vc, g.k_scale, g.v_scale,
                                g.block_table, g.cum_q, g.past, w.cum_q, w.past_lens)
            paq.paged_attn_decode(d, g.query, out, g.kc, g.vc, g.k_scale, g.v_scale,
                                  g.block_table, g.cum_q, g.past, w.cum_q, w.past_lens, 0.0,
                                  splits, ws)
        torch.cuda.synchronize()
        if ws is not None:
            assert not ws.view(torch.int32)[:COUNTERS].any(), "counters left non-zero"
        outs.append(out)
    assert torch.equal(ref.kc, fused.kc), "key cache differs from kv_quant_append's"
    assert torch.equal(ref.vc, fused.vc), "value cache differs from kv_quant_append's"
    assert torch.equal(outs[0], outs[1]), "fused output differs from append + decode"
    kc, vc = oracle_caches(w)
    assert (fused.kc.cpu().numpy() == kc).all(), "key cache differs from the oracle"
    out = outs[1]
    return compare.check(out.float().cpu().numpy(), oracle_attention(w, kc, vc), w.q_dtype,
                         w.name)


FORMATS = ["int8", "int4", "fp8"]


@pytest.mark.parametrize("fmt,D,mode,splits", list(itertools.product(
    FORMATS, [64, 128], ["channel", "head"], [1, 5, -7])))
def test_decode_append_matches_two_calls(fmt, D, mode, splits):
    name = "dapp_%s_d%d_%s_s%d" % (fmt, D, mode, splits)
    print("case", name, flush=True)
    # new tokens at tile rows 0, 31, 16, 5 (past % 32), a sequence without
    # one, a one-key sequence and a long one
    past = np.array([64, 95, 48, 700, 37, 0, 1500])
    qlen = np.array([1, 1, 1, 1, 0, 1, 1])
    w = workloads.custom(name, 3001 + 7 * FORMATS.index(fmt) + D + (mode == "head"),
                         batch=len(past), num_heads=16, kv_num_heads=4, head_size=D,
                         block_size=32 if fmt == "int4" else 16, past=past, q_lens=qlen,
                         q_dtype="bf16" if fmt == "fp8" else "f16", kv_format=fmt,
                         scale_mode=mode, num_splits=splits)
    _both(w, splits)


@pytest.mark.parametrize("fmt,D,mode,splits", list(itertools.product(
    FORMATS, [64, 128], ["channel", "head"], [1, 3])))
def test_decode_append_fp32_kernel(fmt, D, mode, splits):
    """fp32 queries take the fp32 kernel, which appends the new rows itself
    too (single pass, and split-KV with its combine)."""
    name = "dapp_f32_%s_d%d_%s_s%d" % (fmt, D, mode, splits)
    print("case", name, flush=True)
    w = workloads.custom(name, 3101 + 5 * FORMATS.index(fmt) + D + splits, batch=4, num_heads=8,
                         kv_num_heads=2, head_size=D, block_size=16,
                         past=np.array([40, 0, 300, 17]), q_lens=np.array([1, 1, 1, 0]),
                         q_dtype="f32", kv_format=fmt, scale_mode=mode, num_splits=splits)
    _both(w, splits)


def test_decode_append_fp32_kernel_large_group():
    """A 16-bit query with a GQA group of 12 takes the fp32 kernel (its
    16-query-head instance) with the append inside."""
    w = workloads.custom("dapp_g12", 3201, batch=3, num_heads=24, kv_num_heads=2,
                         head_size=128, block_size=16, past=np.array([63, 64, 500]),
                         q_lens=np.ones(3, np.int32), q_dtype="bf16", kv_format="int8",
                         num_splits=1)
    _both(w, 1)


@pytest.mark.parametrize("fmt,splits", list(itertools.product(FORMATS, [1, 6])))
def test_decode_append_fp32_rows(fmt, splits):
    """16-bit queries with fp32 new rows: the MFMA decode appends them itself."""
    name = "dapp_rows32_%s_s%d" % (fmt, splits)
    print("case", name, flush=True)
    w = workloads.custom(name, 3301 + 3 * FORMATS.index(fmt) + splits, batch=3, num_heads=8,
                         kv_num_heads=2, head_size=128, block_size=32 if fmt == "int4" else 16,
                         past=np.array([40, 0, 300]), q_lens=np.ones(3, np.int32),
                         q_dtype="bf16" if fmt == "fp8" else "f16", kv_format=fmt,
                         kv_in_dtype="f32", num_splits=splits)
    _both(w, splits)


def test_decode_append_two_launches():
    """fp32 queries with 16-bit new rows take the two operations one after the
    other: same results."""
    w = workloads.custom("dapp_sep", 3311, batch=3, num_heads=8, kv_num_heads=2,
                         head_size=128, block_size=16, past=np.array([40, 0, 300]),
                         q_lens=np.ones(3, np.int32), q_dtype="f32", kv_format="int8",
                         kv_in_dtype="f16", num_splits=1)
    _both(w, 1)


def test_decode_append_int4_long():
    """The whole int4_long step (fp32 new rows, 128 chunks)."""
    w = workloads.make("int4_long")
    _both(w, w.num_splits)


def test_decode_append_tiny_decode():
    """The tiny_decode step (fp32 queries, fp32 kernel)."""
    w = workloads.make("tiny_decode")
    _both(w, w.num_splits)


def test_decode_append_full_int8_decode():
    """The whole int8_decode step in the bench's configuration."""
    w = workloads.make("int8_decode")
    _both(w, w.num_splits)
