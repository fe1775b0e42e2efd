"""The four large workloads at full size, in the launch configuration the
bench times (same workload builders, same num_splits), against the oracle on
sampled outputs.

For each sampled (row, head) the oracle quantizes that row's sequence itself
(past and new keys/values, oracle quantizer), checks that the cache bytes the
GPU wrote for that sequence are the same, then computes the output row from
its own cache (every other sequence's slots left poisoned).  Properties that
hold at any size are checked on the whole output: every element finite, and
no row written past token_count (NaN canaries).
"""

import numpy as np
import pytest
import torch

import workloads
from oracle import attention, quant
from tests import compare
from tests.gpu_cases import Device
from tests.oracle_cases import POISON, f32

pytestmark = pytest.mark.gpu


def _sequence_codes(w, b):
    """Oracle codes (L, Hkv, C) of sequence b's keys and values, positions 0..L-1."""
    p0, p1 = int(w.cum_past[b]), int(w.cum_past[b + 1])
    r0, r1 = int(w.cum_q[b]), int(w.cum_q[b + 1])
    k = np.concatenate([f32(w.past_key[p0:p1]), f32(w.new_key[r0:r1])])
    v = np.concatenate([f32(w.past_value[p0:p1]), f32(w.new_value[r0:r1])])
    hkv, D = w.kv_num_heads, w.head_size
    ks = quant.expand_scale(w.k_scale, hkv, D).astype(np.float32)
    vs = quant.expand_scale(w.v_scale, hkv, D).astype(np.float32)
    kc = quant.encode_rows(quant.quantize(k, ks[None], w.kv_format), w.kv_format)
    vc = quant.encode_rows(quant.quantize(v, vs[None], w.kv_format), w.kv_format)
    return kc, vc


def _slots(w, b, L):
    bs = w.block_size
    t = np.arange(L)
    return w.block_table[b][t // bs], t % bs


def _samples(w, rng, n):
    """Sampled (row, head) pairs: first and last row of the longest and the
    shortest active sequence, then random rows; heads spread over kv groups."""
    act = [b for b in range(w.batch) if w.q_lens[b] > 0]
    kv = w.past_lens + w.q_lens
    pick = [max(act, key=lambda b: kv[b]), min(act, key=lambda b: kv[b])]
    rows = []
    for b in pick:
        rows += [int(w.cum_q[b]), int(w.cum_q[b + 1]) - 1]
    while len(rows) < n:
        rows.append(int(rng.integers(0, w.token_count)))
    heads = [int(rng.integers(0, w.num_heads)) for _ in rows]
    heads[0], heads[1] = 0, w.num_heads - 1
    return sorted(set(zip(rows, heads)))


@pytest.mark.parametrize("name,n", [("int8_decode", 8), ("int4_long", 6), ("int8_prefill", 10),
                                    ("fp8_prefill", 8)])
def test_full_size_sampled_rows(name, n):
    print("case full-size", name, flush=True)
    w = workloads.make(name)
    g = Device(w).fill()
    out = g.attend()                     # the workload's own num_splits, as benched
    got = out.float().cpu().numpy()
    assert np.isfinite(got).all(), "non-finite outputs"
    gkc, gvc = g.kc.cpu().numpy(), g.vc.cpu().numpy()
    del g
    torch.cuda.empty_cache()
    rng = np.random.default_rng(2024)
    samples = _samples(w, rng, n)
    shape = gkc.shape
    q32 = f32(w.query)
    refs, gots = [], []
    done = {}
    for row, head in samples:
        b = int(np.searchsorted(w.cum_q, row, side="right") - 1)
        L = int(w.past_lens[b] + w.q_lens[b])
        if b not in done:
            kc_b, vc_b = _sequence_codes(w, b)
            blk, off = _slots(w, b, L)
            assert np.array_equal(gkc[blk, off], kc_b), "%s: key cache of sequence %d" % (name, b)
            assert np.array_equal(gvc[blk, off], vc_b), "%s: value cache of sequence %d" % (name, b)
            okc = np.full(shape, POISON, np.uint8)
            ovc = np.full(shape, POISON, np.uint8)
            okc[blk, off] = kc_b
            ovc[blk, off] = vc_b
            done = {b: (okc, ovc)}                  # keep one sequence's cache at a time
        okc, ovc = done[b]
        ref = attention.attention_row(q32, okc, ovc, w.k_scale, w.v_scale,
                                      w.block_table, w.cum_q, w.past_lens, w.kv_format, row, head)
        refs.append(ref)
        gots.append(got[row, head])
        print("  row %d head %d (sequence %d, %d keys)" % (row, head, b, L), flush=True)
    compare.check(np.array(gots), np.array(refs), w.q_dtype, name)
