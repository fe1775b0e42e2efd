"""Pins for oracle.attention: brute force (pure-Python loops), torch's fp64
scaled_dot_product_attention as a library special case, closed forms, and the
invariants the pages rely on (paged == contiguous under any block
permutation, split-KV == single pass, GQA == MHA with repeated kv heads,
prefill rows == decodes, exact max_query_len)."""

import math
import os

import numpy as np
import pytest
import torch

import workloads
from oracle import attention, brute, quant
from tests.oracle_cases import oracle_caches, oracle_attention, f32

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _tiny(fmt, mode="channel", q_dtype="f32", G=2, D=8, bs=4, past=(5, 0, 9), ql=(1, 0, 3),
          seed=0):
    return workloads.custom("t", seed, batch=len(past), num_heads=2 * G, kv_num_heads=2,
                            head_size=D, block_size=bs, past=list(past), q_lens=list(ql),
                            q_dtype=q_dtype, kv_format=fmt, scale_mode=mode)


def _brute(w, kc, vc):
    return brute.paged_attention(
        f32(w.query).tolist(), kc.tolist(), vc.tolist(), w.k_scale.tolist(),
        w.v_scale.tolist(), w.block_table.tolist(), [int(c) for c in w.cum_q],
        [int(p) for p in w.past_lens], w.kv_format, w.num_heads, w.kv_num_heads,
        w.head_size, w.block_size)


@pytest.mark.parametrize("fmt,mode", [("int8", "channel"), ("int4", "channel"),
                                      ("fp8", "head"), ("int4", "head"), ("fp8", "channel")])
def test_vectorised_equals_brute_force(fmt, mode):
    w = _tiny(fmt, mode, D=7 if fmt == "int4" else 8)
    kc, vc = oracle_caches(w)
    out = oracle_attention(w, kc, vc)
    ref = _brute(w, kc, vc)
    assert len(ref) == w.token_count * w.num_heads
    for (r, h), o in ref.items():
        assert np.allclose(out[r, h], o, rtol=0, atol=1e-12 * max(1.0, np.abs(o).max()))


def test_tiny_decode_workload_brute_force():
    w = workloads.make("tiny_decode")
    kc, vc = oracle_caches(w)
    out = oracle_attention(w, kc, vc)
    ref = _brute(w, kc, vc)
    assert sorted(ref) == [(r, h) for r in range(2) for h in range(4)]
    for (r, h), o in ref.items():
        assert np.max(np.abs(out[r, h] - o)) <= 1e-12 * np.abs(o).max()


def _write_codes(codes, table, bs, nb):
    """Test-side scatter of INT8 codes (L, Hkv, D) into a paged cache."""
    L, hkv, D = codes.shape
    cache = np.full((nb, bs, hkv, D), 0x7F, np.uint8)
    for t in range(L):
        cache[table[t // bs], t % bs] = codes[t].astype(np.int8).view(np.uint8)
    return cache


def test_sdpa_library_special_case():
    """Integer-valued K/V with unit scales: paged oracle == torch fp64 SDPA on
    the contiguous tensors, with an explicit end-aligned causal mask and the
    kv heads repeated for GQA."""
    rng = np.random.default_rng(21)
    H, hkv, D, bs = 6, 2, 16, 4
    past, n = 10, 5
    L = past + n
    nb = 6
    table = rng.permutation(nb)
    kcodes = rng.integers(-3, 4, (L, hkv, D))
    vcodes = rng.integers(-50, 51, (L, hkv, D))
    kc, vc = _write_codes(kcodes, table, bs, nb), _write_codes(vcodes, table, bs, nb)
    q = rng.standard_normal((n, H, D))
    ones = np.ones((hkv, D), np.float32)
    out = attention.paged_attention(q, kc, vc, ones, ones, table[None], [0, n], [past], "int8")
    qt = torch.from_numpy(q).permute(1, 0, 2)                           # (H, n, D)
    kt = torch.from_numpy(kcodes.astype(np.float64)).permute(1, 0, 2).repeat_interleave(H // hkv, 0)
    vt = torch.from_numpy(vcodes.astype(np.float64)).permute(1, 0, 2).repeat_interleave(H // hkv, 0)
    mask = torch.arange(L)[None, :] <= (past + torch.arange(n))[:, None]
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask)
    assert np.allclose(out, ref.permute(1, 0, 2).numpy(), rtol=0, atol=1e-11)


@pytest.mark.parametrize("fmt", ["int8", "int4", "fp8"])
def test_single_key_returns_its_value(fmt):
    w = _tiny(fmt, "channel", past=(0,), ql=(1,), D=6)
    kc, vc = oracle_caches(w)
    out = oracle_attention(w, kc, vc)
    v = quant.dequantize(vc[w.block_table[0, 0], 0], fmt, w.v_scale, w.head_size)  # (Hkv, D)
    for h in range(w.num_heads):
        assert np.array_equal(out[0, h], v[h // (w.num_heads // w.kv_num_heads)])


def test_identical_keys_give_mean_of_values_and_rows_sum_to_one():
    rng = np.random.default_rng(4)
    hkv, D, bs, L = 1, 8, 4, 11
    table = np.array([2, 0, 1])
    kcodes = np.repeat(rng.integers(-20, 20, (1, hkv, D)), L, axis=0)
    vcodes = rng.integers(-100, 100, (L, hkv, D))
    kc, vc = _write_codes(kcodes, table, bs, 3), _write_codes(vcodes, table, bs, 3)
    sc = np.full((hkv, D), 0.25, np.float32)
    q = rng.standard_normal((1, 2, D))
    out = attention.paged_attention(q, kc, vc, sc, sc, table[None], [0, 1], [L - 1], "int8")
    assert np.allclose(out[0, 0], vcodes[:, 0].mean(axis=0) * 0.25, atol=1e-12)
    # value codes all 1 with unit scale: the output is the softmax row sum
    ones = _write_codes(np.ones((L, hkv, D), np.int64), table, bs, 3)
    kc2 = _write_codes(rng.integers(-120, 120, (L, hkv, D)), table, bs, 3)
    o1 = attention.paged_attention(q, kc2, ones, sc, np.ones((hkv, D), np.float32),
                                   table[None], [0, 1], [L - 1], "int8")
    assert np.all(np.abs(o1 - 1.0) <= 1e-12)


def test_dominant_logit_selects_its_value():
    rng = np.random.default_rng(8)
    hkv, D, bs, L = 1, 4, 4, 9
    table = np.array([1, 2, 0])
    kcodes = np.zeros((L, hkv, D), np.int64)
    kcodes[6] = 127
    vcodes = rng.integers(-100, 100, (L, hkv, D))
    kc, vc = _write_codes(kcodes, table, bs, 3), _write_codes(vcodes, table, bs, 3)
    q = np.full((1, 1, D), 1.0)
    sc = np.ones((hkv, D), np.float32)
    out = attention.paged_attention(q, kc, vc, sc, sc, table[None], [0, 1], [L - 1], "int8",
                                    softmax_scale=1.0)
    assert np.allclose(out[0, 0], vcodes[6, 0], atol=1e-100)


@pytest.mark.parametrize("fmt", ["int8", "int4", "fp8"])
def test_block_permutation_invariance(fmt):
    w = _tiny(fmt, past=(13, 6, 2), ql=(2, 1, 4), seed=3)
    kc, vc = oracle_caches(w)
    out = oracle_attention(w, kc, vc)
    rng = np.random.default_rng(99)
    perm = rng.permutation(w.num_blocks)           # new id of physical block i
    kc2, vc2 = np.empty_like(kc), np.empty_like(vc)
    kc2[perm], vc2[perm] = kc, vc
    bt2 = np.where(w.block_table >= 0, perm[np.maximum(w.block_table, 0)], -1)
    out2 = attention.paged_attention(f32(w.query), kc2, vc2, w.k_scale, w.v_scale, bt2,
                                     w.cum_q, w.past_lens, fmt)
    assert np.array_equal(out, out2)


@pytest.mark.parametrize("splits", [1, 2, 7, 128])
def test_split_kv_equals_single_pass(splits):
    w = _tiny("int8", past=(40, 3, 0, 17), ql=(1, 1, 1, 2), bs=4, seed=5)
    kc, vc = oracle_caches(w)
    one = oracle_attention(w, kc, vc)
    sp = oracle_attention(w, kc, vc, num_splits=splits)
    assert np.max(np.abs(one - sp)) <= 1e-12 * np.abs(one).max()


def test_chunk_partition_is_balanced_and_covers():
    for nb, S in [(1025, 128), (7, 3), (3, 7), (1, 1)]:
        r = attention.chunk_block_ranges(nb, S)
        assert r[0][0] == 0 and r[-1][1] == nb
        assert all(a[1] == b[0] for a, b in zip(r, r[1:]))
        sizes = [b - a for a, b in r]
        assert max(sizes) - min(sizes) <= 1
    assert sorted(b - a for a, b in attention.chunk_block_ranges(1025, 128)) == [8] * 127 + [9]


def test_gqa_equals_mha_with_repeated_kv_heads():
    w = _tiny("int8", G=3, past=(9, 4), ql=(2, 1), seed=6)
    kc, vc = oracle_caches(w)
    out = oracle_attention(w, kc, vc)
    G = w.num_heads // w.kv_num_heads
    kc_m = np.repeat(kc, G, axis=2)
    vc_m = np.repeat(vc, G, axis=2)
    out_m = attention.paged_attention(f32(w.query), kc_m, vc_m, np.repeat(w.k_scale, G, 0),
                                      np.repeat(w.v_scale, G, 0), w.block_table, w.cum_q,
                                      w.past_lens, "int8")
    assert np.array_equal(out, out_m)


def test_prefill_rows_equal_decodes():
    w = _tiny("fp8", "head", past=(7,), ql=(5,), seed=9)
    kc, vc = oracle_caches(w)
    out = oracle_attention(w, kc, vc)
    q = f32(w.query)
    for i in range(5):
        d = attention.paged_attention(q[i:i + 1], kc, vc, w.k_scale, w.v_scale, w.block_table,
                                      [0, 1], [7 + i], "fp8")
        assert np.allclose(d[0], out[i], rtol=0, atol=1e-13)   # BLAS order may differ
        for h in range(w.num_heads):
            r = attention.attention_row(q, kc, vc, w.k_scale, w.v_scale, w.block_table,
                                        w.cum_q, w.past_lens, "fp8", i, h)
            assert np.allclose(r, out[i, h], rtol=0, atol=1e-13)


def test_zero_token_sequences_produce_no_rows_and_do_not_disturb_others():
    w = _tiny("int8", past=(5, 8, 3), ql=(2, 0, 1), seed=10)
    kc, vc = oracle_caches(w)
    out = oracle_attention(w, kc, vc)
    assert out.shape[0] == 3
    keep = [0, 2]
    out2 = attention.paged_attention(f32(w.query), kc, vc, w.k_scale, w.v_scale,
                                     w.block_table[keep], [0, 2, 3], w.past_lens[keep], "int8")
    assert np.array_equal(out, out2)


def test_max_query_len_golden_and_brute_force():
    with open(os.path.join(GOLDEN, "max_query_len_cases.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            ql, exact, heur = [x.strip() for x in line.split(";")]
            ql = [int(x) for x in ql.split(",")]
            cum = np.concatenate([[0], np.cumsum(ql)])
            assert attention.max_query_len(cum) == int(exact)
            assert attention.heuristic_max_query_len(int(cum[-1]), len(ql)) == int(heur)
    rng = np.random.default_rng(2)
    for _ in range(200):
        ql = rng.integers(0, 6, rng.integers(1, 9))
        cum = np.concatenate([[0], np.cumsum(ql)])
        assert attention.max_query_len(cum) == max(ql)
    assert attention.max_query_len([0]) == 0


def test_combine_handles_empty_chunks():
    o = np.array([[1.0, 2.0]])
    e = np.zeros((1, 2))
    out, lse = attention.combine_partials([e, o, e], [np.array([-np.inf]), np.array([0.3]),
                                                      np.array([-np.inf])])
    assert np.array_equal(out, o) and lse[0] == 0.3
    out, lse = attention.combine_partials([e, e], [np.array([-np.inf])] * 2)
    assert np.all(out == 0) and lse[0] == -np.inf
    # two equal-weight chunks average, and lse adds log 2
    out, lse = attention.combine_partials([o, 3 * o], [np.array([1.0]), np.array([1.0])])
    assert np.allclose(out, 2 * o) and math.isclose(lse[0], 1.0 + math.log(2))
