"""Pins for oracle.sparse: selecting every block is dense attention; any
selection equals dense attention over a cache re-packed (independently, here)
with only the selected blocks; a selected partial last block gives the
closed-form two-key softmax; the selection order does not matter."""

import numpy as np

import workloads
from oracle import attention, sparse
from tests.oracle_cases import f32, oracle_caches


def _w(seed=3, fmt="int8"):
    return workloads.custom("sp_pin", seed, batch=3, num_heads=8, kv_num_heads=2, head_size=64,
                            block_size=16, past=np.array([70, 0, 33]),
                            q_lens=np.array([1, 0, 1]), q_dtype="f32", kv_format=fmt)


def test_all_blocks_selected_is_dense():
    w = _w()
    kc, vc = oracle_caches(w)
    nb = -(-(w.past_lens + 1) // 16)
    sel = np.zeros((3, nb.max()), np.int32)
    for b in range(3):
        sel[b, :nb[b]] = np.arange(nb[b])
    got = sparse.block_sparse_decode(f32(w.query), kc, vc, w.k_scale, w.v_scale, w.block_table,
                                     w.cum_q, w.past_lens, w.kv_format, sel, nb)
    ref = attention.paged_attention(f32(w.query), kc, vc, w.k_scale, w.v_scale, w.block_table,
                                    w.cum_q, w.past_lens, w.kv_format)
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-13)


def test_selection_equals_dense_over_repacked_blocks():
    w = _w(5, "int4")
    kc, vc = oracle_caches(w)
    sel = np.array([[0, 2, 4], [0, 0, 0], [1, 2, 0]], np.int32)     # seq 0: blocks 0,2,4 (4 is partial)
    num = np.array([3, 0, 2], np.int32)
    got = sparse.block_sparse_decode(f32(w.query), kc, vc, w.k_scale, w.v_scale, w.block_table,
                                     w.cum_q, w.past_lens, w.kv_format, sel, num)
    # re-pack: a fresh cache holding only the selected blocks, in order, with
    # the partial last block last; dense attention over it
    for b, r in ((0, 0), (2, 1)):
        L = int(w.past_lens[b]) + 1
        blocks = [int(x) for x in sel[b, :num[b]]]
        nk = sum(min(16, L - 16 * x) for x in blocks)
        ck = np.stack([kc[w.block_table[b][x]] for x in blocks])
        cv = np.stack([vc[w.block_table[b][x]] for x in blocks])
        table = np.arange(len(blocks), dtype=np.int32)[None]
        ref = attention.paged_attention(f32(w.query)[r:r + 1], ck, cv, w.k_scale, w.v_scale, table,
                                        np.array([0, 1]), np.array([nk - 1]), w.kv_format)
        np.testing.assert_allclose(got[r], ref[0], rtol=1e-12, atol=1e-12)


def test_partial_last_block_alone_is_a_two_key_softmax():
    w = _w(7)
    kc, vc = oracle_caches(w)
    # sequence 2 has 34 keys; its last block (2) holds keys 32 and 33 only
    sel = np.zeros((3, 1), np.int32)
    num = np.array([1, 0, 1], np.int32)
    sel[2, 0] = 2                                            # keys 32, 33 of sequence 2
    got = sparse.block_sparse_decode(f32(w.query), kc, vc, w.k_scale, w.v_scale, w.block_table,
                                     w.cum_q, w.past_lens, w.kv_format, sel, num)
    V = attention.sequence_kv(vc, w.kv_format, w.v_scale, w.block_table[2], 34, 64)
    K = attention.sequence_kv(kc, w.kv_format, w.k_scale, w.block_table[2], 34, 64)
    q = f32(w.query)[1]
    for h in range(8):
        g = h // 4
        s = attention.default_scale(64) * (K[32:34, g] @ q[h])
        p = np.exp(s - s.max())
        np.testing.assert_allclose(got[1, h], (p[0] * V[32, g] + p[1] * V[33, g]) / p.sum(),
                                   rtol=1e-12)


def test_selection_order_does_not_matter():
    w = _w(9, "fp8")
    kc, vc = oracle_caches(w)
    a = np.array([[0, 3, 4], [0, 0, 0], [0, 2, 0]], np.int32)
    b = np.array([[4, 0, 3], [0, 0, 0], [2, 0, 0]], np.int32)
    num = np.array([3, 0, 2], np.int32)
    args = (f32(w.query), kc, vc, w.k_scale, w.v_scale, w.block_table, w.cum_q, w.past_lens,
            w.kv_format)
    np.testing.assert_allclose(sparse.block_sparse_decode(*args, a, num),
                               sparse.block_sparse_decode(*args, b, num), rtol=1e-13)


# ---- block-sparse prefill ----

def _wp(seed=11, fmt="int8"):
    # past 70 (block 4 shared by cached and new keys), 0 (no earlier block),
    # 48 (block-aligned), 0 new rows, 37
    return workloads.custom("spp_pin", seed, batch=5, num_heads=8, kv_num_heads=2, head_size=64,
                            block_size=16, past=np.array([70, 0, 48, 20, 37]),
                            q_lens=np.array([9, 5, 6, 0, 20]), q_dtype="f32", kv_format=fmt)


def _prefill(w, kc, vc, sel, num):
    return sparse.block_sparse_prefill(f32(w.query), kc, vc, w.k_scale, w.v_scale,
                                       w.block_table, w.cum_q, w.past_lens, w.kv_format, sel, num)


def test_prefill_every_earlier_block_selected_is_dense():
    w = _wp()
    kc, vc = oracle_caches(w)
    nfb = w.past_lens // 16
    sel = np.zeros((5, max(1, nfb.max())), np.int32)
    for b in range(5):
        sel[b, :nfb[b]] = np.arange(nfb[b])
    got = _prefill(w, kc, vc, sel, nfb)
    ref = attention.paged_attention(f32(w.query), kc, vc, w.k_scale, w.v_scale, w.block_table,
                                    w.cum_q, w.past_lens, w.kv_format)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


def test_prefill_equals_dense_over_repacked_blocks():
    w = _wp(13, "int4")
    kc, vc = oracle_caches(w)
    sel = np.array([[0, 3], [0, 0], [1, 0], [0, 0], [1, 0]], np.int32)
    num = np.array([2, 0, 1, 0, 1], np.int32)
    got = _prefill(w, kc, vc, sel, num)
    # re-pack (independently of the oracle's mask): selected blocks, then the
    # blocks holding new tokens; the chunk then starts at n * bs + past % bs
    # and dense causal prefill over the re-packed cache is the same attention
    for b in (0, 1, 2, 4):
        past, q = int(w.past_lens[b]), int(w.cum_q[b + 1] - w.cum_q[b])
        blocks = [int(x) for x in sel[b, :num[b]]] + list(range(past // 16, -(-(past + q) // 16)))
        ck = np.stack([kc[w.block_table[b][x]] for x in blocks])
        cv = np.stack([vc[w.block_table[b][x]] for x in blocks])
        table = np.arange(len(blocks), dtype=np.int32)[None]
        r0 = int(w.cum_q[b])
        ref = attention.paged_attention(f32(w.query)[r0:r0 + q], ck, cv, w.k_scale, w.v_scale,
                                        table, np.array([0, q]),
                                        np.array([int(num[b]) * 16 + past % 16]), w.kv_format)
        np.testing.assert_allclose(got[r0:r0 + q], ref, rtol=1e-12, atol=1e-13)


def test_prefill_first_row_alone_sees_its_own_key():
    # block-aligned past, nothing selected: row 0 sees only key `past`
    w = _wp(17, "fp8")
    kc, vc = oracle_caches(w)
    got = _prefill(w, kc, vc, np.zeros((5, 1), np.int32), np.zeros(5, np.int32))
    for b in (1, 2):
        past = int(w.past_lens[b])
        V = attention.sequence_kv(vc, w.kv_format, w.v_scale, w.block_table[b], past + 1, 64)
        for h in range(8):
            np.testing.assert_allclose(got[int(w.cum_q[b]), h], V[past, h // 4], rtol=1e-14)


def test_prefill_single_rows_match_the_sparse_decode():
    # one new row per sequence: the decode over the selection plus the
    # blocks holding the new token
    w = workloads.custom("spp_dec", 19, batch=3, num_heads=8, kv_num_heads=2, head_size=64,
                         block_size=16, past=np.array([70, 47, 33]), q_lens=np.array([1, 1, 1]),
                         q_dtype="f32", kv_format="int8")
    kc, vc = oracle_caches(w)
    sel = np.array([[1, 2], [0, 0], [1, 0]], np.int32)
    num = np.array([2, 0, 1], np.int32)
    got = _prefill(w, kc, vc, sel, num)
    dsel = np.zeros((3, 4), np.int32)
    dnum = np.zeros(3, np.int32)
    for b in range(3):
        past = int(w.past_lens[b])
        blocks = [int(x) for x in sel[b, :num[b]]] + list(range(past // 16, past // 16 + 1))
        dsel[b, :len(blocks)] = blocks
        dnum[b] = len(blocks)
    ref = sparse.block_sparse_decode(f32(w.query), kc, vc, w.k_scale, w.v_scale, w.block_table,
                                     w.cum_q, w.past_lens, w.kv_format, dsel, dnum)
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-14)


def test_prefill_ignores_unselected_blocks_only():
    w = _wp(23)
    kc, vc = oracle_caches(w)
    sel = np.array([[1, 0], [0, 0], [2, 0], [0, 0], [0, 0]], np.int32)
    num = np.array([1, 0, 1, 0, 0], np.int32)
    base = _prefill(w, kc, vc, sel, num)
    r0, r1 = int(w.cum_q[0]), int(w.cum_q[1])

    def poke(block, row):
        k2, v2 = kc.copy(), vc.copy()
        k2[w.block_table[0][block], row] ^= 0x15
        v2[w.block_table[0][block], row] ^= 0x15
        return _prefill(w, k2, v2, sel, num)[r0:r1]

    # sequence 0 (past 70): block 0 unselected -> no effect; block 1 selected
    # and block 4 (cached keys 64..69 beside the new ones) -> both matter
    np.testing.assert_array_equal(poke(0, 3), base[r0:r1])
    assert np.abs(poke(1, 3) - base[r0:r1]).max() > 1e-6
    assert np.abs(poke(4, 2) - base[r0:r1]).max() > 1e-6
