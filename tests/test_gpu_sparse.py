"""Block-sparse decode on the GPU (paged_attn_decode_sparse) vs the oracle's
block_sparse_decode: formats x query dtypes x single pass / split-KV, with
local-window + strided selections, every block, a lone partial last block,
and sequences without a new row."""

import numpy as np
import pytest
import torch

import attention_paged_quantized_amd as paq
import workloads
from oracle import sparse
from tests import compare
from tests.gpu_cases import Device, desc_for
from tests.oracle_cases import f32, oracle_caches

pytestmark = pytest.mark.gpu


def selection(w, pattern, rng):
    """Ascending selected logical blocks per sequence (and counts)."""
    nb = -(-(w.past_lens + 1) // w.block_size)
    rows = []
    for b in range(w.batch):
        n = int(nb[b])
        if pattern == "all":
            s = list(range(n))
        elif pattern == "last":
            s = [n - 1]
        else:                        # local window of 2 blocks + every 3rd earlier block
            s = sorted(set(list(range(max(0, n - 2), n)) + list(range(0, n, 3))))
            if pattern == "random":
                s = sorted(set(rng.choice(n, max(1, n // 2), replace=False).tolist()))
        rows.append(s)
    m = max(len(r) for r in rows)
    sel = np.zeros((w.batch, m), np.int32)
    num = np.array([len(r) for r in rows], np.int32)
    for b, r in enumerate(rows):
        sel[b, :len(r)] = r
    return sel, num


def _run(w, pattern, splits, seed=0):
    rng = np.random.default_rng(seed)
    sel, num = selection(w, pattern, rng)
    g = Device(w).fill()
    desc = desc_for(w, w.token_count)
    nbytes = paq.paged_attn_decode_sparse_workspace_size(desc, w.cum_q, w.past_lens, num,
                                                         sel.shape[1], splits)
    ws = torch.zeros(nbytes // 4 + 1, dtype=torch.float32, device="cuda")
    out = torch.full_like(g.query, float("nan"))
    paq.paged_attn_decode_sparse(desc, g.query, out, g.kc, g.vc, g.k_scale, g.v_scale,
                                 g.block_table, g.cum_q, g.past, w.cum_q, w.past_lens,
                                 torch.from_numpy(sel).cuda(), torch.from_numpy(num).cuda(), num,
                                 0.0, splits, ws)
    torch.cuda.synchronize()
    kc, vc = oracle_caches(w)
    ref = sparse.block_sparse_decode(f32(w.query), kc, vc, w.k_scale, w.v_scale, w.block_table,
                                     w.cum_q, w.past_lens, w.kv_format, sel, num)
    compare.check(out.float().cpu().numpy(), ref, w.q_dtype, w.name)


@pytest.mark.parametrize("fmt", ["int8", "int4", "fp8"])
@pytest.mark.parametrize("qdt", ["f16", "bf16"])
@pytest.mark.parametrize("splits", [1, 4])
@pytest.mark.parametrize("pattern", ["window", "random"])
def test_sparse_decode(fmt, qdt, splits, pattern):
    name = "sp_%s_%s_s%d_%s" % (fmt, qdt, splits, pattern)
    print("case", name, flush=True)
    w = workloads.custom(name, 41 + splits, batch=5, num_heads=16, kv_num_heads=4,
                         head_size=128, block_size=16, past=np.array([300, 15, 0, 90, 129]),
                         q_lens=np.array([1, 1, 1, 0, 1]), q_dtype=qdt, kv_format=fmt,
                         scale_mode="head" if fmt == "fp8" else "channel")
    _run(w, pattern, splits, seed=7)


@pytest.mark.parametrize("pattern", ["all", "last"])
def test_sparse_decode_all_and_last_block(pattern):
    print("case sparse", pattern, flush=True)
    w = workloads.custom("sp_" + pattern, 9, batch=3, num_heads=8, kv_num_heads=2, head_size=64,
                         block_size=32, past=np.array([100, 31, 64]),
                         q_lens=np.ones(3, np.int32), q_dtype="f16", kv_format="int4")
    _run(w, pattern, 0)


def test_sparse_decode_full_size_window():
    """int8_decode shape (32 sequences of 1k-4k keys) with the window+strided
    selection, single pass as benched for the dense decode."""
    print("case sparse full", flush=True)
    w = workloads.make("int8_decode")
    _run(w, "window", 1)


# ---- block-sparse prefill (paged_attn_prefill_sparse vs block_sparse_prefill) ----

def prefill_selection(w, pattern, rng):
    """Ascending selected earlier blocks (each below past // block_size)."""
    nfb = w.past_lens // w.block_size
    rows = []
    for b in range(w.batch):
        n = int(nfb[b])
        if pattern == "all":
            s = list(range(n))
        elif pattern == "window":        # the 2 blocks before the local ones + every 3rd
            s = sorted(set(list(range(max(0, n - 2), n)) + list(range(0, n, 3))))
        else:                            # random half
            s = sorted(rng.choice(n, n // 2, replace=False).tolist()) if n else []
        rows.append(s)
    m = max(1, max(len(r) for r in rows))
    sel = np.zeros((w.batch, m), np.int32)
    num = np.array([len(r) for r in rows], np.int32)
    for b, r in enumerate(rows):
        sel[b, :len(r)] = r
    return sel, num


def _run_prefill(w, pattern, seed=0, seqs=None):
    rng = np.random.default_rng(seed)
    if pattern == "none":
        sel, num = None, np.zeros(w.batch, np.int32)
    else:
        sel, num = prefill_selection(w, pattern, rng)
    max_sel = 0 if sel is None else sel.shape[1]
    g = Device(w).fill()
    desc = desc_for(w, w.token_count)
    nbytes = paq.paged_attn_prefill_sparse_workspace_size(desc, w.cum_q, w.past_lens, num,
                                                          max_sel)
    ws = torch.zeros(nbytes // 4 + 1, dtype=torch.float32, device="cuda")
    out = torch.full_like(g.query, float("nan"))
    dsel = None if sel is None else torch.from_numpy(sel).cuda()
    dnum = None if sel is None else torch.from_numpy(num).cuda()
    paq.paged_attn_prefill_sparse(desc, g.query, out, g.kc, g.vc, g.k_scale, g.v_scale,
                                  g.block_table, g.cum_q, g.past, w.cum_q, w.past_lens, dsel,
                                  dnum, num, 0.0, ws)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    kc, vc = oracle_caches(w)
    osel = np.zeros((w.batch, 1), np.int32) if sel is None else sel
    seqs = range(w.batch) if seqs is None else seqs
    # the oracle per sequence (sequences are independent): the sampled ones
    rows = np.concatenate([np.arange(w.cum_q[b], w.cum_q[b + 1]) for b in seqs]).astype(int)
    qlen = np.array([w.cum_q[b + 1] - w.cum_q[b] for b in seqs])
    cum = np.concatenate([[0], np.cumsum(qlen)]).astype(np.int32)
    ref = sparse.block_sparse_prefill(f32(w.query)[rows], kc, vc, w.k_scale, w.v_scale,
                                      w.block_table[list(seqs)], cum, w.past_lens[list(seqs)],
                                      w.kv_format, osel[list(seqs)], num[list(seqs)])
    compare.check(got[rows], ref, w.q_dtype, w.name)
    if len(rows) == got.shape[0]:
        return
    assert np.all(np.isfinite(got)), "non-finite rows outside the sample"


def _wp(fmt, qdt, D, seed):
    return workloads.custom("sparse_prefill", seed, batch=6, num_heads=32, kv_num_heads=8,
                            head_size=D, block_size=16,
                            past=np.array([70, 0, 48, 20, 37, 300]),
                            q_lens=np.array([9, 5, 40, 0, 70, 33]), q_dtype=qdt,
                            kv_format=fmt, kind="prefill",
                            scale_mode="head" if fmt == "fp8" else "channel")


@pytest.mark.parametrize("fmt", ["int8", "int4", "fp8"])
@pytest.mark.parametrize("qdt", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("pattern", ["window", "random", "none"])
def test_sparse_prefill(fmt, qdt, pattern):
    print("case sparse prefill", fmt, qdt, pattern, flush=True)
    _run_prefill(_wp(fmt, qdt, 128, 31), pattern, seed=5)


@pytest.mark.parametrize("fmt", ["int8", "int4"])
def test_sparse_prefill_head64_and_all_blocks(fmt):
    print("case sparse prefill D64 all", fmt, flush=True)
    _run_prefill(_wp(fmt, "f16", 64, 37), "all")


def test_sparse_prefill_full_size_window():
    """int8_prefill shape (64 ragged sequences, pasts up to 2048) with the
    window + strided selection; the oracle on 6 sequences, every row and
    head, the longest included."""
    print("case sparse prefill full", flush=True)
    w = workloads.make("int8_prefill")
    qlen = np.diff(w.cum_q)
    order = np.argsort(-(qlen * 4096 + w.past_lens))
    seqs = sorted(set(order[:3].tolist()) | set(np.random.default_rng(3).choice(
        w.batch, 3, replace=False).tolist()))
    _run_prefill(w, "window", seqs=seqs)
