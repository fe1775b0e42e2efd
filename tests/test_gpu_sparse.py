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
