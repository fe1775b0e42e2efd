"""Cache pools beyond 4 GiB: every kernel addresses blocks with 64-bit byte
offsets.  The sequences' blocks are moved to the highest block ids of a pool
larger than 5 GiB (per cache); the GPU's cache bytes there must equal the
oracle's compact cache, and the outputs must match the oracle's attention on
the compact layout (the oracle is pinned to be invariant under block
permutation)."""

import dataclasses

import numpy as np
import pytest
import torch

import attention_paged_quantized_amd as paq
import workloads
from oracle import rotary
from tests import compare
from tests.gpu_cases import Device, desc_for
from tests.oracle_cases import POISON, f32, oracle_attention, oracle_caches

pytestmark = pytest.mark.gpu


def _moved_to_top(w, pool_bytes=5 << 30):
    """w with its physical blocks renumbered to the top of a pool of more than
    pool_bytes per cache; returns (moved workload, old id -> new id)."""
    row = w.block_size * w.kv_num_heads * w.cache_head_size
    big = pool_bytes // row + 64
    new_id = (big - 1 - np.arange(w.num_blocks)).astype(np.int32)
    bt = np.where(w.block_table >= 0, new_id[np.clip(w.block_table, 0, None)], -1)
    return dataclasses.replace(w, block_table=bt.astype(np.int32), num_blocks=int(big)), new_id


@pytest.mark.parametrize("fmt", ["int8", "int4"])
@pytest.mark.parametrize("kind,splits", [("decode", 1), ("decode", 4), ("prefill", 1)])
def test_blocks_beyond_4gib(fmt, kind, splits):
    name = "big_%s_%s_s%d" % (fmt, kind, splits)
    print("case", name, flush=True)
    if kind == "decode":
        past, qlen = np.array([300, 47, 129]), np.ones(3, np.int32)
    else:
        past, qlen = np.array([0, 70, 16]), np.array([40, 9, 33])
    w = workloads.custom(name, 606, batch=3, num_heads=16, kv_num_heads=4, head_size=128,
                         block_size=16, past=past, q_lens=qlen, q_dtype="f16", kv_format=fmt,
                         kind=kind, num_splits=splits)
    wb, new_id = _moved_to_top(w)
    g = Device(wb).fill()
    out = g.attend()
    torch.cuda.synchronize()
    kc, vc = oracle_caches(w)
    ids = torch.from_numpy(new_id.astype(np.int64)).cuda()
    assert np.array_equal(g.kc[ids].cpu().numpy(), kc), "key blocks at the top of the pool"
    assert np.array_equal(g.vc[ids].cpu().numpy(), vc), "value blocks at the top of the pool"
    assert g.kc.numel() > (4 << 30)
    ref = oracle_attention(w, kc, vc)
    compare.check(out.float().cpu().numpy(), ref, w.q_dtype, name)


def test_rotary_append_beyond_4gib():
    print("case big rotary", flush=True)
    w = workloads.custom("big_rot", 607, batch=2, num_heads=8, kv_num_heads=2, head_size=128,
                         block_size=32, past=np.array([5, 40]), q_lens=np.array([30, 7]),
                         q_dtype="bf16", kv_format="fp8", scale_mode="head", kind="prefill")
    wb, new_id = _moved_to_top(w)
    dev = "cuda"
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    cos, sin = workloads.rope_tables(64, 64)
    shape = (wb.num_blocks, w.block_size, w.kv_num_heads, w.cache_head_size)
    kc = torch.full(shape, POISON, dtype=torch.uint8, device=dev)
    vc = torch.full(shape, POISON, dtype=torch.uint8, device=dev)
    q = w.query.to(dev).contiguous()
    paq.kv_quant_append_rotary(desc_for(wb, w.token_count), w.kv_in_dtype, q, w.new_key.to(dev),
                               w.new_value.to(dev), kc, vc, d(w.k_scale), d(w.v_scale),
                               d(wb.block_table), d(w.cum_q), d(w.past_lens), w.cum_q,
                               w.past_lens, d(cos), d(sin), 64, True)
    torch.cuda.synchronize()
    cshape = (w.num_blocks, w.block_size, w.kv_num_heads, w.cache_head_size)
    kc0 = np.full(cshape, POISON, np.uint8)
    rkc, rvc, rq = rotary.rotary_append(kc0, kc0, f32(w.query), f32(w.new_key), f32(w.new_value),
                                        w.k_scale, w.v_scale, w.block_table, w.cum_q,
                                        w.past_lens, w.kv_format, cos, sin, 64, True, "bf16")
    ids = torch.from_numpy(new_id.astype(np.int64)).cuda()
    assert np.array_equal(kc[ids].cpu().numpy(), rkc)
    assert np.array_equal(vc[ids].cpu().numpy(), rvc)
    assert np.array_equal(q.float().cpu().numpy().view(np.uint32), rq.view(np.uint32))
