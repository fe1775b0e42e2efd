"""paged_attn_decode_noalloc -- the decode for callers that cannot allocate
(its workspace is the library's own per-GPU scratch array) -- against
paged_attn_decode with a caller workspace: same kernels and partition, so the
outputs must be identical, and both must meet the oracle's tolerance.  Two
calls in a row use the one scratch array, the second with a smaller input;
a single pass (no workspace at all) runs between them."""

import numpy as np
import pytest
import torch

import attention_paged_quantized_amd as paq
import workloads
from tests import compare
from tests.gpu_cases import Device, desc_for
from tests.oracle_cases import oracle_attention, oracle_caches

pytestmark = pytest.mark.gpu


def _noalloc_vs_workspace(w, splits):
    print("case noalloc", w.name, splits, flush=True)
    g = Device(w).fill()
    ref = g.attend(num_splits=splits)              # paged_attn_decode, zeroed workspace
    buf = torch.full((w.token_count + 2, w.num_heads, w.head_size), float("nan"),
                     dtype=ref.dtype, device="cuda")
    out = buf[:w.token_count]
    paq.paged_attn_decode_noalloc(desc_for(w, w.token_count), g.query, out, g.kc, g.vc,
                                  g.k_scale, g.v_scale, g.block_table, g.cum_q, g.past, w.cum_q,
                                  w.past_lens, 0.0, splits)
    torch.cuda.synchronize()
    assert torch.isnan(buf[w.token_count:]).all(), "rows past token_count written"
    assert torch.equal(out, ref), "%s: differs from paged_attn_decode" % w.name
    kc, vc = oracle_caches(w)
    compare.check(out.float().cpu().numpy(), oracle_attention(w, kc, vc), w.q_dtype, w.name)


def test_noalloc_decode_matches_workspace_decode():
    big = workloads.custom("noalloc_big", 2101, batch=6, num_heads=32, kv_num_heads=8,
                           head_size=128, block_size=16,
                           past=np.array([3000, 600, 40, 1200, 0, 777]),
                           q_lens=np.array([1, 1, 1, 1, 0, 1]), q_dtype="f16", kv_format="int8",
                           num_splits=-37)
    single = workloads.custom("noalloc_single", 2102, batch=3, num_heads=16, kv_num_heads=4,
                              head_size=64, block_size=32, past=np.array([100, 5, 70]),
                              q_lens=np.ones(3, np.int32), q_dtype="bf16", kv_format="fp8",
                              scale_mode="head", num_splits=1)
    small = workloads.custom("noalloc_small", 2103, batch=2, num_heads=8, kv_num_heads=2,
                             head_size=128, block_size=32, past=np.array([500, 90]),
                             q_lens=np.ones(2, np.int32), q_dtype="f16", kv_format="int4",
                             num_splits=5)
    for w in (big, single, small):
        _noalloc_vs_workspace(w, w.num_splits)
