"""The four large workloads at full size, in the launch configuration the
bench times (same workload builders, same num_splits), against the oracle on
the whole output tensor.

The GPU fills its cache pools with kv_quant_append; every byte of both pools
must equal the oracle's own pools (oracle quantizer, same poison in the unused
slots).  The oracle then computes every output row from its own pools, and the
GPU output must meet the comparison rule element by element.  Rows past
token_count (NaN canaries) must survive.

For the decode workloads the library's host decode (paged_attn_decode_host,
"GQA GEMV decode", sections 2-3) also runs over the caches the GPU wrote,
copied to host memory, and must meet the fp32 tolerance against the same
oracle output.
"""

import os

import numpy as np
import pytest
import torch

import attention_paged_quantized_amd as paq
import workloads
from tests import compare
from tests.gpu_cases import Device, desc_for
from tests.oracle_cases import oracle_attention, oracle_caches

pytestmark = pytest.mark.gpu


def _host_decode(w, kc, vc):
    d = desc_for(w, w.token_count)
    d.q_dtype = paq.DTYPES["f32"]
    q = np.ascontiguousarray(w.query.float().numpy())        # exact widening of the f16 query
    out = np.full_like(q, np.nan)
    threads = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else 8
    paq.paged_attn_decode_host(d, q, out, kc, vc, np.ascontiguousarray(w.k_scale),
                               np.ascontiguousarray(w.v_scale),
                               np.ascontiguousarray(w.block_table),
                               np.ascontiguousarray(w.cum_q), np.ascontiguousarray(w.past_lens),
                               num_threads=max(1, min(16, threads)))
    return out


@pytest.mark.parametrize("name", ["int8_decode", "int4_long", "int8_prefill", "fp8_prefill"])
def test_full_size_whole_output(name):
    print("case full-size", name, flush=True)
    w = workloads.make(name)
    g = Device(w).fill()
    out = g.attend()                     # the workload's own num_splits, as benched
    got = out.float().cpu().numpy()
    gkc, gvc = g.kc.cpu().numpy(), g.vc.cpu().numpy()
    del g, out
    torch.cuda.empty_cache()
    kc, vc = oracle_caches(w)
    assert np.array_equal(gkc, kc), "%s: key cache differs from the oracle" % name
    assert np.array_equal(gvc, vc), "%s: value cache differs from the oracle" % name
    print("  caches byte-identical; oracle attention over %d rows" % w.token_count, flush=True)
    ref = oracle_attention(w, kc, vc)
    rel, n_ulp = compare.check(got, ref, w.q_dtype, name)
    print("  %s: max rel err %.3g (%d elements needed the output ulp)" % (name, rel, n_ulp),
          flush=True)
    if w.kind == "decode":
        host = _host_decode(w, gkc, gvc)
        rel, _ = compare.check(host, ref, "f32", name + " host decode")
        print("  %s host decode: max rel err %.3g" % (name, rel), flush=True)
