"""Every kernel path the planner can choose, on the GPU against the fp64 oracle.

The planner sends a call to the 16-bit MFMA kernels when their shape rules
allow it and to the portable fp32 kernel otherwise ("ONNX Runtime: INT4 Paged
KV Cache", reviewer-feedback section: the safe FP32 kernel).  The format
matrix covers the common shapes; these cases cover the rest:

* fp32 queries in prefill (ragged, causal, zero-token sequences) -> fp32 kernel;
* fp16/bf16 decode with GQA groups 9..16 -> fp32 kernel (single pass and
  split-KV with its combine), and groups 3, 5, 7 -> MFMA decode;
* fp16/bf16 prefill with groups that are not powers of two (3, 5, 6) ->
  fp32 kernel; group 32 -> MFMA prefill with one token per wave;
* groups above 16 on the fp32 path are refused on the host before launch;
* the length-balanced decode partition (long sequences cut into more parts,
  merged by the last part to arrive, in the same launch), explicit and
  automatic, and a workspace reused across calls of different shapes.

Each case is small enough for the oracle to finish in well under a second
and spans several key tiles with a ragged tail.
"""

import itertools

import numpy as np
import pytest

import attention_paged_quantized_amd as paq
import workloads
from tests import compare
from tests.gpu_cases import Device
from tests.oracle_cases import oracle_attention, oracle_caches

pytestmark = pytest.mark.gpu

FORMATS = ["int8", "int4", "fp8"]


def _run(w, splits=None):
    g = Device(w).fill()
    out = g.attend(num_splits=splits)
    kc, vc = oracle_caches(w)
    assert (g.kc.cpu().numpy() == kc).all(), "key cache differs from the oracle"
    assert (g.vc.cpu().numpy() == vc).all(), "value cache differs from the oracle"
    ref = oracle_attention(w, kc, vc)
    return compare.check(out.float().cpu().numpy(), ref, w.q_dtype, w.name)


def _plan_path(w, splits):
    d = paq.make_desc(w.batch, w.token_count, w.num_heads, w.kv_num_heads, w.head_size,
                      w.block_size, w.num_blocks, w.max_blocks_per_seq, w.q_dtype,
                      w.kv_format, w.scale_mode)
    if w.kind == "decode":
        return paq.PATHS[paq.paq_plan_decode(d, w.cum_q, w.past_lens, splits).path]
    return paq.PATHS[paq.paq_plan_prefill(d, w.cum_q, w.past_lens).path]


@pytest.mark.parametrize("fmt,D,mode", list(itertools.product(FORMATS, [64, 128],
                                                              ["channel", "head"])))
def test_prefill_f32_queries(fmt, D, mode):
    name = "pf32_%s_d%d_%s" % (fmt, D, mode)
    print("case", name, flush=True)
    # ragged new rows with two empty sequences, pasts across block edges
    past = np.array([0, 37, 16, 5, 0, 300])
    qlen = np.array([70, 1, 0, 33, 0, 9])
    seed = 1201 + 7 * FORMATS.index(fmt) + D + (mode == "head")
    w = workloads.custom(name, seed, batch=6, num_heads=8, kv_num_heads=2, head_size=D,
                         block_size=16, past=past, q_lens=qlen, q_dtype="f32", kv_format=fmt,
                         scale_mode=mode, kind="prefill")
    assert _plan_path(w, 0) == "f32_prefill"
    _run(w)


@pytest.mark.parametrize("G", [12, 16])
@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("qdt", ["f16", "bf16"])
@pytest.mark.parametrize("splits", [1, 4])
def test_decode_large_groups(G, fmt, qdt, splits):
    """Groups above the MFMA decode's 8 columns take the fp32 kernel."""
    name = "dec_g%d_%s_%s_s%d" % (G, fmt, qdt, splits)
    print("case", name, flush=True)
    hkv = 2
    w = workloads.custom(name, 1301 + G + 5 * FORMATS.index(fmt) + splits, batch=4,
                         num_heads=G * hkv, kv_num_heads=hkv, head_size=128, block_size=16,
                         past=np.array([130, 0, 47, 16]), q_lens=np.array([1, 1, 0, 1]),
                         q_dtype=qdt, kv_format=fmt, num_splits=splits)
    assert _plan_path(w, splits) == ("f32_split" if splits > 1 else "f32_single")
    _run(w)


@pytest.mark.parametrize("G", [3, 5, 7])
@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("splits", [1, 3])
def test_decode_odd_groups(G, fmt, splits):
    """Groups that are not powers of two fill G of the MFMA decode's columns."""
    name = "dec_odd_g%d_%s_s%d" % (G, fmt, splits)
    print("case", name, flush=True)
    hkv = 2
    w = workloads.custom(name, 1401 + G + 5 * FORMATS.index(fmt) + splits, batch=3,
                         num_heads=G * hkv, kv_num_heads=hkv, head_size=128, block_size=32,
                         past=np.array([200, 31, 64]), q_lens=np.ones(3, np.int32),
                         q_dtype="bf16" if G == 5 else "f16", kv_format=fmt,
                         num_splits=splits)
    _run(w)


@pytest.mark.parametrize("G", [3, 5, 6, 32])
@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("qdt", ["f16", "bf16"])
def test_prefill_group_paths(G, fmt, qdt):
    """Groups 3, 5, 6 take the fp32 kernel with 16-bit queries; group 32 the
    MFMA prefill with one token per wave."""
    name = "pf_g%d_%s_%s" % (G, fmt, qdt)
    print("case", name, flush=True)
    hkv = 1 if G == 32 else 2
    w = workloads.custom(name, 1501 + G + 5 * FORMATS.index(fmt) + (qdt == "bf16"), batch=4,
                         num_heads=G * hkv, kv_num_heads=hkv, head_size=128, block_size=16,
                         past=np.array([0, 21, 90, 3]), q_lens=np.array([37, 0, 11, 5]),
                         q_dtype=qdt, kv_format=fmt, kind="prefill",
                         scale_mode="head" if fmt == "fp8" else "channel")
    assert _plan_path(w, 0) == ("prefill" if G == 32 else "f32_prefill")
    _run(w)


def test_groups_beyond_the_fp32_kernel_are_refused():
    """A 16-bit decode with group 32 has no kernel: the host refuses it with
    PAQ_ERR_UNSUPPORTED before anything is launched."""
    w = workloads.custom("dec_g32", 1601, batch=2, num_heads=64, kv_num_heads=2,
                         head_size=128, block_size=16, past=np.array([40, 7]),
                         q_lens=np.ones(2, np.int32), q_dtype="f16", kv_format="int8")
    with pytest.raises(paq.PaqError) as e:
        _plan_path(w, 1)
    assert e.value.status == paq.PAQ_ERR_UNSUPPORTED


@pytest.mark.parametrize("groups", [3, 16, 37, 256])
@pytest.mark.parametrize("fmt", FORMATS)
def test_decode_balanced_parts(groups, fmt):
    """num_splits = -N: the 32-key tiles of all (sequence, head group) pairs
    dealt out to N workgroups in equal runs -- runs that cover several whole
    segments, runs inside one segment, segments cut into up to ~N pieces."""
    name = "dec_bal_%d_%s" % (groups, fmt)
    print("case", name, flush=True)
    past = np.array([0, 31, 32, 600, 1500, 70, 299])
    qlen = np.array([1, 1, 1, 0, 1, 1, 1])
    w = workloads.custom(name, 1701 + groups + 3 * FORMATS.index(fmt), batch=7, num_heads=16,
                         kv_num_heads=4, head_size=128, block_size=32 if fmt == "int4" else 16,
                         past=past, q_lens=qlen, q_dtype="bf16" if fmt == "fp8" else "f16",
                         kv_format=fmt, num_splits=-groups,
                         scale_mode="head" if fmt == "fp8" else "channel")
    assert _plan_path(w, -groups) == "balanced"
    _run(w)


@pytest.mark.parametrize("D,fmt", [(128, "int8"), (64, "int4"), (64, "int8")])
def test_decode_balanced_automatic(D, fmt):
    """The automatic choice on a batch whose (sequence, head group) units
    under-fill the device and whose lengths are skewed is the length-balanced
    partition."""
    name = "dec_bal_auto_d%d_%s" % (D, fmt)
    print("case", name, flush=True)
    past = np.array([3000, 600, 700, 650, 800, 620])           # longest > 1.5 x mean
    w = workloads.custom(name, 1802 + D, batch=6, num_heads=32, kv_num_heads=8, head_size=D,
                         block_size=16, past=past, q_lens=np.ones(6, np.int32), q_dtype="f16",
                         kv_format=fmt, num_splits=0)
    assert _plan_path(w, 0) == "balanced"
    _run(w)


def test_workspace_reused_across_shapes():
    """One workspace, zeroed once, serves split and balanced calls of different
    shapes in a row: every call leaves the arrival counters zero, and every
    result matches the oracle."""
    import torch
    from tests.gpu_cases import COUNTERS, desc_for
    cases = [
        workloads.custom("reuse_a", 1901, batch=5, num_heads=8, kv_num_heads=2, head_size=128,
                         block_size=16, past=np.array([400, 7, 900, 0, 33]),
                         q_lens=np.array([1, 1, 1, 0, 1]), q_dtype="f16", kv_format="int8",
                         num_splits=6),
        workloads.custom("reuse_b", 1902, batch=2, num_heads=32, kv_num_heads=8, head_size=128,
                         block_size=32, past=np.array([2000, 100]), q_lens=np.ones(2, np.int32),
                         q_dtype="f16", kv_format="int4", num_splits=-64),
        workloads.custom("reuse_c", 1903, batch=9, num_heads=16, kv_num_heads=4, head_size=64,
                         block_size=16, past=np.arange(9) * 70 + 5, q_lens=np.ones(9, np.int32),
                         q_dtype="bf16", kv_format="fp8", num_splits=3),
    ]
    need = max(paq.paged_attn_decode_workspace_size(desc_for(w, w.token_count), w.cum_q,
                                                    w.past_lens, w.num_splits) for w in cases)
    ws = torch.zeros(need // 4 + 1, dtype=torch.float32, device="cuda")
    for rep in range(2):
        for w in cases:
            print("case reuse", w.name, rep, flush=True)
            g = Device(w).fill()
            out = torch.full((w.token_count, w.num_heads, w.head_size), float("nan"),
                             dtype=g.query.dtype, device="cuda")
            paq.paged_attn_decode(desc_for(w, w.token_count), g.query, out, g.kc, g.vc,
                                  g.k_scale, g.v_scale, g.block_table, g.cum_q, g.past, w.cum_q,
                                  w.past_lens, 0.0, w.num_splits, ws)
            torch.cuda.synchronize()
            assert not ws.view(torch.int32)[:COUNTERS].any(), "counters left non-zero"
            kc, vc = oracle_caches(w)
            compare.check(out.float().cpu().numpy(), oracle_attention(w, kc, vc), w.q_dtype,
                          w.name)


@pytest.mark.parametrize("name", ["int8_prefill_small", "fp8_prefill_small"])
def test_prefill_padded_grid_matches_exact(name):
    """A grid sized from token_count - batch + 1 for every (sequence, kv head)
    pair (the pre-fix sizing of "PagedAttention FA path: exact
    max_query_len") runs the same tiles plus tiles that exit at once: the
    output is bit-identical to the exact grid's.  A max_query_len below the
    exact maximum is refused before launch."""
    import torch
    from tests.gpu_cases import desc_for
    print("case padded grid", name, flush=True)
    w = workloads.make(name)
    g = Device(w).fill()
    exact = g.attend()
    out = torch.full_like(exact, float("nan"))
    args = (desc_for(w, w.token_count), g.query, out, g.kc, g.vc, g.k_scale, g.v_scale,
            g.block_table, g.cum_q, g.past, w.cum_q, w.past_lens)
    paq.paged_attn_prefill_padded(*args, w.token_count - w.batch + 1)
    torch.cuda.synchronize()
    assert torch.equal(out, exact)
    with pytest.raises(paq.PaqError) as e:
        paq.paged_attn_prefill_padded(*args, int(w.q_lens.max()) - 1)
    assert e.value.status == paq.PAQ_ERR_INVALID_ARG


def _k_per_use_case(w):
    import torch
    from tests.gpu_cases import desc_for
    g = Device(w).fill()
    exact = g.attend()
    out = torch.full_like(exact, float("nan"))
    paq.paged_attn_prefill_k_per_use(desc_for(w, w.token_count), g.query, out, g.kc, g.vc,
                                     g.k_scale, g.v_scale, g.block_table, g.cum_q, g.past,
                                     w.cum_q, w.past_lens)
    torch.cuda.synchronize()
    kc, vc = oracle_caches(w)
    compare.check(out.float().cpu().numpy(), oracle_attention(w, kc, vc), w.q_dtype, w.name)
    # the same exact 16-bit operands in the same products: identical output
    assert torch.equal(out, exact)


@pytest.mark.parametrize("name", ["int8_prefill_small", "fp8_prefill_small"])
def test_prefill_k_per_use_matches(name):
    """The comparison staging scheme (K codes raw in LDS, converted by every
    wave at each use) against the oracle, and bit-identical to the default
    (convert once) path."""
    print("case k per use", name, flush=True)
    _k_per_use_case(workloads.make(name))


@pytest.mark.parametrize("fmt", ["int8", "fp8"])
@pytest.mark.parametrize("qdt", ["f16", "bf16"])
@pytest.mark.parametrize("mode", ["channel", "head"])
def test_prefill_k_per_use_formats(fmt, qdt, mode):
    print("case k per use", fmt, qdt, mode, flush=True)
    w = workloads.custom("kpu", 41, batch=4, num_heads=16, kv_num_heads=4, head_size=128,
                         block_size=32, past=np.array([0, 77, 150, 5]),
                         q_lens=np.array([70, 0, 101, 33]), q_dtype=qdt, kv_format=fmt,
                         scale_mode=mode, kind="prefill")
    _k_per_use_case(w)
