"""kv_quant_append_rotary on the GPU vs the oracle (rotate at each row's
position, then the pinned quantize-append): key and value caches byte for
byte, every untouched byte still poisoned, and the in-place rotated query bit
for bit in its dtype; then prefill over the rotated rows against the oracle's
attention.  Includes zero-token sequences placed so that the heuristic
max_query_len = token_count - batch + 1 would miss rows."""

import numpy as np
import pytest
import torch

import attention_paged_quantized_amd as paq
import workloads
from oracle import rotary
from tests import compare
from tests.gpu_cases import TORCH_DT, desc_for
from tests.oracle_cases import POISON, f32

pytestmark = pytest.mark.gpu


def _case(name, seed, fmt, qdt, kvin, D, past, qlens, H=8, Hkv=2, bs=16, mode="channel"):
    return workloads.custom(name, seed, batch=len(past), num_heads=H, kv_num_heads=Hkv,
                            head_size=D, block_size=bs, past=np.array(past),
                            q_lens=np.array(qlens), q_dtype=qdt, kv_format=fmt,
                            scale_mode=mode, kv_in_dtype=kvin, kind="prefill")


def _run(w, rd, il, with_query=True):
    """Rotary-append the workload's new rows on the GPU and in the oracle;
    returns (gpu kc, vc, q) and (oracle kc, vc, q) as numpy arrays."""
    dev = "cuda"
    key, value, q = w.new_key, w.new_value, w.query
    cum, past = w.cum_q, w.past_lens
    maxpos = int((w.past_lens + w.q_lens).max()) + 1
    cos, sin = workloads.rope_tables(maxpos, rd)
    shape = (w.num_blocks, w.block_size, w.kv_num_heads, w.cache_head_size)
    kc = torch.full(shape, POISON, dtype=torch.uint8, device=dev)
    vc = torch.full(shape, POISON, dtype=torch.uint8, device=dev)
    qd = q.to(dev).contiguous()
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    T = key.shape[0]
    paq.kv_quant_append_rotary(desc_for(w, T), w.kv_in_dtype, qd if with_query else None,
                               key.to(dev), value.to(dev), kc, vc, d(w.k_scale), d(w.v_scale),
                               d(w.block_table), d(cum), d(past), cum, past, d(cos), d(sin), rd, il)
    torch.cuda.synchronize()
    kc0 = np.full(shape, POISON, np.uint8)
    rkc, rvc, rq = rotary.rotary_append(kc0, kc0, f32(q), f32(key), f32(value), w.k_scale,
                                        w.v_scale, w.block_table, cum, past, w.kv_format, cos,
                                        sin, rd, il, w.q_dtype)
    return (kc.cpu().numpy(), vc.cpu().numpy(), qd.float().cpu().numpy()), (rkc, rvc, rq)


FORMATS = ["int8", "int4", "fp8"]
DTYPES = [("f16", "f16"), ("bf16", "bf16"), ("f32", "f32"), ("f16", "f32")]


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("qdt,kvin", DTYPES)
@pytest.mark.parametrize("il", [0, 1])
@pytest.mark.parametrize("rd_frac", [1, 2, 8])
def test_rotary_append_bit_exact(fmt, qdt, kvin, il, rd_frac):
    D = 128
    rd = D // rd_frac
    name = "rot_%s_%s_%s_il%d_rd%d" % (fmt, qdt, kvin, il, rd)
    print("case", name, flush=True)
    # ragged new rows (one sequence without any), pasts across block edges
    seed = 31 + FORMATS.index(fmt) * 7 + DTYPES.index((qdt, kvin)) * 3 + il + rd
    w = _case(name, seed, fmt, qdt, kvin, D, past=[0, 37, 16, 5, 0], qlens=[70, 1, 0, 33, 3])
    (kc, vc, q), (rkc, rvc, rq) = _run(w, rd, il)
    assert np.array_equal(kc, rkc), "key cache differs"
    assert np.array_equal(vc, rvc), "value cache differs"
    assert np.array_equal(q.view(np.uint32), rq.view(np.uint32)), "rotated query differs"


@pytest.mark.parametrize("il", [0, 1])
def test_rotary_keys_only_and_head_size_64(il):
    print("case rot keys only", il, flush=True)
    w = _case("rot_konly_%d" % il, 77 + il, "int4", "f16", "f16", 64, past=[3, 0, 130],
              qlens=[20, 9, 1], H=12, Hkv=3, bs=32, mode="head")
    (kc, vc, q), (rkc, rvc, _) = _run(w, 32, il, with_query=False)
    assert np.array_equal(kc, rkc) and np.array_equal(vc, rvc)
    assert np.array_equal(q, f32(w.query)), "query must be untouched"


def test_rotary_rows_the_heuristic_grid_would_drop():
    """q_lens (0, 0, 0, 61): token_count - batch + 1 = 58 < 61."""
    print("case rot heuristic", flush=True)
    w = _case("rot_heur", 91, "int8", "f16", "f16", 128, past=[5, 0, 9, 40], qlens=[0, 0, 0, 61])
    (kc, vc, q), (rkc, rvc, rq) = _run(w, 128, 0)
    assert np.array_equal(kc, rkc) and np.array_equal(vc, rvc)
    assert np.array_equal(q.view(np.uint32), rq.view(np.uint32))
    # the last rows (positions 40+58 .. 40+60) were rotated, not left as input
    assert not np.array_equal(q[58:], f32(w.query)[58:])


@pytest.mark.parametrize("fmt,qdt", [("int8", "f16"), ("fp8", "bf16"), ("int4", "f16")])
def test_prefill_over_rotated_rows(fmt, qdt):
    """Past rows rotated at 0..past-1 and new rows at past..: prefill on the
    GPU over its own rotated query and cache vs the oracle's attention over
    the oracle's rotated query and cache."""
    from oracle import attention
    print("case rot prefill", fmt, qdt, flush=True)
    w = _case("rot_pf_%s" % fmt, 55, fmt, qdt, qdt, 128, past=[0, 37, 16, 5],
              qlens=[40, 1, 0, 33], mode="head" if fmt == "fp8" else "channel")
    dev = "cuda"
    rd, il = 128, 0
    maxpos = int((w.past_lens + w.q_lens).max()) + 1
    cos, sin = workloads.rope_tables(maxpos, rd)
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    shape = (w.num_blocks, w.block_size, w.kv_num_heads, w.cache_head_size)
    kc = torch.full(shape, POISON, dtype=torch.uint8, device=dev)
    vc = torch.full(shape, POISON, dtype=torch.uint8, device=dev)
    P = int(w.cum_past[-1])
    zeros = np.zeros(w.batch, np.int32)
    paq.kv_quant_append_rotary(desc_for(w, P), w.kv_in_dtype, None, w.past_key.to(dev),
                               w.past_value.to(dev), kc, vc, d(w.k_scale), d(w.v_scale),
                               d(w.block_table), d(w.cum_past), d(zeros), w.cum_past, zeros,
                               d(cos), d(sin), rd, il)
    q = w.query.to(dev).contiguous()
    T = w.token_count
    paq.kv_quant_append_rotary(desc_for(w, T), w.kv_in_dtype, q, w.new_key.to(dev),
                               w.new_value.to(dev), kc, vc, d(w.k_scale), d(w.v_scale),
                               d(w.block_table), d(w.cum_q), d(w.past_lens), w.cum_q,
                               w.past_lens, d(cos), d(sin), rd, il)
    out = torch.empty_like(q)
    paq.paged_attn_prefill(desc_for(w, T), q, out, kc, vc, d(w.k_scale), d(w.v_scale),
                           d(w.block_table), d(w.cum_q), d(w.past_lens), w.cum_q, w.past_lens)
    torch.cuda.synchronize()
    kc0 = np.full(shape, POISON, np.uint8)
    rkc, rvc, _ = rotary.rotary_append(kc0, kc0, np.zeros((P, w.num_heads, 128), np.float32),
                                       f32(w.past_key), f32(w.past_value), w.k_scale, w.v_scale,
                                       w.block_table, w.cum_past, zeros, w.kv_format, cos, sin,
                                       rd, il, w.q_dtype)
    rkc, rvc, rq = rotary.rotary_append(rkc, rvc, f32(w.query), f32(w.new_key), f32(w.new_value),
                                        w.k_scale, w.v_scale, w.block_table, w.cum_q,
                                        w.past_lens, w.kv_format, cos, sin, rd, il, w.q_dtype)
    assert np.array_equal(kc.cpu().numpy(), rkc) and np.array_equal(vc.cpu().numpy(), rvc)
    ref = attention.paged_attention(rq, rkc, rvc, w.k_scale, w.v_scale, w.block_table, w.cum_q,
                                    w.past_lens, w.kv_format)
    compare.check(out.float().cpu().numpy(), ref, w.q_dtype, w.name)


def test_rotary_append_full_ragged_prefill_step():
    """The ragged prefill step at full size (64 sequences, ~15k new rows, 32
    heads over 8 kv heads, INT8 per channel, 6 sequences with no new row):
    every cache byte and every query element exact."""
    print("case rot full int8_prefill", flush=True)
    w = workloads.make("int8_prefill")
    (kc, vc, q), (rkc, rvc, rq) = _run(w, 128, 0)
    assert np.array_equal(kc, rkc) and np.array_equal(vc, rvc)
    assert np.array_equal(q.view(np.uint32), rq.view(np.uint32))
