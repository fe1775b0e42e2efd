"""paged_attn_decode_host (the CPU GEMV decode with flash decoding across
threads) against the fp64 oracle: formats x scale modes x thread counts x
chunk counts, GQA layouts, zero-token and one-key sequences, extreme key
scales, and the C-ABI checks of the entry point.  Runs on the CPU only."""

import numpy as np
import pytest

import attention_paged_quantized_amd as paq
import workloads
from tests import compare
from tests.gpu_cases import desc_for
from tests.oracle_cases import f32, oracle_attention, oracle_caches


def _host(w, splits=0, threads=0):
    kc, vc = oracle_caches(w)
    q = np.ascontiguousarray(f32(w.query))
    out = np.full_like(q, np.nan)
    i32 = lambda x: np.ascontiguousarray(x, dtype=np.int32)
    f = lambda x: np.ascontiguousarray(x, dtype=np.float32)
    paq.paged_attn_decode_host(desc_for(w, w.token_count), q, out, kc, vc, f(w.k_scale),
                               f(w.v_scale), i32(w.block_table), i32(w.cum_q), i32(w.past_lens),
                               0.0, splits, threads)
    return out, oracle_attention(w, kc, vc)


FORMATS = ["int8", "int4", "fp8"]


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("mode", ["channel", "head"])
@pytest.mark.parametrize("threads,splits", [(1, 1), (4, 0), (8, 5), (3, 40)])
def test_host_decode_formats(fmt, mode, threads, splits):
    past = np.array([0, 15, 16, 300, 90, 47])
    qlen = np.array([1, 1, 1, 1, 0, 1])
    w = workloads.custom("host_%s_%s" % (fmt, mode), 61 + FORMATS.index(fmt), batch=6,
                         num_heads=16, kv_num_heads=4, head_size=128, block_size=16, past=past,
                         q_lens=qlen, q_dtype="f32", kv_format=fmt, scale_mode=mode)
    out, ref = _host(w, splits, threads)
    compare.check(out, ref, "f32", w.name)


@pytest.mark.parametrize("H,Hkv,D", [(4, 4, 64), (16, 2, 128), (12, 3, 64), (8, 1, 128)])
def test_host_decode_head_layouts(H, Hkv, D):
    w = workloads.custom("host_heads_%d_%d_%d" % (H, Hkv, D), 70 + H + D, batch=3, num_heads=H,
                         kv_num_heads=Hkv, head_size=D, block_size=32,
                         past=np.array([100, 33, 64]), q_lens=np.ones(3, np.int32),
                         q_dtype="f32", kv_format="int8")
    out, ref = _host(w, 0, 8)
    compare.check(out, ref, "f32", w.name)


def test_host_decode_tiny_config_and_split_agreement():
    w = workloads.make("tiny_decode")
    single, ref = _host(w, 1, 1)
    compare.check(single, ref, "f32", "tiny single")
    split, _ = _host(w, 7, 8)
    compare.check(split, ref, "f32", "tiny split")


def test_host_decode_extreme_key_scales():
    rng = np.random.default_rng(9)
    ks = np.exp(rng.uniform(np.log(1e-3), np.log(6e4), (4, 128))).astype(np.float32)
    w = workloads.custom("host_ext", 91, batch=2, num_heads=16, kv_num_heads=4, head_size=128,
                         block_size=32, past=np.array([700, 33]), q_lens=np.ones(2, np.int32),
                         q_dtype="f32", kv_format="int4", kv_in_dtype="f32", key_scale=ks)
    out, ref = _host(w, 0, 8)
    compare.check(out, ref, "f32", w.name)


def test_host_decode_argument_checks():
    w = workloads.custom("host_args", 5, batch=2, num_heads=8, kv_num_heads=2, head_size=64,
                         block_size=16, past=np.array([3, 4]), q_lens=np.ones(2, np.int32),
                         q_dtype="f16", kv_format="int8")
    kc, vc = oracle_caches(w)
    q = np.zeros((2, 8, 64), np.float32)
    out = np.zeros_like(q)
    args = (kc, vc, w.k_scale.astype(np.float32), w.v_scale.astype(np.float32),
            w.block_table.astype(np.int32), w.cum_q.astype(np.int32), w.past_lens.astype(np.int32))
    with pytest.raises(RuntimeError, match="fp32"):          # 16-bit queries: not this path
        paq.paged_attn_decode_host(desc_for(w, 2), q, out, *args)
    with pytest.raises(ValueError):                          # host arrays only
        paq.paged_attn_decode_host(desc_for(w, 2), q.astype(np.float64), out, *args)
