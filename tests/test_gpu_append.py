"""kv_quant_append on the GPU vs the oracle quantizer: byte-exact caches,
including every byte the step must not touch (poisoned slots, other
sequences' blocks, spare blocks)."""

import numpy as np
import pytest
import torch

import attention_paged_quantized_amd as paq
import workloads
from oracle import quant
from tests.gpu_cases import Device, desc_for
from tests.oracle_cases import POISON, f32, oracle_caches

pytestmark = pytest.mark.gpu


def _all_finite(dtype):
    bits = torch.arange(0, 1 << 16, dtype=torch.int32).to(torch.int16)
    v = bits.view(dtype)
    return v[torch.isfinite(v.float())]


@pytest.mark.parametrize("fmt", ["int8", "int4", "fp8"])
@pytest.mark.parametrize("src", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("mode", ["channel", "head"])
def test_append_exhaustive_inputs_bit_exact(fmt, src, mode):
    """Every finite fp16 (or bf16) value, as append rows, at log-uniform
    per-channel / per-head scales (plus powers of two): codes byte-identical."""
    print("case append", fmt, src, mode, flush=True)
    dt = torch.float16 if src in ("f16", "f32") else torch.bfloat16
    vals = _all_finite(dt)
    hkv, D, bs = 4, 128, 16
    per_tok = hkv * D
    n_tok = -(-vals.numel() // per_tok)
    rng = np.random.default_rng(17)
    pad = vals[torch.from_numpy(rng.integers(0, vals.numel(), n_tok * per_tok - vals.numel()))]
    x = torch.cat([vals, pad])[torch.from_numpy(rng.permutation(n_tok * per_tok))]
    x = x.reshape(n_tok, hkv, D)
    if src == "f32":
        x = x.float() * torch.from_numpy(rng.uniform(0.5, 2.0, x.shape).astype(np.float32))
    # two sequences: one appended after a past of 5 tokens, one from scratch
    q1 = n_tok // 3
    qlens = [q1, n_tok - q1]
    past = [5, 0]
    kv = [p + q for p, q in zip(past, qlens)]
    mb = max(-(-k // bs) for k in kv)
    nb = sum(-(-k // bs) for k in kv) + 3
    perm = rng.permutation(nb).astype(np.int32)
    table = np.full((2, mb), -1, np.int32)
    n0 = -(-kv[0] // bs)
    table[0, :n0] = perm[:n0]
    table[1, :-(-kv[1] // bs)] = perm[n0:n0 + -(-kv[1] // bs)]
    if mode == "channel":
        s = np.exp(rng.uniform(np.log(1e-3), np.log(6e4), (hkv, D))).astype(np.float32)
        s[0, :8] = 2.0 ** np.arange(-4, 4)
    else:
        s = np.array([1e-3, 0.37, 1.0, 6e4], np.float32)
    cum = np.array([0, qlens[0], n_tok], np.int32)
    fmt_c = (D // 2) if fmt == "int4" else D
    kc0 = np.full((nb, bs, hkv, fmt_c), POISON, np.uint8)
    xo = x.float().numpy()
    ref_k, ref_v = quant.quant_append(kc0, kc0, xo, -xo, s, s[::-1].copy() if mode == "head"
                                      else s, table, cum, past, fmt)
    dev = "cuda"
    kc = torch.full(kc0.shape, POISON, dtype=torch.uint8, device=dev)
    vc = torch.full(kc0.shape, POISON, dtype=torch.uint8, device=dev)
    desc = paq.make_desc(2, n_tok, hkv, hkv, D, bs, nb, mb, "f16", fmt, mode)
    sv = s[::-1].copy() if mode == "head" else s
    xd = x.to(dev)
    paq.kv_quant_append(desc, src, xd, (-xd).contiguous(), kc, vc,
                        torch.from_numpy(s).to(dev), torch.from_numpy(sv).to(dev),
                        torch.from_numpy(table).to(dev), torch.from_numpy(cum).to(dev),
                        torch.tensor(past, dtype=torch.int32, device=dev), cum, past)
    torch.cuda.synchronize()
    assert np.array_equal(kc.cpu().numpy(), ref_k)
    assert np.array_equal(vc.cpu().numpy(), ref_v)


@pytest.mark.parametrize("name", ["tiny_decode", "int8_decode_small", "int4_long_small",
                                  "int8_prefill_small", "fp8_prefill_small", "int8_decode"])
def test_append_workloads_bit_exact(name):
    print("case append workload", name, flush=True)
    w = workloads.make(name)
    g = Device(w).fill()
    torch.cuda.synchronize()
    kc, vc = oracle_caches(w)
    assert np.array_equal(g.kc.cpu().numpy(), kc)
    assert np.array_equal(g.vc.cpu().numpy(), vc)


def test_append_zero_token_step_is_a_no_op():
    w = workloads.make("int8_prefill_small")
    g = Device(w)
    before = g.kc.clone()
    zeros = np.zeros(w.batch, np.int32)
    cum0 = np.zeros(w.batch + 1, np.int32)
    e = torch.empty(0, w.kv_num_heads, w.head_size, dtype=torch.float16, device="cuda")
    paq.kv_quant_append(desc_for(w, 0), "f16", e, e, g.kc, g.vc, g.k_scale, g.v_scale,
                        g.block_table, torch.from_numpy(cum0).cuda(), g.zeros, cum0, zeros)
    torch.cuda.synchronize()
    assert torch.equal(before, g.kc)
