"""The algorithmic numerators of the bench's rooflines against brute-force
counts: decode KV bytes (dense and block-sparse), prefill flops (4 * D * H per
visible causal pair, dense and block-sparse), append bytes.  CPU only."""

import numpy as np
import pytest

import bench
import workloads


def _visible_pairs(w, attended=None):
    """Brute force: (row, key) pairs with key <= past + i (and, block-sparse,
    the key's block attended)."""
    n = 0
    for b in range(w.batch):
        past, q = int(w.past_lens[b]), int(w.q_lens[b])
        for i in range(q):
            for t in range(past + i + 1):
                if attended is None or attended(b, t):
                    n += 1
    return n


@pytest.mark.parametrize("name", ["int8_prefill_small", "fp8_prefill_small"])
def test_prefill_flops_count_causal_pairs(name):
    w = workloads.make(name)
    assert bench.prefill_flops(w) == 4 * w.head_size * w.num_heads * _visible_pairs(w)


def test_sparse_prefill_flops_count_attended_pairs():
    w = workloads.make("int8_prefill_small")
    sel, num = bench.sparse_selection(w)
    bs = w.block_size
    for b in range(w.batch):                  # the selection's own contract
        assert all(0 <= x < w.past_lens[b] // bs for x in sel[b, :num[b]])

    def attended(b, t):
        return t // bs >= w.past_lens[b] // bs or t // bs in set(sel[b, :num[b]].tolist())

    assert bench.prefill_flops(w, num) == 4 * w.head_size * w.num_heads * \
        _visible_pairs(w, attended)


@pytest.mark.parametrize("name", ["int8_decode_small", "int4_long_small", "tiny_decode"])
def test_decode_kv_bytes(name):
    w = workloads.make(name)
    keys = sum(int(w.past_lens[b]) + 1 for b in range(w.batch) if w.q_lens[b] > 0)
    assert bench.kv_bytes(w) == keys * w.kv_num_heads * 2 * w.cache_head_size


@pytest.mark.parametrize("name", ["int8_decode_small", "int4_long_small"])
def test_sparse_decode_bytes(name):
    w = workloads.make(name)
    sel, num = bench.sparse_selection(w)
    keys = 0
    for b in range(w.batch):
        if w.q_lens[b] == 0:
            continue
        chosen = set(sel[b, :num[b]].tolist())
        keys += sum(1 for t in range(int(w.past_lens[b]) + 1) if t // w.block_size in chosen)
    assert bench.sparse_kv_bytes(w, sel, num) == keys * w.kv_num_heads * 2 * w.cache_head_size


@pytest.mark.parametrize("rotary", [False, True])
def test_append_bytes(rotary):
    w = workloads.make("int8_prefill_small")
    T = w.token_count
    size = {"f32": 4, "f16": 2, "bf16": 2}
    rows_in = 2 * T * w.kv_num_heads * w.head_size * size[w.kv_in_dtype]      # new K and V read
    codes_out = 2 * T * w.kv_num_heads * w.cache_head_size                    # their codes written
    extra = 0
    if rotary:
        extra = 2 * T * w.num_heads * w.head_size * size[w.q_dtype]           # query read + written
        extra += T * 2 * (w.head_size // 2) * 4                               # cos and sin rows
    assert bench.append_bytes(w, T, rotary) == rows_in + codes_out + extra


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), (["--gpus", "8"], {}),
                                      ([], {"WORLD_SIZE": "2"})])
def test_bench_refuses_more_than_one_gpu(argv, env):
    """The bench measures one GPU: asked for more, it exits with status 2 and
    says so before touching a device."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    p = subprocess.run([sys.executable, os.path.join(root, "bench.py")] + argv,
                       capture_output=True, text=True, timeout=60, cwd=root,
                       env=dict(os.environ, **env))
    assert p.returncode == 2
    assert "one GPU only" in p.stderr
    assert p.stdout == ""
