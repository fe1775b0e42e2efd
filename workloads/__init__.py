"""Seeded synthetic inputs for paged quantized-KV attention.

This module only draws inputs: batch structure (past lengths, query lengths,
zero-token sequences), physical block tables (seeded permutations of a block
pool), queries, real-valued keys/values to be appended, and the calibrated
fp32 scales.  It holds none of the attention or quantization arithmetic, and
both the HIP path and the CPU oracle consume what it returns.

The shapes and distributions follow the five workloads of the study:
  tiny_decode   batch 3, heads 4/2, D 64, block 16, 24 blocks, fp32 Q, INT8
                per-channel; past {37,100,0}, q_len {1,1,0}
  int8_decode   batch 32, heads 32/8, D 128, block 16, fp16 Q, INT8
                per-channel; past U{1024..4096}, q_len 1; one launch, the
                library's automatic partition (length-balanced parts)
  int4_long     batch 4, heads 32/8, D 128 (64 packed bytes), block 32, fp16
                Q, INT4 per-channel, past 32768, q_len 1; k_scale log-uniform
                in [1e-3, 6e4]; 128-way split-KV
  int8_prefill  batch 64, heads 32/8, D 128, block 16, fp16 Q, INT8
                per-channel; q_len U{1..512} with 6 of 64 at 0, past
                U{0..2048}, causal
  fp8_prefill   batch 4, q_len 2048, past 0, heads 32/8, D 128, block 64,
                bf16 Q, FP8 E4M3 with one fp32 scale per kv head, causal
Each also has a "_small" variant (same head/format structure, fewer tokens)
sized for CPU-oracle parity runs that still span several tiles and a ragged
tail.

Value recipe: Q ~ N(0,1); K, V ~ N(0,1) times a per-(kv head, channel) gain
drawn from LogNormal(0, 0.5) (FP8: no gain); values are rounded (torch RNE
casts) to the model dtype, and the scales are amax / qmax over every token of
every sequence (per kv head and channel, or per kv head for FP8), qmax = 127,
7 or 448; an all-zero channel gets scale 1.  int4_long instead draws k_scale
log-uniformly over [1e-3, 6e4] and keys as 2 * k_scale * N(0,1) in fp32
(fp16 cannot hold them).
"""

from dataclasses import dataclass, field

import numpy as np
import torch

QMAX = {"int8": 127.0, "int4": 7.0, "fp8": 448.0}
DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclass
class Workload:
    name: str
    batch: int
    num_heads: int
    kv_num_heads: int
    head_size: int
    block_size: int
    num_blocks: int
    max_blocks_per_seq: int
    q_dtype: str                 # "f32" | "f16" | "bf16"  (query and output)
    kv_format: str               # "int8" | "int4" | "fp8"
    scale_mode: str              # "channel" | "head"
    kv_in_dtype: str             # dtype of the key/value rows to append
    past_lens: np.ndarray        # int32 (B,)
    q_lens: np.ndarray           # int32 (B,)
    cum_q: np.ndarray            # int32 (B+1,)
    cum_past: np.ndarray         # int32 (B+1,) offsets of past rows
    block_table: np.ndarray      # int32 (B, max_blocks_per_seq), -1 padded
    query: torch.Tensor          # (T, H, D) in q_dtype, CPU
    past_key: torch.Tensor       # (sum past, Hkv, D) in kv_in_dtype, CPU
    past_value: torch.Tensor
    new_key: torch.Tensor        # (T, Hkv, D) in kv_in_dtype, CPU
    new_value: torch.Tensor
    k_scale: np.ndarray          # float32 (Hkv, D) or (Hkv,)
    v_scale: np.ndarray
    num_splits: int = 1          # 0 auto, 1 single pass, >1 split-KV chunks, -K balanced
    kind: str = "decode"         # "decode" | "prefill"
    seed: int = 0
    notes: dict = field(default_factory=dict)

    @property
    def token_count(self):
        return int(self.cum_q[-1])

    @property
    def kv_lens(self):
        return self.past_lens + self.q_lens

    @property
    def cache_head_size(self):
        d = self.head_size
        return (d + 1) // 2 if self.kv_format == "int4" else d


def _cast(x64, dtype):
    return torch.from_numpy(np.ascontiguousarray(x64)).to(DTYPES[dtype])


def _block_table(rng, kv_lens, bs, max_blocks, spare):
    need = [-(-int(L) // bs) for L in kv_lens]
    total = sum(need) + spare
    perm = rng.permutation(total).astype(np.int32)
    bt = np.full((len(kv_lens), max_blocks), -1, dtype=np.int32)
    pos = 0
    for b, n in enumerate(need):
        bt[b, :n] = perm[pos:pos + n]
        pos += n
    return bt, total


def _calibrate(x, kv_format, scale_mode):
    """amax / qmax over all rows, per (kv head, channel) or per kv head."""
    a = x.abs().to(torch.float64)
    amax = a.amax(dim=0) if scale_mode == "channel" else a.amax(dim=(0, 2))
    s = (amax / QMAX[kv_format]).to(torch.float32).numpy()
    s[s == 0] = 1.0
    return s.astype(np.float32)


def make(name, seed=None):
    """Build the named workload with its default seed (or the given one)."""
    return _BUILDERS[name](seed)


def _finish(name, rng, seed, *, batch, H, Hkv, D, bs, past, qlen, q_dtype, kv_format,
            scale_mode, kv_in_dtype, num_splits, kind, spare=8, num_blocks=None,
            block_table=None, gains=True, key_scale_override=None, key_code_sigma=2.0,
            max_blocks=None):
    past = np.asarray(past, dtype=np.int32)
    qlen = np.asarray(qlen, dtype=np.int32)
    kv_lens = past + qlen
    if max_blocks is None:
        max_blocks = max(1, int(-(-int(kv_lens.max()) // bs)))
    if block_table is None:
        bt, nblk = _block_table(rng, kv_lens, bs, max_blocks, spare)
    else:
        bt, nblk = block_table, num_blocks
    cum_q = np.concatenate([[0], np.cumsum(qlen)]).astype(np.int32)
    cum_past = np.concatenate([[0], np.cumsum(past)]).astype(np.int32)
    T, P = int(cum_q[-1]), int(cum_past[-1])
    q = _cast(rng.standard_normal((T, H, D)), q_dtype)
    kg = rng.lognormal(0.0, 0.5, (Hkv, D)) if gains else np.ones((Hkv, D))
    vg = rng.lognormal(0.0, 0.5, (Hkv, D)) if gains else np.ones((Hkv, D))
    if key_scale_override is not None:
        k_scale = key_scale_override.astype(np.float32)
        ks = k_scale.astype(np.float64)
        ks = ks[None] if ks.ndim == 2 else ks[None, :, None]
        kall = key_code_sigma * ks * rng.standard_normal((P + T, Hkv, D))
    else:
        kall = rng.standard_normal((P + T, Hkv, D)) * kg[None]
    vall = rng.standard_normal((P + T, Hkv, D)) * vg[None]
    kall = _cast(kall, kv_in_dtype)
    vall = _cast(vall, kv_in_dtype)
    if key_scale_override is None:
        k_scale = _calibrate(kall, kv_format, scale_mode)
    v_scale = _calibrate(vall, kv_format, scale_mode)
    return Workload(
        name=name, batch=batch, num_heads=H, kv_num_heads=Hkv, head_size=D,
        block_size=bs, num_blocks=int(nblk), max_blocks_per_seq=int(bt.shape[1]),
        q_dtype=q_dtype, kv_format=kv_format, scale_mode=scale_mode,
        kv_in_dtype=kv_in_dtype, past_lens=past, q_lens=qlen, cum_q=cum_q,
        cum_past=cum_past, block_table=bt, query=q,
        past_key=kall[:P].contiguous(), past_value=vall[:P].contiguous(),
        new_key=kall[P:].contiguous(), new_value=vall[P:].contiguous(),
        k_scale=k_scale, v_scale=v_scale, num_splits=num_splits, kind=kind, seed=seed)


def _tiny_decode(seed):
    seed = 1001 if seed is None else seed
    rng = np.random.default_rng(seed)
    bt = rng.permutation(24).astype(np.int32).reshape(3, 8)
    return _finish("tiny_decode", rng, seed, batch=3, H=4, Hkv=2, D=64, bs=16,
                   past=[37, 100, 0], qlen=[1, 1, 0], q_dtype="f32", kv_format="int8",
                   scale_mode="channel", kv_in_dtype="f32", num_splits=1, kind="decode",
                   num_blocks=24, block_table=bt)


def _int8_decode(seed, small=False):
    seed = 1002 if seed is None else seed
    rng = np.random.default_rng(seed)
    B = 5 if small else 32
    lo, hi = (20, 300) if small else (1024, 4096)
    past = rng.integers(lo, hi + 1, B)
    return _finish("int8_decode" + ("_small" if small else ""), rng, seed, batch=B, H=32,
                   Hkv=8, D=128, bs=16, past=past, qlen=np.ones(B, np.int32), q_dtype="f16",
                   kv_format="int8", scale_mode="channel", kv_in_dtype="f16",
                   num_splits=0, kind="decode")


def _int4_long(seed, small=False):
    seed = 1003 if seed is None else seed
    rng = np.random.default_rng(seed)
    B = 2 if small else 4
    past = np.full(B, 700 if small else 32768)
    ks = np.exp(rng.uniform(np.log(1e-3), np.log(6e4), (8, 128)))
    return _finish("int4_long" + ("_small" if small else ""), rng, seed, batch=B, H=32,
                   Hkv=8, D=128, bs=32, past=past, qlen=np.ones(B, np.int32), q_dtype="f16",
                   kv_format="int4", scale_mode="channel", kv_in_dtype="f32",
                   num_splits=7 if small else 128, kind="decode",
                   key_scale_override=ks)


def _int8_prefill(seed, small=False):
    seed = 1004 if seed is None else seed
    rng = np.random.default_rng(seed)
    B = 6 if small else 64
    nzero = 2 if small else 6
    qmax_, pmax = (70, 200) if small else (512, 2048)
    qlen = rng.integers(1, qmax_ + 1, B)
    qlen[rng.choice(B, nzero, replace=False)] = 0
    past = rng.integers(0, pmax + 1, B)
    return _finish("int8_prefill" + ("_small" if small else ""), rng, seed, batch=B, H=32,
                   Hkv=8, D=128, bs=16, past=past, qlen=qlen, q_dtype="f16",
                   kv_format="int8", scale_mode="channel", kv_in_dtype="f16",
                   num_splits=1, kind="prefill",
                   max_blocks=-(-(pmax + qmax_) // 16))


def _fp8_prefill(seed, small=False):
    seed = 1005 if seed is None else seed
    rng = np.random.default_rng(seed)
    B = 2 if small else 4
    n = 130 if small else 2048
    return _finish("fp8_prefill" + ("_small" if small else ""), rng, seed, batch=B, H=32,
                   Hkv=8, D=128, bs=64, past=np.zeros(B, np.int32),
                   qlen=np.full(B, n), q_dtype="bf16", kv_format="fp8",
                   scale_mode="head", kv_in_dtype="bf16", num_splits=1, kind="prefill",
                   gains=False)


_BUILDERS = {
    "tiny_decode": _tiny_decode,
    "int8_decode": lambda s: _int8_decode(s),
    "int8_decode_small": lambda s: _int8_decode(s, True),
    "int4_long": lambda s: _int4_long(s),
    "int4_long_small": lambda s: _int4_long(s, True),
    "int8_prefill": lambda s: _int8_prefill(s),
    "int8_prefill_small": lambda s: _int8_prefill(s, True),
    "fp8_prefill": lambda s: _fp8_prefill(s),
    "fp8_prefill_small": lambda s: _fp8_prefill(s, True),
}

NAMES = tuple(_BUILDERS)


def custom(name, seed, *, batch, num_heads, kv_num_heads, head_size, block_size,
           past, q_lens, q_dtype, kv_format, scale_mode="channel", kv_in_dtype=None,
           num_splits=1, kind="decode", spare=4, key_scale=None, key_code_sigma=2.0):
    """A workload with explicit structure, for edge-case tests.  `key_scale`
    (fp32, (kv_num_heads, head_size) or (kv_num_heads,)) replaces the
    calibrated key scales; keys are then drawn as key_code_sigma * scale * N(0,1)
    in kv_in_dtype (use "f32" for scales outside the 16-bit ranges)."""
    rng = np.random.default_rng(seed)
    return _finish(name, rng, seed, batch=batch, H=num_heads, Hkv=kv_num_heads,
                   D=head_size, bs=block_size, past=past, qlen=q_lens, q_dtype=q_dtype,
                   kv_format=kv_format, scale_mode=scale_mode,
                   kv_in_dtype=kv_in_dtype or ("f32" if q_dtype == "f32" else q_dtype),
                   num_splits=num_splits, kind=kind, spare=spare,
                   gains=kv_format != "fp8", key_scale_override=key_scale,
                   key_code_sigma=key_code_sigma)


def rope_tables(max_position, rotary_dim, base=10000.0):
    """fp32 cos/sin tables (max_position, rotary_dim // 2) of the usual rotary
    angles p * base^(-2k / rotary_dim), computed in fp64 and rounded: inputs
    of the rotary append, like the other seeded inputs here."""
    k = np.arange(rotary_dim // 2, dtype=np.float64)
    ang = np.arange(max_position, dtype=np.float64)[:, None] * base ** (-2.0 * k / rotary_dim)
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)
