"""Test-side helpers that drive the HIP library through its binding.

The device cache pools start poisoned exactly like the oracle's (0x7F), the
past tokens and then the step's new tokens are appended with kv_quant_append,
and the attention call runs on the current torch stream.  Output buffers get
two extra canary rows (NaN) that must survive the call.
"""

import numpy as np
import torch

import attention_paged_quantized_amd as paq

POISON = 0x7F          # same poison byte as the oracle-side pools
COUNTERS = 16384       # int32 arrival counters at the head of a decode workspace

TORCH_DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def desc_for(w, token_count):
    return paq.make_desc(w.batch, token_count, w.num_heads, w.kv_num_heads, w.head_size,
                         w.block_size, w.num_blocks, w.max_blocks_per_seq, w.q_dtype,
                         w.kv_format, w.scale_mode)


class Device:
    """Device-resident copy of a workload's inputs and caches."""

    def __init__(self, w, dev="cuda"):
        self.w = w
        self.dev = dev
        d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
        self.block_table = d(w.block_table)
        self.cum_q = d(w.cum_q)
        self.past = d(w.past_lens)
        self.cum_past = d(w.cum_past)
        self.zeros = torch.zeros(w.batch, dtype=torch.int32, device=dev)
        self.k_scale = d(w.k_scale)
        self.v_scale = d(w.v_scale)
        shape = (w.num_blocks, w.block_size, w.kv_num_heads, w.cache_head_size)
        self.kc = torch.full(shape, POISON, dtype=torch.uint8, device=dev)
        self.vc = torch.full(shape, POISON, dtype=torch.uint8, device=dev)
        self.query = w.query.to(dev)

    def append_past(self):
        w = self.w
        P = int(w.cum_past[-1])
        if P == 0:
            return
        paq.kv_quant_append(desc_for(w, P), w.kv_in_dtype, w.past_key.to(self.dev),
                            w.past_value.to(self.dev), self.kc, self.vc, self.k_scale,
                            self.v_scale, self.block_table, self.cum_past, self.zeros,
                            w.cum_past, np.zeros(w.batch, np.int32))

    def append_new(self):
        w = self.w
        paq.kv_quant_append(desc_for(w, w.token_count), w.kv_in_dtype, w.new_key.to(self.dev),
                            w.new_value.to(self.dev), self.kc, self.vc, self.k_scale,
                            self.v_scale, self.block_table, self.cum_q, self.past, w.cum_q,
                            w.past_lens)

    def fill(self):
        self.append_past()
        self.append_new()
        return self

    def attend(self, num_splits=None, kind=None, softmax_scale=0.0, canary=True):
        """Run decode or prefill; returns the output (T, H, D) on the device and
        checks the canary rows behind it."""
        w = self.w
        T = w.token_count
        kind = kind or w.kind
        S = w.num_splits if num_splits is None else num_splits
        buf = torch.full((T + 2, w.num_heads, w.head_size), float("nan"),
                         dtype=TORCH_DT[w.q_dtype], device=self.dev)
        out = buf[:T]
        desc = desc_for(w, T)
        if kind == "decode":
            nbytes = paq.paged_attn_decode_workspace_size(desc, w.cum_q, w.past_lens, S)
            ws = torch.zeros(max(1, nbytes // 4), dtype=torch.float32, device=self.dev) \
                if nbytes else None
            paq.paged_attn_decode(desc, self.query, out, self.kc, self.vc, self.k_scale,
                                  self.v_scale, self.block_table, self.cum_q, self.past, w.cum_q,
                                  w.past_lens, softmax_scale, S, ws)
            if ws is not None:
                torch.cuda.synchronize()
                # the arrival counters at the head of the workspace are zero again
                assert not ws.view(torch.int32)[:COUNTERS].any(), "counters left non-zero"
        else:
            paq.paged_attn_prefill(desc, self.query, out, self.kc, self.vc, self.k_scale,
                                   self.v_scale, self.block_table, self.cum_q, self.past,
                                   w.cum_q, w.past_lens, softmax_scale)
        torch.cuda.synchronize()
        if canary:
            assert torch.isnan(buf[T:]).all(), "output rows past token_count were written"
        return out
