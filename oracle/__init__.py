"""Plain fp64 CPU oracle for paged attention over a quantized KV cache.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code,
headers, tables or constants with the HIP library under
``attention_paged_quantized_amd/``; the two meet only through the seeded input
generators in ``workloads/``, which hold none of the method's arithmetic.

Sources.  The operation is defined by five web pages on one subject:
  P1 "ONNX Runtime: INT4 Paged KV Cache" (onnxruntime PR 32515) -- cache shape
     with cache_head_size, nibble packing, per-channel scales folded into Q.
  P2 "INT8-KV Tensor-Core DynamicSparseAttention" (onnxruntime PR 33707) --
     fp32 accumulation checked against an fp64 reference.
  P3 "PagedAttention FA path: exact max_query_len" (onnxruntime PR 28409) --
     cumulative query lengths, exact host maximum, zero-token sequences.
  P4 "GQA GEMV decode kernel" (onnxruntime PR 29216) -- flash decoding
     (split-KV) vs single pass, naive-vs-flash parity.
  P5 "FlashInfer FP8 KV-cache prefill repack" (flashinfer PR 3485) -- FP8 KV.

Modules
  codecs     OCP E4M3 encode/decode, packed INT4 layout.
  quant      symmetric quantizers and the quantize-and-append step.
  attention  paged gather, exact attention, chunked (split-KV) attention,
             exact max_query_len.
  brute      pure-Python scalar-loop attention for tiny inputs.
  rotary     rotary position embedding of the new rows and the fused
             rotate-then-quantize append.
  sparse     block-sparse decode over selected KV blocks.

Every function is pinned by ``tests/test_oracle_*.py`` against closed forms,
library special cases, exhaustive enumeration or brute force.  Nothing here is
"parity unpinned".
"""

from . import codecs, quant, attention, brute, rotary, sparse  # noqa: F401
