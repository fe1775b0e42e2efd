"""Paged attention over a quantized (INT8 / packed INT4 / FP8 E4M3) KV cache
for AMD MI355X (gfx950).

A thin ctypes binding of the C ABI in include/paq.h: the functions below have
the same names and arguments as the C entry points and only marshal them
(device tensors -> data pointers, host arrays -> int32 buffers, the current
torch stream -> hipStream_t).  Every step of the computation runs in the HIP
kernels of libpaq.so; there is no Python or CPU fallback, and importing the
functions fails loudly when the library has not been built
(``python -m attention_paged_quantized_amd.build``).
"""

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpaq.so")

PAQ_OK, PAQ_ERR_INVALID_ARG, PAQ_ERR_UNSUPPORTED, PAQ_ERR_WORKSPACE, PAQ_ERR_HIP = range(5)
DTYPES = {"f32": 0, "f16": 1, "bf16": 2}
KV_FORMATS = {"int8": 0, "int4": 1, "fp8": 2}
SCALE_MODES = {"channel": 0, "head": 1}
PATHS = {0: "none", 1: "single", 2: "split", 3: "f32_single", 4: "f32_split", 5: "prefill",
         6: "f32_prefill", 7: "balanced"}
ABI_VERSION = 2

# Every symbol include/paq.h declares.
EXPORTS = ("paq_abi_version", "paq_status_string", "paq_last_error", "paq_plan_decode",
           "paq_plan_prefill", "paged_attn_decode_workspace_size", "paged_attn_decode",
           "paged_attn_prefill", "kv_quant_append", "kv_quant_append_rotary",
           "paged_attn_decode_host", "paged_attn_decode_sparse",
           "paged_attn_decode_sparse_workspace_size", "paged_attn_prefill_padded",
           "paged_attn_decode_noalloc", "paged_attn_prefill_sparse",
           "paged_attn_prefill_sparse_workspace_size", "paged_attn_prefill_k_per_use",
           "paged_attn_decode_append")


class PaqDesc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "token_count", "num_heads", "kv_num_heads", "head_size", "block_size",
        "num_blocks", "max_blocks_per_seq", "q_dtype", "kv_format", "scale_mode")]


class PaqPlan(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "max_query_len", "max_kv_len", "active_seqs", "work_units", "num_splits", "path",
        "grid_x", "grid_y", "grid_z", "waves_per_group", "parts", "parts_per_seq",
        "chunks_per_part", "keys_per_group")] + [
        ("total_tiles", ctypes.c_int64), ("workspace_bytes", ctypes.c_uint64)]


class PaqError(RuntimeError):
    def __init__(self, status, message):
        super().__init__("paq status %d (%s): %s" % (status, status_string(status), message))
        self.status = status


_lib_handle = None
_I32P = ctypes.POINTER(ctypes.c_int32)
_VP = ctypes.c_void_p


def lib():
    """The loaded libpaq.so (raises if it has not been built)."""
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libpaq.so is not built: run "
                              "`python -m attention_paged_quantized_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        L.paq_abi_version.restype = ctypes.c_int32
        L.paq_status_string.restype = ctypes.c_char_p
        L.paq_status_string.argtypes = [ctypes.c_int32]
        L.paq_last_error.restype = ctypes.c_char_p
        L.paq_plan_decode.restype = ctypes.c_int32
        L.paq_plan_decode.argtypes = [ctypes.POINTER(PaqDesc), _I32P, _I32P, ctypes.c_int32,
                                      ctypes.c_int32, ctypes.POINTER(PaqPlan)]
        L.paq_plan_prefill.restype = ctypes.c_int32
        L.paq_plan_prefill.argtypes = [ctypes.POINTER(PaqDesc), _I32P, _I32P,
                                       ctypes.POINTER(PaqPlan)]
        L.paged_attn_decode_workspace_size.restype = ctypes.c_size_t
        L.paged_attn_decode_workspace_size.argtypes = [ctypes.POINTER(PaqDesc), _I32P, _I32P,
                                                       ctypes.c_int32]
        attn = [ctypes.POINTER(PaqDesc), _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                _I32P, _I32P, ctypes.c_float]
        L.paged_attn_decode.restype = ctypes.c_int32
        L.paged_attn_decode.argtypes = attn + [ctypes.c_int32, _VP, ctypes.c_size_t, _VP]
        L.paged_attn_decode_noalloc.restype = ctypes.c_int32
        L.paged_attn_decode_noalloc.argtypes = attn + [ctypes.c_int32, _VP]
        L.paged_attn_prefill.restype = ctypes.c_int32
        L.paged_attn_prefill.argtypes = attn + [_VP]
        L.paged_attn_prefill_k_per_use.restype = ctypes.c_int32
        L.paged_attn_prefill_k_per_use.argtypes = attn + [_VP]
        L.paged_attn_prefill_padded.restype = ctypes.c_int32
        L.paged_attn_prefill_padded.argtypes = attn + [ctypes.c_int32, _VP]
        L.kv_quant_append.restype = ctypes.c_int32
        L.kv_quant_append.argtypes = [ctypes.POINTER(PaqDesc), ctypes.c_int32, _VP, _VP, _VP,
                                      _VP, _VP, _VP, _VP, _VP, _VP, _I32P, _I32P, _VP]
        L.paged_attn_decode_append.restype = ctypes.c_int32
        L.paged_attn_decode_append.argtypes = [ctypes.POINTER(PaqDesc), ctypes.c_int32, _VP,
                                               _VP] + attn[1:] + [ctypes.c_int32, _VP,
                                                                  ctypes.c_size_t, _VP]
        L.paged_attn_decode_sparse.restype = ctypes.c_int32
        L.paged_attn_decode_sparse.argtypes = attn[:-1] + [_VP, _VP, _I32P, ctypes.c_int32,
                                                           ctypes.c_float, ctypes.c_int32, _VP,
                                                           ctypes.c_size_t, _VP]
        L.paged_attn_decode_sparse_workspace_size.restype = ctypes.c_size_t
        L.paged_attn_decode_sparse_workspace_size.argtypes = [ctypes.POINTER(PaqDesc), _I32P,
                                                              _I32P, _I32P, ctypes.c_int32,
                                                              ctypes.c_int32]
        L.paged_attn_prefill_sparse.restype = ctypes.c_int32
        L.paged_attn_prefill_sparse.argtypes = attn[:-1] + [_VP, _VP, _I32P, ctypes.c_int32,
                                                            ctypes.c_float, _VP, ctypes.c_size_t,
                                                            _VP]
        L.paged_attn_prefill_sparse_workspace_size.restype = ctypes.c_size_t
        L.paged_attn_prefill_sparse_workspace_size.argtypes = [ctypes.POINTER(PaqDesc), _I32P,
                                                               _I32P, _I32P, ctypes.c_int32]
        L.paged_attn_decode_host.restype = ctypes.c_int32
        L.paged_attn_decode_host.argtypes = [ctypes.POINTER(PaqDesc), _VP, _VP, _VP, _VP, _VP,
                                             _VP, _VP, _VP, _VP, ctypes.c_float,
                                             ctypes.c_int32, ctypes.c_int32]
        L.kv_quant_append_rotary.restype = ctypes.c_int32
        L.kv_quant_append_rotary.argtypes = [ctypes.POINTER(PaqDesc), ctypes.c_int32, _VP, _VP,
                                             _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _I32P,
                                             _I32P, _VP, _VP, ctypes.c_int32, ctypes.c_int32,
                                             ctypes.c_int32, _VP]
        _lib_handle = L
    return _lib_handle


def status_string(status):
    return lib().paq_status_string(int(status)).decode()


def paq_status_string(status):
    return status_string(status)


def paq_last_error():
    return lib().paq_last_error().decode()


def paq_abi_version():
    return int(lib().paq_abi_version())


def make_desc(batch, token_count, num_heads, kv_num_heads, head_size, block_size, num_blocks,
              max_blocks_per_seq, q_dtype, kv_format, scale_mode):
    """A PaqDesc from Python values (dtype/format/mode names or enum ints)."""
    def enum(v, table):
        return table[v] if isinstance(v, str) else int(v)
    return PaqDesc(int(batch), int(token_count), int(num_heads), int(kv_num_heads),
                   int(head_size), int(block_size), int(num_blocks), int(max_blocks_per_seq),
                   enum(q_dtype, DTYPES), enum(kv_format, KV_FORMATS),
                   enum(scale_mode, SCALE_MODES))


def _host_i32(a):
    """Host int32 array -> (keepalive, pointer); None -> NULL."""
    if a is None:
        return None, None
    if hasattr(a, "cpu") and hasattr(a, "numpy"):
        a = a.cpu().numpy()
    arr = np.ascontiguousarray(np.asarray(a, dtype=np.int32))
    return arr, arr.ctypes.data_as(_I32P)


def _dev(t):
    """Device tensor -> data pointer (None -> NULL)."""
    if t is None:
        return None
    if not getattr(t, "is_cuda", False):
        raise ValueError("expected a device (cuda/hip) tensor")
    if not t.is_contiguous():
        raise ValueError("device tensors must be contiguous")
    return t.data_ptr()


def _stream(stream):
    if stream is not None:
        return getattr(stream, "cuda_stream", stream)
    import torch
    return torch.cuda.current_stream().cuda_stream


def _check(status):
    if status != PAQ_OK:
        raise PaqError(status, paq_last_error())


def paq_plan_decode(desc, cum_q_host, past_lens_host, num_splits=0, num_cus=0):
    a, pa = _host_i32(cum_q_host)
    b, pb = _host_i32(past_lens_host)
    plan = PaqPlan()
    _check(lib().paq_plan_decode(ctypes.byref(desc), pa, pb, int(num_splits), int(num_cus),
                                 ctypes.byref(plan)))
    return plan


def paq_plan_prefill(desc, cum_q_host, past_lens_host):
    a, pa = _host_i32(cum_q_host)
    b, pb = _host_i32(past_lens_host)
    plan = PaqPlan()
    _check(lib().paq_plan_prefill(ctypes.byref(desc), pa, pb, ctypes.byref(plan)))
    return plan


def paged_attn_decode_workspace_size(desc, cum_q_host, past_lens_host, num_splits=0):
    a, pa = _host_i32(cum_q_host)
    b, pb = _host_i32(past_lens_host)
    return int(lib().paged_attn_decode_workspace_size(ctypes.byref(desc), pa, pb,
                                                      int(num_splits)))


def paged_attn_decode(desc, query, out, key_cache, value_cache, k_scale, v_scale, block_table,
                      cum_q, past_lens, cum_q_host, past_lens_host, softmax_scale=0.0,
                      num_splits=0, workspace=None, stream=None):
    """GQA decode through the C ABI.  `workspace` (device tensor of at least
    paged_attn_decode_workspace_size() bytes, or None for a single pass) must
    be zero-filled when allocated: its leading arrival counters have to be
    zero when a split call starts, and every call leaves them zero."""
    a, pa = _host_i32(cum_q_host)
    b, pb = _host_i32(past_lens_host)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().paged_attn_decode(
        ctypes.byref(desc), _dev(query), _dev(out), _dev(key_cache), _dev(value_cache),
        _dev(k_scale), _dev(v_scale), _dev(block_table), _dev(cum_q), _dev(past_lens), pa, pb,
        float(softmax_scale), int(num_splits), _dev(workspace), ws_bytes, _stream(stream)))


def paged_attn_decode_append(desc, kv_in_dtype, key, value, query, out, key_cache, value_cache,
                             k_scale, v_scale, block_table, cum_q, past_lens, cum_q_host,
                             past_lens_host, softmax_scale=0.0, num_splits=0, workspace=None,
                             stream=None):
    """kv_quant_append of the step's new key/value rows followed by
    paged_attn_decode, in one call (the decode kernel appends the rows itself
    where it can).  Same workspace rule as paged_attn_decode."""
    a, pa = _host_i32(cum_q_host)
    b, pb = _host_i32(past_lens_host)
    dt = DTYPES[kv_in_dtype] if isinstance(kv_in_dtype, str) else int(kv_in_dtype)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().paged_attn_decode_append(
        ctypes.byref(desc), dt, _dev(key), _dev(value), _dev(query), _dev(out), _dev(key_cache),
        _dev(value_cache), _dev(k_scale), _dev(v_scale), _dev(block_table), _dev(cum_q),
        _dev(past_lens), pa, pb, float(softmax_scale), int(num_splits), _dev(workspace), ws_bytes,
        _stream(stream)))


def paged_attn_decode_noalloc(desc, query, out, key_cache, value_cache, k_scale, v_scale,
                              block_table, cum_q, past_lens, cum_q_host, past_lens_host,
                              softmax_scale=0.0, num_splits=0, stream=None):
    """paged_attn_decode with the library's own per-GPU scratch as workspace
    (no allocation; calls on one GPU must not overlap)."""
    a, pa = _host_i32(cum_q_host)
    b, pb = _host_i32(past_lens_host)
    _check(lib().paged_attn_decode_noalloc(
        ctypes.byref(desc), _dev(query), _dev(out), _dev(key_cache), _dev(value_cache),
        _dev(k_scale), _dev(v_scale), _dev(block_table), _dev(cum_q), _dev(past_lens), pa, pb,
        float(softmax_scale), int(num_splits), _stream(stream)))


def paged_attn_prefill(desc, query, out, key_cache, value_cache, k_scale, v_scale, block_table,
                       cum_q, past_lens, cum_q_host, past_lens_host, softmax_scale=0.0,
                       stream=None):
    a, pa = _host_i32(cum_q_host)
    b, pb = _host_i32(past_lens_host)
    _check(lib().paged_attn_prefill(
        ctypes.byref(desc), _dev(query), _dev(out), _dev(key_cache), _dev(value_cache),
        _dev(k_scale), _dev(v_scale), _dev(block_table), _dev(cum_q), _dev(past_lens), pa, pb,
        float(softmax_scale), _stream(stream)))


def paged_attn_prefill_padded(desc, query, out, key_cache, value_cache, k_scale, v_scale,
                              block_table, cum_q, past_lens, cum_q_host, past_lens_host,
                              max_query_len, softmax_scale=0.0, stream=None):
    """paged_attn_prefill with the grid sized from max_query_len (>= the exact
    maximum) for every (sequence, kv head) pair."""
    a, pa = _host_i32(cum_q_host)
    b, pb = _host_i32(past_lens_host)
    _check(lib().paged_attn_prefill_padded(
        ctypes.byref(desc), _dev(query), _dev(out), _dev(key_cache), _dev(value_cache),
        _dev(k_scale), _dev(v_scale), _dev(block_table), _dev(cum_q), _dev(past_lens), pa, pb,
        float(softmax_scale), int(max_query_len), _stream(stream)))


def paged_attn_prefill_k_per_use(desc, query, out, key_cache, value_cache, k_scale, v_scale,
                                 block_table, cum_q, past_lens, cum_q_host, past_lens_host,
                                 softmax_scale=0.0, stream=None):
    """paged_attn_prefill with K codes kept raw in LDS and converted by every
    wave at each use (the staging scheme the default is compared with)."""
    a, pa = _host_i32(cum_q_host)
    b, pb = _host_i32(past_lens_host)
    _check(lib().paged_attn_prefill_k_per_use(
        ctypes.byref(desc), _dev(query), _dev(out), _dev(key_cache), _dev(value_cache),
        _dev(k_scale), _dev(v_scale), _dev(block_table), _dev(cum_q), _dev(past_lens), pa, pb,
        float(softmax_scale), _stream(stream)))


def kv_quant_append(desc, kv_in_dtype, key, value, key_cache, value_cache, k_scale, v_scale,
                    block_table, cum_q, past_lens, cum_q_host, past_lens_host, stream=None):
    a, pa = _host_i32(cum_q_host)
    b, pb = _host_i32(past_lens_host)
    dt = DTYPES[kv_in_dtype] if isinstance(kv_in_dtype, str) else int(kv_in_dtype)
    _check(lib().kv_quant_append(
        ctypes.byref(desc), dt, _dev(key), _dev(value), _dev(key_cache), _dev(value_cache),
        _dev(k_scale), _dev(v_scale), _dev(block_table), _dev(cum_q), _dev(past_lens), pa, pb,
        _stream(stream)))


def kv_quant_append_rotary(desc, kv_in_dtype, query, key, value, key_cache, value_cache,
                           k_scale, v_scale, block_table, cum_q, past_lens, cum_q_host,
                           past_lens_host, cos_cache, sin_cache, rotary_dim, interleaved=False,
                           stream=None):
    """kv_quant_append with rotary embedding of the new query (in place; None
    skips it) and key rows first.  cos_cache/sin_cache: fp32 device tensors
    (max_position, rotary_dim // 2)."""
    a, pa = _host_i32(cum_q_host)
    b, pb = _host_i32(past_lens_host)
    dt = DTYPES[kv_in_dtype] if isinstance(kv_in_dtype, str) else int(kv_in_dtype)
    max_position = int(cos_cache.shape[0]) if cos_cache is not None else 0
    _check(lib().kv_quant_append_rotary(
        ctypes.byref(desc), dt, _dev(query), _dev(key), _dev(value), _dev(key_cache),
        _dev(value_cache), _dev(k_scale), _dev(v_scale), _dev(block_table), _dev(cum_q),
        _dev(past_lens), pa, pb, _dev(cos_cache), _dev(sin_cache), max_position, int(rotary_dim),
        1 if interleaved else 0, _stream(stream)))


def paged_attn_decode_host(desc, query, out, key_cache, value_cache, k_scale, v_scale,
                           block_table, cum_q, past_lens, softmax_scale=0.0, num_splits=0,
                           num_threads=0):
    """Decode on the host CPU.  Every array is a host numpy array: query/out
    float32 (T, H, D), caches uint8, scales float32, table/cum_q/past int32
    (C-contiguous; out is written)."""
    import numpy as np

    def host(x, dtype):
        if not isinstance(x, np.ndarray) or x.dtype != dtype or not x.flags["C_CONTIGUOUS"]:
            raise ValueError("expected a C-contiguous %s numpy array" % np.dtype(dtype).name)
        return x.ctypes.data

    if not out.flags["WRITEABLE"]:
        raise ValueError("out must be writeable")
    _check(lib().paged_attn_decode_host(
        ctypes.byref(desc), host(query, np.float32), host(out, np.float32),
        host(key_cache, np.uint8), host(value_cache, np.uint8), host(k_scale, np.float32),
        host(v_scale, np.float32), host(block_table, np.int32), host(cum_q, np.int32),
        host(past_lens, np.int32), float(softmax_scale), int(num_splits), int(num_threads)))


def paged_attn_decode_sparse_workspace_size(desc, cum_q_host, past_lens_host, num_sel_host,
                                            max_sel, num_splits=0):
    a, pa = _host_i32(cum_q_host)
    b, pb = _host_i32(past_lens_host)
    c, pc = _host_i32(num_sel_host)
    return int(lib().paged_attn_decode_sparse_workspace_size(ctypes.byref(desc), pa, pb, pc,
                                                             int(max_sel), int(num_splits)))


def paged_attn_decode_sparse(desc, query, out, key_cache, value_cache, k_scale, v_scale,
                             block_table, cum_q, past_lens, cum_q_host, past_lens_host,
                             sel_blocks, num_sel, num_sel_host, softmax_scale=0.0, num_splits=0,
                             workspace=None, stream=None):
    """Block-sparse decode: sel_blocks (batch, max_sel) and num_sel (batch) are
    int32 device tensors; num_sel_host their host copy."""
    a, pa = _host_i32(cum_q_host)
    b, pb = _host_i32(past_lens_host)
    c, pc = _host_i32(num_sel_host)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().paged_attn_decode_sparse(
        ctypes.byref(desc), _dev(query), _dev(out), _dev(key_cache), _dev(value_cache),
        _dev(k_scale), _dev(v_scale), _dev(block_table), _dev(cum_q), _dev(past_lens), pa, pb,
        _dev(sel_blocks), _dev(num_sel), pc, int(sel_blocks.shape[1]), float(softmax_scale),
        int(num_splits), _dev(workspace), ws_bytes, _stream(stream)))


def paged_attn_prefill_sparse_workspace_size(desc, cum_q_host, past_lens_host, num_sel_host,
                                             max_sel):
    a, pa = _host_i32(cum_q_host)
    b, pb = _host_i32(past_lens_host)
    c, pc = _host_i32(num_sel_host)
    return int(lib().paged_attn_prefill_sparse_workspace_size(ctypes.byref(desc), pa, pb, pc,
                                                              int(max_sel)))


def paged_attn_prefill_sparse(desc, query, out, key_cache, value_cache, k_scale, v_scale,
                              block_table, cum_q, past_lens, cum_q_host, past_lens_host,
                              sel_blocks, num_sel, num_sel_host, softmax_scale=0.0,
                              workspace=None, stream=None):
    """Block-sparse prefill: sel_blocks (batch, max_sel) and num_sel (batch) are
    int32 device tensors (None, None with max_sel 0: local blocks only);
    num_sel_host their host copy."""
    a, pa = _host_i32(cum_q_host)
    b, pb = _host_i32(past_lens_host)
    c, pc = _host_i32(num_sel_host)
    max_sel = 0 if sel_blocks is None else int(sel_blocks.shape[1])
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().paged_attn_prefill_sparse(
        ctypes.byref(desc), _dev(query), _dev(out), _dev(key_cache), _dev(value_cache),
        _dev(k_scale), _dev(v_scale), _dev(block_table), _dev(cum_q), _dev(past_lens), pa, pb,
        _dev(sel_blocks), _dev(num_sel), pc, max_sel, float(softmax_scale), _dev(workspace),
        ws_bytes, _stream(stream)))
