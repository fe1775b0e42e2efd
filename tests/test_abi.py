"""CPU tests of the C-ABI library: it loads, exports every symbol the header
declares, and its host logic (validation, exact max_query_len, split planning,
workspace sizing) behaves as documented.  No kernel is launched: every call
here either fails validation or has nothing to launch."""

import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import attention_paged_quantized_amd as paq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "paq.h")
FAKE = 0x10000          # a non-NULL "device" pointer that is never dereferenced


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_symbol():
    L = paq.lib()
    names = _declared_functions()
    assert sorted(names) == sorted(paq.EXPORTS)
    for n in names:
        assert hasattr(L, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", paq.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert set(names) <= exported


def test_abi_version_and_status_strings():
    assert paq.paq_abi_version() == paq.ABI_VERSION == 2
    assert paq.paq_status_string(0) == "ok"
    assert "workspace" in paq.paq_status_string(3)
    assert paq.paq_status_string(99) == "unknown status"


def _desc(B, T, H=32, hkv=8, D=128, bs=16, nb=100, mb=10, q="f16", fmt="int8", mode="channel"):
    return paq.make_desc(B, T, H, hkv, D, bs, nb, mb, q, fmt, mode)


def _cum(qlens):
    return np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)


def _align(x, a=256):
    return (x + a - 1) // a * a


COUNTER_BYTES = 16384 * 4      # arrival counters at the head of every decode workspace


def test_plan_decode_paths_and_workspace():
    # tiny decode: fp32 queries -> the portable fp32 kernel, one pass
    d = paq.make_desc(3, 2, 4, 2, 64, 16, 24, 8, "f32", "int8", "channel")
    p = paq.paq_plan_decode(d, [0, 1, 2, 2], [37, 100, 0], 0, 256)
    assert (p.max_query_len, p.max_kv_len, p.active_seqs, p.work_units) == (1, 101, 2, 4)
    assert paq.PATHS[p.path] == "f32_single" or paq.PATHS[p.path] == "f32_split"
    # long INT4 decode with 128 chunks: one wave per pair of INT4 kv heads (a
    # 128-byte line) -> 4 head groups; 4 sequences x 4 groups = 16 units, so
    # about one workgroup per CU needs 16 parts of 8 chunks per sequence
    d = _desc(4, 4, bs=32, nb=4200, mb=1025, fmt="int4")
    p = paq.paq_plan_decode(d, _cum([1] * 4), [32768] * 4, 128, 256)
    assert paq.PATHS[p.path] == "split" and p.num_splits == 128
    assert (p.parts_per_seq, p.chunks_per_part, p.parts) == (16, 8, 64)
    assert (p.grid_x, p.grid_y, p.grid_z, p.waves_per_group) == (64 * 4, 1, 1, 8)
    # workspace: counters, then one partial (D fp32) and one (max, sum) pair per
    # part and query head
    slots = 64 * 32
    al = lambda x: -(-x // 256) * 256
    assert p.workspace_bytes == COUNTER_BYTES + al(slots * 128 * 4) + al(slots * 2 * 4)
    # (sizing without a plan of its own uses the device's compute units, or
    # 256 when no GPU is visible -- as here, and as on an MI355X)
    assert paq.paged_attn_decode_workspace_size(d, _cum([1] * 4), [32768] * 4, 128) == \
        p.workspace_bytes
    # 256 (sequence, kv head) units fill 256 CUs: the automatic choice is one pass
    d = _desc(32, 32, mb=257, nb=6000)
    past = [1024 + 96 * b for b in range(32)]
    p = paq.paq_plan_decode(d, _cum([1] * 32), past, 0, 256)
    assert paq.PATHS[p.path] == "single" and p.workspace_bytes == 0
    # under-filled with near-uniform lengths: block-aligned chunks, about two
    # workgroups per CU (4 sequences x 4 INT4 head groups = 16 units -> 32)
    d4 = _desc(4, 4, bs=32, nb=4200, mb=1025, fmt="int4")
    p = paq.paq_plan_decode(d4, _cum([1] * 4), [32768] * 4, 0, 256)
    assert paq.PATHS[p.path] == "split" and p.num_splits == 32
    # under-filled with skewed lengths (longest > 1.5 x mean): the
    # length-balanced partition over one workgroup per CU, each streaming an
    # equal share of the 32-key tiles of all (sequence, kv head) pairs; a
    # workgroup keeps partials for its first and last pieces
    dk = _desc(4, 4, mb=2000, nb=9000)
    pk = [30000, 100, 200, 300]
    p = paq.paq_plan_decode(dk, _cum([1] * 4), pk, 0, 256)
    assert paq.PATHS[p.path] == "balanced" and p.num_splits == 0
    total = sum(-(-(x + 1) // 32) for x in pk) * 8
    assert p.total_tiles == total and p.parts == 256 and p.grid_x == 256
    assert p.keys_per_group == 32 * -(-total // 256)
    rows = 2 * 256 * 4                  # slots x query heads per head group
    assert p.workspace_bytes == COUNTER_BYTES + al(rows * 128 * 4) + al(rows * 2 * 4)
    # an explicit length-balanced split: -N workgroups
    p = paq.paq_plan_decode(d, _cum([1] * 32), past, -100, 256)
    assert paq.PATHS[p.path] == "balanced" and p.parts == 100 and p.grid_x == 100
    # enough units for the dispatcher alone: one pass, no workspace
    d = _desc(256, 256, mb=257, nb=60000)
    p = paq.paq_plan_decode(d, _cum([1] * 256), [2000] * 256, 0, 256)
    assert paq.PATHS[p.path] == "single" and p.workspace_bytes == 0
    # short sequences are not split
    p = paq.paq_plan_decode(_desc(2, 2), _cum([1, 1]), [10, 100], 0, 256)
    assert p.num_splits == 1 and paq.PATHS[p.path] == "single"


@pytest.mark.parametrize("cus", [32, 256, 304])
def test_plan_decode_split_follows_the_compute_units(cus):
    """The split partition is sized for the compute units it is planned for,
    and the plan carries everything the launch uses: parts x chunks per part
    cover every chunk, the grid is parts x head groups, and the workspace
    holds a partial for every part and query head."""
    d = _desc(4, 4, bs=32, nb=4200, mb=1025, fmt="int4")
    p = paq.paq_plan_decode(d, _cum([1] * 4), [32768] * 4, 128, cus)
    assert p.parts_per_seq * p.chunks_per_part >= 128
    assert (p.parts_per_seq - 1) * p.chunks_per_part < 128
    assert p.parts == 4 * p.parts_per_seq and p.grid_x == 4 * p.parts
    assert p.grid_x >= min(cus, 4 * 4 * 128) * 0.5
    al = lambda x: -(-x // 256) * 256
    slots = p.parts * 32
    assert p.workspace_bytes == COUNTER_BYTES + al(slots * 128 * 4) + al(slots * 2 * 4)


def test_plan_decode_rejects_bad_balanced_requests():
    d = _desc(2, 2)
    with pytest.raises(paq.PaqError):
        paq.paq_plan_decode(d, _cum([1, 1]), [100, 300], -257, 256)      # > 256 workgroups
    # fewer tiles than workgroups: one workgroup per tile at most
    p = paq.paq_plan_decode(d, _cum([1, 1]), [10, 40], -200, 256)
    assert p.parts == p.total_tiles == (1 + 2) * 8


def test_plan_prefill_uses_exact_max_query_len():
    # q_lens {5,0,0}: the heuristic token_count-batch+1 would give 3
    d = _desc(3, 5, mb=4)
    p = paq.paq_plan_prefill(d, _cum([5, 0, 0]), [0, 7, 3])
    assert p.max_query_len == 5 and p.active_seqs == 1
    # one 32-token query tile (4 waves x 8 tokens at group 4) for each kv head of
    # the one sequence with rows: one workgroup on each of the 8 XCDs, none for
    # the empty sequences
    assert (p.grid_x, p.grid_y, p.grid_z) == (8, 1, 1)
    # ragged: q_lens {70, 1, 33} -> 3 + 1 + 2 tiles for every kv head; with 8 kv
    # heads XCD x takes head x of every sequence: 6 items each
    p = paq.paq_plan_prefill(_desc(3, 104, mb=8), _cum([70, 1, 33]), [0, 5, 9])
    assert p.grid_x == 8 * 6
    # 2 kv heads x 5 sequences = 10 pairs: XCDs 0 and 1 take pairs {0, 8} and
    # {1, 9} (sequences 0 and 4), the others one pair each
    p = paq.paq_plan_prefill(_desc(5, 140, H=8, hkv=2, mb=8), _cum([64, 0, 0, 0, 76]),
                             [0] * 5)
    assert p.grid_x == 8 * (2 + 3)
    # the exact maximum sizes the grid: 2048 tokens -> 64 query tiles per pair
    p = paq.paq_plan_prefill(_desc(4, 8192, mb=128), _cum([2048] * 4), [0] * 4)
    assert p.grid_x == 64 * 8 * 4
    # {1,0,0,0}: the heuristic would be -2 (an invalid grid)
    p = paq.paq_plan_prefill(_desc(4, 1, mb=4), _cum([1, 0, 0, 0]), [3, 0, 0, 0])
    assert p.max_query_len == 1
    # every sequence empty: nothing to launch
    p = paq.paq_plan_prefill(_desc(3, 0, mb=4), _cum([0, 0, 0]), [5, 0, 2])
    assert paq.PATHS[p.path] == "none"


def _call_decode(d, cum, past, splits=1, ws=None, ws_bytes=0, ptr=FAKE):
    L = paq.lib()
    a, pa = paq._host_i32(cum)
    b, pb = paq._host_i32(past)
    return L.paged_attn_decode(ctypes.byref(d), ptr, ptr, ptr, ptr, ptr, ptr, ptr, ptr, ptr,
                               pa, pb, 0.0, splits, ws, ws_bytes, None)


def _call_prefill(d, cum, past, ptr=FAKE):
    L = paq.lib()
    a, pa = paq._host_i32(cum)
    b, pb = paq._host_i32(past)
    return L.paged_attn_prefill(ctypes.byref(d), ptr, ptr, ptr, ptr, ptr, ptr, ptr, ptr, ptr,
                                pa, pb, 0.0, None)


def _call_append(d, cum, past, in_dtype=1, ptr=FAKE):
    L = paq.lib()
    a, pa = paq._host_i32(cum)
    b, pb = paq._host_i32(past)
    return L.kv_quant_append(ctypes.byref(d), in_dtype, ptr, ptr, ptr, ptr, ptr, ptr, ptr, ptr,
                             ptr, pa, pb, None)


def _call_rotary(d, cum, past, rd=64, il=0, maxpos=4096, ptr=FAKE, cs=FAKE, query=FAKE):
    L = paq.lib()
    a, pa = paq._host_i32(cum)
    b, pb = paq._host_i32(past)
    return L.kv_quant_append_rotary(ctypes.byref(d), 1, query, ptr, ptr, ptr, ptr, ptr, ptr, ptr,
                                    ptr, ptr, pa, pb, cs, cs, maxpos, rd, il, None)


BAD_CASES = [
    # (description, desc kwargs, q_lens/cum, past, expected status)
    ("cum_q decreases", dict(B=3, T=2), [0, 2, 1, 2], [1, 1, 1], paq.PAQ_ERR_INVALID_ARG),
    ("cum_q[B] != token_count", dict(B=2, T=5), [0, 1, 2], [1, 1], paq.PAQ_ERR_INVALID_ARG),
    ("cum_q[0] != 0", dict(B=2, T=2), [1, 1, 2], [1, 1], paq.PAQ_ERR_INVALID_ARG),
    ("negative past", dict(B=2, T=2), [0, 1, 2], [1, -1], paq.PAQ_ERR_INVALID_ARG),
    ("block table too short", dict(B=2, T=2, mb=2), [0, 1, 2], [31, 32],
     paq.PAQ_ERR_INVALID_ARG),
    ("H not a multiple of Hkv", dict(B=1, T=1, H=30), [0, 1], [4], paq.PAQ_ERR_INVALID_ARG),
    ("head_size 96", dict(B=1, T=1, D=96), [0, 1], [4], paq.PAQ_ERR_UNSUPPORTED),
    ("block_size 8", dict(B=1, T=1, bs=8), [0, 1], [4], paq.PAQ_ERR_UNSUPPORTED),
    ("negative batch", dict(B=-1, T=0), [0], [0], paq.PAQ_ERR_INVALID_ARG),
    ("no blocks but tokens", dict(B=1, T=1, nb=0), [0, 1], [4], paq.PAQ_ERR_INVALID_ARG),
]


@pytest.mark.parametrize("name,kw,cum,past,status", BAD_CASES, ids=[c[0] for c in BAD_CASES])
def test_invalid_arguments_are_rejected_before_launch(name, kw, cum, past, status):
    d = _desc(**kw)
    assert _call_decode(d, cum, past) == status, paq.paq_last_error()
    assert paq.paq_last_error()
    assert _call_prefill(d, cum, past) == status
    assert _call_append(d, cum, past) == status
    assert _call_rotary(d, cum, past) == status


def test_rotary_specific_checks():
    d = _desc(2, 2)
    cum, past = [0, 1, 2], [4, 9]
    for rd in (0, -16, 3, 130, 144):                     # odd, non-positive, > head_size
        assert _call_rotary(d, cum, past, rd=rd) == paq.PAQ_ERR_INVALID_ARG, rd
    assert _call_rotary(d, cum, past, rd=24) == paq.PAQ_ERR_UNSUPPORTED
    assert "multiple of 16" in paq.paq_last_error()
    assert _call_rotary(d, cum, past, il=2) == paq.PAQ_ERR_INVALID_ARG
    assert _call_rotary(d, cum, past, maxpos=0) == paq.PAQ_ERR_INVALID_ARG
    # the last new row of sequence 1 sits at position 9: a table of 9 rows is short
    assert _call_rotary(d, cum, past, maxpos=9) == paq.PAQ_ERR_INVALID_ARG
    assert "position 9" in paq.paq_last_error()
    # an empty sequence needs no table row, whatever its past
    assert _call_rotary(_desc(2, 1), [0, 1, 1], [4, 1000], maxpos=5, cs=FAKE + 4) == \
        paq.PAQ_ERR_INVALID_ARG                          # misaligned tables
    assert "aligned" in paq.paq_last_error()
    assert _call_rotary(d, cum, past, cs=None) == paq.PAQ_ERR_INVALID_ARG
    assert _call_rotary(d, cum, past, ptr=None) == paq.PAQ_ERR_INVALID_ARG
    # nothing to do: no launch, NULL pointers accepted
    assert _call_rotary(_desc(2, 0), [0, 0, 0], [4, 9], ptr=None, cs=None, query=None) == \
        paq.PAQ_OK


def test_decode_specific_checks():
    d = _desc(2, 3)
    assert _call_decode(d, [0, 2, 3], [4, 4]) == paq.PAQ_ERR_INVALID_ARG     # q_len 2
    assert "q_len" in paq.paq_last_error()
    assert _call_decode(_desc(1, 1), [0, 1], [4], splits=-257) == paq.PAQ_ERR_UNSUPPORTED
    # split decode without (or with too small) a workspace
    assert _call_decode(_desc(1, 1), [0, 1], [100], splits=4) == paq.PAQ_ERR_WORKSPACE
    assert _call_decode(_desc(1, 1), [0, 1], [100], splits=4, ws=FAKE, ws_bytes=64) == \
        paq.PAQ_ERR_WORKSPACE
    # NULL device pointers are caught once there is work
    assert _call_decode(_desc(1, 1), [0, 1], [4], ptr=None) == paq.PAQ_ERR_INVALID_ARG


def _call_decode_append(d, cum, past, kv_in=1, key=FAKE, splits=1, ws=None, ws_bytes=0):
    L = paq.lib()
    a, pa = paq._host_i32(cum)
    b, pb = paq._host_i32(past)
    return L.paged_attn_decode_append(ctypes.byref(d), kv_in, key, FAKE, FAKE, FAKE, FAKE, FAKE,
                                      FAKE, FAKE, FAKE, FAKE, FAKE, pa, pb, 0.0, splits, ws,
                                      ws_bytes, None)


def test_decode_append_checks():
    """The fused decode step refuses what either of its operations refuses,
    before anything is launched."""
    d = _desc(2, 3)
    assert _call_decode_append(d, [0, 2, 3], [4, 4]) == paq.PAQ_ERR_INVALID_ARG   # q_len 2
    d = _desc(1, 1)
    assert _call_decode_append(d, [0, 1], [4], kv_in=9) == paq.PAQ_ERR_INVALID_ARG
    assert "kv_in_dtype" in paq.paq_last_error()
    assert _call_decode_append(d, [0, 1], [4], key=None) == paq.PAQ_ERR_INVALID_ARG
    assert _call_decode_append(d, [0, 1], [100], splits=4) == paq.PAQ_ERR_WORKSPACE
    assert _call_decode_append(d, [0, 1], [100], splits=4, ws=FAKE, ws_bytes=64) == \
        paq.PAQ_ERR_WORKSPACE
    # no new token: nothing to append or attend, NULL rows accepted
    assert _call_decode_append(_desc(1, 0), [0, 0], [4], key=None) == paq.PAQ_OK


def test_bad_enums_and_null_host_arrays():
    assert _call_decode(_desc(1, 1, q="f16", fmt=7), [0, 1], [0]) == paq.PAQ_ERR_INVALID_ARG
    assert _call_decode(_desc(1, 1, mode=5), [0, 1], [0]) == paq.PAQ_ERR_INVALID_ARG
    assert _call_append(_desc(1, 1), [0, 1], [0], in_dtype=9) == paq.PAQ_ERR_INVALID_ARG
    L = paq.lib()
    d = _desc(1, 1)
    assert L.paged_attn_prefill(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                FAKE, None, None, 0.0, None) == paq.PAQ_ERR_INVALID_ARG


def test_nothing_to_do_returns_ok_without_touching_the_device():
    # zero-token step (every q_len 0): no launch, even with NULL device pointers
    d = _desc(3, 0)
    assert _call_decode(d, [0, 0, 0, 0], [5, 0, 9], ptr=None) == paq.PAQ_OK
    assert _call_prefill(d, [0, 0, 0, 0], [5, 0, 9], ptr=None) == paq.PAQ_OK
    assert _call_append(d, [0, 0, 0, 0], [5, 0, 9], ptr=None) == paq.PAQ_OK
    # empty batch
    d = _desc(0, 0)
    assert _call_decode(d, [0], [], ptr=None) == paq.PAQ_OK
    assert _call_prefill(d, [0], [], ptr=None) == paq.PAQ_OK


def test_binding_refuses_host_tensors():
    import torch
    d = _desc(1, 1)
    x = torch.zeros(4)
    with pytest.raises(ValueError):
        paq.paged_attn_prefill(d, x, x, x, x, x, x, x, x, x, [0, 1], [0], stream=0)


def test_sparse_decode_checks():
    L = paq.lib()
    d = _desc(2, 2)
    cum, past = [0, 1, 2], [40, 9]                    # 41 and 10 keys: 3 and 1 blocks of 16
    assert paq.paged_attn_decode_sparse_workspace_size(d, cum, past, [2, 1], 3, 1) > 0
    assert paq.paged_attn_decode_sparse_workspace_size(d, cum, past, [4, 1], 4, 1) == 0  # > 3 blocks
    assert paq.paged_attn_decode_sparse_workspace_size(d, cum, past, [0, 1], 3, 1) == 0  # none
    assert paq.paged_attn_decode_sparse_workspace_size(d, cum, past, [2, 1], 1, 1) == 0  # > max_sel
    a, pa = paq._host_i32(cum)
    b, pb = paq._host_i32(past)
    c, pc = paq._host_i32([2, 2])                    # sequence 1 has only one block
    rc = L.paged_attn_decode_sparse(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                    FAKE, FAKE, pa, pb, FAKE, FAKE, pc, 3, 0.0, 1, FAKE, 1 << 20,
                                    None)
    assert rc == paq.PAQ_ERR_INVALID_ARG and "selects 2 blocks" in paq.paq_last_error()
    c, pc = paq._host_i32([2, 1])
    rc = L.paged_attn_decode_sparse(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                    FAKE, FAKE, pa, pb, FAKE, FAKE, pc, 3, 0.0, 1, FAKE, 16, None)
    assert rc == paq.PAQ_ERR_WORKSPACE
    # the host key counts of a sparse call are upper bounds (the device knows
    # the exact ones), so the length-balanced partition, which cuts tiles by
    # the host counts, is refused; the automatic choice never takes it
    rc = L.paged_attn_decode_sparse(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                    FAKE, FAKE, pa, pb, FAKE, FAKE, pc, 3, 0.0, -4, FAKE, 1 << 20,
                                    None)
    assert rc == paq.PAQ_ERR_UNSUPPORTED and "exact key counts" in paq.paq_last_error()
    assert paq.paged_attn_decode_sparse_workspace_size(d, cum, past, [2, 1], 3, -4) == 0


def test_sparse_decode_automatic_never_balanced():
    """A skewed batch under-filling the device: the dense decode plans the
    length-balanced partition, the sparse decode over the same lengths a
    chunk partition."""
    d = _desc(6, 6, nb=2000, mb=200)
    cum = list(range(7))
    past = [3000, 600, 700, 650, 800, 620]
    p = paq.paq_plan_decode(d, cum, past, 0)
    assert paq.PATHS[p.path] == "balanced"
    ws = paq.paged_attn_decode_sparse_workspace_size(d, cum, past, [188, 38, 44, 41, 50, 39],
                                                     188, 0)
    assert ws > 0


def test_sparse_prefill_checks():
    """Selections reach only blocks before the first new token; the workspace
    holds the compact table (max_sel + the most local blocks per row) and the
    effective past lengths; refusals come before any launch."""
    L = paq.lib()
    d = _desc(3, 25)
    cum, past = [0, 10, 10, 25], [40, 5, 16]       # local blocks: 2..3, none, 1..1
    # 40 // 16 = 2 earlier blocks for sequence 0, 1 for sequence 2
    ws = paq.paged_attn_prefill_sparse_workspace_size(d, cum, past, [2, 0, 1], 2)
    assert ws == _align(3 * (2 + 2) * 4) + _align(3 * 4)
    assert paq.paged_attn_prefill_sparse_workspace_size(d, cum, past, None, 0) == \
        _align(3 * 2 * 4) + _align(3 * 4)
    assert paq.paged_attn_prefill_sparse_workspace_size(d, cum, past, [3, 0, 1], 3) == 0
    assert paq.paged_attn_prefill_sparse_workspace_size(d, cum, past, [0, 0, 2], 2) == 0
    assert paq.paged_attn_prefill_sparse_workspace_size(d, cum, past, [2, 0, 1], 1) == 0
    # sequence 1 has no new row: its count is not read
    assert paq.paged_attn_prefill_sparse_workspace_size(d, cum, past, [2, 99, 1], 2) > 0
    a, pa = paq._host_i32(cum)
    b, pb = paq._host_i32(past)
    c, pc = paq._host_i32([0, 0, 2])
    rc = L.paged_attn_prefill_sparse(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                     FAKE, FAKE, pa, pb, FAKE, FAKE, pc, 2, 0.0, FAKE, 1 << 20,
                                     None)
    assert rc == paq.PAQ_ERR_INVALID_ARG and "selects 2 blocks" in paq.paq_last_error()
    c, pc = paq._host_i32([2, 0, 1])
    rc = L.paged_attn_prefill_sparse(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                     FAKE, FAKE, pa, pb, FAKE, FAKE, pc, 2, 0.0, FAKE, 16, None)
    assert rc == paq.PAQ_ERR_WORKSPACE
    rc = L.paged_attn_prefill_sparse(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                     FAKE, FAKE, pa, pb, None, None, pc, 2, 0.0, FAKE, 1 << 20,
                                     None)
    assert rc == paq.PAQ_ERR_INVALID_ARG and "sel_blocks" in paq.paq_last_error()


def test_prefill_k_per_use_refusals():
    """The per-use K conversion variant exists for 16-bit queries over 1-byte
    codes at head size 128; anything else is refused before launch."""
    L = paq.lib()
    cum, past = [0, 5], [10]
    a, pa = paq._host_i32(cum)
    b, pb = paq._host_i32(past)
    for kw in ({"fmt": "int4"}, {"D": 64}, {"q": "f32"}):
        d = _desc(1, 5, **kw)
        rc = L.paged_attn_prefill_k_per_use(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                            FAKE, FAKE, FAKE, pa, pb, 0.0, None)
        assert rc == paq.PAQ_ERR_UNSUPPORTED, kw
        assert "per-use" in paq.paq_last_error()


def test_noalloc_decode_refuses_plans_beyond_its_scratch():
    """The allocation-free decode holds 16 MiB of scratch per GPU: a plan that
    needs more is refused before anything is launched (no GPU involved)."""
    L = paq.lib()
    d = _desc(64, 64, mb=300, nb=20000, q="f32")      # fp32 kernel: partials per chunk
    cum, past = _cum([1] * 64), [4000] * 64
    need = paq.paged_attn_decode_workspace_size(d, cum, past, 64)
    assert need > 16 << 20
    a, pa = paq._host_i32(cum)
    b, pb = paq._host_i32(past)
    rc = L.paged_attn_decode_noalloc(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                     FAKE, FAKE, pa, pb, 0.0, 64, None)
    assert rc == paq.PAQ_ERR_WORKSPACE and "allocation-free" in paq.paq_last_error()
