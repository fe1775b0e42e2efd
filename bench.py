#!/usr/bin/env python3
"""Throughput of the paged quantized-KV attention path on one MI355X.

One step = the whole hot path over one batch: host planning, kv_quant_append
of the step's new tokens, then paged_attn_decode or paged_attn_prefill.
Inputs are seeded synthetic workloads (workloads/), resident in HBM before the
timed region.  The KV cache is rotated over several pools (>= ~1.1 GiB in
total) so that every step reads it cold from HBM rather than from the 256 MB
Infinity Cache.

Prints one JSON line.  The headline (`value`, `roofline`, `cpu_baseline`) is
the --workload (default int8_decode, the GQA INT8 decode the metric is quoted
on): decode KV-cache bandwidth (algorithmic KV bytes read per step / step
time, GB/s), or the algorithmic MFMA rate (TFLOP/s, unmasked causal pairs
only) for prefill.  `roofline` is measured for the attention call with HIP
events on its stream.  Unless --only is given, `configs` holds the same
measurement for the other four workloads (tiny_decode's latency in us
included) and `ablations` the comparisons: single pass against the automatic
partition on the two decode workloads, the exact prefill grid against one
sized from token_count - batch + 1, K codes converted once into LDS against
converted by every wave at each use, and the block-sparse decode and prefill.
"""

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode KV-cache GB/s (frac of HBM peak) + tokens/s; prefill MFMA util"
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
MFMA_PEAK_TFLOPS = {"f16": 2516.6, "bf16": 2516.6}   # dense, 256 CU x 4096 flop/clk x 2.4 GHz
KERNEL_SOURCES = {
    "decode": ["decode_mfma.hip", "combine.hip", "device.hpp", "launch.hpp"],
    "prefill": ["prefill_mfma.hip", "device.hpp", "launch.hpp"],
    "quant_append_kernel": ["quant_append.hip", "append.hpp", "device.hpp", "launch.hpp"],
    "rotary_append_kernel": ["rotary_append.hip", "append.hpp", "device.hpp", "launch.hpp"],
}
MAIN_KERNEL = {"decode": "decode_stream_kernel", "prefill": "prefill_mfma_kernel"}


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="int8_decode",
                    choices=["int8_decode", "int4_long", "tiny_decode", "int8_prefill",
                             "fp8_prefill"])
    ap.add_argument("--pools", type=int, default=0, help="KV pools to rotate (0 = auto)")
    ap.add_argument("--splits", type=int, default=None, help="override num_splits (decode)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--skip-warm", action="store_true",
                    help="skip the cache-warm reference calls (profiler runs)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run the plain copy kernel that scales HBM counters")
    ap.add_argument("--summarize-stats", metavar="CSV",
                    help="no GPU: turn a rocprofv3 --stats kernel_stats.csv into a "
                         "profiles/ summary for --workload and exit")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no GPU: turn two rocprofv3 --pmc runs (FETCH_SIZE, then "
                         "WRITE_SIZE) into profiles/counters_<workload>.json and exit")
    ap.add_argument("--summarize-mfma", metavar="DIR",
                    help="no GPU: turn a rocprofv3 --pmc run of the MFMA counters (" +
                         " ".join(MFMA_COUNTERS) + ") over a prefill workload into "
                         "profiles/prefill_mfma_kernel_<workload>_mfma.json and exit")
    ap.add_argument("--command", default="", help="command line recorded in a summary")
    ap.add_argument("--sparse", action="store_true",
                    help="block-sparse attention: decode over a local window of 2 blocks plus "
                         "every 3rd earlier block (paged_attn_decode_sparse); prefill over the "
                         "blocks holding new tokens, the 2 before them and every 3rd earlier "
                         "block (paged_attn_prefill_sparse); value counts the "
                         "selected KV bytes (decode) or the visible pairs' flops (prefill)")
    ap.add_argument("--rotary", action="store_true",
                    help="the step's append is kv_quant_append_rotary (rotary embedding of "
                         "the new query and key rows over all head_size channels)")
    ap.add_argument("--padded-grid", action="store_true",
                    help="prefill: size the grid from token_count - batch + 1 for every "
                         "(sequence, kv head) pair (paged_attn_prefill_padded)")
    ap.add_argument("--k-per-use", action="store_true",
                    help="prefill: K codes kept raw in LDS and converted by every wave at "
                         "each use (paged_attn_prefill_k_per_use), the staging scheme the "
                         "default is compared with")
    ap.add_argument("--separate", action="store_true",
                    help="decode: the step as kv_quant_append then paged_attn_decode (two "
                         "calls) instead of one paged_attn_decode_append call")
    ap.add_argument("--only", action="store_true",
                    help="measure the --workload alone (no configs / ablations)")
    return ap.parse_args()


def kv_bytes(w):
    act = w.q_lens > 0
    return int((w.kv_lens[act].astype(np.int64)).sum()) * w.kv_num_heads * 2 * w.cache_head_size


def append_bytes(w, T, rotary):
    """Algorithmic HBM bytes of one append: the new key and value rows read,
    their codes written; with the rotary embedding also the query rows read
    and written back and one cos and one sin table row per new row."""
    ib = {"f32": 4, "f16": 2, "bf16": 2}
    n = 2 * T * w.kv_num_heads * (w.head_size * ib[w.kv_in_dtype] + w.cache_head_size)
    if rotary:
        n += 2 * T * w.num_heads * w.head_size * ib[w.q_dtype] + T * w.head_size * 4
    return int(n)


def prefill_flops(w, num_sel=None):
    """4 * D * H per visible (query, key) pair; with num_sel (block-sparse
    prefill) a row sees the selected earlier blocks and its local blocks up
    to itself: num_sel * bs + past % bs + i + 1 keys."""
    n = w.q_lens.astype(np.int64)
    p = w.past_lens.astype(np.int64)
    if num_sel is not None:
        p = np.asarray(num_sel, np.int64) * w.block_size + p % w.block_size
    pairs = (n * p + n * (n + 1) // 2).sum()
    return int(4 * w.head_size * w.num_heads * pairs)


def source_sha(kind):
    """Hash of the code of a kernel's sources, comments and whitespace left
    out: a counter file stays valid across comment edits and goes stale when
    the code changes."""
    import re
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, "attention_paged_quantized_amd", "csrc", f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)     # block comments
        text = re.sub(r"//[^\n]*", " ", text)                  # line comments
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def counters(workload, kind):
    """HBM traffic per launch from committed rocprofv3 counter runs of the
    workload's main kernel of this kind (decode, prefill, or an append kernel's
    name), if they were taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "%s_%s_counters.json" %
                        (MAIN_KERNEL.get(kind, kind), workload))
    if not os.path.exists(path):
        return None
    with open(path) as f:
        c = json.load(f)
    if c.get("source_sha") != source_sha(kind):
        return None
    return int((c["fetch_kib"] * c["fetch_factor"] + c["write_kib"] * c["write_factor"]) * 1024)


def cpu_kernel(w, g, desc, calls=5):
    """The library's own host decode (paged_attn_decode_host: fp32 GEMV decode,
    flash decoding across threads) on the whole workload, with the caches the
    GPU wrote copied to host memory: a fast CPU figure beside the oracle's."""
    import attention_paged_quantized_amd as paq
    threads = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    threads = max(1, min(16, threads))
    kc, vc = g.kc.cpu().numpy(), g.vc.cpu().numpy()
    q = np.ascontiguousarray(w.query.float().numpy())
    out = np.empty_like(q)
    args = (kc, vc, np.ascontiguousarray(w.k_scale, np.float32),
            np.ascontiguousarray(w.v_scale, np.float32),
            np.ascontiguousarray(w.block_table, np.int32), np.ascontiguousarray(w.cum_q, np.int32),
            np.ascontiguousarray(w.past_lens, np.int32))
    d32 = paq.make_desc(desc.batch, desc.token_count, desc.num_heads, desc.kv_num_heads,
                        desc.head_size, desc.block_size, desc.num_blocks,
                        desc.max_blocks_per_seq, "f32", desc.kv_format, desc.scale_mode)
    paq.paged_attn_decode_host(d32, q, out, *args, num_threads=threads)       # warm
    t0 = time.perf_counter()
    for _ in range(calls):
        paq.paged_attn_decode_host(d32, q, out, *args, num_threads=threads)
    sec = (time.perf_counter() - t0) / calls
    kvb = kv_bytes(w)
    return {"kernel": "paged_attn_decode_host", "value": round(kvb / sec / 1e9, 2),
            "unit": "GB/s", "ms_per_call": round(sec * 1e3, 3), "threads": threads,
            "tokens_per_s": round(int((w.q_lens > 0).sum()) / sec, 1)}


def host_stream_gbs(threads, nbytes=2 ** 31):
    """Streaming-read bandwidth of the host with `threads` threads (numpy sums
    over disjoint slices of a 2 GiB array; numpy releases the GIL in them):
    the roofline of the host decode."""
    import concurrent.futures
    a = np.ones(nbytes // 4, np.float32)
    parts = np.array_split(a, threads)
    with concurrent.futures.ThreadPoolExecutor(threads) as ex:
        list(ex.map(np.sum, parts))                      # touch / warm
        best = 0.0
        for _ in range(3):
            t0 = time.perf_counter()
            list(ex.map(np.sum, parts))
            best = max(best, nbytes / (time.perf_counter() - t0) / 1e9)
    return round(best, 2)


def cpu_baseline(w, seconds):
    """The oracle as it stands, on the host cores, over a bounded sample of the
    same workload: its sequences one after another (cycling through the batch)
    until the time budget is spent; each costs one oracle quant_append of the
    sequence's new rows plus its oracle attention.  Each sequence gets a pool
    of its own blocks only (gathered before timing), so the oracle's append
    copies that sequence's cache, not the whole batch's."""
    import threadpoolctl
    from oracle import attention, quant
    from tests.oracle_cases import f32, oracle_caches

    kc, vc = oracle_caches(w)
    kin, vin = f32(w.new_key), f32(w.new_value)
    q = f32(w.query)
    info = threadpoolctl.threadpool_info()
    threads = max([i.get("num_threads", 1) for i in info] or [1])
    active = [b for b in range(w.batch) if w.q_lens[b] > 0]
    pools = {}
    for b in active:
        nb = -(-int(w.kv_lens[b]) // w.block_size)
        blocks = w.block_table[b, :nb]
        pools[b] = (kc[blocks], vc[blocks], np.arange(nb, dtype=np.int32)[None])
    done_kv = done_flops = done_tok = nseq = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        b = active[nseq % len(active)]
        r0, r1 = int(w.cum_q[b]), int(w.cum_q[b + 1])
        cq = np.array([0, r1 - r0], np.int32)
        pl = w.past_lens[b:b + 1]
        pk, pv, bt = pools[b]
        kc2, vc2 = quant.quant_append(pk, pv, kin[r0:r1], vin[r0:r1], w.k_scale, w.v_scale,
                                      bt, cq, pl, w.kv_format)
        attention.paged_attention(q[r0:r1], kc2, vc2, w.k_scale, w.v_scale, bt, cq, pl,
                                  w.kv_format)
        n, p = r1 - r0, int(w.past_lens[b])
        done_kv += (p + n) * w.kv_num_heads * 2 * w.cache_head_size
        done_flops += 4 * w.head_size * w.num_heads * (n * p + n * (n + 1) // 2)
        done_tok += 1 if w.kind == "decode" else n
        nseq += 1
    el = time.perf_counter() - t0
    res = {"cores": int(threads), "kind": "oracle",
           "sample": "%d sequences of %s (cycling through the batch; fp64 oracle "
                     "quant_append of the sequence's new rows into a pool of its own blocks, "
                     "then its attention), %.1f s wall" % (nseq, w.name, el),
           "tokens_per_s": round(done_tok / el, 3)}
    if w.kind == "decode":
        res.update({"value": round(done_kv / el / 1e9, 5), "unit": "GB/s"})
    else:
        res.update({"value": round(done_flops / el / 1e12, 6), "unit": "TFLOP/s"})
    return res


# Kernels of one attention call, by workload kind (substrings of the symbol).
CALL_KERNELS = {"decode": ("decode_stream_kernel", "combine_kernel", "attn_f32_kernel",
                           "sparse_compact_kernel"),
                "prefill": ("prefill_mfma_kernel", "attn_f32_kernel",
                            "sparse_prefill_compact_kernel")}
CALIB_KERNEL = "neg_kernel"


def _short(name):
    for k in ("decode_stream_kernel", "combine_kernel", "attn_f32_kernel",
              "prefill_mfma_kernel", "quant_append_kernel", "rotary_append_kernel",
              "sparse_prefill_compact_kernel", "sparse_compact_kernel", CALIB_KERNEL):
        if k in name:
            return k
    return name[:48]


def summarize_stats(args):
    """rocprofv3 --kernel-trace --stats CSV -> profiles/<kernel>_<workload>.txt"""
    import csv
    import workloads
    w = workloads.make(args.workload)
    rows = list(csv.DictReader(open(args.summarize_stats)))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    if args.rotary:
        return summarize_append_stats(args, w, rows, "rotary_append_kernel")
    call = [r for r in rows if any(k in r["Name"] for k in CALL_KERNELS[w.kind])]
    main = [r for r in call if "compact" not in r["Name"]]
    main_k = _short(main[0]["Name"]) if main else "none"
    lines = ["rocprofv3 kernel statistics, workload %s (%s)%s" %
             (w.name, w.kind, (", variant " + variant(args)[1:]) if variant(args) else ""),
             "command: %s" % (args.command or "(not recorded)"),
             "kernel sources sha256[:16]: %s" % source_sha(w.kind), "",
             "%-22s %7s %12s %12s %12s %12s" % ("kernel", "calls", "avg_us", "min_us",
                                                 "max_us", "total_us")]
    for r in rows[:12]:
        lines.append("%-22s %7d %12.3f %12.3f %12.3f %12.1f" % (
            _short(r["Name"]), int(r["Calls"]), float(r["AverageNs"]) / 1e3,
            float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3, float(r["TotalDurationNs"]) / 1e3))
    tot = sum(float(r["AverageNs"]) for r in call) / 1e3
    lines += ["", "attention call (%s): %.3f us average per call" %
              (" + ".join(_short(r["Name"]) for r in call), tot)]
    if args.sparse:
        sel, num = sparse_selection(w)
    if w.kind == "decode":
        kvb = sparse_kv_bytes(w, sel, num) if args.sparse else kv_bytes(w)
        lines.append("algorithmic KV bytes per call %d -> %.1f GB/s, %.4f of 8000 GB/s" %
                     (kvb, kvb / (tot * 1e3), kvb / (tot * 1e3) / HBM_PEAK_GBS))
    else:
        fl = prefill_flops(w, num if args.sparse else None)
        lines.append("algorithmic flops per call %d -> %.1f TFLOP/s, %.4f of %.1f" %
                     (fl, fl / (tot * 1e-6) / 1e12, fl / (tot * 1e-6) / 1e12 /
                      MFMA_PEAK_TFLOPS[w.q_dtype], MFMA_PEAK_TFLOPS[w.q_dtype]))
    out = os.path.join(ROOT, "profiles", "%s_%s%s.txt" % (main_k, w.name, variant(args)))
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("wrote", out)


def summarize_append_stats(args, w, rows, kernel):
    """The append kernel's line of a kernel-statistics run ->
    profiles/<kernel>_<workload>.txt"""
    mine = [r for r in rows if kernel in r["Name"]]
    r = mine[0]
    avg = float(r["AverageNs"]) / 1e3
    ab = append_bytes(w, w.token_count, kernel == "rotary_append_kernel")
    lines = ["rocprofv3 kernel statistics, workload %s, %s" % (w.name, kernel),
             "command: %s" % (args.command or "(not recorded)"),
             "kernel sources sha256[:16]: %s" % source_sha(kernel), "",
             "%-22s %7s %12s %12s %12s %12s" % ("kernel", "calls", "avg_us", "min_us",
                                                 "max_us", "total_us")]
    for q in rows[:12]:
        lines.append("%-22s %7d %12.3f %12.3f %12.3f %12.1f" % (
            _short(q["Name"]), int(q["Calls"]), float(q["AverageNs"]) / 1e3,
            float(q["MinNs"]) / 1e3, float(q["MaxNs"]) / 1e3, float(q["TotalDurationNs"]) / 1e3))
    lines += ["", "%s: %.3f us average per call (min %.3f)" % (kernel, avg,
                                                               float(r["MinNs"]) / 1e3),
              "algorithmic bytes per call %d -> %.1f GB/s, %.4f of %.0f GB/s" %
              (ab, ab / (avg * 1e3), ab / (avg * 1e3) / HBM_PEAK_GBS, HBM_PEAK_GBS)]
    out = os.path.join(ROOT, "profiles", "%s_%s.txt" % (kernel, w.name))
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("wrote", out)


MFMA_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_F16",
                 "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_BUSY_CYCLES", "SQ_ACTIVE_INST_VALU",
                 "GRBM_GUI_ACTIVE")


def summarize_mfma(args):
    """One rocprofv3 --pmc run of MFMA_COUNTERS over a prefill workload ->
    profiles/prefill_mfma_kernel_<workload>[variant]_mfma.json: matrix-core
    busy fraction (SQ_VALU_MFMA_BUSY_CYCLES over 4 SIMDs x 256 CUs x the
    per-XCD active cycles), the MFMA flops issued (MOPS x 512) against the
    algorithmic flops, and the VALU-active fraction, medians over dispatches."""
    import csv
    import glob
    import workloads
    w = workloads.make(args.workload)
    vals = {}
    for f in glob.glob(os.path.join(args.summarize_mfma, "**", "*counter_collection.csv"),
                       recursive=True):
        for r in csv.DictReader(open(f)):
            if "prefill_mfma_kernel" in r["Kernel_Name"] and r["Counter_Name"] in MFMA_COUNTERS:
                vals.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    med = {k: sorted(v)[len(v) // 2] for k, v in vals.items()}
    n_xcd, cus = 8, 256
    active = med["GRBM_GUI_ACTIVE"] / n_xcd             # cycles the kernel kept the GPU busy
    mops = med.get("SQ_INSTS_VALU_MFMA_MOPS_F16", 0.0) + med.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0)
    fl = prefill_flops(w, sparse_selection(w)[1] if args.sparse else None)
    res = {"workload": w.name, "variant": variant(args)[1:] or "default",
           "source_sha": source_sha("prefill"), "command": args.command,
           "dispatches": len(vals.get("GRBM_GUI_ACTIVE", [])),
           "counters_median": med,
           "mfma_busy_frac": round(med["SQ_VALU_MFMA_BUSY_CYCLES"] / (active * cus * 4), 4),
           "valu_active_frac": round(med["SQ_ACTIVE_INST_VALU"] / (active * cus), 4)
           if "SQ_ACTIVE_INST_VALU" in med else None,
           "mfma_flops_issued": mops * 512,
           "algorithmic_flops": fl,
           "issued_over_algorithmic": round(mops * 512 / fl, 4),
           "active_cycles_per_xcd": active,
           "definitions": "mfma_busy_frac = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 x "
                          "256 CU x 4 SIMD); valu_active_frac = SQ_ACTIVE_INST_VALU / "
                          "(GRBM_GUI_ACTIVE / 8 x 256); flops issued = MOPS x 512 (the "
                          "profiler's MFMA FLOPs unit)"}
    out = os.path.join(ROOT, "profiles", "prefill_mfma_kernel_%s%s_mfma.json" %
                       (w.name, variant(args)))
    with open(out, "w") as f:
        json.dump(res, f, indent=1)
    print("wrote", out, json.dumps(res))


def summarize_pmc(args):
    """Two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) -> per-call HBM bytes of
    the attention kernels, scaled by the counters of a 256 MiB copy, written to
    profiles/counters_<workload>.json"""
    import csv
    import glob
    import workloads
    w = workloads.make(args.workload)

    def medians(d, counter):
        vals = {}
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                if r["Counter_Name"] == counter:
                    vals.setdefault(_short(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
        return {k: sorted(v)[len(v) // 2] for k, v in vals.items()}

    fetch = medians(args.summarize_pmc[0], "FETCH_SIZE")
    write = medians(args.summarize_pmc[1], "WRITE_SIZE")
    calib_kib = CALIB_ELEMS * 4 / 1024.0
    ff = calib_kib / fetch[CALIB_KERNEL]
    wf = calib_kib / write[CALIB_KERNEL]
    ks = [k for k in CALL_KERNELS[w.kind] if k in fetch]
    if args.rotary:
        ks = []                     # a rotary run records its append kernel only
    res = {"workload": w.name, "source_sha": source_sha(w.kind), "command": args.command,
           "calibration": "torch.neg over %d fp32 (%.0f KiB read, %.0f KiB written): "
                          "FETCH_SIZE %.1f KiB, WRITE_SIZE %.1f KiB" %
                          (CALIB_ELEMS, calib_kib, calib_kib, fetch[CALIB_KERNEL],
                           write[CALIB_KERNEL]),
           "fetch_factor": round(ff, 5), "write_factor": round(wf, 5),
           "kernels": {k: {"fetch_kib": fetch[k], "write_kib": write.get(k, 0.0)} for k in ks},
           "fetch_kib": sum(fetch[k] for k in ks), "write_kib": sum(write.get(k, 0.0) for k in ks)}
    hbm = (res["fetch_kib"] * ff + res["write_kib"] * wf) * 1024
    res["hbm_bytes_per_call"] = int(hbm)
    if w.kind == "decode":
        kvb = sparse_kv_bytes(w, *sparse_selection(w)) if args.sparse else kv_bytes(w)
        res["algorithmic_kv_bytes_per_call"] = kvb
        res["traffic_over_algorithmic"] = round(hbm / kvb, 4)
    if ks:
        out = os.path.join(ROOT, "profiles", "%s_%s%s_counters.json" % (ks[0], w.name,
                                                                          variant(args)))
        with open(out, "w") as f:
            json.dump(res, f, indent=1)
        print("wrote", out, json.dumps(res))
    # the append kernel of the same runs, on its own
    for k in ("rotary_append_kernel",) if args.rotary else ("quant_append_kernel",):
        if k not in fetch:
            continue
        r = {"workload": w.name, "source_sha": source_sha(k), "command": args.command,
             "calibration": res["calibration"], "fetch_factor": res["fetch_factor"],
             "write_factor": res["write_factor"], "fetch_kib": fetch[k],
             "write_kib": write.get(k, 0.0)}
        r["hbm_bytes_per_call"] = int((r["fetch_kib"] * ff + r["write_kib"] * wf) * 1024)
        ab = append_bytes(w, w.token_count, k == "rotary_append_kernel")
        r["algorithmic_bytes_per_call"] = ab
        r["traffic_over_algorithmic"] = round(r["hbm_bytes_per_call"] / ab, 4)
        out = os.path.join(ROOT, "profiles", "%s_%s_counters.json" % (k, w.name))
        with open(out, "w") as f:
            json.dump(r, f, indent=1)
        print("wrote", out, json.dumps(r))


CALIB_ELEMS = 2 ** 26          # fp32 elements of the counter-calibration copy (256 MiB)


def sparse_selection(w):
    """The benched block-sparse selections, (sel (batch, max_sel), num (batch)):
    decode, a 2-block local window plus every 3rd earlier block of each
    sequence; prefill, the 2 blocks before the ones holding new tokens plus
    every 3rd earlier block (the local blocks are always attended)."""
    if w.kind == "decode":
        n_all = -(-(w.past_lens + 1) // w.block_size)
    else:
        n_all = w.past_lens // w.block_size
    rows = [sorted(set(list(range(max(0, n - 2), n)) + list(range(0, n, 3)))) for n in n_all]
    sel = np.zeros((w.batch, max(1, max(len(r) for r in rows))), np.int32)
    num = np.array([len(r) for r in rows], np.int32)
    for b, r in enumerate(rows):
        sel[b, :len(r)] = r
    return sel, num


def sparse_kv_bytes(w, sel, num):
    """Selected KV bytes of a block-sparse decode (whole blocks, the last one up
    to kv_len), over the sequences with a new row."""
    keys = 0
    for b in range(w.batch):
        if w.q_lens[b] > 0:
            keys += sum(min(w.block_size, int(w.past_lens[b]) + 1 - w.block_size * int(x))
                        for x in sel[b, :num[b]])
    return keys * w.kv_num_heads * 2 * w.cache_head_size


def variant(args):
    """File-name suffix of a profiled variant ("" for the default call)."""
    v = ""
    if args.splits is not None:
        v += "_splits%d" % args.splits
    if args.padded_grid:
        v += "_padded"
    if args.k_per_use:
        v += "_k_per_use"
    if args.sparse:
        v += "_sparse"
    return v


def sleep_rate(stream):
    """Cycles per second of torch.cuda._sleep on this device: the fastest of a
    few calibrations (its cycles follow the shader clock, which may still be
    ramping up at the first ones; the fastest rate gives the shortest sleep
    per cycle, so holds sized from it are never too short)."""
    import torch
    rates = []
    for _ in range(3):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        torch.cuda._sleep(2_000_000)
        e1.record(stream)
        torch.cuda.synchronize()
        rates.append(2_000_000 / (e0.elapsed_time(e1) / 1e3))
    return max(rates)


_WORKLOADS = {}          # workloads built so far (the ablations reuse them)


def measure(args, name, splits=None, padded=False, rotary=False, sparse=False, warm=True,
            append_loop=True, k_per_use=False, separate=False):
    """Time `steps` steps (append + attention) of workload `name` after
    `warmup` untimed ones; returns the measurement as a dict, plus the
    workload, one filled Device and the descriptor (for the CPU figures).
    A dense decode step is one paged_attn_decode_append call (the decode
    kernel appends the step's rows itself where it can); separate=True runs
    kv_quant_append and paged_attn_decode instead."""
    import torch
    import attention_paged_quantized_amd as paq
    import workloads
    from tests.gpu_cases import Device, desc_for

    dev = torch.device("cuda:0")
    if name not in _WORKLOADS:
        _WORKLOADS[name] = workloads.make(name)
    w = _WORKLOADS[name]
    kind = w.kind
    S = w.num_splits if splits is None else splits
    T = w.token_count
    print("[bench] workload %s: batch %d, tokens %d, kv bytes %.1f MB" %
          (w.name, w.batch, T, kv_bytes(w) / 1e6), file=sys.stderr, flush=True)

    pool_bytes = 2 * w.num_blocks * w.block_size * w.kv_num_heads * w.cache_head_size
    pools = args.pools or int(min(16, max(2, -(-(1.1 * 2 ** 30) // pool_bytes))))
    devs = [Device(w, dev).fill() for _ in range(pools)]
    torch.cuda.synchronize()
    print("[bench] %d KV pools of %.1f MB filled" % (pools, pool_bytes / 1e6), file=sys.stderr,
          flush=True)

    desc = desc_for(w, T)
    if rotary:
        rcos, rsin = workloads.rope_tables(int(w.kv_lens.max()) + 1, w.head_size)
        rcos, rsin = torch.from_numpy(rcos).to(dev), torch.from_numpy(rsin).to(dev)
    kin = w.new_key.to(dev)
    vin = w.new_value.to(dev)
    outs = [torch.empty_like(g.query) for g in devs]
    ws = None
    plan = None
    if kind == "decode":
        plan = paq.paq_plan_decode(desc, w.cum_q, w.past_lens, S)
        nbytes = paq.paged_attn_decode_workspace_size(desc, w.cum_q, w.past_lens, S)
        if nbytes:
            ws = torch.zeros(nbytes // 4 + 1, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    heuristic_mql = T - w.batch + 1
    if sparse and kind == "prefill":
        sel_np, num_np = sparse_selection(w)
        sel_d, num_d = torch.from_numpy(sel_np).to(dev), torch.from_numpy(num_np).to(dev)
        nbytes = paq.paged_attn_prefill_sparse_workspace_size(desc, w.cum_q, w.past_lens,
                                                              num_np, sel_np.shape[1])
        ws = torch.zeros(nbytes // 4 + 1, dtype=torch.float32, device=dev)
    elif sparse:
        sel_np, num_np = sparse_selection(w)
        sel_d, num_d = torch.from_numpy(sel_np).to(dev), torch.from_numpy(num_np).to(dev)
        nbytes = paq.paged_attn_decode_sparse_workspace_size(desc, w.cum_q, w.past_lens, num_np,
                                                             sel_np.shape[1], S)
        ws = torch.zeros(nbytes // 4 + 1, dtype=torch.float32, device=dev)

    fused = kind == "decode" and not sparse and not rotary and not separate

    def attention(g, out):
        if fused:
            paq.paged_attn_decode_append(desc, w.kv_in_dtype, kin, vin, g.query, out, g.kc, g.vc,
                                         g.k_scale, g.v_scale, g.block_table, g.cum_q, g.past,
                                         w.cum_q, w.past_lens, 0.0, S, ws, stream)
        elif kind == "decode" and sparse:
            paq.paged_attn_decode_sparse(desc, g.query, out, g.kc, g.vc, g.k_scale, g.v_scale,
                                         g.block_table, g.cum_q, g.past, w.cum_q, w.past_lens,
                                         sel_d, num_d, num_np, 0.0, S, ws, stream)
        elif kind == "decode":
            paq.paged_attn_decode(desc, g.query, out, g.kc, g.vc, g.k_scale, g.v_scale,
                                  g.block_table, g.cum_q, g.past, w.cum_q, w.past_lens, 0.0, S,
                                  ws, stream)
        elif sparse:
            paq.paged_attn_prefill_sparse(desc, g.query, out, g.kc, g.vc, g.k_scale, g.v_scale,
                                          g.block_table, g.cum_q, g.past, w.cum_q, w.past_lens,
                                          sel_d, num_d, num_np, 0.0, ws, stream)
        elif k_per_use:
            paq.paged_attn_prefill_k_per_use(desc, g.query, out, g.kc, g.vc, g.k_scale,
                                             g.v_scale, g.block_table, g.cum_q, g.past, w.cum_q,
                                             w.past_lens, 0.0, stream)
        elif padded:
            paq.paged_attn_prefill_padded(desc, g.query, out, g.kc, g.vc, g.k_scale, g.v_scale,
                                          g.block_table, g.cum_q, g.past, w.cum_q, w.past_lens,
                                          heuristic_mql, 0.0, stream)
        else:
            paq.paged_attn_prefill(desc, g.query, out, g.kc, g.vc, g.k_scale, g.v_scale,
                                   g.block_table, g.cum_q, g.past, w.cum_q, w.past_lens, 0.0,
                                   stream)

    def append(g):
        if rotary:
            paq.kv_quant_append_rotary(desc, w.kv_in_dtype, g.query, kin, vin, g.kc, g.vc,
                                       g.k_scale, g.v_scale, g.block_table, g.cum_q, g.past,
                                       w.cum_q, w.past_lens, rcos, rsin, w.head_size, False,
                                       stream)
        else:
            paq.kv_quant_append(desc, w.kv_in_dtype, kin, vin, g.kc, g.vc, g.k_scale,
                                g.v_scale, g.block_table, g.cum_q, g.past, w.cum_q,
                                w.past_lens, stream)

    def step(i, ev=None):
        g = devs[i % pools]
        if not fused:
            append(g)
        if ev is not None:
            ev[0].record(stream)
        attention(g, outs[i % pools])
        if ev is not None:
            ev[1].record(stream)

    # Warm up, and measure how long the host takes to queue one step (with
    # per-call events, the slower of the two loops below).
    wevs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in range(args.warmup)]
    torch.cuda.synchronize()
    h0 = time.perf_counter()
    for i in range(args.warmup):
        step(i, wevs[i])
    host_ms = (time.perf_counter() - h0) * 1e3 / max(1, args.warmup)
    torch.cuda.synchronize()
    hz = sleep_rate(stream)

    def hold(n_steps):
        # keep the stream busy while the host queues n_steps, so that the
        # events below time the GPU and not the Python launch rate
        # (a generous margin: the sleep is outside the timed region)
        torch.cuda._sleep(int((6.0 * n_steps * host_ms + 20.0) * 1e-3 * hz))

    # The timed steps: append + attention, bracketed by two events only (an
    # event recorded between kernels costs GPU time of its own).
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    hold(args.steps)
    t_start.record(stream)
    for i in range(args.steps):
        step(i)
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_total = t_start.elapsed_time(t_end)
    ms_step = ms_total / args.steps
    # The attention call's average time: the calls alone, back to back over
    # the same pools, between two events on their stream.
    k0 = torch.cuda.Event(enable_timing=True)
    k1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    hold(args.steps)
    k0.record(stream)
    for i in range(args.steps):
        attention(devs[i % pools], outs[i % pools])
    k1.record(stream)
    torch.cuda.synchronize()
    kern_avg = k0.elapsed_time(k1) / args.steps
    # Their spread: the steps again with an event pair around each call (each
    # pair adds its own overhead, so these run longer than the average above).
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    hold(args.steps)
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    kern_ms = [a.elapsed_time(b) for a, b in evs]
    kern_sorted = sorted(kern_ms)
    app_avg = None
    if append_loop:
        # the append on its own: per-call events over the same pools, outside
        # the timed steps (its events would add to their time)
        aevs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                for _ in range(args.steps)]
        torch.cuda.synchronize()
        hold(args.steps)
        for i, (e0, e1) in enumerate(aevs):
            e0.record(stream)
            append(devs[i % pools])
            e1.record(stream)
        torch.cuda.synchronize()
        app_avg = sum(a.elapsed_time(b) for a, b in aevs) / len(aevs)

    # warm (cache-resident) reference: the same pool every call, per-call events
    warm_ms = None
    if warm and not args.skip_warm:
        for i in range(5):
            attention(devs[0], outs[0])
        wev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(20)]
        torch.cuda.synchronize()
        hold(len(wev))
        for e0, e1 in wev:
            e0.record(stream)
            attention(devs[0], outs[0])
            e1.record(stream)
        torch.cuda.synchronize()
        warm_ms = sorted(e0.elapsed_time(e1) for e0, e1 in wev)[len(wev) // 2]

    r = {"workload": w.name, "ms_per_step": round(ms_step, 6)}
    cfg = {"workload": w.name, "batch": w.batch, "num_heads": w.num_heads,
           "kv_num_heads": w.kv_num_heads, "head_size": w.head_size,
           "block_size": w.block_size, "kv_format": w.kv_format, "scale_mode": w.scale_mode,
           "q_dtype": w.q_dtype, "token_count": T, "kv_pools": pools}
    p10p90 = [round(kern_sorted[len(kern_ms) // 10] * 1e3, 3),
              round(kern_sorted[9 * len(kern_ms) // 10] * 1e3, 3)]
    if kind == "decode":
        kvb = kv_bytes(w)
        if sparse:
            kvb = sparse_kv_bytes(w, sel_np, num_np)
        act = int((w.q_lens > 0).sum())
        r.update({"value": round(kvb / (ms_step / 1e3) / 1e9, 2), "unit": "GB/s",
                  "tokens_per_s": round(act / (ms_step / 1e3), 1),
                  "hbm_frac": round(kvb / (ms_step / 1e3) / 1e9 / HBM_PEAK_GBS, 4)})
        cfg.update({"num_splits": S, "path": paq.PATHS[plan.path],
                    "parts": plan.parts, "keys_per_group": plan.keys_per_group,
                    "kv_bytes_per_step": kvb, "max_kv_len": int(w.kv_lens.max())})
        achieved = kvb / (kern_avg / 1e3) / 1e9
        traffic = None if sparse else counters(w.name, "decode")
        call = "decode_stream_kernel" if plan.path in (1, 2, 7) else \
            "attn_f32_kernel" + (" + combine_kernel" if plan.path == 4 else "")
        r["roofline"] = {"bound": "hbm", "achieved": round(achieved, 2),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                         "kernel": ("paged_attn_decode_sparse call (sparse_compact_kernel + %s)"
                                    if sparse else
                                    "paged_attn_decode_append call (%s%s)" % (
                                        "%s", ", the step's append inside"
                                        if w.kv_in_dtype == w.q_dtype or
                                        (w.kv_in_dtype == "f32" and
                                         call == "decode_stream_kernel") else
                                        " after quant_append_kernel")
                                    if fused else "paged_attn_decode call (%s)") % call,
                         "kernel_us_avg": round(kern_avg * 1e3, 3),
                         "per_call_events_us_p10_p90": p10p90,
                         "warm_cache_us": round(warm_ms * 1e3, 3) if warm_ms else None,
                         "algorithmic_bytes_per_launch": kvb}
    else:
        fl = prefill_flops(w, num_np if sparse else None)
        peak = MFMA_PEAK_TFLOPS[w.q_dtype]
        r.update({"value": round(fl / (ms_step / 1e3) / 1e12, 3), "unit": "TFLOP/s",
                  "tokens_per_s": round(T / (ms_step / 1e3), 1)})
        achieved = fl / (kern_avg / 1e3) / 1e12
        r["roofline"] = {"bound": "mfma", "achieved": round(achieved, 3), "peak": peak,
                         "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                         "traffic": None if padded or sparse or k_per_use
                         else counters(w.name, "prefill"),
                         "kernel": "paged_attn_prefill%s call (%sprefill_mfma_kernel)" %
                                   ("_padded" if padded else "_sparse" if sparse else
                                    "_k_per_use" if k_per_use else "",
                                    "sparse_prefill_compact_kernel + " if sparse else ""),
                         "kernel_us_avg": round(kern_avg * 1e3, 3),
                         "per_call_events_us_p10_p90": p10p90,
                         "warm_cache_us": round(warm_ms * 1e3, 3) if warm_ms else None,
                         "algorithmic_flops_per_launch": fl}
        cfg.update({"max_query_len": int(w.q_lens.max()), "causal": True,
                    "grid": "token_count - batch + 1 = %d for every pair" % heuristic_mql
                            if padded else "exact"})
    r["config"] = cfg
    if app_avg is not None:
        ab = append_bytes(w, T, rotary)
        r["append"] = {"kernel": "rotary_append_kernel" if rotary else "quant_append_kernel",
                       "bound": "hbm", "us_avg": round(app_avg * 1e3, 3),
                       "algorithmic_bytes": ab,
                       "achieved": round(ab / (app_avg / 1e3) / 1e9, 2), "unit": "GB/s",
                       "frac": round(ab / (app_avg / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                       "traffic": counters(w.name, "rotary_append_kernel" if rotary
                                           else "quant_append_kernel")}
    if sparse and kind == "decode":
        cfg["sparse"] = "2-block local window + every 3rd earlier block; %d of %d KV bytes" % (
            kvb, kv_bytes(w))
    elif sparse:
        cfg["sparse"] = ("the blocks holding new tokens + the 2 blocks before them + every 3rd "
                         "earlier block; %d of %d causal (query, key) pairs" %
                         (fl // (4 * w.head_size * w.num_heads),
                          prefill_flops(w) // (4 * w.head_size * w.num_heads)))
    keep = devs[0]
    del devs, outs, ws
    torch.cuda.empty_cache()
    return r, w, keep, desc


def summary(r):
    """The per-configuration line of a measurement."""
    rf = r["roofline"]
    out = {"ms_per_step": r["ms_per_step"], "value": r["value"], "unit": r["unit"],
           "tokens_per_s": r["tokens_per_s"], "kernel_us_avg": rf["kernel_us_avg"],
           "per_call_events_us_p10_p90": rf["per_call_events_us_p10_p90"], "achieved": rf["achieved"],
           "roofline_unit": rf["unit"], "bound": rf["bound"], "frac": rf["frac"],
           "traffic": rf["traffic"], "kernel": rf["kernel"], "config": r["config"]}
    if r["config"]["workload"] == "tiny_decode":
        out["latency_us"] = rf["kernel_us_avg"]
    if "append" in r:
        out["append_us"] = r["append"]["us_avg"]
    return out


def main():
    args = parse()
    if args.summarize_stats:
        summarize_stats(args)
        return
    if args.summarize_pmc:
        summarize_pmc(args)
        return
    if args.summarize_mfma:
        summarize_mfma(args)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(requested --gpus %d, WORLD_SIZE %d)" % (args.gpus, world), file=sys.stderr)
        sys.exit(2)

    import torch
    import attention_paged_quantized_amd as paq

    torch.cuda.set_device(0)
    paq.lib()
    r, w, g0, desc = measure(args, args.workload, splits=args.splits, padded=args.padded_grid,
                             rotary=args.rotary, sparse=args.sparse, k_per_use=args.k_per_use,
                             separate=args.separate)
    result = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
              "ms_per_step": r["ms_per_step"], "higher_is_better": True, "scaling": "weak",
              "vs_baseline": None, "dtype": {"f32": "f32", "bf16": "bf16"}.get(w.q_dtype, "f16"),
              "data": "synthetic (seeded; workloads/%s)" % w.name}
    for k in ("value", "unit", "tokens_per_s", "hbm_frac", "roofline", "config", "append"):
        if k in r:
            result[k] = r[k]

    # the copy rate of this GPU for context (read + write bytes / time); with
    # --calib-copy also the 256 MiB copy whose counters scale FETCH/WRITE_SIZE
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    src = torch.empty(2 ** 28, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    for _ in range(5):
        dst.copy_(src)
    c1.record(stream)
    torch.cuda.synchronize()
    result["hbm_copy_GBs"] = round(2 * src.numel() * 4 * 5 / (c0.elapsed_time(c1) / 1e3) / 1e9, 1)
    if args.calib_copy:
        for _ in range(3):
            torch.neg(src[:CALIB_ELEMS], out=dst[:CALIB_ELEMS])
        torch.cuda.synchronize()
    del src, dst

    if not args.only and not args.sparse and not args.rotary and not args.k_per_use and \
            not args.separate:
        # every configuration, then the ablations (short timings each)
        configs = {}
        for name in ("tiny_decode", "int8_decode", "int4_long", "int8_prefill", "fp8_prefill"):
            if name == w.name:
                configs[name] = summary(r)
                continue
            cr = measure(args, name, warm=False)[0]
            configs[name] = summary(cr)
        result["configs"] = configs
        abl = {}
        for label, name, kw in (
                ("int8_decode single pass (num_splits 1)", "int8_decode", {"splits": 1}),
                ("int4_long single pass (num_splits 1)", "int4_long", {"splits": 1}),
                ("int8_prefill grid from token_count - batch + 1", "int8_prefill",
                 {"padded": True}),
                ("fp8_prefill grid from token_count - batch + 1", "fp8_prefill",
                 {"padded": True}),
                ("int8_prefill K codes converted per use", "int8_prefill", {"k_per_use": True}),
                ("fp8_prefill K codes converted per use", "fp8_prefill", {"k_per_use": True}),
                ("int8_decode block-sparse (2-block window + every 3rd block)", "int8_decode",
                 {"sparse": True}),
                ("int8_prefill block-sparse (local blocks + 2 before + every 3rd)",
                 "int8_prefill", {"sparse": True}),
                ("int8_decode step as two calls (kv_quant_append, then paged_attn_decode)",
                 "int8_decode", {"separate": True})):
            ar = measure(args, name, warm=False, append_loop=False, **kw)[0]
            s = summary(ar)
            ref = configs[name]
            s["time_vs_default"] = round(s["kernel_us_avg"] / ref["kernel_us_avg"], 3)
            s["step_vs_default"] = round(s["ms_per_step"] / ref["ms_per_step"], 3)
            abl[label] = s
        result["ablations"] = abl

    if w.kind == "decode" and not args.no_cpu_baseline and not args.sparse:
        threads = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") \
            else os.cpu_count()
        threads = max(1, min(16, threads))
        ck = cpu_kernel(w, g0, desc)
        ck["host_stream_GBs"] = host_stream_gbs(threads)
        ck["frac_of_host_stream"] = round(ck["value"] / ck["host_stream_GBs"], 4)
        result["cpu_kernel"] = ck
    del g0
    if not args.no_cpu_baseline:
        print("[bench] timing the fp64 oracle on the host (%.0f s budget)" % args.cpu_seconds,
              file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
