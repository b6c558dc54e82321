#!/usr/bin/env python3
"""Benchmark of the paged decode-attention hot path on one MI355X.

One step = one call of the C-ABI entry point (partition kernel + log-sum-exp
merge kernel) over one batch of the chosen synthetic workload, with every
input already resident in HBM.  The KV pools are rotated over several
device copies so that each call reads its K/V from HBM rather than from the
256 MB Infinity Cache.  Prints one JSON line.

    python bench.py [--steps K] [--warmup W] [--config long_ctx] [--only]

Default workload: the batch-1 long-context decode (1 sequence, 131072
tokens, 64 query / 8 kv heads, head_dim 128, bf16 KV).  Unless --only is
given, the same line also carries the fp8-KV workload (16 sequences,
contexts 512..32768, head_dim 64, e4m3fn with per-token scales) measured
the same way ("fp8_config") and the read rate of a plain streaming kernel
at both calls' byte counts ("read_ceiling"); each decode entry also
carries "gather_ceiling", a plain kernel reading exactly the blocks the
call reads (the paged access pattern's own ceiling).  --op stream sweeps the
streaming probe's launch shapes alone.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged decode attention: KV GB/s (% of HBM peak) and µs/call at batch 1"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E peak, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, TFLOP/s
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
# per operation: the kernel source and the host code that validates and
# plans its launch; a counter record is valid only for the digest it was
# taken under
_CSRC = os.path.join(ROOT, "paged_attention_decode_attn_amd", "csrc")
KERNEL_SOURCES = {op: [os.path.join(_CSRC, f) for f in (*k, "pa_host.cpp", "pa_internal.h")]
                  for op, k in (("decode", ("pa_device.hip",)), ("cache_write", ("pa_cache.hip",)),
                                ("prefill", ("pa_prefill.hip", "pa_prefill_host.cpp", "pa_prefill_internal.h")))}


def parse_args():
    from paged_attention_decode_attn_amd.workloads import CONFIG_ORDER, NEXT_CONFIG_ORDER, PREFILL_CONFIGS
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="long_ctx", choices=CONFIG_ORDER + NEXT_CONFIG_ORDER + list(PREFILL_CONFIGS))
    ap.add_argument("--op", default="decode", choices=["decode", "cache_write", "prefill", "stream"],
                    help="decode: the attention call (default); cache_write: the paged KV-cache "
                         "write before it, on --config's decode step or a bulk write (--bulk); "
                         "prefill: packed prefill chunks over the paged cache (--config prefill_8k or "
                         "chunked_prefill); stream: the streaming-read probe's ceiling over launch "
                         "shapes")
    ap.add_argument("--write-pieces", type=int, default=0,
                    help="with --op cache_write: 16-byte pieces per thread (0 = the library's choice)")
    ap.add_argument("--bulk", type=int, default=0,
                    help="with --op cache_write: write this many tokens to distinct random slots "
                         "of a large pool instead of the config's decode step")
    ap.add_argument("--workgroups", type=int, default=0, help="partition-kernel grid (0 = the planner's)")
    ap.add_argument("--min-share", type=int, default=0, help="smallest share in 32-token chunks (0 = the planner's)")
    ap.add_argument("--copies", type=int, default=0, help="rotated KV copies (0 = enough for >= 1 GiB)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--ceiling", action="store_true",
                    help="also time the gather probe over the workload's own blocks (on by default for the "
                         "full long_ctx run)")
    ap.add_argument("--only", action="store_true",
                    help="with the default long_ctx workload: measure it alone (no fp8 config, no read ceiling)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run plain 1 GiB device copies (HBM counter calibration)")
    ap.add_argument("--summarize", nargs=5, metavar=("TRACE", "FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE"),
                    help="turn rocprofv3 output directories of this workload into the text "
                         "summary and traffic record under profiles/ (no GPU needed)")
    ap.add_argument("--command", default="", help="with --summarize: the commands that made the runs")
    ap.add_argument("--counters", nargs="*", default=[], metavar="DIR",
                    help="with --summarize: rocprofv3 --pmc output directories of SQ/TA/TCP/GRBM counter "
                         "passes of the same workload, summarised with derived figures")
    return ap.parse_args()


def source_digest(op: str) -> str:
    """Digest of the code (comments and whitespace left out) of the sources
    an operation's kernels and launch plan come from: a stored traffic
    figure holds while this digest is unchanged."""
    h = hashlib.sha256()
    for path in KERNEL_SOURCES[op]:
        with open(path, encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, op: str = "decode"):
    """HBM bytes per launch of the operation's main kernel from the committed
    rocprofv3 counter summary, or None when its sources changed since."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(workload)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("kernel_source_sha256_16") != source_digest(op):
        return None
    return rec.get("hbm_bytes_per_launch")


def _db_rows(path, sql):
    import glob
    import sqlite3
    rows = []
    for db in sorted(glob.glob(os.path.join(path, "**", "*.db"), recursive=True)):
        con = sqlite3.connect(db)
        rows += con.execute(sql).fetchall()
        con.close()
    return rows


def cache_write_workload(args):
    """(spec, inputs, workload name, algorithmic bytes) of the cache write
    that ``--op cache_write`` times: the config's decode step, or ``--bulk``
    tokens to distinct random slots of a pool of at least twice as many."""
    from paged_attention_decode_attn_amd.workloads import CONFIGS, generate_cache_write, write_bytes
    spec = CONFIGS[args.config]
    if args.bulk:
        pool = max(spec.pool_blocks, -(-2 * args.bulk // spec.block_size))
        spec = spec.replace(batch=1, ctx_lo=16, ctx_hi=16, pool_blocks=pool)
    cw = generate_cache_write(spec, bulk_tokens=args.bulk or None)
    name = (f"bulk{args.bulk}_" if args.bulk else "decode_step_") + spec.name
    wb = write_bytes(cw.slot_mapping, spec.hkv, spec.head_dim, spec.kv_dtype, spec.pool_blocks,
                     spec.block_size)
    return spec, cw, name, wb


def summarize(args):
    """Kernel-trace statistics and calibrated HBM traffic of one workload."""
    from paged_attention_decode_attn_amd.workloads import CONFIGS, generate, kv_bytes
    trace, fetch, write, cfetch, cwrite = args.summarize
    flops = None
    if args.op == "prefill":
        from paged_attention_decode_attn_amd.workloads import PREFILL_CONFIGS, generate_prefill, prefill_flops
        pspec = PREFILL_CONFIGS[args.config]
        pf = generate_prefill(pspec)
        spec, wname = pspec, pspec.name
        flops = prefill_flops(pf.cache.context_lens, pf.chunk_lens, pspec.hq, pspec.head_dim, pspec.sliding_window)
        kvb = prefill_bytes(pf)
        kname, title, unit = "prefill_kernel", "paged prefill attention", "bytes (q, K/V once, out)"
        kernels = (("%prefill_kernel%", "prefill_kernel"),)
    elif args.op == "cache_write":
        spec, _, wname, kvb = cache_write_workload(args)
        kname, title, unit = "cache_write_kernel", "paged KV-cache write", "bytes (rows read + cache written)"
        kernels = (("%cache_write_kernel%", "cache_write_kernel"),)
    else:
        spec = CONFIGS[args.config]
        wname = spec.name
        w0 = generate(spec)
        kvb = kv_bytes(w0.context_lens, spec.hkv, spec.head_dim, spec.kv_dtype, w0.query_lens,
                       spec.sliding_window)
        kname, title, unit = "partition_kernel", "paged decode attention", "KV bytes"
        kernels = (("%partition_kernel%", "partition_kernel"), ("%reduce_kernel%", "reduce_kernel"))
    stats = _db_rows(trace, "select name, count(*), avg(duration), min(duration), max(duration) "
                            "from kernels group by name")

    def counter(path, name, like):
        r = _db_rows(path, f"select avg(value), count(*) from counters_collection where "
                           f"counter_name = '{name}' and kernel_name like '{like}'")
        return r[0] if r and r[0][0] is not None else (None, 0)
    n_copy = 1 << 30
    cf = n_copy / (counter(cfetch, "FETCH_SIZE", "%copyBuffer%")[0] * 1024)
    cw = n_copy / (counter(cwrite, "WRITE_SIZE", "%copyBuffer%")[0] * 1024)
    lines = [f"# rocprofv3 summary: {title}, workload {wname}", "",
             "Commands (run from the repository root on one MI355X):", ""]
    lines += ["    " + c for c in args.command.split(" ;; ") if c]
    lines += ["", f"Algorithmic {unit} per call: {kvb}", "",
              "Kernel trace (durations in ns):", "",
              "| kernel | calls | avg | min | max |", "|---|---|---|---|---|"]
    for name, n, avg, mn, mx in sorted(stats, key=lambda r: -r[2] * r[1]):
        short = name.replace("void ", "").replace("(anonymous namespace)::", "").split("(")[0]
        lines.append(f"| {short} | {n} | {avg:.0f} | {mn:.0f} | {mx:.0f} |")
    lines += ["", f"HBM counter calibration with a plain 1 GiB device copy: FETCH_SIZE x {cf:.3f}, "
              f"WRITE_SIZE x {cw:.3f} gives true bytes.", "",
              "| kernel | FETCH_SIZE KiB/dispatch | WRITE_SIZE KiB/dispatch | calibrated HBM bytes/dispatch |",
              "|---|---|---|---|"]
    record = {}
    for like, label in kernels:
        fk, nf = counter(fetch, "FETCH_SIZE", like)
        wk, nw = counter(write, "WRITE_SIZE", like)
        if fk is None or wk is None:
            continue
        hbm = fk * 1024 * cf + wk * 1024 * cw
        lines.append(f"| {label} | {fk:.0f} | {wk:.0f} | {hbm:.0f} |")
        record[label] = hbm
    part = [r for r in stats if kname in r[0]]
    if part and flops is not None:
        avg_ns = part[0][2]
        lines += ["", f"Algorithmic flops per call: {flops}", "",
                  f"{kname}: {flops / avg_ns / 1e3:.1f} TFLOP/s algorithmic "
                  f"({100 * flops / avg_ns / 1e3 / MFMA_BF16_PEAK_TFLOPS:.1f}% of the 2.5 PFLOP/s dense bf16 "
                  f"peak) at the traced average duration; HBM traffic {record.get(kname, 0) / kvb:.3f} x the "
                  f"bytes that must move once (q, the chunks' K/V, out)."]
    elif part:
        avg_ns = part[0][2]
        lines += ["", f"{kname}: {kvb / avg_ns:.1f} GB/s algorithmic "
                      f"({100 * kvb / avg_ns / HBM_PEAK_GBS:.1f}% of 8 TB/s) at the traced average "
                      f"duration; HBM traffic {record.get(kname, 0) / kvb:.3f} x the "
                      f"algorithmic bytes."]
    if args.counters:
        lines += counter_lines(args.counters, kernels)
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    fname = f"{kname}_{args.config}{'_bulk' + str(args.bulk) if args.op == 'cache_write' and args.bulk else ''}.md"
    with open(os.path.join(os.path.dirname(TRAFFIC_FILE), fname), "w") as f:
        f.write("\n".join(lines) + "\n")
    try:
        with open(TRAFFIC_FILE) as f:
            allrec = json.load(f)
    except (OSError, ValueError):
        allrec = {}
    if kname in record:
        allrec[wname] = {"kernel_source_sha256_16": source_digest(args.op),
                             "hbm_bytes_per_launch": round(record[kname]),
                             "algorithmic_bytes": kvb,
                             "calibration": {"fetch": round(cf, 4), "write": round(cw, 4)}}
        if flops is not None:
            allrec[wname]["algorithmic_flops"] = flops
        with open(TRAFFIC_FILE, "w") as f:
            json.dump(allrec, f, indent=1, sort_keys=True)
    print("\n".join(lines))


XCDS, CUS, SIMDS_PER_CU = 8, 256, 4     # MI355X


def counter_lines(dirs, kernels):
    """Per-dispatch averages of the counter passes and figures derived from
    them.  GRBM_GUI_ACTIVE is summed over the XCDs, so the kernel's own
    cycles are GRBM_GUI_ACTIVE / 8; SIMD-cycles are those times 1024 SIMDs."""
    vals = {}
    for d in dirs:
        for name, cname, v in _db_rows(d, "select kernel_name, counter_name, avg(value) from counters_collection "
                                          "group by kernel_name, counter_name"):
            for like, label in kernels:
                if like.strip("%") in name:
                    vals.setdefault(label, {})[cname] = v
    out = ["", "Counters (rocprofv3 --pmc, averages per dispatch; derived figures below the table):", "",
           "| kernel | counter | value |", "|---|---|---|"]
    for label, cs in vals.items():
        for c in sorted(cs):
            out.append(f"| {label} | {c} | {cs[c]:.0f} |")
    out += [""]
    for label, cs in vals.items():
        cyc = cs.get("GRBM_GUI_ACTIVE", 0) / XCDS
        simd_cyc = cyc * CUS * SIMDS_PER_CU
        fig = []
        if cyc:
            fig.append(f"kernel cycles (GRBM_GUI_ACTIVE / {XCDS}) {cyc:.0f}")
        if simd_cyc and "SQ_VALU_MFMA_BUSY_CYCLES" in cs:
            fig.append(f"MFMA busy {100 * cs['SQ_VALU_MFMA_BUSY_CYCLES'] / simd_cyc:.1f} % of SIMD-cycles")
        if simd_cyc and "SQ_ACTIVE_INST_VALU" in cs:
            fig.append(f"VALU busy {100 * 4 * cs['SQ_ACTIVE_INST_VALU'] / simd_cyc:.1f} % of SIMD-cycles "
                       f"(SQ_ACTIVE_INST_VALU x 4)")
        if cs.get("SQ_INSTS_MFMA"):
            fig.append(f"{cs['SQ_INSTS_VALU'] / cs['SQ_INSTS_MFMA']:.1f} VALU instructions per MFMA")
        if cs.get("SQ_WAVES"):
            fig.append(f"per wave: {cs.get('SQ_INSTS_VALU', 0) / cs['SQ_WAVES']:.0f} VALU, "
                       f"{cs.get('SQ_INSTS_MFMA', 0) / cs['SQ_WAVES']:.0f} MFMA, "
                       f"{cs.get('SQ_INSTS_VMEM_RD', 0) / cs['SQ_WAVES']:.0f} vector-memory reads")
        if cs.get("TCP_TCC_READ_REQ_sum"):
            fig.append(f"average L2 read latency {cs['TCP_TCC_READ_REQ_LATENCY_sum'] / cs['TCP_TCC_READ_REQ_sum']:.0f} "
                       f"cycles (TCP_TCC_READ_REQ_LATENCY / TCP_TCC_READ_REQ)")
        if cyc and "TA_BUSY_avr" in cs:
            fig.append(f"TA busy {100 * cs['TA_BUSY_avr'] / cyc:.0f} % of cycles")
        if cyc and "TA_ADDR_STALLED_BY_TC_CYCLES_sum" in cs:
            fig.append(f"TA address path stalled by the L1 {100 * cs['TA_ADDR_STALLED_BY_TC_CYCLES_sum'] / CUS / cyc:.0f} "
                       f"% of cycles (per CU)")
        if simd_cyc and "SQ_VALU_MFMA_COEXEC_CYCLES" in cs:
            fig.append(f"VALU issued while the MFMA unit is busy {100 * cs['SQ_VALU_MFMA_COEXEC_CYCLES'] / simd_cyc:.1f} "
                       f"% of SIMD-cycles")
        if cyc and "SQ_LDS_IDX_ACTIVE" in cs:
            fig.append(f"LDS active {100 * cs['SQ_LDS_IDX_ACTIVE'] / CUS / cyc:.0f} % of cycles (per CU), "
                       f"bank-conflict cycles {100 * cs.get('SQ_LDS_BANK_CONFLICT', 0) / max(cs['SQ_LDS_IDX_ACTIVE'], 1):.0f} "
                       f"% of LDS-active cycles")
        if cs.get("SQ_INSTS_LDS") and "SQ_WAIT_INST_LDS" in cs:
            fig.append(f"waves waiting on LDS results {cs['SQ_WAIT_INST_LDS'] / max(cs['SQ_INSTS_LDS'], 1):.1f} "
                       f"wave-cycles (in units of 4) per LDS instruction")
        out.append(f"{label}: " + "; ".join(fig) + ".")
    return out


def calibrate_copy():
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "device copy", "bytes_read_per_copy": n,
                      "bytes_written_per_copy": n, "copies": 5}), flush=True)


def cpu_baseline(w, seconds: float):
    """The float64 oracle as it stands, on whole sequences of the same
    workload, until about `seconds` of CPU time (at least one sequence)."""
    from threadpoolctl import threadpool_limits

    from oracle import paged_decode_attention
    from paged_attention_decode_attn_amd.workloads import kv_bytes
    inputs = w.numpy_inputs()
    spec = w.spec
    done_bytes, done_seqs, t = 0, 0, 0.0
    with threadpool_limits(limits=1):
        b = 0
        while True:
            t0 = time.perf_counter()
            paged_decode_attention(**inputs, batch_subset=[b])
            t += time.perf_counter() - t0
            done_bytes += kv_bytes(w.context_lens[b:b + 1], spec.hkv, spec.head_dim, spec.kv_dtype,
                                   w.query_lens[b:b + 1], spec.sliding_window)
            done_seqs += 1
            b = (b + 1) % spec.batch
            if t >= seconds:
                break
    return {"value": done_bytes / t / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{done_seqs} whole-sequence oracle calls of this workload "
                      f"({done_bytes} KV bytes, {t:.1f} s, 1 thread; "
                      f"{len(os.sched_getaffinity(0))} host cores visible)",
            "seconds": t}


WRITE_METRIC = "paged KV-cache write: GB/s (% of HBM peak) and µs/call"
PREFILL_METRIC = "paged prefill attention: TFLOP/s (% of dense bf16 MFMA peak) and ms/call"


def prefill_bytes(pf) -> int:
    """Bytes a prefill call must move at least once: the packed q rows and
    outputs, and the K/V rows of every attended token (each sequence's
    whole context, or from its first row's window on) for every kv head."""
    s = pf.spec
    w = s.sliding_window
    tokens = 0
    for L, n in zip(pf.cache.context_lens.tolist(), pf.chunk_lens.tolist()):
        tokens += L - (max(0, L - n - w + 1) if w > 0 and n > 0 else 0)
    per_token = s.hkv * (s.head_dim * 2 * (1 if s.kv_dtype == "fp8_e4m3fn" else 2)
                         + (8 if s.kv_dtype == "fp8_e4m3fn" else 0))
    return 2 * pf.q.numel() * 2 + tokens * per_token


def bench_prefill(args):
    """Packed prefill chunks over the paged cache: one call per step, timed
    eagerly and as a replayed HIP graph; the roofline is the matrix peak."""
    import torch

    from paged_attention_decode_attn_amd import binding as B
    from paged_attention_decode_attn_amd.workloads import PREFILL_CONFIGS, generate_prefill, prefill_flops

    spec = PREFILL_CONFIGS[args.config]
    print(f"[bench] generating {spec.name}", file=sys.stderr, flush=True)
    pf = generate_prefill(spec)
    flops = prefill_flops(pf.cache.context_lens, pf.chunk_lens, spec.hq, spec.head_dim, spec.sliding_window)
    nbytes = prefill_bytes(pf)
    d = pf.to("cuda")
    c = d.cache
    out = torch.empty_like(d.q)
    ext = spec.sliding_window > 0 or c.sinks is not None

    def call(stream=None):
        if ext:
            B.paged_attn_prefill_ext(d.q, c.k_cache, c.v_cache, c.block_tables, c.context_lens, d.cu_seqlens,
                                     pf.max_query_len, pf.scale, spec.sliding_window, c.sinks, out, stream=stream,
                                     k_scale=c.k_scale, v_scale=c.v_scale)
        else:
            B.paged_attn_prefill(d.q, c.k_cache, c.v_cache, c.block_tables, c.context_lens, d.cu_seqlens,
                                 pf.max_query_len, pf.scale, out, stream=stream, k_scale=c.k_scale, v_scale=c.v_scale)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    start.record()
    for _ in range(args.steps):
        call()
    stop.record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms = start.elapsed_time(stop) / args.steps
    gs = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=gs):
        for _ in range(args.steps):
            call(stream=gs)
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    start.record()
    graph.replay()
    stop.record()
    torch.cuda.synchronize()
    ms_graph = start.elapsed_time(stop) / args.steps
    del graph
    value = flops / (ms * 1e-3) / 1e12
    achieved = flops / (min(ms, ms_graph) * 1e-3) / 1e12
    res = {
        "metric": PREFILL_METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8_e4m3fn-kv/bf16-mfma" if spec.kv_dtype == "fp8_e4m3fn" else "bf16", "data": "synthetic",
        "config": {"workload": spec.name, "batch": spec.batch, "q_heads": spec.hq, "kv_heads": spec.hkv,
                   "head_dim": spec.head_dim, "kv_dtype": spec.kv_dtype, "block_size": spec.block_size,
                   "sliding_window": spec.sliding_window or None, "sinks": spec.sinks,
                   "context_lens": [int(x) for x in pf.cache.context_lens],
                   "chunk_lens": [int(x) for x in pf.chunk_lens]},
        "ms_per_call_graph": round(ms_graph, 6), "flops_per_call": flops, "bytes_per_call": nbytes,
        "wall_s_timed_region": round(t_wall, 4),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": measured_traffic(spec.name, "prefill"), "algorithmic_flops": flops,
                     "kernel": "prefill_kernel",
                     "timing": "faster of the eager and graph-replayed timed steps (one kernel per call)"},
    }
    if not args.no_cpu_baseline:
        from threadpoolctl import threadpool_limits

        from oracle import paged_prefill_attention
        h = pf.cache

        def bits(t):
            return t.view(torch.int16).numpy().view("uint16") if t.dtype == torch.bfloat16 else t.numpy()
        qb, kb, vb = bits(pf.q), bits(h.k_cache), bits(h.v_cache)
        fp8 = h.k_scale is not None
        kscale = h.k_scale.numpy() if fp8 else None
        vscale = h.v_scale.numpy() if fp8 else None
        tables, ctx, cu = h.block_tables.numpy(), h.context_lens.numpy(), pf.cu_seqlens.numpy()
        sinks = None if h.sinks is None else h.sinks.numpy()
        w = spec.sliding_window
        done, rows_done, t, r = 0, 0, 0.0, 0
        b = spec.batch - 1
        n = int(pf.chunk_lens[b])
        with threadpool_limits(limits=1):
            while t < args.cpu_seconds and rows_done < n:
                rows = list(range(n - 1 - r, max(n - 1 - r - 8, -1), -1))    # the longest rows first
                t0 = time.perf_counter()
                paged_prefill_attention(qb, kb, vb, tables, ctx, cu, pf.scale, kscale, vscale,
                                        "fp8_e4m3fn" if fp8 else "bf16", batch_subset=[b], row_subset=rows,
                                        sliding_window=w, sinks=sinks)
                t += time.perf_counter() - t0
                L = int(ctx[b])
                done += sum(4 * spec.head_dim * spec.hq * (min(L - n + x + 1, w) if w > 0 else L - n + x + 1)
                            for x in rows)
                rows_done += len(rows)
                r += len(rows)
        res["cpu_baseline"] = {"value": done / t / 1e12, "unit": "TFLOP/s", "cores": 1, "kind": "oracle",
                               "sample": f"{rows_done} rows of sequence {b} evaluated one by one by the oracle "
                                         f"({done} flops, {t:.1f} s, 1 thread)"}
    print(json.dumps(res), flush=True)


def bench_cache_write(args):
    """The paged KV-cache write: the new tokens' K/V rows of the config's
    decode step (or ``--bulk`` tokens to random slots of a large pool) into
    the cache, timed like the attention call; rows rotated over copies so
    they are read from HBM."""
    import torch

    from paged_attention_decode_attn_amd import binding as B
    from paged_attention_decode_attn_amd.workloads import write_bytes

    spec, cw, name, wb = cache_write_workload(args)
    B.paged_attn_set_write_pieces(args.write_pieces)
    d = cw.to("cuda")
    w = d.base
    row_bytes = 2 * d.k_new.numel() * 2
    copies = max(2, min(64, math.ceil((1 << 30) / max(row_bytes, 1)) + 1))
    rows = [(d.k_new.clone(), d.v_new.clone()) for _ in range(copies)]

    def call(i):
        kn, vn = rows[i % copies]
        B.paged_attn_reshape_and_cache(kn, vn, d.slot_mapping, w.k_cache, w.v_cache, w.k_scale, w.v_scale)

    for i in range(args.warmup):
        call(i)
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(args.steps):
        call(i)
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / args.steps
    gs = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=gs):
        for i in range(args.steps):
            call(i)
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    start.record()
    graph.replay()
    stop.record()
    torch.cuda.synchronize()
    ms_graph = start.elapsed_time(stop) / args.steps
    del graph
    value = wb / (ms * 1e-3) / 1e9
    # one kernel per call: its launch duration is the faster of the two
    # timings (eager calls are host-bound when the write is small)
    achieved = wb / (min(ms, ms_graph) * 1e-3) / 1e9
    res = {
        "metric": WRITE_METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16->fp8_e4m3fn+fp32 scales" if spec.kv_dtype == "fp8_e4m3fn" else "bf16",
        "data": "synthetic",
        "config": {"workload": name, "tokens": int(cw.k_new.shape[0]), "kv_heads": spec.hkv,
                   "head_dim": spec.head_dim, "kv_dtype": spec.kv_dtype, "pool_blocks": spec.pool_blocks,
                   "row_copies_rotated": copies},
        "us_per_call": round(ms * 1e3, 3), "us_per_call_graph": round(ms_graph * 1e3, 3),
        "bytes_per_call": wb,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(name, "cache_write"),
                     "algorithmic_bytes": wb,
                     "kernel": "cache_write_kernel",
                     "timing": "faster of the eager and graph-replayed timed steps"},
    }
    if not args.no_cpu_baseline:
        from threadpoolctl import threadpool_limits

        from oracle.cache_write import reshape_and_cache
        h = cw.base

        def bits(t):
            return t.view(torch.int16).numpy().view("uint16") if t.dtype == torch.bfloat16 else t.numpy()
        n = min(cw.k_new.shape[0], 4096)
        t0 = time.perf_counter()
        with threadpool_limits(limits=1):
            reshape_and_cache(bits(cw.k_new[:n]), bits(cw.v_new[:n]), cw.slot_mapping[:n].numpy(),
                              bits(h.k_cache), bits(h.v_cache),
                              None if h.k_scale is None else h.k_scale.numpy(),
                              None if h.v_scale is None else h.v_scale.numpy(), spec.kv_dtype)
        t = time.perf_counter() - t0
        nb = write_bytes(cw.slot_mapping[:n], spec.hkv, spec.head_dim, spec.kv_dtype, spec.pool_blocks,
                         spec.block_size)
        res["cpu_baseline"] = {"value": nb / t / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
                               "sample": f"oracle write of {n} tokens ({nb} bytes, {t:.2f} s incl. "
                                         f"copying the pool, 1 thread)"}
    print(json.dumps(res), flush=True)


def stream_ceiling(nbytes_list=(1 << 30,), steps: int = 20, warmup: int = 3):
    """The streaming-read probe over launch shapes (workgroups, threads,
    loads in flight, contiguous or grid-stride ranges) on buffers of the
    given sizes: the best rate per size is the achievable read ceiling."""
    import torch

    from paged_attention_decode_attn_amd import binding as B
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    shapes = [(cus * k, t, u, g) for k in (1, 2, 4, 8) for t in (256, 512) for u in (4, 8) for g in (0, 1)
              if k * t <= 2048]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    out = {}
    for nbytes in nbytes_list:
        bufs = [torch.zeros(nbytes // 4, dtype=torch.int32, device="cuda") for _ in range(2)]
        rows = []
        for wg, t, u, g in shapes:
            for i in range(warmup):
                B.paged_attn_probe_stream_read(bufs[i % 2], wg, t, u, g, sink)
            torch.cuda.synchronize()
            start.record()
            for i in range(steps):
                B.paged_attn_probe_stream_read(bufs[i % 2], wg, t, u, g, sink)
            stop.record()
            torch.cuda.synchronize()
            us = start.elapsed_time(stop) * 1e3 / steps
            rows.append({"workgroups": wg, "threads": t, "loads_in_flight": u,
                         "layout": "grid_stride" if g else "contiguous", "us": round(us, 3),
                         "GBs": round(nbytes / us / 1e3, 1)})
        best = max(rows, key=lambda r: r["GBs"])
        out[str(nbytes)] = {"best_GBs": best["GBs"], "best_frac_of_peak": round(best["GBs"] / HBM_PEAK_GBS, 4),
                            "best_shape": best, "shapes": rows}
        del bufs
    return out


def gather_ceiling(spec, w, pools, steps: int = 10, warmup: int = 2):
    """Read rate of the gather probe over exactly the bytes and places a
    decode call of this workload reads: every used block (all kv heads) of
    K, V and, for fp8, both scale arrays, from the same rotated pool copies;
    the best of a sweep of launch shapes."""
    import torch

    from paged_attention_decode_attn_amd import binding as B
    bt = w.block_tables.cpu()
    ids = []
    for b in range(spec.batch):
        L = int(w.context_lens[b])
        ids.append(bt[b, :(L + spec.block_size - 1) // spec.block_size])
    ids = torch.cat(ids).to(torch.int32).cuda()
    k0 = pools[0][0]
    nb = k0.shape[0]
    kvb = k0.stride(0) * k0.element_size()
    arrays = []
    for kc, vc, ks, vs in pools:
        a = [(kc, kvb, kvb), (vc, kvb, kvb)]
        if ks is not None:
            sb = ks.stride(0) * 4
            a += [(ks, sb, sb), (vs, sb, sb)]
        arrays.append(a)
    nbytes = ids.numel() * sum(x[2] for x in arrays[0])
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    rows = []
    for wg in (cus, 2 * cus, 4 * cus):
        for t in (256, 512, 1024):
            for u in (4, 8, 16):
                for i in range(warmup):
                    B.paged_attn_probe_gather_read(arrays[i % len(arrays)], ids, nb, wg, t, u, sink)
                torch.cuda.synchronize()
                start.record()
                for i in range(steps):
                    B.paged_attn_probe_gather_read(arrays[i % len(arrays)], ids, nb, wg, t, u, sink)
                stop.record()
                torch.cuda.synchronize()
                us = start.elapsed_time(stop) * 1e3 / steps
                rows.append((nbytes / us / 1e3, us, wg, t, u))
    best = max(rows)
    return {"bytes": nbytes, "blocks": int(ids.numel()), "best_GBs": round(best[0], 1),
            "best_frac_of_peak": round(best[0] / HBM_PEAK_GBS, 4), "best_us": round(best[1], 3),
            "best_shape": {"workgroups": best[2], "threads": best[3], "loads_in_flight": best[4]}}


def bench_decode(args, config: str, cpu_seconds: float, ceiling: bool = False):
    """One decode workload: eager steps (the value), the same steps with
    per-kernel HIP events (the roofline's kernel time), and a graph replay."""
    import torch

    from paged_attention_decode_attn_amd import binding as B
    from paged_attention_decode_attn_amd.workloads import CONFIGS, generate, kv_bytes

    spec = CONFIGS[config]
    print(f"[bench] generating {spec.name}", file=sys.stderr, flush=True)
    w = generate(spec)
    kvb = kv_bytes(w.context_lens, spec.hkv, spec.head_dim, spec.kv_dtype, w.query_lens, spec.sliding_window)
    dev = w.to("cuda")
    pool_bytes = 2 * dev.k_cache.numel() * dev.k_cache.element_size()
    copies = args.copies or min(64, max(2, math.ceil((1 << 30) / kvb) + 1))
    copies = max(1, min(copies, int((64 << 30) // max(pool_bytes, 1))))
    pools = [(dev.k_cache, dev.v_cache, dev.k_scale, dev.v_scale)]
    for _ in range(copies - 1):
        ks = None if dev.k_scale is None else dev.k_scale.permute(0, 2, 1).clone().permute(0, 2, 1)
        vs = None if dev.v_scale is None else dev.v_scale.permute(0, 2, 1).clone().permute(0, 2, 1)
        pools.append((dev.k_cache.clone(), dev.v_cache.clone(), ks, vs))
    out = torch.empty_like(dev.q)
    B.paged_attn_set_workgroups(args.workgroups)
    B.paged_attn_set_min_share(args.min_share)
    # the most tokens a sequence's rows read (the table's reach, or the
    # window plus the query rows over one more chunk)
    max_ctx = spec.block_size * spec.table_width
    if spec.sliding_window > 0:
        max_ctx = min(max_ctx, 32 * (-(-(spec.sliding_window + spec.qlen - 1) // 32) + 1))
    plan = B.paged_attn_plan(spec.batch, spec.hq, spec.hkv, spec.head_dim, spec.qlen, max_ctx, spec.kv_dtype,
                             torch.cuda.get_device_properties(0).multi_processor_count)
    ext = spec.sliding_window > 0 or dev.sinks is not None

    def call(i):
        kc, vc, ks, vs = pools[i % copies]
        if ext:
            B.paged_attn_decode_ext(dev.q, kc, vc, dev.block_tables, dev.context_lens, dev.query_lens,
                                    dev.scale, ks, vs, spec.sliding_window, dev.sinks, out)
        else:
            B.paged_attn_decode(dev.q, kc, vc, dev.block_tables, dev.context_lens, dev.query_lens,
                                dev.scale, ks, vs, out)

    print(f"[bench] {config}: warmup {args.warmup}, copies {copies}, plan {plan}", file=sys.stderr, flush=True)
    for i in range(args.warmup):
        call(i)
    torch.cuda.synchronize()

    # timed region: exactly K steps, bracketed by synchronisation
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record()
    for i in range(args.steps):
        call(i)
    stop.record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms_per_step = start.elapsed_time(stop) / args.steps

    # the same K steps again with HIP events recorded by the library around
    # each of its kernels, on the stream the kernels run on: per-kernel
    # durations for the roofline (events between launches add their own
    # gaps, so the step time above is measured without them)
    B.paged_attn_profile_begin(args.steps)
    torch.cuda.synchronize()
    start.record()
    for i in range(args.steps):
        call(i)
    stop.record()
    torch.cuda.synchronize()
    prof = B.paged_attn_profile_end()
    ms_with_events = start.elapsed_time(stop) / args.steps
    B.paged_attn_set_workgroups(0)
    B.paged_attn_set_min_share(0)

    # the same K steps captured into one HIP graph and replayed: the device
    # time of a call without the host's per-call launch cost (the pages'
    # engine replays its decode step as a graph); the workspace exists on
    # the capture stream before capture begins
    gs = torch.cuda.Stream()
    with torch.cuda.stream(gs):
        for i in range(2):
            call(i)
    gs.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=gs):
        for i in range(args.steps):
            call(i)
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    start.record()
    graph.replay()
    stop.record()
    torch.cuda.synchronize()
    ms_graph = start.elapsed_time(stop) / args.steps
    del graph

    part_ms = prof["partition_ms"] / max(prof["calls"], 1)
    red_ms = prof["reduce_ms"] / max(prof["calls"], 1)
    value = kvb / (ms_per_step * 1e-3) / 1e9
    achieved = kvb / (part_ms * 1e-3) / 1e9
    traffic = measured_traffic(spec.name)
    res = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8_e4m3fn-kv/bf16-mfma" if spec.kv_dtype == "fp8_e4m3fn" else "bf16",
        "data": "synthetic",
        "config": {"workload": spec.name, "batch": spec.batch,
                   "query_len": (f"U[{spec.qlen_lo}, {spec.qlen}] (seed {spec.seed})" if spec.qlen_lo
                                 else spec.qlen),
                   "q_heads": spec.hq, "kv_heads": spec.hkv, "head_dim": spec.head_dim,
                   "kv_dtype": spec.kv_dtype, "block_size": spec.block_size,
                   "sliding_window": spec.sliding_window or None, "sinks": spec.sinks,
                   "context_lens": ([int(x) for x in w.context_lens] if spec.batch <= 4
                                    else f"U[{spec.ctx_lo}, {spec.ctx_hi}] (seed {spec.seed})"),
                   "workgroups": plan["workgroups"], "heads_per_group": plan["heads_per_group"],
                   "min_share_chunks": plan["min_share_chunks"], "kv_copies_rotated": copies},
        "us_per_call": round(ms_per_step * 1e3, 3),
        "us_per_call_with_kernel_events": round(ms_with_events * 1e3, 3),
        "us_per_call_graph": round(ms_graph * 1e3, 3),
        "kv_GBs_graph": round(kvb / (ms_graph * 1e-3) / 1e9, 2),
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "kv_bytes_per_call": kvb,
        "kernel_us": {"partition": round(part_ms * 1e3, 3), "reduce": round(red_ms * 1e3, 3)},
        "wall_s_timed_region": round(t_wall, 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "algorithmic_bytes": kvb,
                     "kernel": "partition_kernel"},
    }
    if ceiling and spec.sliding_window == 0:
        print(f"[bench] {config}: gather-probe ceiling", file=sys.stderr, flush=True)
        res["gather_ceiling"] = gather_ceiling(spec, w, pools)
    if cpu_seconds > 0:
        print(f"[bench] {config}: cpu baseline (oracle)", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(w, cpu_seconds)
    del pools, dev
    torch.cuda.empty_cache()
    return res


def main():
    args = parse_args()
    if args.summarize:
        summarize(args)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE {world}); the decode-attention path has no multi-GPU mode here.",
              file=sys.stderr, flush=True)
        sys.exit(2)

    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.op == "cache_write":
        bench_cache_write(args)
        return
    if args.op == "prefill":
        bench_prefill(args)
        return
    if args.op == "stream":
        print("[bench] streaming-read probe", file=sys.stderr, flush=True)
        print(json.dumps({"op": "stream_read_ceiling", "unit": "GB/s", "peak": HBM_PEAK_GBS,
                          "sizes": stream_ceiling((1 << 30, 536870912, 266846144), steps=args.steps,
                                                  warmup=args.warmup)}), flush=True)
        return

    cpu_s = 0.0 if args.no_cpu_baseline else args.cpu_seconds
    full = args.config == "long_ctx" and not args.only
    res = bench_decode(args, args.config, cpu_s, ceiling=full or args.ceiling)
    if full:
        # the second target configuration, measured the same way in the
        # same run, and the read ceiling of a plain streaming kernel at the
        # two calls' byte counts
        res["fp8_config"] = bench_decode(args, "fp8", min(cpu_s, 5.0), ceiling=True)
        print("[bench] streaming-read probe", file=sys.stderr, flush=True)
        ceil = stream_ceiling((res["kv_bytes_per_call"], res["fp8_config"]["kv_bytes_per_call"]),
                              steps=max(5, min(args.steps, 20)), warmup=3)
        res["read_ceiling"] = {k: {"best_GBs": v["best_GBs"], "best_frac_of_peak": v["best_frac_of_peak"],
                                   "best_shape": v["best_shape"]} for k, v in ceil.items()}
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
