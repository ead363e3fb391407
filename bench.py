#!/usr/bin/env python3
"""Benchmark of the CSA2 hot path on one MI355X.

One step = the whole Full-layer hot path over one decode batch of the
long-context workload (4 sequences x 1,048,576 compressed entries, one query
each): indexer scan -> exact top-512 -> FP4 gather/dequant + joint sparse and
sliding-window attention.  Inputs are seeded synthetic tensors resident in HBM
before timing starts.  Prints one JSON line.

Also reported, outside the headline: per-stage times (HIP events on the
launch stream), the Reuse-mode attention of three later layers over the same
selection, the roofline of the dominant kernel (the indexer scan), and the CPU
oracle timed on this host's cores on the same batch.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
WORKLOADS = {
    "long_decode": dict(B=4, N=1 << 20),
    "batched_decode": dict(B=64, N=131072),
    "tiny_decode": dict(B=1, N=2048),
    # one Full layer (index, top-512, attention) and three Reuse layers over its selection
    "reuse_group": dict(B=32, N=262144),
    # 4096 query tokens after a 65536-token prefix, compression ratio 2
    "causal_prefill": dict(B=1, N=34816, q_per_seq=4096, ratio=2, prefix=65536),
}
# the workloads reported beside the headline in the default run (sub-objects of its line)
SIDE_WORKLOADS = ("batched_decode", "reuse_group", "causal_prefill")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="long_decode", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing leg")
    ap.add_argument("--no-side-workloads", action="store_true",
                    help="time only the headline workload (by default the batched-decode, reuse-group and "
                         "causal-prefill workloads follow it as sub-objects of the same line)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run torch.neg over 1 GiB of fp32 (reads and writes 1 GiB: the reference dispatch "
                         "that scales rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE to bytes)")
    ap.add_argument("--summarize-counters", nargs="+", metavar="ARG",
                    help="KERNEL DIR...: per-dispatch means of every counter that rocprofv3 --pmc runs "
                         "wrote under the DIRs, for the kernels whose name contains KERNEL")
    ap.add_argument("--summarize", nargs="+", metavar="DIR",
                    help="print the profile summary of rocprofv3 CSV output (kernel stats, the FETCH_SIZE run, the "
                         "WRITE_SIZE run and optionally the MFMA-counter run) instead of benchmarking")
    return ap.parse_args()


# Sources of the one-query scan kernel: the recorded traffic holds only while they and its compile
# flags are unchanged (of the public header, only its constants count: its documentation does not
# change the kernel).
SCAN_SOURCES = ["compressed_sparse_attention_02_amd/csrc/index.hip", "compressed_sparse_attention_02_amd/csrc/idx_tile.h",
                "compressed_sparse_attention_02_amd/csrc/idx_plan.h",
                "compressed_sparse_attention_02_amd/csrc/csa2_common.h", "include/csa2.h"]
PMC_SUMMARY = os.path.join(ROOT, "profiles", "idx_scan_kernel_long_decode_hbm_traffic.md")
CAL_BYTES = 1 << 30          # bytes the calibration dispatch reads, and writes


def scan_sources_sha256():
    import hashlib
    from compressed_sparse_attention_02_amd import build as hip_build
    h = hashlib.sha256()
    for f in SCAN_SOURCES:
        data = open(os.path.join(ROOT, f), "rb").read()
        if f.endswith("csa2.h"):
            data = b"".join(l for l in data.splitlines(keepends=True) if l.lstrip().startswith(b"#define"))
        h.update(data)
    h.update(repr((hip_build.FLAGS, hip_build.FILE_FLAGS.get("index.hip", []))).encode())
    return h.hexdigest()


def recorded_traffic():
    """HBM bytes per scan launch from the committed counter summary, or None when it is missing
    or was taken on other kernel sources."""
    try:
        text = open(PMC_SUMMARY).read()
    except OSError:
        return None
    fields = dict(line.split(":", 1) for line in text.splitlines() if line.startswith("- ") and ":" in line)
    fields = {k[2:].strip(): v.strip().strip("`") for k, v in fields.items()}
    if fields.get("scan sources sha256") != scan_sources_sha256():
        return None
    try:
        return float(fields["HBM bytes per launch"])
    except (KeyError, ValueError):
        return None


def summarize_counters(kernel, dirs):
    """Markdown table of the per-dispatch mean of each counter in rocprofv3 --pmc CSV output,
    over the dispatches of the kernels whose name contains `kernel`."""
    import csv
    import glob
    from collections import defaultdict
    vals = defaultdict(lambda: defaultdict(list))
    for d in dirs:
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                if kernel in r["Kernel_Name"]:
                    vals[r["Kernel_Name"]][r["Counter_Name"]].append(float(r["Counter_Value"]))
    for name, cs in sorted(vals.items()):
        print(f"### {name}\n\n| counter | per dispatch | dispatches |\n|---|---|---|")
        for c, v in sorted(cs.items()):
            print(f"| {c} | {sum(v) / len(v):.4g} | {len(v)} |")
        print()
    return 0


def summarize(stats_dir, fetch_dir=None, write_dir=None, mfma_dir=None):
    """Markdown summary of rocprofv3 CSV output: per-kernel durations of the bench run and the
    per-dispatch FETCH_SIZE / WRITE_SIZE of the scan, scaled by the calibration dispatch."""
    import csv
    import glob

    def rows(d, suffix):
        out = []
        for f in glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True):
            out += list(csv.DictReader(open(f)))
        return out

    print("### Kernel durations (rocprofv3 --kernel-trace --stats)\n")
    print("| kernel | calls | average us | min us | max us |\n|---|---|---|---|---|")
    for r in sorted(rows(stats_dir, "kernel_stats.csv"), key=lambda r: -float(r["TotalDurationNs"])):
        name = r["Name"].split("(")[0]
        if "csa2" in name:
            print(f"| {name} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | {float(r['MinNs']) / 1e3:.1f} | "
                  f"{float(r['MaxNs']) / 1e3:.1f} |")

    def per_dispatch(d, counter):
        acc = {}
        data = [r for r in rows(d, "counter_collection.csv") if r["Counter_Name"] == counter]
        # the benchmarked scan is the largest-grid one (a Reindex pass scans its pools with a smaller grid)
        scan_grid = max((int(r["Grid_Size"]) for r in data if "idx_scan_kernel" in r["Kernel_Name"]), default=0)
        # the calibration is the 1 GiB torch.neg, the largest neg dispatch (the input generator runs smaller ones)
        cal_grid = max((int(r["Grid_Size"]) for r in data if "neg_kernel" in r["Kernel_Name"]), default=0)
        for r in data:
            name = r["Kernel_Name"]
            key = ("scan" if "idx_scan_kernel" in name and int(r["Grid_Size"]) == scan_grid else
                   "scan_mx" if "idx_scan_mx_kernel" in name else
                   "cal" if "neg_kernel" in name and int(r["Grid_Size"]) == cal_grid else
                   "combine" if "attend_combine" in name else
                   "attend" if ("attend_kernel" in name or "attend_cs_kernel" in name) else None)
            if key:
                acc.setdefault(key, {}).setdefault(r["Dispatch_Id"], 0.0)
                acc[key][r["Dispatch_Id"]] += float(r["Counter_Value"])
        return {k: sum(v.values()) / len(v) for k, v in acc.items()}, {k: len(v) for k, v in acc.items()}

    if not fetch_dir or not write_dir:
        return 0
    f, fn = per_dispatch(fetch_dir, "FETCH_SIZE")
    w, wn = per_dispatch(write_dir, "WRITE_SIZE")
    f_scale = CAL_BYTES / (f["cal"] * 1024)
    w_scale = CAL_BYTES / (w["cal"] * 1024)
    traffic = f["scan"] * 1024 * f_scale + w["scan"] * 1024 * w_scale
    print("\n### HBM traffic of idx_scan_kernel (rocprofv3 --pmc)\n")
    print(f"- FETCH_SIZE KiB per scan dispatch: {f['scan']:.0f} (mean of {fn['scan']})")
    print(f"- WRITE_SIZE KiB per scan dispatch: {w['scan']:.0f} (mean of {wn['scan']})")
    print(f"- calibration dispatch (torch.neg, reads and writes {CAL_BYTES} B): FETCH_SIZE {f['cal']:.0f} KiB, "
          f"WRITE_SIZE {w['cal']:.0f} KiB")
    print(f"- FETCH scale: {f_scale:.4f}")
    print(f"- WRITE scale: {w_scale:.4f}")
    print(f"- HBM bytes per launch: {traffic:.0f}")
    print(f"- scan sources sha256: `{scan_sources_sha256()}`")
    if "scan_mx" in f and "scan_mx" in w:
        mx = f["scan_mx"] * 1024 * f_scale + w["scan_mx"] * 1024 * w_scale
        print("\n### HBM traffic of idx_scan_mx_kernel (MXFP4 indexer, same runs and scales)\n")
        print(f"- FETCH_SIZE KiB per dispatch: {f['scan_mx']:.0f} (mean of {fn['scan_mx']})")
        print(f"- WRITE_SIZE KiB per dispatch: {w['scan_mx']:.0f} (mean of {wn['scan_mx']})")
        print(f"- HBM bytes per launch: {mx:.0f}")
    # attention kernels, split by grid size (the single-layer call and the
    # three-layer Reuse call launch different grids)
    def by_grid(d, counter, kernel):
        acc = {}
        for r in rows(d, "counter_collection.csv"):
            if r["Counter_Name"] == counter and any(k in r["Kernel_Name"] for k in kernel.split("|")):
                g = acc.setdefault((r["Kernel_Name"].split("(")[0].replace("void csa2::", "").replace("csa2::", ""),
                                    int(r["Grid_Size"])), {})
                v = g.setdefault(r["Dispatch_Id"], [0.0, int(r["End_Timestamp"]) - int(r["Start_Timestamp"])])
                v[0] += float(r["Counter_Value"])
        return {k: (sum(x[0] for x in v.values()) / len(v), sum(x[1] for x in v.values()) / len(v), len(v))
                for k, v in acc.items()}

    kinds = "attend_kernel|attend_cs_kernel|attend_combine_kernel"
    print("\n### attention kernels per launch shape (same FETCH / WRITE runs and scales)\n")
    fa, wa = by_grid(fetch_dir, "FETCH_SIZE", kinds), by_grid(write_dir, "WRITE_SIZE", kinds)
    for key in sorted(fa, key=lambda k: (k[1], k[0])):
        if key in wa:
            print(f"- {key[0]}, grid {key[1]} threads: FETCH {fa[key][0] * 1024 * f_scale:.0f} B, "
                  f"WRITE {wa[key][0] * 1024 * w_scale:.0f} B per dispatch (means of {fa[key][2]})")
    if mfma_dir:
        print("\n### MFMA work of the attention kernels (rocprofv3 --pmc SQ_INSTS_VALU_MFMA_MOPS_BF16)\n")
        mo = by_grid(mfma_dir, "SQ_INSTS_VALU_MFMA_MOPS_BF16", "attend_kernel|attend_cs_kernel")
        for key in sorted(mo, key=lambda k: (k[1], k[0])):
            flops, ns, n = mo[key][0] * 512, mo[key][1], mo[key][2]
            print(f"- {key[0]}, grid {key[1]} threads: {flops:.4g} bf16 MFMA flop per dispatch, {ns / 1e3:.1f} us per "
                  f"dispatch under counter collection -> {flops / ns / 1e3:.2f} TFLOP/s = "
                  f"{flops / ns / 1e3 / MFMA_BF16_PEAK_TFLOPS:.4f} of 2.5 PFLOP/s (means of {n})")
    return 0


def main():
    args = parse()
    if args.summarize:
        return summarize(*args.summarize)
    if args.summarize_counters:
        return summarize_counters(args.summarize_counters[0], args.summarize_counters[1:])
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
              "the data-parallel path would shard sequences across GPUs with no exchange", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import compressed_sparse_attention_02_amd as csa
    import csa2_gen as G

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.workload == "causal_prefill":
        return prefill_main(args, dev)
    if args.workload == "reuse_group":
        line = {"metric": METRIC, **reuse_group_section(args, dev)}
        if args.copy_calibration:
            copy_calibration(dev)
        print(json.dumps(line), flush=True)
        return 0
    wl = WORKLOADS[args.workload]
    B, N = wl["B"], wl["N"]
    print(f"[bench] generating {args.workload}: B={B} N={N}", file=sys.stderr, flush=True)
    # large generation chunks: the generator is counter-based per element, so the bytes do not
    # depend on the chunking, and fewer chunks keep the dispatch count down under a profiler
    c = G.make_case(args.workload, B=B, N=N, n_layers=4, seed=0, device=dev, chunk_rows=1 << 19)
    print("[bench] inputs generated", file=sys.stderr, flush=True)
    T = c.T
    q_idx = c.q_idx.view(torch.bfloat16)
    k_idx = c.k_idx.view(torch.bfloat16)
    q0 = c.q[0].view(torch.bfloat16)
    swa0 = c.swa[0].view(torch.bfloat16)
    q_re = c.q[1:].view(torch.bfloat16).contiguous()
    swa_re = c.swa[1:].view(torch.bfloat16).contiguous()

    # long rows: the scan writes only tile maxima and the selection re-derives candidate
    # scores (a score matrix would save the candidate pass its key re-reads, but writing it
    # slows the scan by more at every batch measured); short rows keep the score matrix and
    # select in LDS
    rows = N <= csa.TOPK_ROW_MAX
    scores = torch.empty((T, N), dtype=torch.float32, device=dev) if rows else None
    tile_max = torch.empty((T, csa.tile_max_ld(N)), dtype=torch.float32, device=dev)
    stats = torch.empty(csa.index_stats_bytes(T, 1, N) // 4, dtype=torch.int32, device=dev)
    idx = torch.empty((T, 512), dtype=torch.int32, device=dev)
    idx_b = torch.empty((T, 512), dtype=torch.int32, device=dev)
    out = torch.empty((T, 64, 512), dtype=torch.bfloat16, device=dev)
    out_re = torch.empty((3, T, 64, 512), dtype=torch.bfloat16, device=dev)
    ws_t = torch.empty(max(1, csa.topk_workspace_bytes(T, N)), dtype=torch.uint8, device=dev)
    ws_a = torch.empty(max(1, csa.attend_workspace_bytes(T)), dtype=torch.uint8, device=dev)
    ws_r = torch.empty(max(1, csa.attend_workspace_bytes(T, n_layers=3)), dtype=torch.uint8, device=dev)
    ws_a = ws_a if csa.attend_workspace_bytes(T) else None

    # Every timed call is bound once (csa.bind): the same library launches with the binding's
    # argument checks and marshalling done up front, so per-call Python stays out of the timing.
    do_index = csa.bind(csa.csa2_index, q_idx, c.w_idx, k_idx, c.q_pos, 1, 1, want_scores=rows, scores=scores,
                        tile_max=tile_max, stats=stats)
    do_topk = csa.bind(csa.csa2_topk, scores, tile_max, stats, q_idx, c.w_idx, k_idx, c.q_pos, 1, 1, indices=idx,
                       workspace=ws_t)
    do_topk_bf16 = csa.bind(csa.csa2_topk, scores, tile_max, stats, q_idx, c.w_idx, k_idx, c.q_pos, 1, 1,
                            indices=idx_b, workspace=ws_t, select=csa.SELECT_BF16)
    do_attend = csa.bind(csa.csa2_attend_fp4, q0, c.kv_codes, c.kv_scales, idx, swa0, c.swa_end, None,
                         c.softmax_scale, 1, 128, out=out, workspace=ws_a)
    do_reuse = csa.bind(csa.csa2_reuse_attend, q_re, c.kv_codes, c.kv_scales, idx, swa_re, c.swa_end, None,
                        c.softmax_scale, 1, 128, out=out_re, workspace=ws_r)

    # hierarchical sparse indexer: the Full layer's candidate pool, then a Reindex layer's
    # own top-512 within it (its indexer query drawn under another seed)
    pool = torch.empty((T, csa.HSI_POOL), dtype=torch.int32, device=dev)
    ws_p = torch.empty(csa.hsi_pool_workspace_bytes(T, N), dtype=torch.uint8, device=dev)
    ws_x = torch.empty(csa.reindex_workspace_bytes(T), dtype=torch.uint8, device=dev)
    idx_x = torch.empty((T, 512), dtype=torch.int32, device=dev)
    q_x = G.normal_bf16(1, G.ST_QIDX, 0, T * csa.IDX_HEADS * csa.IDX_DIM, dev).view(
        T, csa.IDX_HEADS, csa.IDX_DIM).view(torch.bfloat16)
    w_x = G.uniform_f32(1, G.ST_W, 0, T * csa.IDX_HEADS, dev).view(T, csa.IDX_HEADS)

    do_pool = csa.bind(csa.csa2_hsi_pool, tile_max, stats, q_idx, c.w_idx, k_idx, c.q_pos, 1, 1, pool=pool,
                       workspace=ws_p)
    do_reindex = csa.bind(csa.csa2_reindex, pool, q_x, w_x, k_idx, 1, indices=idx_x, workspace=ws_x)

    def step():
        do_index()
        do_topk()
        do_attend()

    stream = torch.cuda.current_stream(dev)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # ---- headline: K whole steps, wall clock between synchronisations
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    print(f"[bench] {args.steps} steps timed: {ms_step:.4f} ms per step", file=sys.stderr, flush=True)

    # ---- per-stage timing with events on the launch stream
    def timed(fn, reps):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, b in ev:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        ts = sorted(a.elapsed_time(b) * 1e3 for a, b in ev)
        return ts[len(ts) // 2], sum(ts) / len(ts)

    reps = max(10, args.steps)
    idx_med, idx_avg = timed(do_index, reps)
    topk_med, _ = timed(do_topk, reps)
    do_index()
    topk_bf16_med, _ = timed(do_topk_bf16, reps)
    do_index()
    do_topk()
    att_med, att_avg = timed(do_attend, reps)
    do_reuse()
    reuse_med, _ = timed(do_reuse, reps)
    do_index()
    do_pool()
    do_reindex()
    pool_med, _ = timed(do_pool, reps)
    reindex_med, _ = timed(do_reindex, reps)
    print("[bench] stages timed", file=sys.stderr, flush=True)

    # dominant kernel: the indexer scan (csa2_index is that one kernel).
    # Algorithmic bytes per launch: each sequence's keys once (256 B/entry),
    # q_idx (8 KiB) and w (128 B) per query, its outputs (tile maxima, 4 B per
    # 16 entries; the score matrix, 4 B per entry, only for short rows) and
    # the 16-byte summary header per query.
    idx_bytes = B * N * 256 + T * (8192 + 128 + 16) + T * csa.tile_max_ld(N) * 4 + (T * N * 4 if rows else 0)
    achieved = idx_bytes / (idx_avg * 1e-6) / 1e9
    step_bytes = T * G.algorithmic_bytes_decode_query(N)

    # the attention call (gather + dequant + attention, plus its merge): per
    # query 512 FP4 rows (272 B), 128 window rows (1 KiB), q and out (64 KiB
    # each), the indices (2 KiB); 2 x 64 heads x 640 rows x 512 x 2 flop
    att_bytes = T * (512 * 272 + 128 * 1024 + 65536 + 65536 + 512 * 4)
    att_flops = T * 2 * (2 * 64 * 640 * 512)
    att_gbps = att_bytes / (att_avg * 1e-6) / 1e9
    att_tflops = att_flops / (att_avg * 1e-6) / 1e12

    # ---- the same step with the MXFP4 indexer (FP4 queries and keys, 68 B per key)
    mx = mxfp4_step(c, G, csa, args, stream, timed, idx, out, ws_t, ws_a)
    print("[bench] MXFP4-indexer and deployed-format steps timed", file=sys.stderr, flush=True)

    # ---- the KV write (compressor, indexer-K projection, RoPE, FP4 cache) for this batch's new
    # entries and for a prefill chunk
    kvw = kv_write_section(csa, G, dev, B)
    print("[bench] KV write timed", file=sys.stderr, flush=True)

    # plain copy bandwidth of this machine (context for the roofline fraction)
    x = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    y = torch.empty_like(x)
    y.copy_(x)
    cp_med, _ = timed(lambda: y.copy_(x), 10)
    copy_gbps = 2 * (1 << 30) / (cp_med * 1e-6) / 1e9
    del x, y
    if args.copy_calibration:
        copy_calibration(dev)

    line = {
        "metric": METRIC,
        "value": T / (ms_step * 1e-3),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "batch": B, "entries_per_seq": N, "queries_per_seq": 1,
                   "indexer": "32x128 bf16", "topk": 512, "heads": 64, "head_dim": 512, "window": 128,
                   "main_kv": "MXFP4 E2M1+E8M0/32", "parallelism": "none (1 GPU)"},
        "step_hbm_GBps": step_bytes / (ms_step * 1e-3) / 1e9,
        "step_frac_of_peak": step_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "roofline": {"kernel": "idx_scan_kernel (all of csa2_index)", "bound": "hbm", "achieved": achieved,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": recorded_traffic() if args.workload == "long_decode" else None,
                     "algorithmic_bytes_per_launch": idx_bytes, "avg_launch_us": idx_avg},
        "stages_us": {"index": idx_med, "topk": topk_med, "attend": att_med, "reuse_3_layers": reuse_med,
                      "topk_bf16_select": topk_bf16_med},
        "hierarchical_us": {"pool": pool_med, "reindex": reindex_med,
                            "note": "outside the step: a Full layer's 16384-entry candidate pool (after its scan) "
                                    "and one Reindex layer's top-512 within it"},
        "attention": {"call": "csa2_attend_fp4 (attend + merge kernels)", "avg_us": att_avg,
                      "algorithmic_bytes": att_bytes, "GBps": att_gbps, "frac_hbm": att_gbps / HBM_PEAK_GBPS,
                      "flops": att_flops, "TFLOPs": att_tflops, "frac_mfma_bf16": att_tflops / MFMA_BF16_PEAK_TFLOPS},
        "mxfp4_indexer": mx,
        "kv_write": kvw,
        "copy_GBps": copy_gbps,
    }

    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(c, G)
    if args.workload == "long_decode" and not args.no_side_workloads:
        # the other workloads, each on its own inputs (the headline's are freed first)
        del c, q_idx, k_idx, q0, swa0, q_re, swa_re, scores, tile_max, stats, out, out_re, ws_t, ws_a, ws_r
        del pool, ws_p, ws_x, q_x, w_x, do_index, do_topk, do_topk_bf16, do_attend, do_reuse, do_pool, do_reindex
        torch.cuda.empty_cache()
        side = {}
        for name in SIDE_WORKLOADS:
            print(f"[bench] side workload {name}", file=sys.stderr, flush=True)
            if name == "causal_prefill":
                side[name] = prefill_section(args, dev)
            elif name == "reuse_group":
                side[name] = reuse_group_section(args, dev)
            else:
                side[name] = decode_section(args, dev, name)
            torch.cuda.empty_cache()
            print(f"[bench] side workload {name}: {side[name]['ms_per_step']:.4f} ms per step", file=sys.stderr,
                  flush=True)
        line["workloads"] = side
    print(json.dumps(line), flush=True)
    return 0


METRIC = "decode queries/s + achieved HBM GB/s (% peak), CSA2 top-512 FP4 attn at 1 GPU"


def copy_calibration(dev):
    """torch.neg over CAL_BYTES of fp32 (reads and writes CAL_BYTES): the reference dispatch
    that scales rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE to bytes."""
    import torch
    xf = torch.ones(CAL_BYTES // 4, dtype=torch.float32, device=dev)
    yf = torch.empty_like(xf)
    torch.neg(xf, out=yf)
    torch.cuda.synchronize()
    del xf, yf


def _timer(stream):
    """Median and mean duration (us) of fn() over reps runs, from HIP events recorded on the
    launch stream around each run."""
    import torch

    def timed(fn, reps):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, b in ev:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        ts = sorted(a.elapsed_time(b) * 1e3 for a, b in ev)
        return ts[len(ts) // 2], sum(ts) / len(ts)
    return timed


def _wall_ms(step, steps, warmup):
    """Wall-clock ms per step over `steps` steps after `warmup`, between synchronisations."""
    import torch
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def _full_layer(csa, c, dev, T, N, n_layers_reuse=0):
    """Bound calls of one Full layer over case c (index -> top-512 -> attention), and the
    buffers they write; long rows take the tile regime (no score matrix)."""
    import torch
    bf = torch.bfloat16
    rows = N <= csa.TOPK_ROW_MAX
    with_scores = rows
    scores = torch.empty((T, N), dtype=torch.float32, device=dev) if with_scores else None
    tile_max = torch.empty((T, csa.tile_max_ld(N)), dtype=torch.float32, device=dev)
    stats = torch.empty(csa.index_stats_bytes(T, c.q_per_seq, N) // 4, dtype=torch.int32, device=dev)
    idx = torch.empty((T, 512), dtype=torch.int32, device=dev)
    out = torch.empty((T, 64, 512), dtype=bf, device=dev)
    ws_t = torch.empty(max(1, csa.topk_workspace_bytes(T, N)), dtype=torch.uint8, device=dev)
    ws_a = torch.empty(max(1, csa.attend_workspace_bytes(T)), dtype=torch.uint8, device=dev)
    ix = (c.q_idx.view(bf), c.w_idx, c.k_idx.view(bf), c.q_pos, c.ratio, c.q_per_seq)
    calls = dict(
        index=csa.bind(csa.csa2_index, *ix, want_scores=with_scores, scores=scores, tile_max=tile_max, stats=stats),
        topk=csa.bind(csa.csa2_topk, scores, tile_max, stats, *ix, indices=idx, workspace=ws_t),
        attend=csa.bind(csa.csa2_attend_fp4, c.q[0].view(bf), c.kv_codes, c.kv_scales, idx, c.swa[0].view(bf),
                        c.swa_end, None, c.softmax_scale, c.q_per_seq, c.window, out=out, workspace=ws_a))
    return calls, idx, with_scores


def decode_section(args, dev, name):
    """A decode workload other than the headline (batched decode: 64 sequences x 131072 entries):
    the same Full-layer step, timed the same way, with the step's algorithmic bytes against 8 TB/s."""
    import torch

    import compressed_sparse_attention_02_amd as csa
    import csa2_gen as G

    wl = WORKLOADS[name]
    B, N = wl["B"], wl["N"]
    c = G.make_case(name, B=B, N=N, n_layers=1, seed=0, device=dev, chunk_rows=1 << 19)
    T = c.T
    calls, idx, rows = _full_layer(csa, c, dev, T, N)

    def step():
        calls["index"]()
        calls["topk"]()
        calls["attend"]()

    ms = _wall_ms(step, args.steps, args.warmup)
    timed = _timer(torch.cuda.current_stream(dev))
    reps = max(10, args.steps)
    st = {k: timed(calls[k], reps) for k in ("index", "topk", "attend")}
    step_bytes = T * G.algorithmic_bytes_decode_query(N)
    idx_bytes = B * N * 256 + T * (8192 + 128 + 16) + T * csa.tile_max_ld(N) * 4 + (T * N * 4 if rows else 0)
    scan_gbps = idx_bytes / (st["index"][1] * 1e-6) / 1e9
    att_bytes = T * (512 * 272 + 128 * 1024 + 65536 + 65536 + 512 * 4)
    return {
        "value": T / (ms * 1e-3), "unit": "queries/s", "ms_per_step": ms, "steps": args.steps,
        "config": {"workload": name, "batch": B, "entries_per_seq": N, "queries_per_seq": 1, "topk": 512,
                   "main_kv": "MXFP4 E2M1+E8M0/32", "indexer": "32x128 bf16"},
        "algorithmic_bytes_per_step": step_bytes,
        "step_hbm_GBps": step_bytes / (ms * 1e-3) / 1e9,
        "step_frac_of_peak": step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "roofline": {"kernel": "idx_scan_kernel (all of csa2_index)", "bound": "hbm", "achieved": scan_gbps,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": scan_gbps / HBM_PEAK_GBPS,
                     "algorithmic_bytes_per_launch": idx_bytes, "avg_launch_us": st["index"][1]},
        "stages_us": {k: v[0] for k, v in st.items()},
        "attention": {"avg_us": st["attend"][1], "algorithmic_bytes": att_bytes,
                      "GBps": att_bytes / (st["attend"][1] * 1e-6) / 1e9,
                      "frac_hbm": att_bytes / (st["attend"][1] * 1e-6) / 1e9 / HBM_PEAK_GBPS},
    }


def reuse_group_section(args, dev):
    """The cross-layer reuse group (report sec. 2.3.1): one Full layer (index, top-512, attention)
    over 32 sequences x 262144 entries, then three Reuse layers, each with its own queries and
    window, attending over the Full layer's selection and KV.  Timed two ways: as the model runs
    them (three single-layer calls, since a Reuse layer's query depends on the previous layer's
    output) and as one fused three-layer call (each selected row gathered once)."""
    import torch

    import compressed_sparse_attention_02_amd as csa
    import csa2_gen as G

    wl = WORKLOADS["reuse_group"]
    B, N = wl["B"], wl["N"]
    c = G.make_case("reuse_group", B=B, N=N, n_layers=4, seed=0, device=dev, chunk_rows=1 << 19)
    T = c.T
    bf = torch.bfloat16
    calls, idx, rows = _full_layer(csa, c, dev, T, N)
    ws_1 = torch.empty(max(1, csa.attend_workspace_bytes(T)), dtype=torch.uint8, device=dev)
    ws_3 = torch.empty(max(1, csa.attend_workspace_bytes(T, n_layers=3)), dtype=torch.uint8, device=dev)
    out_1 = torch.empty((3, 1, T, 64, 512), dtype=bf, device=dev)
    out_3 = torch.empty((3, T, 64, 512), dtype=bf, device=dev)
    single = [csa.bind(csa.csa2_reuse_attend, c.q[l:l + 1].view(bf), c.kv_codes, c.kv_scales, idx,
                       c.swa[l:l + 1].view(bf), c.swa_end, None, c.softmax_scale, 1, 128, out=out_1[l - 1],
                       workspace=ws_1) for l in (1, 2, 3)]
    fused = csa.bind(csa.csa2_reuse_attend, c.q[1:].view(bf).contiguous(), c.kv_codes, c.kv_scales, idx,
                     c.swa[1:].view(bf).contiguous(), c.swa_end, None, c.softmax_scale, 1, 128, out=out_3,
                     workspace=ws_3)

    def full():
        calls["index"]()
        calls["topk"]()
        calls["attend"]()

    def step():  # as the model runs it: Full, then three single-layer Reuse calls
        full()
        for s in single:
            s()

    def step_fused():
        full()
        fused()

    ms = _wall_ms(step, args.steps, args.warmup)
    ms_fused = _wall_ms(step_fused, args.steps, args.warmup)
    # both forms compute the same attention; their split-K merges may round differently
    d3, d1 = out_3.float(), out_1[:, 0].float()
    same = {"bitwise_equal": bool(torch.equal(out_3, out_1[:, 0])),
            "max_abs_diff": float((d3 - d1).abs().max()),
            "within_bf16_tolerance": bool(((d3 - d1).abs() <= 1e-2 + 2e-2 * d1.abs()).all())}
    timed = _timer(torch.cuda.current_stream(dev))
    reps = max(10, args.steps)
    st = {k: timed(calls[k], reps) for k in ("index", "topk", "attend")}
    st["reuse_l1_x3"] = timed(lambda: [s() for s in single], reps)
    st["reuse_l3"] = timed(fused, reps)
    full_bytes = T * G.algorithmic_bytes_decode_query(N)
    layer_bytes = T * (512 * 272 + 128 * 1024 + 65536 + 65536 + 512 * 4)   # 403,456 B per query
    step_bytes = full_bytes + 3 * layer_bytes
    reuse_flops = 3 * T * 2 * (2 * 64 * 640 * 512)

    def att(us, nbytes, flops):
        return {"avg_us": us, "algorithmic_bytes": nbytes, "GBps": nbytes / (us * 1e-6) / 1e9,
                "frac_hbm": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, "flops": flops,
                "TFLOPs": flops / (us * 1e-6) / 1e12,
                "frac_mfma_bf16": flops / (us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS}

    idx_bytes = B * N * 256 + T * (8192 + 128 + 16) + T * csa.tile_max_ld(N) * 4 + (T * N * 4 if rows else 0)
    scan_gbps = idx_bytes / (st["index"][1] * 1e-6) / 1e9
    return {
        "value": T / (ms * 1e-3), "unit": "queries/s (groups of 1 Full + 3 Reuse layers)", "ms_per_step": ms,
        "steps": args.steps,
        "config": {"workload": "reuse_group", "batch": B, "entries_per_seq": N, "queries_per_seq": 1,
                   "layers": "1 Full + 3 Reuse", "topk": 512, "main_kv": "MXFP4 E2M1+E8M0/32",
                   "indexer": "32x128 bf16"},
        "algorithmic_bytes_per_step": step_bytes,
        "step_hbm_GBps": step_bytes / (ms * 1e-3) / 1e9,
        "step_frac_of_peak": step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "fused_reuse_step": {"ms_per_step": ms_fused, "value": T / (ms_fused * 1e-3),
                             "step_frac_of_peak": step_bytes / (ms_fused * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                             "outputs_vs_single_layer_calls": same},
        "roofline": {"kernel": "idx_scan_kernel (all of csa2_index)", "bound": "hbm", "achieved": scan_gbps,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": scan_gbps / HBM_PEAK_GBPS,
                     "algorithmic_bytes_per_launch": idx_bytes, "avg_launch_us": st["index"][1]},
        "stages_us": {k: v[0] for k, v in st.items()},
        "reuse_attention": {"3 x L=1": att(st["reuse_l1_x3"][1], 3 * layer_bytes, reuse_flops),
                            "1 x L=3": att(st["reuse_l3"][1], 3 * layer_bytes, reuse_flops)},
    }


def mxfp4_step(c, G, csa, args, stream, timed, idx, out, ws_t, ws_a):
    """The decode step with MXFP4 indexer queries and keys (the generator's quantisation of
    the same bf16 ones): csa2_index_mxfp4 + csa2_topk_mxfp4 + csa2_attend_fp4."""
    import torch
    B, N, T = c.B, c.N, c.T
    qc, qs, kc, ks = G.mx_indexer(c, chunk_rows=1 << 19)
    dev = qc.device
    tile_max = torch.empty((T, csa.tile_max_ld(N)), dtype=torch.float32, device=dev)
    stats = torch.empty(csa.index_mxfp4_stats_bytes(T, 1, N) // 4, dtype=torch.int32, device=dev)
    q0 = c.q[0].view(torch.bfloat16)
    swa0 = c.swa[0].view(torch.bfloat16)

    do_index = csa.bind(csa.csa2_index_mxfp4, qc, qs, c.w_idx, kc, ks, c.q_pos, 1, 1, want_scores=False,
                        tile_max=tile_max, stats=stats)
    do_topk = csa.bind(csa.csa2_topk_mxfp4, None, tile_max, stats, c.w_idx, kc, ks, c.q_pos, 1, 1, indices=idx,
                       workspace=ws_t)
    do_attend = csa.bind(csa.csa2_attend_fp4, q0, c.kv_codes, c.kv_scales, idx, swa0, c.swa_end, None,
                         c.softmax_scale, 1, 128, out=out, workspace=ws_a)

    def step():
        do_index()
        do_topk()
        do_attend()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    reps = max(10, args.steps)
    idx_med, idx_avg = timed(do_index, reps)
    topk_med, _ = timed(do_topk, reps)
    # algorithmic bytes of the FP4 scan per launch: 68 B per key, per query the FP4 query
    # (2048 + 128 B), w (128 B), the header (16 B), the dequantised query it leaves for the
    # selection (8192 B) and its tile maxima
    scan_bytes = B * N * 68 + T * (2048 + 128 + 128 + 16 + 8192) + T * csa.tile_max_ld(N) * 4
    step_bytes = T * (68 * N + 2048 + 128 + 128 + 512 * 272 + 128 * 1024 + 65536 + 65536 + 512 * 4)
    scan_gbps = scan_bytes / (idx_avg * 1e-6) / 1e9
    # the report's deployed formats end to end: MXFP4 indexer, E2M1 + E4M3/16 main KV (288 B per
    # entry), FP8 window rows (584 B), output rotated at -pos before the cast
    nv_codes, nv_scales = G.kv_e4m3_16(c, chunk_rows=1 << 19)
    f8, rp, s8 = (x[0].contiguous() for x in G.window_fp8(c))
    rp = rp.view(torch.bfloat16)

    do_attend_dep = csa.bind(csa.csa2_attend_ex, q0, nv_codes, nv_scales, idx, c.swa_end, None, c.softmax_scale, 1,
                             128, kv_format=csa.KV_E4M3_16, swa_fp8=f8, swa_rope=rp, swa_scales=s8,
                             rope_pos=c.q_pos, out=out, workspace=ws_a)

    def step_dep():
        do_index()
        do_topk()
        do_attend_dep()

    for _ in range(args.warmup):
        step_dep()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step_dep()
    torch.cuda.synchronize()
    ms_dep = (time.perf_counter() - t0) * 1e3 / args.steps
    att_med, att_avg = timed(do_attend_dep, reps)
    att_bytes = T * (512 * 288 + 128 * 584 + 65536 + 65536 + 512 * 4)
    dep = {"value": T / (ms_dep * 1e-3), "unit": "queries/s", "ms_per_step": ms_dep,
           "main_kv": "E2M1 + E4M3/16 (288 B)", "window": "FP8: 448 E4M3 + E8M0/64, 64 bf16 (584 B)",
           "output": "inverse RoPE of channels 448..511 at -pos, fused",
           "attention_us": {"median": att_med, "mean": att_avg, "algorithmic_bytes": att_bytes,
                            "GBps": att_bytes / (att_avg * 1e-6) / 1e9},
           "step_hbm_GBps": T * (68 * N + 2048 + 128 + 128 + 512 * 288 + 128 * 584 + 65536 + 65536 + 512 * 4)
           / (ms_dep * 1e-3) / 1e9}
    return {"value": T / (ms_step * 1e-3), "unit": "queries/s", "ms_per_step": ms_step,
            "indexer": "32x128 MXFP4 (E2M1 + E8M0/32), 68 B per key",
            "scan": {"kernel": "idx_scan_mx_kernel (all of csa2_index_mxfp4)", "bound": "hbm",
                     "achieved": scan_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": scan_gbps / HBM_PEAK_GBPS,
                     "algorithmic_bytes_per_launch": scan_bytes, "avg_launch_us": idx_avg},
            "stages_us": {"index": idx_med, "topk": topk_med},
            "step_hbm_GBps": step_bytes / (ms_step * 1e-3) / 1e9,
            "step_frac_of_peak": step_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS,
            "deployed_formats_step": dep,
            "note": "same workload and selection semantics with FP4 indexer operands; not the headline"}


def kv_write_section(csa, G, dev, B, d=5120, calls=20, reps=5):
    """csa2_kv_write at the model's hidden size: one decode step's new entries (one per sequence,
    the decoder's ratio m = 1) and a 4096-token prefill chunk at the encoder's ratio m = 2.
    A graph of `calls` back-to-back calls is captured and replayed, so the time per call is the
    GPU's (both kernels and the gaps between launches), not the binding's or a replay's."""
    import torch
    res = {}
    for name, (n, m) in {"decode": (B, 1), "prefill_chunk": (2048, 2)}.items():
        inp = G.kv_write_inputs(3, n, m, d, device=dev)
        bf = lambda t: None if t is None else t.view(torch.bfloat16)
        codes = torch.empty((n, 256), dtype=torch.uint8, device=dev)
        scales = torch.empty((n, 16), dtype=torch.uint8, device=dev)
        k = torch.empty((n, 128), dtype=torch.bfloat16, device=dev)
        ws = torch.empty(csa.kv_write_workspace_bytes(n, m, d), dtype=torch.uint8, device=dev)

        def call():
            csa.csa2_kv_write(bf(inp["h"]), bf(inp["w_kv"]), bf(inp["w_ik"]), inp["pos"], m=m, w_z=bf(inp["w_z"]),
                              kv_codes=codes, kv_scales=scales, k_out=k, workspace=ws)

        call()
        torch.cuda.synchronize()
        ref = (codes.clone(), scales.clone(), k.clone())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(calls):
                call()
        g.replay()
        torch.cuda.synchronize()
        same = all(torch.equal(a, b) for a, b in zip(ref, (codes, scales, k)))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / (reps * calls)
        nproj = 2 if m > 1 else 1
        byts = n * m * d * 2 + nproj * 512 * d * 2 + 128 * 512 * 2 + 4 * n + n * (256 + 16 + 256)
        flops = 2 * n * m * d * 512 * nproj + 2 * n * 512 * 128
        res[name] = {"entries": n, "m": m, "d": d, "us": us, "algorithmic_bytes": byts,
                     "GBps": byts / (us * 1e-6) / 1e9, "frac_hbm": byts / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS,
                     "flops": flops, "TFLOPs": flops / (us * 1e-6) / 1e12,
                     "frac_mfma_bf16": flops / (us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                     "graph_replay_matches_eager": same}
        del g
    res["formats"] = "MXFP4 cache (E2M1 + E8M0/32), bf16 indexer K"
    return res


def host_cpu():
    """This host's logical CPU count, the CPUs this process may run on, and the CPU model name."""
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    if model is None:
        try:
            import subprocess
            out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
            model = next((l.split(":", 1)[1].strip() for l in out.splitlines() if l.startswith("Model name")), None)
        except (OSError, subprocess.SubprocessError):
            pass
    return {"nproc": os.cpu_count(), "affinity": len(os.sched_getaffinity(0)), "model": model}


def cpu_baseline(c, G, min_seconds=10.0, max_seconds=30.0, one_core_seconds=4.0):
    """The oracle (as is) on this host's cores: the same step (index over every visible entry,
    top-512, attention), repeated for about min_seconds with all of its OpenMP threads, then on
    one thread over the first query only (the same per-query work) for about one_core_seconds.
    The index phase spreads (query, 4096-entry chunk) pairs over every thread; top-512 and
    attention run one thread per query."""
    import numpy as np

    import oracle

    def u16(t):
        return np.ascontiguousarray(t.cpu().view(__import__("torch").int16).numpy().view(np.uint16))

    q_idx, w, k = u16(c.q_idx), c.w_idx.cpu().numpy(), u16(c.k_idx)
    q_pos = c.q_pos.cpu().numpy()
    q, swa = u16(c.q[0]), u16(c.swa[0])
    codes, scales, swa_end = c.kv_codes.cpu().numpy(), c.kv_scales.cpu().numpy(), c.swa_end.cpu().numpy()
    oracle.lib()
    threads = oracle.max_threads()

    def run(nq, seconds, cap):
        reps, t0 = 0, time.perf_counter()
        while True:
            sc = oracle.index(q_idx[:nq], w[:nq], k[:nq], q_pos[:nq], c.ratio, c.q_per_seq)
            sel = oracle.topk(sc, q_pos[:nq], c.ratio, c.k)
            oracle.attend(q[:nq], codes[:nq], scales[:nq], sel, swa[:nq], swa_end[:nq], None, c.softmax_scale,
                          c.q_per_seq, c.window)
            reps += 1
            dt = time.perf_counter() - t0
            if dt >= seconds or dt * (reps + 1) / reps > cap:
                return reps, dt

    reps, dt = run(c.T, min_seconds, max_seconds)
    prev = oracle.set_threads(1)
    try:
        reps1, dt1 = run(1, one_core_seconds, 3 * one_core_seconds)
    finally:
        oracle.set_threads(prev)
    cpu = host_cpu()
    return {"value": reps * c.T / dt, "unit": "queries/s", "cores": threads, "kind": "oracle",
            "one_core": {"value": reps1 / dt1, "unit": "queries/s", "cores": 1,
                         "sample": f"{reps1} repetitions of the first query's step, {dt1:.1f} s wall"},
            "threads_by_phase": {"index": threads, "topk": min(c.T, threads), "attention": min(c.T, threads)},
            "host": cpu,
            "sample": f"{reps} repetitions of the full {c.T}-query step of the same workload (index over all "
                      f"{c.N} entries per sequence, top-512, attention), {dt:.1f} s wall with {threads} OpenMP "
                      f"threads on {cpu['affinity']} of {cpu['nproc']} CPUs ({cpu['model']})"}


def prefill_main(args, dev):
    """The causal prefill chunk as its own line (--workload causal_prefill)."""
    sec = prefill_section(args, dev)
    line = {"metric": METRIC, "value": sec.pop("value"), "unit": sec.pop("unit"), "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": sec.pop("ms_per_step"),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic", **sec}
    print(json.dumps(line), flush=True)
    return 0


def prefill_section(args, dev):
    """The causal prefill chunk: csa2_index (score matrix written) + csa2_topk (row regime) +
    csa2_attend_fp4 for 4096 queries over 34816 compressed entries (ratio 2), with the scan
    and the attention against the bf16 MFMA roofline (both are dense products here) and the
    step against the MFMA bound of their flops."""
    import torch

    import compressed_sparse_attention_02_amd as csa
    import csa2_gen as G

    wl = WORKLOADS["causal_prefill"]
    print("[bench] generating causal_prefill", file=sys.stderr, flush=True)
    c = G.make_case("causal_prefill", **wl, seed=0, device=dev, chunk_rows=1 << 19)
    T, N = c.T, c.N
    calls, idx, rows = _full_layer(csa, c, dev, T, N)

    def step():
        calls["index"]()
        calls["topk"]()
        calls["attend"]()

    steps = max(3, min(args.steps, 20))
    ms_step = _wall_ms(step, steps, max(1, min(args.warmup, 3)))
    print(f"[bench] prefill: {steps} steps timed: {ms_step:.4f} ms per step", file=sys.stderr, flush=True)
    timed = _timer(torch.cuda.current_stream(dev))
    reps = max(5, min(args.steps, 20))
    idx_med, idx_avg = timed(calls["index"], reps)
    topk_med, _ = timed(calls["topk"], reps)
    att_med, att_avg = timed(calls["attend"], reps)
    # the indexer GEMM: 2 x 32 heads x 128 channels per visible (query, entry) pair
    n_vis = sum(min(N, (p + 1) // c.ratio) for p in c.q_pos.tolist())
    idx_flops = 2 * 32 * 128 * n_vis
    att_flops = T * 2 * (2 * 64 * (512 + c.window) * 512)
    idx_tflops = idx_flops / (idx_avg * 1e-6) / 1e12
    bound_ms = (idx_flops + att_flops) / (MFMA_BF16_PEAK_TFLOPS * 1e12) * 1e3
    sec = {
        "value": T / (ms_step * 1e-3), "unit": "query tokens/s", "ms_per_step": ms_step, "steps": steps,
        "config": {"workload": "causal_prefill", "queries": T, "prefix_tokens": 65536, "ratio": c.ratio,
                   "entries": N, "indexer": "32x128 bf16", "topk": 512, "heads": 64, "head_dim": 512,
                   "window": c.window, "main_kv": "MXFP4 E2M1+E8M0/32", "parallelism": "none (1 GPU)"},
        "roofline": {"kernel": "idx_scan_kernel (all of csa2_index, score matrix written)", "bound": "mfma",
                     "achieved": idx_tflops, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": idx_tflops / MFMA_BF16_PEAK_TFLOPS, "traffic": None,
                     "algorithmic_flops_per_launch": idx_flops, "avg_launch_us": idx_avg},
        "stages_us": {"index": idx_med, "topk_rows": topk_med, "attend": att_med},
        "attention": {"call": "csa2_attend_fp4", "avg_us": att_avg, "flops": att_flops,
                      "TFLOPs": att_flops / (att_avg * 1e-6) / 1e12,
                      "frac_mfma_bf16": att_flops / (att_avg * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS},
        "mfma_bound_ms": bound_ms,
        "step_frac_of_mfma_bound": bound_ms / ms_step,
    }
    if args.workload == "causal_prefill" and not args.no_cpu_baseline:
        sec["cpu_baseline"] = cpu_baseline_prefill(c, G)
    return sec


def cpu_baseline_prefill(c, G, n_sample=8, min_seconds=10.0, max_seconds=30.0):
    """The oracle (as is) on this host's cores over a sample of the chunk's queries (the last
    n_sample, which see the most entries): index, row top-512, attention."""
    import numpy as np

    import oracle

    def u16(t):
        return np.ascontiguousarray(t.cpu().view(__import__("torch").int16).numpy().view(np.uint16))

    t0_q = c.T - n_sample
    q_idx, w = u16(c.q_idx[t0_q:]), c.w_idx[t0_q:].cpu().numpy()
    k = u16(c.k_idx)
    q_pos = c.q_pos[t0_q:].cpu().numpy()
    q, swa = u16(c.q[0][t0_q:]), u16(c.swa[0])
    codes, scales = c.kv_codes.cpu().numpy(), c.kv_scales.cpu().numpy()
    swa_end = c.swa_end[t0_q:].cpu().numpy()
    oracle.lib()
    reps, t0 = 0, time.perf_counter()
    while True:
        sc = oracle.index(q_idx, w, k, q_pos, c.ratio, n_sample)
        sel = oracle.topk(sc, q_pos, c.ratio, c.k)
        oracle.attend(q, codes, scales, sel, swa, swa_end, None, c.softmax_scale, n_sample, c.window)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds or dt * (reps + 1) / reps > max_seconds:
            break
    cores = oracle.max_threads()      # the index phase spreads (query, entry chunk) pairs over all threads
    return {"value": reps * n_sample / dt, "unit": "queries/s", "cores": cores, "kind": "oracle", "host": host_cpu(),
            "sample": f"{reps} repetitions of the chunk's last {n_sample} queries (index over their "
                      f"{int(q_pos[-1] + 1) // c.ratio} visible entries, top-512, attention), {dt:.1f} s wall "
                      f"on {cores} threads"}


if __name__ == "__main__":
    sys.exit(main())
