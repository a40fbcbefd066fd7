"""Benchmark of the KVSlimmer merge path on one MI355X.

One step = the whole hot path on one Llama-3.1-8B-shaped layer at 32K context
(8 KV heads x 128, 32 query heads, bf16): one merge round to 50% with the 32
most recent tokens kept, in kvs_score_merge (window statistics, Hessian-norm
sums, closed-form weights, merge and compaction), then kvs_decode_attn (one
decode query per head over the merged cache).  The same round through the
separate calls kvs_score -> kvs_merge_weights -> kvs_merge_compact is timed
beside it, outside the step.  Inputs are resident in HBM before timing starts; steps
rotate over several input layers whose total exceeds the 256 MB Infinity
Cache, so every step reads its K/V from HBM.

Prints one JSON line (rank 0).  Usage: python bench.py [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KV tokens merged/sec + achieved HBM GB/s (Llama-3.1-8B layer, 32K ctx)"
HBM_PEAK_GBS = 8000.0
PEAK_MFMA_BF16_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak
SIMDS = 1024                    # 256 CUs x 4 SIMDs
PEAK_CLOCK_GHZ = 2.4


def kernel_bytes(N, H, D, P, T, GW, has_n=False, elt=2):
    """Algorithmic HBM bytes per launch of each kernel: what the method must move, once.
    row = one K row + one V row of one (batch, kv-head) slot."""
    row = 2 * D * elt
    nb = 4 if has_n else 0
    return {
        "score_pass1": N * H * (row + nb),                        # K, V once (lse/O partials are not counted)
        "combine": 0,
        "score_pass2": N * H * (row + nb) + (N + P) * H * 4,       # K, V once; g_self, g_cross out
        "select": 0,                                              # a full round selects by rule
        "merge_compact": N * H * (row + 4 + nb) + P * H * 4 + T * H * (row + 4 + 4),
        # pass 2 with the merge folded in: K, V once; g_self, g_cross and the compacted cache out
        "score_pass2_merge": N * H * (row + nb) + (N + P) * H * 4 + T * H * (row + 4 + 4),
        "decode": T * H * (row + 4),
    }


# rocprofv3 kernel names -> the labels the library gives its launches
KERNEL_LABELS = (("p1_mfma_kernel", "score_pass1"), ("pass1_valu_kernel", "score_pass1"),
                 ("p2_mfma_kernel", "score_pass2"), ("pass2_valu_kernel", "score_pass2"),
                 ("combine_kernel", "combine"), ("pair_cos_kernel", "pair_cos"),
                 ("combine_wave_kernel", "combine"), ("qsum_kernel", "qsum"), ("select_fixed_kernel", "select"),
                 ("select_small_kernel", "select"), ("sel_clear_kernel", "select"), ("sel_hist_kernel", "select"),
                 ("sel_count_kernel", "select"), ("sel_final_kernel", "select"), ("append_kernel", "append"),
                 ("pack_kernel", "pack"), ("exact_e_kernel", "exact_e"), ("spectral_proj_kernel", "spectral_proj"),
                 ("spectral_pair_kernel", "spectral_pair"),
                 ("merge_compact_kernel", "merge_compact"), ("decode_mfma_kernel", "decode"),
                 ("decode_kernel", "decode"))
COPY_BYTES = 1 << 30            # calibration copy: reads and writes this many bytes
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_c2_layer32k.md")


def kernel_label(rocprof_name):
    if "kvs::" not in rocprof_name:
        return None
    # pass 2 with the merge folded in: p2_mfma_kernel<D, HAS_N, MERGE = true, ...>
    if re.search(r"kvs::p2_mfma_kernel<\d+, (true|false), true", rocprof_name):
        return "score_pass2_merge"
    for key, label in KERNEL_LABELS:
        if "kvs::" + key in rocprof_name:
            return label
    return None


def sources_digest():
    """Digest of every source the kernels are built from; counter figures taken on other
    sources no longer describe the kernels and are not reported."""
    import hashlib
    h = hashlib.sha256()
    for d in (os.path.join(ROOT, "long_context_kv_kvslimmer_amd", "csrc"), os.path.join(ROOT, "include")):
        for f in sorted(os.listdir(d)):
            if f.endswith((".hip", ".h", ".cpp")):
                h.update(f.encode())
                with open(os.path.join(d, f), "rb") as fh:
                    h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic(label):
    """HBM bytes per launch of `label` from the committed counter summary, if it was
    taken on the current sources; else None."""
    try:
        lines = open(TRAFFIC_FILE).read().splitlines()
    except OSError:
        return None
    vals = dict(l.strip("` ").split(" = ", 1) for l in lines if l.startswith("`") and " = " in l)
    if vals.get("sources") != sources_digest():
        return None
    v = vals.get(f"traffic_bytes[{label}]")
    return None if v is None else int(v)


def summarize_counters(fetch_csv, write_csv, cmd):
    """Markdown summary of two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of
    `bench.py --copy-calibration`: per-dispatch KiB of each library kernel, scaled by
    what the same counter reads for the calibration copy of COPY_BYTES."""
    import csv
    import statistics

    def load(path, counter):
        per = {}
        copy = []
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            v = float(r["Counter_Value"])
            if "neg_kernel" in r["Kernel_Name"] and int(r["Grid_Size"]) >= (1 << 20):
                copy.append(v)
            lab = kernel_label(r["Kernel_Name"])
            if lab:
                per.setdefault(lab, []).append(v)
        return {k: statistics.mean(v) for k, v in per.items()}, statistics.mean(copy)

    fetch, fcopy = load(fetch_csv, "FETCH_SIZE")
    write, wcopy = load(write_csv, "WRITE_SIZE")
    ff = COPY_BYTES / (fcopy * 1024)
    fw = COPY_BYTES / (wcopy * 1024)
    out = ["# HBM traffic per launch, C2 layer (32K ctx, 8x128 KV heads, bf16)", "",
           "Made by:", "", "```", cmd, "```", "",
           f"Calibration: a plain elementwise copy (torch.neg) reads and writes {COPY_BYTES} B; FETCH_SIZE "
           f"reads {fcopy:.1f} KiB for it, WRITE_SIZE {wcopy:.1f} KiB.  Scale factors: fetch {ff:.4f}, "
           f"write {fw:.4f}.", "",
           "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled read MB | scaled write MB | traffic MB |",
           "|---|---:|---:|---:|---:|---:|"]
    lines = []
    for lab in sorted(set(fetch) | set(write)):
        r = fetch.get(lab, 0.0) * 1024 * ff
        w = write.get(lab, 0.0) * 1024 * fw
        out.append(f"| {lab} | {fetch.get(lab, 0):.1f} | {write.get(lab, 0):.1f} | {r / 1e6:.2f} | {w / 1e6:.2f} | "
                   f"{(r + w) / 1e6:.2f} |")
        lines.append(f"`traffic_bytes[{lab}] = {int(round(r + w))}`")
    out += ["", "Machine-read values (bytes per launch; valid for these sources only):", "",
            f"`sources = {sources_digest()}`", ""] + lines
    return "\n".join(out) + "\n"


def summarize_trace(stats_csv, bench_json, cmd):
    """Markdown summary of a rocprofv3 --kernel-trace --stats run of bench.py next to the
    per-kernel HIP-event times of a bench.py run with the same arguments and no profiler
    (under the profiler the event-timed launches read a few microseconds long)."""
    import csv
    rows = {}
    for r in csv.DictReader(open(stats_csv)):
        lab = kernel_label(r["Name"])
        if lab:
            c, t = rows.get(lab, (0, 0.0))
            rows[lab] = (c + int(r["Calls"]), t + float(r["TotalDurationNs"]))
    line = json.loads([l for l in open(bench_json).read().splitlines() if l.startswith("{")][-1])
    ev = line.get("kernels_ranked", {})
    out = ["# Kernel durations, C2 layer (32K ctx, 8x128 KV heads, bf16)", "", "Made by:", "", "```", cmd, "```",
           "", "rocprofv3 averages over every launch of the profiled run.  The HIP-event columns and the last "
           "line come from a run of the same bench.py command without the profiler: medians over the ranking "
           "steps (every launch timed by its own start/stop events, after the warm-up), and the roofline object "
           "of the timed region (only the dominant kernel timed).", "",
           "| kernel | launches | rocprofv3 avg us | HIP-event median us | algorithmic MB | GB/s (events) |",
           "|---|---:|---:|---:|---:|---:|"]
    for lab, (c, t) in sorted(rows.items(), key=lambda kv: -kv[1][1]):
        e = ev.get(lab, {})
        out.append(f"| {lab} | {c} | {t / c / 1e3:.2f} | {e.get('median_ms', float('nan')) * 1e3:.2f} | "
                   f"{e.get('algorithmic_MB', 0)} | {e.get('GBps')} |")
    out += ["", f"ms_per_step {line['ms_per_step']}, value {line['value']} {line['unit']}, roofline "
            f"{json.dumps(line['roofline'])}"]
    return "\n".join(out) + "\n"


def summarize_stats(stats_csv, title, cmd):
    """Markdown table of a rocprofv3 --kernel-trace --stats run: launches, mean and total
    duration per kernel label."""
    import csv
    rows = {}
    for r in csv.DictReader(open(stats_csv)):
        lab = kernel_label(r["Name"])
        if lab == "combine":   # the two variants serve different callers (window statistics, decode)
            lab += " (one wave per row)" if "combine_wave_kernel" in r["Name"] else " (one workgroup per row)"
        if lab:
            c, t = rows.get(lab, (0, 0.0))
            rows[lab] = (c + int(r["Calls"]), t + float(r["TotalDurationNs"]))
    out = [f"# {title}", "", "Made by:", "", "```", cmd, "```", "",
           "| kernel | launches | rocprofv3 avg us | total ms |", "|---|---:|---:|---:|"]
    for lab, (c, t) in sorted(rows.items(), key=lambda kv: -kv[1][1]):
        out.append(f"| {lab} | {c} | {t / c / 1e3:.2f} | {t / 1e6:.3f} |")
    return "\n".join(out) + "\n"


def summarize_mfma(sq_csv, stats_csv, cmd):
    """Markdown summary of a rocprofv3 --pmc run with SQ_INSTS_VALU_MFMA_MOPS_BF16,
    SQ_INSTS_VALU_MFMA_MOPS_F16 and SQ_VALU_MFMA_BUSY_CYCLES (per-dispatch sums over the
    chip) next to each kernel's mean duration from a kernel-trace run: 16-bit MFMA work per
    launch (bf16 and f16 products, which have the same dense peak), achieved rate against
    that peak, and matrix-core busy cycles per SIMD against the launch duration."""
    import csv
    import statistics
    per = {}
    for r in csv.DictReader(open(sq_csv)):
        lab = kernel_label(r["Kernel_Name"])
        if lab:
            per.setdefault((lab, r["Counter_Name"]), []).append(float(r["Counter_Value"]))
    dur = {}
    for r in csv.DictReader(open(stats_csv)):
        lab = kernel_label(r["Name"])
        if lab:
            c, t = dur.get(lab, (0, 0.0))
            dur[lab] = (c + int(r["Calls"]), t + float(r["TotalDurationNs"]))
    out = ["# MFMA work and utilisation of the scorer, C2 layer (32K ctx, 8x128 KV heads, bf16)", "", "Made by:", "",
           "```", cmd, "```", "",
           f"Peak: dense bf16 / f16 MFMA {PEAK_MFMA_BF16_TFLOPS} TFLOP/s; {SIMDS} SIMDs at {PEAK_CLOCK_GHZ} GHz.  FLOP "
           "per launch = (SQ_INSTS_VALU_MFMA_MOPS_BF16 + SQ_INSTS_VALU_MFMA_MOPS_F16) x 512 (the counters' unit).  "
           "Busy = SQ_VALU_MFMA_BUSY_CYCLES / SIMDs / (mean duration x peak clock).", "",
           "| kernel | MFMA instructions | bf16 GFLOP | f16 GFLOP | GFLOP per launch | mean us | TFLOP/s | of peak | "
           "MFMA busy per SIMD |",
           "|---|---:|---:|---:|---:|---:|---:|---:|---:|"]
    for lab in sorted({k[0] for k in per}):
        mb = statistics.mean(per.get((lab, "SQ_INSTS_VALU_MFMA_MOPS_BF16"), [0.0]))
        mh = statistics.mean(per.get((lab, "SQ_INSTS_VALU_MFMA_MOPS_F16"), [0.0]))
        if mb + mh == 0 or lab not in dur:
            continue
        flop = (mb + mh) * 512
        inst = statistics.mean(per.get((lab, "SQ_INSTS_MFMA"), [float("nan")]))
        busy = statistics.mean(per.get((lab, "SQ_VALU_MFMA_BUSY_CYCLES"), [float("nan")]))
        c, t = dur[lab]
        us = t / c / 1e3
        tf = flop / (us * 1e-6) / 1e12
        frac_busy = busy / SIMDS / (us * 1e-6 * PEAK_CLOCK_GHZ * 1e9)
        out.append(f"| {lab} | {inst:.0f} | {mb * 512 / 1e9:.2f} | {mh * 512 / 1e9:.2f} | {flop / 1e9:.2f} | {us:.2f} | "
                   f"{tf:.1f} | {tf / PEAK_MFMA_BF16_TFLOPS:.3f} | {frac_busy:.3f} |")
    return "\n".join(out) + "\n"


def summarize_pmc(csvs, stats_csv, cmd, title):
    """Markdown summary of several rocprofv3 --pmc runs (comma-separated counter_collection
    CSVs) next to a kernel-trace stats CSV: per kernel label, the mean per-dispatch value of
    every counter, then the ratios that show which pipe binds.  GRBM_GUI_ACTIVE is summed
    over the 8 XCDs in the CSV, so one eighth of it is the dispatch's active cycles."""
    import csv
    import statistics
    per = {}
    for path in csvs.split(","):
        for r in csv.DictReader(open(path)):
            lab = kernel_label(r["Kernel_Name"])
            if lab:
                per.setdefault(lab, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    dur = {}
    for r in csv.DictReader(open(stats_csv)):
        lab = kernel_label(r["Name"])
        if lab:
            c, t = dur.get(lab, (0, 0.0))
            dur[lab] = (c + int(r["Calls"]), t + float(r["TotalDurationNs"]))
    names = sorted({n for d in per.values() for n in d})
    out = [f"# {title}", "", "Made by:", "", "```", cmd, "```", "",
           "Mean value per dispatch (sums over the chip as rocprofv3 reports them).", "",
           "| counter | " + " | ".join(sorted(per)) + " |", "|---|" + "---:|" * len(per)]
    for n in names:
        out.append(f"| {n} | " + " | ".join(f"{statistics.mean(per[k][n]):.4g}" if n in per[k] else "" for k in
                                            sorted(per)) + " |")
    out += ["", "Derived (SIMDs = 1024; cycles = GRBM_GUI_ACTIVE / 8; quad-cycle counters x 4):", "",
            "| kernel | mean us | active cycles | VALU instr per SIMD | trans share | VALU busy | MFMA busy | "
            "MFMA-VALU co-exec / MFMA busy | LDS busy | LDS bank-conflict rate | wave wait share |",
            "|---|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|"]

    def m(k, n):
        v = per[k].get(n)
        return statistics.mean(v) if v else float("nan")
    for k in sorted(per):
        cyc = m(k, "GRBM_GUI_ACTIVE") / 8
        us = dur[k][1] / dur[k][0] / 1e3 if k in dur else float("nan")
        valu = m(k, "SQ_INSTS_VALU") / SIMDS
        trans = m(k, "SQ_INSTS_VALU_TRANS_F32") / max(m(k, "SQ_INSTS_VALU"), 1)
        vbusy = m(k, "SQ_ACTIVE_INST_VALU") * 4 / SIMDS / cyc
        mbusy = m(k, "SQ_VALU_MFMA_BUSY_CYCLES") / SIMDS / cyc
        coex = m(k, "SQ_VALU_MFMA_COEXEC_CYCLES") / max(m(k, "SQ_VALU_MFMA_BUSY_CYCLES"), 1)
        lbusy = m(k, "SQ_ACTIVE_INST_LDS") * 4 / SIMDS / cyc
        bc = m(k, "SQ_LDS_BANK_CONFLICT") / max(m(k, "SQ_LDS_IDX_ACTIVE") - m(k, "SQ_LDS_BANK_CONFLICT"), 1)
        wait = m(k, "SQ_WAIT_ANY") / max(m(k, "SQ_WAVE_CYCLES"), 1)
        out.append(f"| {k} | {us:.2f} | {cyc:.0f} | {valu:.0f} | {trans:.3f} | {vbusy:.3f} | {mbusy:.3f} | {coex:.3f} | "
                   f"{lbusy:.3f} | {bc:.4f} | {wait:.3f} |")
    return "\n".join(out) + "\n"


def summarize_per_config(jsonl, cmd):
    """Markdown table of the JSON lines printed by `bench.py --per-config`."""
    allrows = [json.loads(line) for line in open(jsonl) if line.startswith("{")]
    rows = [r for r in allrows if "merge_ms_per_layer" in r]
    streams = [r for r in allrows if "chunk_sweep" in r]
    out = ["# Per-config GPU timings (every layer of each seeded workload)", "", "Made by:", "", "```", cmd, "```", "",
           "Every merge round is one kvs_score_merge call (for partial rounds the selection runs between the "
           "scorer's passes and the merge inside the second).  One layer alone: median of 5 repetitions after a "
           "warm-up, events around the layer's rounds.  All layers: every layer's cache resident, all layers merged "
           "back to back, median of 3 passes, on one stream and with the layers alternating over two streams (the "
           "layers share nothing; both orders give the same merged rows); the whole-model figures use the faster. "
           " Algorithmic MB: K and V read by both scorer passes, merged rows written once.", "",
           "| config | batch x layers | rounds (pairs merged) | merge ms, one layer alone | merge ms, all layers "
           "(one stream / two streams) | per layer in the sequence | tokens/s | algorithmic MB / layer | GB/s |",
           "|---|---|---|---:|---:|---:|---:|---:|---:|"]
    for r in rows:
        if "merge_ms_all_layers_one_stream" in r:
            al = f"{r['merge_ms_all_layers_one_stream']} / {r['merge_ms_all_layers_two_streams']}"
            per = round(r["merge_ms_all_layers"] / r["layers"], 4)
            tps, gbs = r["merge_tokens_per_s_all_layers"], r["merge_GBps_all_layers"]
        else:
            al, per = f"{r['merge_ms_all_layers']}", r["merge_ms_per_layer"]
            tps, gbs = r["merge_tokens_per_s"], r["merge_GBps"]
        out.append(f"| {r['config']} | {r['batch']} x {r['layers']} | {r['rounds']} | {r['merge_ms_per_layer']} | "
                   f"{al} | {per} | {tps:.3g} | {r['merge_algorithmic_MB_per_layer']} | {gbs} |")
    cpu = [r for r in rows if "cpu_oracle" in r]
    if cpu:
        c0 = cpu[0]["cpu_oracle"]
        out += ["", f"CPU oracle on the same layer (fp64 NumPy on the host's {c0['host_cores_available']} cores, "
                    f"{c0['cpu_model']}; worker threads one per slice up to the cores, one BLAS thread each).  A slice "
                    "is one (batch item, KV head) through every round of the layer; configs with a sample of slices "
                    "are scaled to the layer by slices / sample at the sample's thread count (extrapolated).  A "
                    "reported baseline, not a target.", "",
                "| config | slices timed | threads | merge | merge s / layer | merge s, all layers | tokens/s | "
                "GPU speed-up |",
                "|---|---|---:|---|---:|---:|---:|---:|"]
        for r in cpu:
            c = r["cpu_oracle"]
            out.append(f"| {r['config']} | {c['slices']} | {c['cores']} | {c['merge']} | {c['merge_s_per_layer']} | "
                       f"{c['merge_s_all_layers']} | {c['merge_tokens_per_s']:.3g} | "
                       f"{c['merge_s_all_layers'] * 1e3 / r['merge_ms_all_layers']:.0f}x |")
        for r in cpu:
            c = r["cpu_oracle"]
            if "decode_steps" in c:
                out.append("")
                out.append(f"CPU oracle decode ({r['config']}): every step of every query head, measured: "
                           f"{c['decode_ms_per_layer_step']} ms per layer-step, {c['decode_ms_per_step_all_layers']} "
                           f"ms per {r['layers']}-layer step ({c['decode_cores']} worker threads); GPU "
                           f"{r.get('decode_us_per_layer_step', 'n/a')} us per layer-step.")
    out += ["", "Kernel time per layer, summed over the layer's rounds (library event marks, one marked run; each "
                "mark adds ~1 us):", "", "| config | kernels (us) |", "|---|---|"]
    for r in rows:
        ks = ", ".join(f"{k} {v}" for k, v in r.get("kernel_us_per_layer", {}).items())
        out.append(f"| {r['config']} | {ks} |")
    for r in rows:
        if "decode_steps" in r:
            out += ["", f"Decode ({r['config']}): {r['decode_steps']} steps over {r['decode_slots'][0]}.."
                        f"{r['decode_slots'][1]} slots per head.", "",
                    "| measure | value |", "|---|---:|",
                    f"| per layer-step, calls back to back (decode kernel + combine) | "
                    f"{r['decode_us_per_layer_step']} us, {r['decode_step_GBps']} GB/s |",
                    f"| decode kernel (library event marks) | {r['decode_kernel_us']} us, "
                    f"{r['decode_kernel_GBps']} GB/s |",
                    f"| combine (library event marks) | {r['decode_combine_us']} us |",
                    f"| per step, all {r['layers']} layers | {r['decode_ms_per_step_all_layers']} ms |"]
    for r in streams:
        ks = ", ".join(f"{k} {v}" for k, v in r["kernel_us_per_round"].items())
        out += ["", f"Chunked prefill under a cache budget ({r['config']}): {r['tokens']} tokens x "
                    f"{r['layers_folded_into_batch']} layers (folded into the batch) x {r['kv_heads']} KV heads, chunks "
                    f"of {r['chunk']}, budget {r['budget']} slots, {r['n_sink']} kept first tokens; "
                    f"{r['merge_rounds']} partial merge rounds.", "",
                "| measure | value |", "|---|---:|",
                f"| whole loop (appends + rounds, median of 5) | {r['loop_ms']} ms, "
                f"{r['prefill_tokens_per_s']:.3g} tokens/s |",
                f"| per round | {r['ms_per_round']} ms |",
                f"| kernels per round (library event marks) | {ks} |",
                f"| merge-round kernel time, whole loop | {r['merge_kernel_us_total']} us (appends "
                f"{r['append_us_total']} us more) |",
                f"| merge algorithmic MB, whole loop | {r['merge_algorithmic_MB']} ({r['merge_kernel_GBps']} GB/s "
                f"over kernel time) |",
                f"| peak device memory the loop allocates | {r['peak_alloc_MB']} MB (uncompressed cache "
                f"{r['full_cache_MB']} MB) |", "",
                "Peak memory and loop time against chunk size:", "",
                "| chunk | merge rounds | loop ms | peak alloc MB | two caches MB |", "|---:|---:|---:|---:|---:|"]
        for c in r["chunk_sweep"]:
            out.append(f"| {c['chunk']} | {c['rounds']} | {c['loop_ms']} | {c['peak_alloc_MB']} | {c['cache_MB']} |")
    return "\n".join(out) + "\n"


def copy_calibration(dev):
    """A plain copy of known size for scaling the FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst


def cpu_model():
    """The host CPU's model name (first "model name" line of /proc/cpuinfo), or None."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(cfg, K, V, Qw, q):
    """The oracle as it stands on the whole C2 layer: every KV head's merge round and one
    decode query over its merged cache.  The heads are independent slices, so they run on
    a pool of worker threads (one per host core the process may use, at most one per head),
    each with one BLAS thread."""
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits

    from oracle import kvs_oracle as O
    G = cfg.group
    M = cfg.rounds[0]
    scale = 1 / math.sqrt(cfg.head_dim)
    heads = cfg.kv_heads
    slices = []
    for h in range(heads):
        slices.append((K[0, h].double().cpu().numpy(), V[0, h].double().cpu().numpy(),
                       Qw[0, h * G:(h + 1) * G].double().cpu().numpy().reshape(-1, cfg.head_dim),
                       q[0, h * G].double().cpu().numpy()))

    def one(s):
        Ks, Vs, Qs, qd = s
        r = O.merge_round(Ks, Vs, None, Qs, scale, cfg.n_sink, cfg.n_recent, M)
        O.decode(r.K, r.V, r.n, qd, scale)

    workers = max(1, min(heads, len(os.sched_getaffinity(0))))
    t0 = time.perf_counter()
    with threadpool_limits(1):
        with ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(one, slices))
    dt = time.perf_counter() - t0
    tokens = cfg.batch * cfg.n_slots
    return {"value": tokens / dt, "unit": "tokens/s", "cores": workers, "kind": "oracle",
            "cpu_model": cpu_model(), "host_cores_available": len(os.sched_getaffinity(0)),
            "sample": f"the whole C2 layer: all {heads} KV heads (N={cfg.n_slots}, merge of {M} pairs) plus one "
                      f"decode query per KV head over its merged cache, fp64 NumPy, {workers} worker threads "
                      f"(one KV head each, one BLAS thread each; the oracle's Python-level loops hold the "
                      f"interpreter lock), {dt:.1f} s"}


ORACLE_SLICES = {1: None, 2: None, 3: 2, 4: 2, 5: 2}   # None: every slice of the layer


def cpu_oracle_config(cfg, K0, V0, Qws, decode=None):
    """The oracle as it stands on one layer of a config, on the host cores.  A slice is one
    (batch item, KV head) chained through every merge round of the layer (each round's input
    is the oracle's own output of the round before).  Slices run on a pool of worker threads
    (one per host core the process may use, at most one per slice), one BLAS thread each.
    C1 and C2 time every slice of the layer ("measured"); the larger configs time a seeded
    sample of slices and scale the layer by slices / sample ("extrapolated").  `decode`:
    the merged cache, slot counts and per-step queries the GPU decoded; every step of every
    query head runs, in full.  The model-wide figures multiply by the layers, as the GPU's."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import kvs_oracle as O
    G, D = cfg.group, cfg.head_dim
    scale = 1 / math.sqrt(D)
    total = cfg.batch * cfg.kv_heads
    want = ORACLE_SLICES.get(cfg.idx)
    pairs = [(b, h) for b in range(cfg.batch) for h in range(cfg.kv_heads)]
    if want is not None and want < total:
        rs = np.random.RandomState(1000 + cfg.idx)
        pairs = [pairs[i] for i in sorted(rs.choice(total, want, replace=False))]
    cores = len(os.sched_getaffinity(0))
    slices = [(K0[b, h].double().cpu().numpy(), V0[b, h].double().cpu().numpy(),
               [Qw[b, h * G:(h + 1) * G].double().cpu().numpy().reshape(-1, D) for Qw in Qws]) for b, h in pairs]

    def chain(sl):
        Ks, Vs, Qs = sl
        ns = None
        for Qr, M in zip(Qs, cfg.rounds):
            r = O.merge_round(Ks, Vs, ns, Qr, scale, cfg.n_sink, cfg.n_recent, M)
            Ks, Vs, ns = r.K, r.V, r.n

    workers = max(1, min(len(slices), cores))
    t0 = time.perf_counter()
    with threadpool_limits(1):
        with ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(chain, slices))
    wall = time.perf_counter() - t0
    measured = len(slices) == total
    layer_s = wall if measured else wall * total / len(slices)
    tokens = cfg.batch * cfg.n_slots
    res = {"kind": "oracle", "slices": f"{len(slices)} of {total} (batch, KV head) slices per layer",
           "merge": "measured" if measured else "extrapolated", "sample_wall_s": round(wall, 2),
           "merge_s_per_layer": round(layer_s, 2), "merge_s_all_layers": round(layer_s * cfg.layers, 1),
           "merge_tokens_per_s": round(tokens / layer_s, 1), "cores": workers, "host_cores_available": cores,
           "cpu_model": cpu_model()}
    if decode is not None:
        Kc, Vc, nc, qs, slot_counts = decode
        Kh = [Kc[0, h].double().cpu().numpy() for h in range(cfg.kv_heads)]
        Vh = [Vc[0, h].double().cpu().numpy() for h in range(cfg.kv_heads)]
        nh = [nc[0, h].cpu().numpy().astype(np.int64) for h in range(cfg.kv_heads)]
        qh = [q[0].double().cpu().numpy() for q in qs]

        def head(hq):
            h = hq // G
            for t, Nt in enumerate(slot_counts):
                O.decode(Kh[h][:Nt], Vh[h][:Nt], nh[h][:Nt], qh[t][hq], scale)

        dw = max(1, min(cfg.q_heads, cores))
        t0 = time.perf_counter()
        with threadpool_limits(1):
            with ThreadPoolExecutor(max_workers=dw) as ex:
                list(ex.map(head, range(cfg.q_heads)))
        dt = time.perf_counter() - t0
        res.update({"decode": "measured", "decode_steps": len(slot_counts),
                    "decode_ms_per_layer_step": round(dt * 1e3 / len(slot_counts), 3),
                    "decode_ms_per_step_all_layers": round(dt * 1e3 / len(slot_counts) * cfg.layers, 2),
                    "decode_cores": dw})
    return res


def gpu_clock_info():
    """Peak shader clock (HIP device attribute, kHz -> MHz) and, where the driver's sysfs
    table is readable, the current shader clock level; ROCm and HIP versions."""
    import ctypes
    info = {"gpu_peak_sclk_MHz": None, "gpu_sclk_now": None, "rocm_version": None, "hip_runtime": None}
    try:
        import torch
        info["hip_runtime"] = torch.version.hip
        lib = ctypes.CDLL("libamdhip64.so")
        v = ctypes.c_int(0)
        if lib.hipDeviceGetAttribute(ctypes.byref(v), 5, 0) == 0:     # hipDeviceAttributeClockRate
            info["gpu_peak_sclk_MHz"] = v.value // 1000
    except (OSError, AttributeError):
        pass
    try:
        info["rocm_version"] = open("/opt/rocm/.info/version").read().strip()
    except OSError:
        pass
    import glob
    for path in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            cur = [l.strip() for l in open(path) if l.strip().endswith("*")]
        except OSError:
            continue
        if cur:
            info["gpu_sclk_now"] = cur[0]
            break
    return info


def rank_kernels(marks, steps):
    """Per-label launches per step, median launch time and time per step from
    (label, ms) marks of `steps` whole steps.  The median keeps one slow launch (a first
    launch that loads its code object, say) from deciding the ranking."""
    import statistics
    per = {}
    for name, ms in marks:
        per.setdefault(name, []).append(ms)
    out = {}
    for name, v in per.items():
        lps = len(v) / max(steps, 1)
        med = statistics.median(v)
        out[name] = {"launches_per_step": lps, "median_ms": med, "mean_ms": sum(v) / len(v),
                     "ms_per_step": med * lps}
    return out


def dominant_kernel(ranked):
    """The kernel that takes the most time per step."""
    return max(ranked, key=lambda n: ranked[n]["ms_per_step"]) if ranked else None


def per_config(dev, which, reps=5, chunk_sweep=(256, 512, 1024, 2016), cpu=True, all_layers=True):
    """Per-config GPU timings (not the bench line): every merge round of one layer of each
    seeded workload through kvs_score_merge (one call per round), timed with
    events on the library's stream over `reps` repetitions after one warm-up.  Configs with
    several layers are also timed with every layer resident and merged back to back
    (all_layer_timing); the whole-model time is the faster of its one- and two-stream orders.
    The decode workload (C5) appends one token per step and times each kvs_decode_attn.  With
    `cpu`, the oracle is timed on the same layer (cpu_oracle_config) after the GPU."""
    import statistics
    import torch
    from long_context_kv_kvslimmer_amd import configs, pipeline, synth
    from long_context_kv_kvslimmer_amd import kvslim as L
    lines = []
    for idx in which:
        cfg = configs.CONFIGS[idx]
        if cfg.budget:
            res = stream_timing(cfg, dev, reps, chunks=chunk_sweep)
            lines.append(res)
            print(json.dumps(res), flush=True)
            torch.cuda.empty_cache()
            continue
        layer = 0
        K0, V0, last = pipeline.config_cache(cfg, layer, dev)
        elt = K0.element_size()
        row = 2 * cfg.head_dim * elt           # K + V bytes of one slot
        plan = []
        Qws = []
        K, V, n, N = K0, V0, None, cfg.n_slots
        alg = 0
        for r, M in enumerate(cfg.rounds):
            Qw = torch.stack([synth.window_queries(cfg, layer, b, r, dev) for b in range(cfg.batch)])
            Qws.append(Qw)
            cap = N - M + (cfg.decode_steps if r == len(cfg.rounds) - 1 else 0)
            bufs = pipeline.alloc_round(K, cfg.q_heads, cfg.window, cfg.n_sink, cfg.n_recent, M, n_slots=N,
                                        out_capacity=cap, want_flags=False)
            P = L.num_pairs(N, cfg.n_sink, cfg.n_recent)
            full = M == P
            # K and V are read by both scorer passes (the merge runs inside the second), the
            # merged rows are written once
            reads = 2 * N * row + (N * 4 if n is not None else 0)
            alg += cfg.batch * cfg.kv_heads * (reads + (N - M) * (row + 8))
            plan.append((K, V, n, Qw, M, N, full, bufs))
            K, V, n, N = bufs.K, bufs.V, bufs.n, N - M

        def rounds():
            for (Ki, Vi, ni, Qw, M, Ni, full, bufs) in plan:
                pipeline.run_round_fused(Ki, Vi, ni, Qw, cfg.q_heads, cfg.window, cfg.n_sink, cfg.n_recent, M, bufs,
                                         n_slots=Ni)

        rounds()
        torch.cuda.synchronize()
        times = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            rounds()
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        ms = statistics.median(times)
        marks = L.KernelMarks(max_launches=64)
        with marks:
            rounds()
        torch.cuda.synchronize()
        per_kernel = {}
        for name, kms in marks.times():
            per_kernel[name] = round(per_kernel.get(name, 0.0) + kms * 1e3, 2)
        tokens = cfg.batch * cfg.n_slots
        res = {"config": f"C{cfg.idx} {cfg.name}", "batch": cfg.batch, "layers": cfg.layers,
               "rounds": list(cfg.rounds), "merge_ms_per_layer": round(ms, 4),
               "merge_ms_all_layers": round(ms * cfg.layers, 3),
               "merge_tokens_per_s": round(tokens / (ms * 1e-3), 1),
               "merge_algorithmic_MB_per_layer": round(alg / 1e6, 2),
               "merge_GBps": round(alg / (ms * 1e-3) / 1e9, 1),
               "kernel_us_per_layer": per_kernel}
        if all_layers and cfg.layers > 1:
            # all layers measured back to back (the line above scales one isolated layer)
            al = all_layer_timing(cfg, dev, plan)
            best = min(al["merge_ms_all_layers_one_stream"], al["merge_ms_all_layers_two_streams"])
            res.update(al)
            res.update({"merge_ms_all_layers": best, "merge_ms_all_layers_scaled": round(ms * cfg.layers, 3),
                        "merge_tokens_per_s_all_layers": round(tokens * cfg.layers / (best * 1e-3), 1),
                        "merge_GBps_all_layers": round(alg * cfg.layers / (best * 1e-3) / 1e9, 1)})
        if cfg.decode_steps:
            bufs = plan[-1][7]
            Kc, Vc, nc = bufs.K, bufs.V, bufs.n
            steps = cfg.decode_steps
            k_new, v_new = synth.decode_tokens(cfg, layer, 0, last[0], steps, dev)
            # step t reads only the first N + t + 1 slots, so every token can be appended first
            # and the steps enqueued back to back
            Kc[0, :, N:N + steps] = k_new
            Vc[0, :, N:N + steps] = v_new
            nc[0, :, N:N + steps] = 1
            descs = [L.cache_desc(Kc, cfg.q_heads, N + t + 1) for t in range(steps)]
            qs = [synth.decode_query(cfg, layer, 0, t, dev)[None].contiguous() for t in range(steps)]
            ws = torch.zeros(max(L.workspace_bytes(L.KVS_OP_DECODE, descs[-1], None), 16), dtype=torch.uint8,
                             device=dev)
            out = torch.empty(cfg.batch, cfg.q_heads, cfg.head_dim, dtype=torch.float32, device=dev)
            scale = 1.0 / math.sqrt(cfg.head_dim)

            def decode_all():
                for t in range(steps):
                    L.kvs_decode_attn(descs[t], Kc, Vc, nc, qs[t], scale, out, ws)

            decode_all()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            decode_all()
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / steps
            marks = L.KernelMarks(max_launches=4 * steps)
            with marks:
                decode_all()
            torch.cuda.synchronize()
            kt = {}
            for name, kms in marks.times():
                kt.setdefault(name, []).append(kms * 1e3)
            mid = steps // 2
            dbytes = cfg.batch * cfg.kv_heads * (N + mid + 1) * (row + 4)
            kd = statistics.median(kt["decode"])
            res.update({"decode_steps": steps, "decode_slots": [N + 1, N + steps],
                        "decode_us_per_layer_step": round(us, 2),
                        "decode_ms_per_step_all_layers": round(us * cfg.layers / 1e3, 4),
                        "decode_kernel_us": round(kd, 2),
                        "decode_combine_us": round(statistics.median(kt["combine"]), 2),
                        "decode_kernel_GBps": round(dbytes / (kd * 1e-6) / 1e9, 1),
                        "decode_step_GBps": round(dbytes / (us * 1e-6) / 1e9, 1),
                        "decode_note": "per step: kvs_decode_attn calls enqueued back to back (decode kernel + "
                                       "combine); kernel times from library event marks (include ~1 us of mark gap)"})
        if cpu:
            dec = None
            if cfg.decode_steps:
                dec = (Kc, Vc, nc, qs, [N + t + 1 for t in range(steps)])
            res["cpu_oracle"] = cpu_oracle_config(cfg, K0, V0, Qws, dec)
        lines.append(res)
        print(json.dumps(res), flush=True)
        del plan, K0, V0
        torch.cuda.empty_cache()
    return lines


def all_layer_timing(cfg, dev, plan0, reps=3):
    """Every layer of a config merged back to back: the caches of all layers resident at once
    (layer 0's rounds are `plan0`), every layer's rounds enqueued on one stream, then with the
    layers alternating over two streams (pipeline.run_layers_fused; the layers share
    nothing).  Medians over `reps` passes over all layers; both orders must give the same
    merged rows."""
    import statistics
    import torch
    from long_context_kv_kvslimmer_amd import pipeline, synth
    plans = [[(K, V, n, Qw, M, N, bufs) for (K, V, n, Qw, M, N, _, bufs) in plan0]]
    for layer in range(1, cfg.layers):
        K, V, _ = pipeline.config_cache(cfg, layer, dev)
        n, N = None, cfg.n_slots
        p = []
        for r, M in enumerate(cfg.rounds):
            Qw = torch.stack([synth.window_queries(cfg, layer, b, r, dev) for b in range(cfg.batch)])
            bufs = pipeline.alloc_round(K, cfg.q_heads, cfg.window, cfg.n_sink, cfg.n_recent, M, n_slots=N,
                                        out_capacity=N - M, want_flags=False)
            p.append((K, V, n, Qw, M, N, bufs))
            K, V, n, N = bufs.K, bufs.V, bufs.n, N - M
        plans.append(p)

    def run(n_streams):
        return lambda: pipeline.run_layers_fused(plans, cfg.q_heads, cfg.window, cfg.n_sink, cfg.n_recent,
                                                 n_streams=n_streams)

    one_stream, two_streams = run(1), run(2)

    def last_rows():
        torch.cuda.synchronize()
        return [p[-1][-1].K[..., :p[-1][5] - p[-1][4], :].float().sum().item() for p in plans]

    def timed(f):
        f()
        torch.cuda.synchronize()
        times = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            f()
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        return statistics.median(times)

    one_ms = timed(one_stream)
    ref = last_rows()
    two_ms = timed(two_streams)
    same = last_rows() == ref
    del plans[1:]
    torch.cuda.empty_cache()
    return {"merge_ms_all_layers_one_stream": round(one_ms, 3), "merge_ms_all_layers_two_streams": round(two_ms, 3),
            "all_layers_outputs_equal": same}


def stream_timing(cfg, dev, reps=5, chunks=(256, 512, 1024, 2016)):
    """Chunked prefill under a cache budget, all layers folded into the batch: the whole loop
    (chunk appends + one partial merge round per chunk past the budget) timed with events on
    the current stream, the library's kernels split by name with event marks, and the peak
    device memory the loop allocates (two ping-pong caches, round statistics, workspaces)
    measured for several chunk sizes against the uncompressed cache."""
    import statistics
    import torch
    from long_context_kv_kvslimmer_amd import pipeline
    from long_context_kv_kvslimmer_amd import kvslim as L
    K_src, V_src, wq = pipeline.stream_inputs(cfg, dev)
    B, H, total, D = K_src.shape
    row = 2 * D * K_src.element_size()
    full_mb = B * H * total * row / 1e6

    def setup(chunk):
        plan = pipeline.stream_schedule(total, cfg.budget, chunk, cfg.n_sink)
        qws = [wq(c) if s.rounds else None for c, s in enumerate(plan)]
        torch.cuda.synchronize()
        base = torch.cuda.memory_allocated()
        torch.cuda.reset_peak_memory_stats()
        st = pipeline.alloc_stream(B, H, cfg.q_heads, D, K_src.dtype, dev, cfg.window, cfg.n_sink, plan)

        def run():
            return pipeline.run_stream(K_src, V_src, lambda c: qws[c], cfg.q_heads, cfg.window, cfg.n_sink,
                                       plan, st)
        run()
        torch.cuda.synchronize()
        peak = torch.cuda.max_memory_allocated() - base
        return plan, st, run, peak

    def timed(run, n):
        times = []
        for _ in range(n):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            run()
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        return statistics.median(times)

    sweep = []
    for chunk in chunks:
        plan, st, run, peak = setup(chunk)
        ms = timed(run, 3)
        sweep.append({"chunk": chunk, "rounds": sum(len(s.rounds) for s in plan), "loop_ms": round(ms, 3),
                      "peak_alloc_MB": round(peak / 1e6, 1),
                      "cache_MB": round(2 * st.bufs[0].K.numel() * 2 * K_src.element_size() / 1e6, 1)})
        del plan, st, run
        torch.cuda.empty_cache()
    plan, st, run, peak = setup(cfg.chunk)
    ms = timed(run, reps)
    n_rounds = sum(len(s.rounds) for s in plan)
    marks = L.KernelMarks(max_launches=16 * n_rounds + 64)
    with marks:
        run()
    torch.cuda.synchronize()
    per_kernel = {}
    for name, kms in marks.times():
        per_kernel[name] = per_kernel.get(name, 0.0) + kms * 1e3
    kern_us = sum(v for k, v in per_kernel.items() if k != "append")   # the merge rounds' kernels
    # algorithmic bytes of the merge rounds: both scorer passes read K, V and the counts of
    # the N slots (the merge runs inside the second); T slots are written with count and
    # source index
    alg = 0
    for s in plan:
        for N, M in s.rounds:
            alg += B * H * (2 * N * (row + 4) + (N - M) * (row + 8))
    return {"config": f"C{cfg.idx} {cfg.name}", "layers_folded_into_batch": B, "kv_heads": H, "tokens": total,
            "budget": cfg.budget, "chunk": cfg.chunk, "n_sink": cfg.n_sink, "chunks": len(plan),
            "merge_rounds": n_rounds, "loop_ms": round(ms, 3),
            "prefill_tokens_per_s": round(total / (ms * 1e-3), 1),
            "ms_per_round": round(ms / max(n_rounds, 1), 4),
            "kernel_us_per_round": {k: round(v / n_rounds, 2) for k, v in per_kernel.items()},
            "merge_kernel_us_total": round(kern_us, 1),
            "append_us_total": round(per_kernel.get("append", 0.0), 1),
            "merge_algorithmic_MB": round(alg / 1e6, 1),
            "merge_kernel_GBps": round(alg / (kern_us * 1e-6) / 1e9, 1),
            "peak_alloc_MB": round(peak / 1e6, 1), "full_cache_MB": round(full_mb, 1),
            "chunk_sweep": sweep,
            "note": "loop_ms includes the chunk appends (kvs_append, the prefill's cache writes) and host "
                    "launch overhead; kernel times from library event marks"}


def diag_timing(dev, reps=5):
    """The exact-gradient diagnostics on one C2 layer (32K slots, 8 KV heads, 128 window
    queries per head) with an upstream gradient E ~ N(0, 1) per window query: kernel time,
    and what it reports - the norm-weighted cosines cos(E, c11), cos(E, c22), cos(E, c12)
    and how far the forward-only weights land from the exact-Hessian ones."""
    import statistics
    import torch
    from long_context_kv_kvslimmer_amd import configs, pipeline, synth
    from long_context_kv_kvslimmer_amd import kvslim as L
    cfg = configs.C2
    K, V, _ = synth.make_cache(cfg, 0, 0, dev)
    K, V = K[None].contiguous(), V[None].contiguous()
    Qw = synth.window_queries(cfg, 0, 0, 0, dev)[None].contiguous()
    g = torch.Generator(device=dev)
    g.manual_seed(17)
    E = torch.randn(Qw.shape, generator=g, device=dev, dtype=torch.float32)
    S, R, Hq, W = cfg.n_sink, cfg.n_recent, cfg.q_heads, cfg.window
    bufs = pipeline.alloc_round(K, Hq, W, S, R, cfg.rounds[0], want_flags=False)
    pipeline.run_round_fused(K, V, None, Qw, Hq, W, S, R, cfg.rounds[0], bufs)
    lse, O = bufs.lse.clone(), bufs.O.clone()
    pipeline.exact_e_diag(K, V, None, Qw, E, lse, O, Hq, W, S, R)
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        marks = L.KernelMarks(max_launches=4)
        with marks:
            slot, pair = pipeline.exact_e_diag(K, V, None, Qw, E, lse, O, Hq, W, S, R)
        torch.cuda.synchronize()
        times.append(sum(ms for _, ms in marks.times()))
    P = pair.shape[2]
    m = S + 2 * torch.arange(P, device=dev)
    so = slot[0]
    c11 = (so[:, m, 0].sum() / so[:, m, 1].sum()).item()
    c22 = (so[:, m + 1, 0].sum() / so[:, m + 1, 1].sum()).item()
    c12 = (pair[0, :, :, 0].sum() / pair[0, :, :, 1].sum()).item()
    dw = (pair[0, :, :, 3] - pair[0, :, :, 5]).abs()
    ms = statistics.median(times)
    # per window query and unit (pair or single slot), per head-dim element: 9 fma + 3 add
    units = cfg.n_sink + P + (cfg.n_slots - cfg.n_sink - 2 * P)
    flop = cfg.kv_heads * units * cfg.group * W * cfg.head_dim * 21
    tf = flop / (ms * 1e-3) / 1e12
    return {"config": "exact-gradient diagnostics, C2 layer (32K slots x 8 KV heads, 128 window queries per head), "
                      "E ~ N(0, 1)", "kernel_ms": round(ms, 4),
            # the library is built without packed fp32 instructions, so the fp32 vector peak is
            # the unpacked one: 256 CUs x 4 SIMDs x 16 lanes x 2 flop (fma) x 2.4 GHz = 78.6 TFLOP/s
            # (157.3 counts two fp32 operations per lane per packed instruction)
            "roofline": {"bound": "alu", "achieved": round(tf, 1), "peak": 78.6, "unit": "TFLOP/s",
                         "frac": round(tf / 78.6, 3), "flop_per_launch": flop,
                         "peak_note": "unpacked fp32 vector rate; packed fp32 forms are compiled out"},
            "cos_E_c11": round(c11, 4), "cos_E_c22": round(c22, 4), "cos_E_c12": round(c12, 4),
            "median_abs_w_exact_minus_w_fwd": round(dw.median().item(), 4),
            "note": "a random E is no trained model's gradient: the angle relation the forward-only weights "
                    "assume (cos11 = cos22 = -cos12) does not hold for it, so these figures show the diagnostic "
                    "working, not KVSlimmer's accuracy"}


def spectral_timing(dev, T=32768, d=4096, r=128, reps=5):
    """The spectral split on a Llama-3.1-8B-shaped key projection (d_model 4096 -> one KV
    head of 128): 32K synthetic token states (AR(1) in d_model), W with a decaying
    spectrum, its thin SVD as the modes; kernel times and what the split shows (the share
    of the mean adjacent-key cosine carried by the top modes)."""
    import statistics
    import torch
    from long_context_kv_kvslimmer_amd import kvslim as L
    g = torch.Generator(device=dev)
    g.manual_seed(23)
    # AR(1) token states x_t = 0.9 x_{t-1} + eps_t, 256 steps at a time with a
    # lower-triangular power matrix
    eps = torch.randn(T, d, generator=g, device=dev) * 0.44
    coef = torch.tensor(0.9, device=dev)
    X = torch.empty(T, d, device=dev)
    carry = torch.randn(d, generator=g, device=dev)
    blk = 256
    tt = torch.arange(blk, device=dev, dtype=torch.float32)
    Lm = torch.where(tt[:, None] >= tt[None, :], coef ** (tt[:, None] - tt[None, :]), torch.zeros((), device=dev))
    pw = coef ** (tt + 1)
    for b0 in range(0, T, blk):
        y = Lm @ eps[b0:b0 + blk] + pw[:, None] * carry[None, :]
        X[b0:b0 + blk] = y
        carry = y[-1]
    W = torch.randn(d, r, generator=g, device=dev) / torch.sqrt(1 + torch.arange(r, device=dev, dtype=torch.float32))
    U, sig, _ = torch.linalg.svd(W.cpu().double(), full_matrices=False)
    Xb = X.to(torch.bfloat16).contiguous()
    Ub = U.T.contiguous().to(torch.bfloat16).to(dev)
    lam = (sig ** 2).float().to(dev)
    proj = torch.empty(T, r, device=dev)
    contrib = torch.empty(T - 1, r, device=dev)
    cos = torch.empty(T - 1, device=dev)
    L.kvs_spectral_modes(Xb, Ub, lam, proj, contrib, cos)
    torch.cuda.synchronize()
    per = {}
    for _ in range(reps):
        marks = L.KernelMarks(max_launches=4)
        with marks:
            L.kvs_spectral_modes(Xb, Ub, lam, proj, contrib, cos)
        torch.cuda.synchronize()
        for name, ms in marks.times():
            per.setdefault(name, []).append(ms)
    med = {k: statistics.median(v) for k, v in per.items()}
    share = contrib.mean(0) / cos.mean()
    top = torch.sort(share, descending=True).values.cumsum(0)
    proj_bytes = T * d * 2 + r * d * 2 + T * r * 4
    flop = 2 * T * d * r
    pm = med.get("spectral_proj", float("nan"))
    return {"config": f"spectral split, T={T} tokens, d_model={d}, {r} modes (bf16)",
            "kernel_ms": {k: round(v, 4) for k, v in med.items()},
            "roofline": {"kernel": "spectral_proj", "bound": "hbm", "achieved": round(proj_bytes / (pm * 1e-3) / 1e9, 1),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(proj_bytes / (pm * 1e-3) / 1e9 / HBM_PEAK_GBS, 3),
                         "mfma_TFLOPs": round(flop / (pm * 1e-3) / 1e12, 1)},
            "mean_adjacent_cos": round(cos.mean().item(), 4),
            "share_of_mean_cos_top4_top16_modes": [round(top[3].item(), 3), round(top[15].item(), 3)],
            "note": "synthetic W (singular values ~ 1/sqrt(i)) and AR(1) token states: the split shows the tool "
                    "working; the pages' figure needs a trained model's projections"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--sets", type=int, default=4, help="rotating input layers (>= 3 to exceed the MALL)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a plain 1 GiB copy first (counter calibration)")
    ap.add_argument("--summarize-counters", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "CMD"))
    ap.add_argument("--summarize-trace", nargs=3, metavar=("STATS_CSV", "BENCH_JSON", "CMD"))
    ap.add_argument("--summarize-mfma", nargs=3, metavar=("SQ_CSV", "STATS_CSV", "CMD"))
    ap.add_argument("--summarize-pmc", nargs=4, metavar=("CSVS", "STATS_CSV", "CMD", "TITLE"))
    ap.add_argument("--summarize-per-config", nargs=2, metavar=("JSONL", "CMD"))
    ap.add_argument("--summarize-stats", nargs=3, metavar=("STATS_CSV", "TITLE", "CMD"))
    ap.add_argument("--spectral", action="store_true",
                    help="time the spectral split (32K tokens, d_model 4096, 128 modes) instead of the bench line")
    ap.add_argument("--diag", action="store_true",
                    help="time the exact-gradient diagnostics on a C2 layer instead of the bench line")
    ap.add_argument("--no-all-layers", action="store_true",
                    help="with --per-config: time one layer only, not every layer back to back (a profiled run "
                         "then sees no kernels of two streams overlapping)")
    ap.add_argument("--no-chunk-sweep", action="store_true",
                    help="with --per-config 6: time only the 512-token-chunk loop (no chunk-size sweep)")
    ap.add_argument("--per-config", type=str, default=None, metavar="1,2,3,4,5,6",
                    help="print per-config merge and decode timings (one JSON line per config) instead of the bench line")
    args = ap.parse_args()
    if args.summarize_stats:
        sys.stdout.write(summarize_stats(*args.summarize_stats))
        return
    if args.summarize_per_config:
        sys.stdout.write(summarize_per_config(*args.summarize_per_config))
        return
    if args.summarize_mfma:
        sys.stdout.write(summarize_mfma(*args.summarize_mfma))
        return
    if args.summarize_pmc:
        sys.stdout.write(summarize_pmc(*args.summarize_pmc))
        return
    if args.summarize_counters:
        sys.stdout.write(summarize_counters(*args.summarize_counters))
        return
    if args.summarize_trace:
        sys.stdout.write(summarize_trace(*args.summarize_trace))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU's share; --gpus {args.gpus} is not supported (each (batch, layer, "
              f"kv-head) slice is independent: shard by KV head, layer or batch, one process per GPU)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from long_context_kv_kvslimmer_amd import configs, kvslim as L, pipeline, synth

    dev = "cuda:0"
    torch.cuda.set_device(0)
    if args.diag:
        print(json.dumps(diag_timing(dev)), flush=True)
        return
    if args.spectral:
        print(json.dumps(spectral_timing(dev)), flush=True)
        return
    if args.per_config:
        per_config(dev, [int(x) for x in args.per_config.split(",")],
                   chunk_sweep=() if args.no_chunk_sweep else (256, 512, 1024, 2016), cpu=not args.no_cpu_baseline,
                   all_layers=not args.no_all_layers)
        return
    cfg = configs.C2
    if args.copy_calibration:
        copy_calibration(dev)
    B, H, Hq, D, N, W = cfg.batch, cfg.kv_heads, cfg.q_heads, cfg.head_dim, cfg.n_slots, cfg.window
    S, R, M = cfg.n_sink, cfg.n_recent, cfg.rounds[0]
    P = L.num_pairs(N, S, R)
    T = N - M

    sets = []
    for i in range(args.sets):
        K, V, _ = synth.make_cache(cfg, i, 0, dev)
        Qw = synth.window_queries(cfg, i, 0, 0, dev)
        q = synth.decode_query(cfg, i, 0, 0, dev)
        sets.append((K[None].contiguous(), V[None].contiguous(), Qw[None].contiguous(), q[None].contiguous()))
    bufs = pipeline.alloc_round(sets[0][0], Hq, W, S, R, M, want_flags=False)
    dec_cache = L.cache_desc(bufs.K, Hq, T)
    dec_ws = torch.zeros(max(L.workspace_bytes(L.KVS_OP_DECODE, dec_cache, None), 16), dtype=torch.uint8, device=dev)
    dec_out = torch.empty(B, Hq, D, dtype=torch.float32, device=dev)
    cache = L.cache_desc(sets[0][0], Hq, N)
    rnd = L.round_desc(W, S, R, M, 1.0 / math.sqrt(D))
    out_desc = L.cache_desc(bufs.K, Hq, T)
    # the adjacent-key cosine only feeds the selection; a round that merges every
    # candidate pair (or none) has nothing to select, so it is not requested then
    cos_out = bufs.cos if 0 < M < P else None

    def step(i):
        """One round: statistics, weights, merge and compaction in kvs_score_merge (a full
        round: every candidate pair merges), then one decode step over the merged cache."""
        K, V, Qw, q = sets[i % len(sets)]
        L.kvs_score_merge(cache, K, V, None, Qw, rnd, bufs.lse, bufs.O, bufs.g_self, bufs.g_cross, out_desc,
                          bufs.K, bufs.V, bufs.n, bufs.src, bufs.score_ws)
        L.kvs_decode_attn(dec_cache, bufs.K, bufs.V, bufs.n, q, 1.0 / math.sqrt(D), dec_out, dec_ws)

    def step_separate(i):
        """The same round through the separate calls (kvs_score, kvs_merge_weights,
        kvs_merge_compact): measured in warm-up for the standalone merge pass."""
        K, V, Qw, q = sets[i % len(sets)]
        L.kvs_score(cache, K, V, None, Qw, rnd, bufs.lse, bufs.O, bufs.g_self, bufs.g_cross, cos_out, bufs.score_ws)
        L.kvs_merge_weights(cache, rnd, bufs.g_self, bufs.g_cross, cos_out, None, None, bufs.sel_state)
        L.kvs_merge_compact(cache, K, V, None, bufs.g_self, bufs.g_cross, rnd, bufs.sel_state, out_desc,
                            bufs.K, bufs.V, bufs.n, bufs.src)
        L.kvs_decode_attn(dec_cache, bufs.K, bufs.V, bufs.n, q, 1.0 / math.sqrt(D), dec_out, dec_ws)

    # warm-up: W steps (at least one, so that every kernel has loaded its code object
    # before any launch is marked); then, still outside the timed region, a few steps with
    # every launch marked rank the kernels by median time per step
    for i in range(max(args.warmup, 1)):
        step(i)
    n_rank = 3
    every = L.KernelMarks(max_launches=16 * n_rank)
    with every:
        for i in range(n_rank):
            step(args.warmup + i)
    torch.cuda.synchronize()
    ranked = rank_kernels(every.times(), n_rank)
    step_separate(0)            # first launches of these kernels load their code
    torch.cuda.synchronize()
    sep = L.KernelMarks(max_launches=16 * n_rank)
    with sep:
        for i in range(n_rank):
            step_separate(i)
    torch.cuda.synchronize()
    ranked_sep = rank_kernels(sep.times(), n_rank)
    dominant = dominant_kernel(ranked)

    # timed region: K whole steps; the library records HIP events right before and after
    # each launch of the dominant kernel (on its stream), timing that kernel live
    marks = L.KernelMarks(max_launches=4 * args.steps, label=dominant)
    t_start, t_stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    t_start.record()
    with marks:
        for i in range(args.steps):
            step(args.warmup + i)
    t_stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    gpu_ms = t_start.elapsed_time(t_stop) / args.steps
    timed = [ms for _, ms in marks.times()]
    if dominant is None and timed:
        dominant = marks.times()[0][0]
    kb = kernel_bytes(N, H, D, P, T, cfg.group * W)
    kernels = {}
    for name, r in ranked.items():
        by = kb.get(name, 0)
        kernels[name] = {"launches_per_step": r["launches_per_step"], "median_ms": round(r["median_ms"], 4),
                         "algorithmic_MB": round(by / 1e6, 2),
                         "GBps": round(by / (r["median_ms"] * 1e-3) / 1e9, 1) if by else None}
    kernels_separate = {}
    for name, r in ranked_sep.items():
        by = kb.get(name, 0)
        med = r["median_ms"]
        kernels_separate[name] = {"median_ms": round(med, 4), "algorithmic_MB": round(by / 1e6, 2),
                                  "GBps": round(by / (med * 1e-3) / 1e9, 1) if by else None,
                                  "hbm_frac": round(by / (med * 1e-3) / 1e9 / HBM_PEAK_GBS, 4) if by else None}
    dom_ms = sum(timed) / len(timed)
    dom_gbps = kb[dominant] / (dom_ms * 1e-3) / 1e9
    step_bytes = sum(kb[n] * kernels[n]["launches_per_step"] for n in kernels if n in kb)
    line = {
        "metric": METRIC,
        "value": round(B * N / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "C2: one Llama-3.1-8B layer, 32K ctx, merge to 50% keeping 32 recent "
                               "(kvs_score_merge), then one decode step", "batch": B, "kv_heads": H, "q_heads": Hq, "head_dim": D,
                   "n_slots": N, "window": W, "n_merge": M, "out_slots": T, "input_sets": len(sets),
                   "accumulate": "f32"},
        "hbm_GBps_step": round(step_bytes / (ms_step * 1e-3) / 1e9, 1),
        "gpu_ms_per_step": round(gpu_ms, 4),
        "kernels_ranked": kernels,
        "kernels_separate_calls": kernels_separate,
        "roofline": {"kernel": dominant, "avg_ms": round(dom_ms, 4), "launches": len(timed),
                     "algorithmic_bytes": kb[dominant], "bound": "hbm", "achieved": round(dom_gbps, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(dom_gbps / HBM_PEAK_GBS, 4),
                     "traffic": recorded_traffic(dominant)},
    }
    line["given_window_stats"] = given_stats_timing(args, sets, step, bufs, cache, rnd, out_desc, dec_cache, dec_out,
                                                    dec_ws, D, B * N, kb)
    line["machine"] = gpu_clock_info()
    if not args.no_cpu_baseline:
        K, V, Qw, q = sets[0]
        line["cpu_baseline"] = cpu_baseline(cfg, K, V, Qw, q)
    print(json.dumps(line), flush=True)


def given_stats_timing(args, sets, step, bufs, cache, rnd, out_desc, dec_cache, dec_out, dec_ws, D, tokens, kb):
    """The same step when the prefill attention supplies the window statistics: the round
    through kvs_score_merge_stats (no first scorer pass), then the decode step.  Each input
    set's statistics are taken from kvs_score_merge once, before timing."""
    import torch
    from long_context_kv_kvslimmer_amd import kvslim as L
    stats = []
    for i in range(len(sets)):
        step(i)
        stats.append((bufs.lse.clone(), bufs.O.clone()))
    torch.cuda.synchronize()

    def step_stats(i):
        K, V, Qw, q = sets[i % len(sets)]
        lse, O = stats[i % len(sets)]
        L.kvs_score_merge_stats(cache, K, V, None, Qw, rnd, lse, O, bufs.g_self, bufs.g_cross, out_desc,
                                bufs.K, bufs.V, bufs.n, bufs.src, bufs.score_ws)
        L.kvs_decode_attn(dec_cache, bufs.K, bufs.V, bufs.n, q, 1.0 / math.sqrt(D), dec_out, dec_ws)

    for i in range(args.warmup):
        step_stats(i)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(args.steps):
        step_stats(i)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    marks = L.KernelMarks(max_launches=64)
    with marks:
        for i in range(4):
            step_stats(i)
    torch.cuda.synchronize()
    per = {}
    for name, kms in marks.times():
        tot, cnt = per.get(name, (0.0, 0))
        per[name] = (tot + kms, cnt + 1)
    kernels = {}
    for name, (tot, cnt) in per.items():
        avg = tot / cnt
        by = kb.get(name, 0)
        kernels[name] = {"avg_ms": round(avg, 4), "GBps": round(by / (avg * 1e-3) / 1e9, 1) if by else None}
    return {"ms_per_step": round(ms, 4), "tokens_per_s": round(tokens / (ms * 1e-3), 1), "kernels": kernels,
            "note": "kvs_score_merge_stats + kvs_decode_attn per step (GPU events); the window statistics "
                    "are an input here (a prefill attention computes them), so the first scorer pass and its "
                    "combine are not run; not the headline value"}


if __name__ == "__main__":
    main()
