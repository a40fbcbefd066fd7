"""Benchmark of the KVSlimmer merge path on one MI355X.

One step = the whole hot path on one Llama-3.1-8B-shaped layer at 32K context
(8 KV heads x 128, 32 query heads, bf16): kvs_score (window statistics and
Hessian-norm sums) -> kvs_merge_weights -> kvs_merge_compact (merge to 50%,
32 most recent tokens kept) -> kvs_decode_attn (one decode query per head over
the merged cache).  Inputs are resident in HBM before timing starts; steps
rotate over several input layers whose total exceeds the 256 MB Infinity
Cache, so every step reads its K/V from HBM.

Prints one JSON line (rank 0).  Usage: python bench.py [--steps K] [--warmup W]
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

METRIC = "KV tokens merged/sec + achieved HBM GB/s (Llama-3.1-8B layer, 32K ctx)"
HBM_PEAK_GBS = 8000.0


def algorithmic_bytes(N, H, D, P, M, T, has_n=False, elt=2):
    """Bytes each call must move (the method's reads and writes, once each)."""
    row = 2 * D * elt                               # one K row + one V row
    score = 2 * N * H * row + N * H * 4 + P * H * 4   # K,V twice; g_self, g_cross out
    merge = N * H * (row + 4 + (4 if has_n else 0)) + P * H * 4 + T * H * (row + 4 + 4)
    decode = T * H * (row + 4)
    select = 0
    return {"kvs_score": score, "kvs_merge_weights": select, "kvs_merge_compact": merge, "kvs_decode_attn": decode}


def cpu_baseline(cfg, K, V, Qw, heads=2):
    """The oracle as it stands, on `heads` KV heads of one layer (one thread)."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import kvs_oracle as O
    G = cfg.group
    M = cfg.rounds[0]
    t0 = time.perf_counter()
    with threadpool_limits(1):
        for h in range(heads):
            Ks = K[0, h].double().cpu().numpy()
            Vs = V[0, h].double().cpu().numpy()
            Qs = Qw[0, h * G:(h + 1) * G].double().cpu().numpy().reshape(-1, cfg.head_dim)
            r = O.merge_round(Ks, Vs, None, Qs, 1 / math.sqrt(cfg.head_dim), cfg.n_sink, cfg.n_recent, M)
            O.decode(r.K, r.V, r.n, Qs[0], 1 / math.sqrt(cfg.head_dim))
    dt = time.perf_counter() - t0
    tokens = cfg.n_slots * heads / cfg.kv_heads        # share of the layer's token positions
    return {"value": tokens / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{heads} of {cfg.kv_heads} KV heads of one C2 layer (N={cfg.n_slots}), merge round + "
                      f"one decode query, fp64 NumPy, 1 BLAS thread, {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--sets", type=int, default=4, help="rotating input layers (>= 3 to exceed the MALL)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU's share; --gpus {args.gpus} is not supported (each (batch, layer, "
              f"kv-head) slice is independent, see DESIGN.md for how the path shards)", file=sys.stderr)
        sys.exit(2)

    import torch

    from long_context_kv_kvslimmer_amd import configs, kvslim as L, pipeline, synth

    dev = "cuda:0"
    torch.cuda.set_device(0)
    cfg = configs.C2
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
    dec_ws = torch.empty(max(L.workspace_bytes(L.KVS_OP_DECODE, dec_cache, None), 16), dtype=torch.uint8, device=dev)
    dec_out = torch.empty(B, Hq, D, dtype=torch.float32, device=dev)
    cache = L.cache_desc(sets[0][0], Hq, N)
    rnd = L.round_desc(W, S, R, M, 1.0 / math.sqrt(D))
    out_desc = L.cache_desc(bufs.K, Hq, T)
    names = ("kvs_score", "kvs_merge_weights", "kvs_merge_compact", "kvs_decode_attn")
    # the adjacent-key cosine only feeds the selection; a round that merges every
    # candidate pair (or none) has nothing to select, so it is not requested then
    cos_out = bufs.cos if 0 < M < P else None

    def step(i, ev=None):
        K, V, Qw, q = sets[i % len(sets)]
        if ev is not None:
            ev[0].record()
        L.kvs_score(cache, K, V, None, Qw, rnd, bufs.lse, bufs.O, bufs.g_self, bufs.g_cross, cos_out, bufs.score_ws)
        if ev is not None:
            ev[1].record()
        L.kvs_merge_weights(cache, rnd, bufs.g_self, bufs.g_cross, cos_out, None, None, bufs.sel_state)
        if ev is not None:
            ev[2].record()
        L.kvs_merge_compact(cache, K, V, None, bufs.g_self, bufs.g_cross, rnd, bufs.sel_state, out_desc,
                            bufs.K, bufs.V, bufs.n, bufs.src)
        if ev is not None:
            ev[3].record()
        L.kvs_decode_attn(dec_cache, bufs.K, bufs.V, bufs.n, q, 1.0 / math.sqrt(D), dec_out, dec_ws)
        if ev is not None:
            ev[4].record()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # timed region: K whole steps, per-call HIP events on the stream the kernels run on
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_call = {n: 0.0 for n in names}
    for ev in events:
        for k, n in enumerate(names):
            per_call[n] += ev[k].elapsed_time(ev[k + 1])
    gpu_ms = sum(events[i][0].elapsed_time(events[i][4]) for i in range(args.steps))
    ms_step = wall * 1e3 / args.steps
    per_call = {n: v / args.steps for n, v in per_call.items()}
    abytes = algorithmic_bytes(N, H, D, P, M, T)
    kernels = {n: {"ms": round(per_call[n], 4),
                   "algorithmic_MB": round(abytes[n] / 1e6, 2),
                   "GBps": round(abytes[n] / (per_call[n] * 1e-3) / 1e9, 1) if per_call[n] > 0 else None}
               for n in names}
    dominant = max(names, key=lambda n: per_call[n])
    ach = abytes[dominant] / (per_call[dominant] * 1e-3) / 1e9
    step_bytes = sum(abytes.values())
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
        "config": {"workload": "C2: one Llama-3.1-8B layer, 32K ctx, merge to 50% keeping 32 recent, "
                               "then one decode step", "batch": B, "kv_heads": H, "q_heads": Hq, "head_dim": D,
                   "n_slots": N, "window": W, "n_merge": M, "out_slots": T, "input_sets": len(sets),
                   "accumulate": "f32"},
        "hbm_GBps_step": round(step_bytes / (ms_step * 1e-3) / 1e9, 1),
        "gpu_ms_per_step": round(gpu_ms / args.steps, 4),
        "kernels": kernels,
        "roofline": {"kernel": dominant, "bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": None},
    }
    if not args.no_cpu_baseline:
        K, V, Qw, _ = sets[0]
        line["cpu_baseline"] = cpu_baseline(cfg, K, V, Qw)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
