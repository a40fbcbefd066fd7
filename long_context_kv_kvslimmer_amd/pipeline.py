"""One merge round and decode steps through the C ABI, with torch used only to
allocate device buffers.  Every computation runs in libkvslim's HIP kernels."""
from __future__ import annotations

import math
from dataclasses import dataclass

import torch

from . import kvslim as L


@dataclass
class RoundBuffers:
    lse: torch.Tensor
    O: torch.Tensor
    g_self: torch.Tensor
    g_cross: torch.Tensor
    cos: torch.Tensor
    sel_state: torch.Tensor
    score_ws: torch.Tensor
    w: torch.Tensor | None
    selected: torch.Tensor | None
    K: torch.Tensor
    V: torch.Tensor
    n: torch.Tensor
    src: torch.Tensor


def alloc_round(K: torch.Tensor, n_q_heads: int, window: int, n_sink: int, n_recent: int, n_merge: int,
                n_slots: int | None = None, out_dtype=None, out_capacity: int | None = None,
                want_flags: bool = False) -> RoundBuffers:
    B, H, cap, D = K.shape
    N = cap if n_slots is None else n_slots
    P = L.num_pairs(N, n_sink, n_recent)
    T = N - n_merge
    dev = K.device
    f32 = torch.float32
    cache = L.cache_desc(K, n_q_heads, N)
    rnd = L.round_desc(window, n_sink, n_recent, n_merge, 1.0 / math.sqrt(D))
    ws = max(L.workspace_bytes(op, cache, rnd) for op in (L.KVS_OP_SCORE, L.KVS_OP_SCORE_MERGE, L.KVS_OP_STATS_MERGE))
    ss = L.workspace_bytes(L.KVS_OP_SEL_STATE, cache, rnd)
    ocap = T if out_capacity is None else out_capacity
    odt = K.dtype if out_dtype is None else out_dtype
    return RoundBuffers(
        lse=torch.empty(B, n_q_heads, window, dtype=f32, device=dev),
        O=torch.empty(B, n_q_heads, window, D, dtype=f32, device=dev),
        g_self=torch.empty(B, H, N, dtype=f32, device=dev),
        g_cross=torch.empty(B, H, P, dtype=f32, device=dev),
        cos=torch.empty(B, H, P, dtype=f32, device=dev),
        sel_state=torch.empty(max(ss, 16), dtype=torch.uint8, device=dev),
        score_ws=torch.empty(max(ws, 16), dtype=torch.uint8, device=dev),
        w=torch.empty(B, H, P, 2, dtype=f32, device=dev) if want_flags else None,
        selected=torch.empty(B, H, P, dtype=torch.uint8, device=dev) if want_flags else None,
        K=torch.empty(B, H, ocap, D, dtype=odt, device=dev),
        V=torch.empty(B, H, ocap, D, dtype=odt, device=dev),
        n=torch.empty(B, H, ocap, dtype=torch.int32, device=dev),
        src=torch.empty(B, H, ocap, dtype=torch.int32, device=dev),
    )


def run_round(K, V, n, Qw, n_q_heads: int, window: int, n_sink: int, n_recent: int, n_merge: int,
              bufs: RoundBuffers, n_slots: int | None = None):
    """score -> merge_weights -> merge_compact, all enqueued on the current stream."""
    B, H, cap, D = K.shape
    N = cap if n_slots is None else n_slots
    cache = L.cache_desc(K, n_q_heads, N)
    rnd = L.round_desc(window, n_sink, n_recent, n_merge, 1.0 / math.sqrt(D))
    P = L.num_pairs(N, n_sink, n_recent)
    # the cosine feeds only the selection: computed for partial rounds, or when flags are wanted
    cos = bufs.cos if (0 < n_merge < P or bufs.selected is not None) else None
    L.kvs_score(cache, K, V, n, Qw, rnd, bufs.lse, bufs.O, bufs.g_self, bufs.g_cross, cos, bufs.score_ws)
    L.kvs_merge_weights(cache, rnd, bufs.g_self, bufs.g_cross, cos, bufs.w, bufs.selected, bufs.sel_state)
    out = L.cache_desc(bufs.K, n_q_heads, N - n_merge)
    L.kvs_merge_compact(cache, K, V, n, bufs.g_self, bufs.g_cross, rnd, bufs.sel_state, out,
                        bufs.K, bufs.V, bufs.n, bufs.src)
    return bufs


def run_round_fused(K, V, n, Qw, n_q_heads: int, window: int, n_sink: int, n_recent: int, n_merge: int,
                    bufs: RoundBuffers, n_slots: int | None = None):
    """A whole round (any 0 <= n_merge <= P) through kvs_score_merge; selection flags and
    weights are not produced."""
    B, H, cap, D = K.shape
    N = cap if n_slots is None else n_slots
    cache = L.cache_desc(K, n_q_heads, N)
    rnd = L.round_desc(window, n_sink, n_recent, n_merge, 1.0 / math.sqrt(D))
    out = L.cache_desc(bufs.K, n_q_heads, N - n_merge)
    L.kvs_score_merge(cache, K, V, n, Qw, rnd, bufs.lse, bufs.O, bufs.g_self, bufs.g_cross, out,
                      bufs.K, bufs.V, bufs.n, bufs.src, bufs.score_ws)
    return bufs


def run_layers_fused(layers: list, n_q_heads: int, window: int, n_sink: int, n_recent: int,
                     n_streams: int = 2) -> None:
    """Merge rounds of several independent layers, enqueued without a host wait.

    `layers[l]` is the list of layer l's rounds, each (K, V, n, Qw, n_merge, n_slots, bufs) in
    order (round r + 1 reads round r's bufs).  Layer l's rounds go to stream l % n_streams in
    order; the streams start after the work already on the current stream and the current
    stream waits for all of them at the end.  Layers share no buffer, so the order of
    layers across streams does not change a result; what overlaps is one layer's short,
    latency-bound launches (the selection, the combine, kernel tails) with another layer's
    scorer passes.  With n_streams = 1 the layers run in order on the current stream."""
    def rounds(plan):
        for (K, V, n, Qw, M, N, bufs) in plan:
            run_round_fused(K, V, n, Qw, n_q_heads, window, n_sink, n_recent, M, bufs, n_slots=N)

    if n_streams <= 1:
        for plan in layers:
            rounds(plan)
        return
    main = torch.cuda.current_stream()
    side = [torch.cuda.Stream(device=main.device) for _ in range(n_streams)]
    fork = torch.cuda.Event()
    fork.record(main)
    for s in side:
        s.wait_event(fork)
    for i, plan in enumerate(layers):
        with torch.cuda.stream(side[i % n_streams]):
            rounds(plan)
    for s in side:
        join = torch.cuda.Event()
        join.record(s)
        main.wait_event(join)


def run_round_given_stats(K, V, n, Qw, lse, O, n_q_heads: int, window: int, n_sink: int, n_recent: int,
                          n_merge: int, bufs: RoundBuffers, n_slots: int | None = None):
    """A whole round through kvs_score_merge_stats: the window statistics lse [B, H_q, W] and
    O [B, H_q, W, D] come from the caller (the prefill attention); bufs.lse / bufs.O unused."""
    B, H, cap, D = K.shape
    N = cap if n_slots is None else n_slots
    cache = L.cache_desc(K, n_q_heads, N)
    rnd = L.round_desc(window, n_sink, n_recent, n_merge, 1.0 / math.sqrt(D))
    out = L.cache_desc(bufs.K, n_q_heads, N - n_merge)
    L.kvs_score_merge_stats(cache, K, V, n, Qw, rnd, lse, O, bufs.g_self, bufs.g_cross, out,
                            bufs.K, bufs.V, bufs.n, bufs.src, bufs.score_ws)
    return bufs


def exact_e_diag(K, V, n, Qw, E, lse, O, n_q_heads: int, window: int, n_sink: int, n_recent: int,
                 n_slots: int | None = None):
    """Exact-gradient diagnostics of one round (kvs_exact_e_diag): returns slot_out
    [B, H, N, 3] and pair_out [B, H, P, 9]."""
    B, H, cap, D = K.shape
    N = cap if n_slots is None else n_slots
    P = L.num_pairs(N, n_sink, n_recent)
    cache = L.cache_desc(K, n_q_heads, N)
    rnd = L.round_desc(window, n_sink, n_recent, 0, 1.0 / math.sqrt(D))
    slot_out = torch.empty(B, H, N, 3, dtype=torch.float32, device=K.device)
    pair_out = torch.empty(B, H, max(P, 1), 9, dtype=torch.float32, device=K.device)
    L.kvs_exact_e_diag(cache, K, V, n, Qw, rnd, E, lse, O, slot_out, pair_out)
    return slot_out, pair_out[:, :, :P]


def run_full_round_fused(K, V, n, Qw, n_q_heads: int, window: int, n_sink: int, n_recent: int,
                         bufs: RoundBuffers, n_slots: int | None = None):
    """A full round (every candidate pair merges) through kvs_score_merge."""
    N = K.shape[2] if n_slots is None else n_slots
    P = L.num_pairs(N, n_sink, n_recent)
    return run_round_fused(K, V, n, Qw, n_q_heads, window, n_sink, n_recent, P, bufs, n_slots)


def merge_round(K, V, n, Qw, n_q_heads: int, window: int, n_sink: int, n_recent: int, n_merge: int,
                n_slots: int | None = None, out_dtype=None, out_capacity: int | None = None,
                want_flags: bool = True) -> RoundBuffers:
    bufs = alloc_round(K, n_q_heads, window, n_sink, n_recent, n_merge, n_slots, out_dtype, out_capacity,
                       want_flags)
    return run_round(K, V, n, Qw, n_q_heads, window, n_sink, n_recent, n_merge, bufs, n_slots)


def decode(K, V, n, q, n_slots: int | None = None, sm_scale: float | None = None,
           workspace: torch.Tensor | None = None, out: torch.Tensor | None = None) -> torch.Tensor:
    B, H, cap, D = K.shape
    Hq = q.shape[1]
    N = cap if n_slots is None else n_slots
    cache = L.cache_desc(K, Hq, N)
    if workspace is None:
        workspace = torch.zeros(max(L.workspace_bytes(L.KVS_OP_DECODE, cache, None), 16), dtype=torch.uint8,
                                device=K.device)
    if out is None:
        out = torch.empty(B, Hq, D, dtype=torch.float32, device=K.device)
    L.kvs_decode_attn(cache, K, V, n, q, 1.0 / math.sqrt(D) if sm_scale is None else sm_scale, out, workspace)
    return out


# ---------------------------------------------------------------- workloads --
def config_cache(cfg, layer: int, device, batches=None):
    """Seeded raw cache of one layer: K, V [B, H_kv, N, D] and the last raw keys [B, H_kv, D]."""
    from . import synth
    bs = range(cfg.batch) if batches is None else batches
    ks, vs, lasts = [], [], []
    for b in bs:
        k, v, last = synth.make_cache(cfg, layer, b, device)
        ks.append(k)
        vs.append(v)
        lasts.append(last)
    return torch.stack(ks), torch.stack(vs), torch.stack(lasts)


def config_rounds(cfg, layer: int, device, K=None, V=None, batches=None, out_dtype=None, want_flags=True,
                  last_capacity: int = 0):
    """Run every merge round of a workload config on one layer.  Returns a list of
    (K_in, V_in, n_in, Qw, M, bufs) per round; round r + 1 consumes round r's output.
    `last_capacity` extra slots are reserved after the last round's output (decode appends)."""
    from . import synth
    if K is None:
        K, V, _ = config_cache(cfg, layer, device, batches)
    bs = list(range(cfg.batch)) if batches is None else list(batches)
    n = None
    out = []
    N = K.shape[2]
    for r, M in enumerate(cfg.rounds):
        Qw = torch.stack([synth.window_queries(cfg, layer, b, r, device) for b in bs])
        T = N - M
        cap = T + (last_capacity if r == len(cfg.rounds) - 1 else 0)
        bufs = merge_round(K, V, n, Qw, cfg.q_heads, cfg.window, cfg.n_sink, cfg.n_recent, M, n_slots=N,
                           out_dtype=out_dtype, out_capacity=cap, want_flags=want_flags)
        out.append((K, V, n, Qw, M, bufs))
        K, V, n, N = bufs.K, bufs.V, bufs.n, T
    return out


# ------------------------------------------------------ chunked budget loop --
@dataclass
class StreamStep:
    c0: int            # first token of the chunk
    length: int        # tokens in the chunk
    n_after: int       # slots held once the chunk is appended
    rounds: list       # [(N, M), ...]: merge rounds that bring the cache back to the budget


def stream_schedule(total: int, budget: int, chunk: int, n_sink: int) -> list:
    """Host plan of chunked prefill under a cache budget (the evaluation regime of the
    deep-dive's 实验设置): chunk after chunk is appended, and while the cache holds
    N > budget slots a merge round with M = min(N - budget, P) runs, P the candidate pairs
    after the n_sink kept first slots (no recent window is protected).  budget > n_sink
    guarantees every such round has a pair to merge."""
    if chunk < 1 or n_sink < 0 or budget <= n_sink or total < 0:
        raise ValueError("need chunk >= 1, total >= 0 and budget > n_sink >= 0")
    plan, N = [], 0
    for c0 in range(0, total, chunk):
        length = min(chunk, total - c0)
        N += length
        step = StreamStep(c0, length, N, [])
        while N > budget:
            M = min(N - budget, L.num_pairs(N, n_sink, 0))
            step.rounds.append((N, M))
            N -= M
        plan.append(step)
    return plan


@dataclass
class StreamBuffers:
    bufs: tuple        # two RoundBuffers whose K/V/n are the ping-pong caches; statistics shared
    capacity: int      # slots per (b, h) of each cache


def alloc_stream(B: int, H: int, n_q_heads: int, D: int, dtype, device, window: int, n_sink: int,
                 plan: list, want_flags: bool = False) -> StreamBuffers:
    """Two caches of the largest size the plan reaches, and one set of round statistics and
    workspaces sized for the largest round; nothing is allocated while the loop runs."""
    cap = max([s.n_after for s in plan] + [1])
    f32 = torch.float32
    P = L.num_pairs(cap, n_sink, 0)
    ws = ss = 16
    for s in plan:
        for N, M in s.rounds:
            c = L.KvsCache(B, H, n_q_heads, D, N, H * cap * D, cap * D)
            r = L.round_desc(window, n_sink, 0, M, 1.0 / math.sqrt(D))
            ws = max(ws, L.workspace_bytes(L.KVS_OP_SCORE, c, r), L.workspace_bytes(L.KVS_OP_SCORE_MERGE, c, r))
            ss = max(ss, L.workspace_bytes(L.KVS_OP_SEL_STATE, c, r))
    shared = dict(
        lse=torch.empty(B, n_q_heads, window, dtype=f32, device=device),
        O=torch.empty(B, n_q_heads, window, D, dtype=f32, device=device),
        g_self=torch.empty(B * H * cap, dtype=f32, device=device),
        g_cross=torch.empty(max(B * H * P, 1), dtype=f32, device=device),
        cos=torch.empty(max(B * H * P, 1), dtype=f32, device=device),
        sel_state=torch.empty(ss, dtype=torch.uint8, device=device),
        score_ws=torch.empty(ws, dtype=torch.uint8, device=device),
        w=torch.empty(max(B * H * P, 1), 2, dtype=f32, device=device) if want_flags else None,
        selected=torch.empty(max(B * H * P, 1), dtype=torch.uint8, device=device) if want_flags else None,
        src=torch.empty(B, H, cap, dtype=torch.int32, device=device))
    two = tuple(RoundBuffers(K=torch.empty(B, H, cap, D, dtype=dtype, device=device),
                             V=torch.empty(B, H, cap, D, dtype=dtype, device=device),
                             n=torch.empty(B, H, cap, dtype=torch.int32, device=device), **shared)
                for _ in range(2))
    return StreamBuffers(two, cap)


def run_stream(K_src, V_src, window_queries, n_q_heads: int, window: int, n_sink: int, plan: list,
               st: StreamBuffers, on_round=None, fused: bool = True):
    """Run the chunked budget loop on the current stream.  K_src, V_src [B, H_kv, total, D]
    hold the raw tokens (a prefill would write each chunk in turn); window_queries(c) gives
    the observation window [B, H_q, W, D] of chunk c (its last W queries).  Each chunk is
    appended with count 1 to the current cache (kvs_append), then each planned round reads that cache
    and writes the other one, through kvs_score_merge (fused) or the three separate calls.
    on_round(c, K, V, n, Qw, N, M, out) runs after each round is enqueued.  Returns
    (buffers holding the final cache, its slot count)."""
    cur, N = 0, 0
    src = L.cache_desc(K_src, n_q_heads)
    for c, s in enumerate(plan):
        b = st.bufs[cur]
        L.kvs_append(L.cache_desc(b.K, n_q_heads), b.K, b.V, b.n, N, src, K_src, V_src, s.c0, s.length)
        N += s.length
        if not s.rounds:
            continue
        Qw = window_queries(c)
        for Nr, M in s.rounds:
            out = st.bufs[1 - cur]
            step = run_round_fused if fused else run_round
            step(b.K, b.V, b.n, Qw, n_q_heads, window, n_sink, 0, M, out, n_slots=Nr)
            if on_round is not None:
                on_round(c, b.K, b.V, b.n, Qw, Nr, M, out)
            cur, b, N = 1 - cur, out, Nr - M
    return st.bufs[cur], N


def stream_inputs(cfg, device, layers=None):
    """Raw tokens of every layer folded into the batch dimension, [layers, H_kv, N, D], and
    the per-chunk observation windows [layers, H_q, W, D] (drawn per chunk, seeded)."""
    from . import synth
    ls = list(range(cfg.layers)) if layers is None else list(layers)
    K = torch.empty(len(ls), cfg.kv_heads, cfg.n_slots, cfg.head_dim, dtype=synth.TORCH_DTYPE[cfg.dtype],
                    device=device)
    V = torch.empty_like(K)
    for i, layer in enumerate(ls):
        K[i], V[i], _ = synth.make_cache(cfg, layer, 0, device)

    def window_queries(c):
        return torch.stack([synth.window_queries(cfg, layer, 0, c, device) for layer in ls])
    return K, V, window_queries
