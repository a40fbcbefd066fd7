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
    ws = L.workspace_bytes(L.KVS_OP_SCORE, cache, rnd)
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


def run_full_round_fused(K, V, n, Qw, n_q_heads: int, window: int, n_sink: int, n_recent: int,
                         bufs: RoundBuffers, n_slots: int | None = None):
    """A full round (every candidate pair merges) through kvs_score_merge."""
    B, H, cap, D = K.shape
    N = cap if n_slots is None else n_slots
    P = L.num_pairs(N, n_sink, n_recent)
    cache = L.cache_desc(K, n_q_heads, N)
    rnd = L.round_desc(window, n_sink, n_recent, P, 1.0 / math.sqrt(D))
    out = L.cache_desc(bufs.K, n_q_heads, N - P)
    L.kvs_score_merge(cache, K, V, n, Qw, rnd, bufs.lse, bufs.O, bufs.g_self, bufs.g_cross, out,
                      bufs.K, bufs.V, bufs.n, bufs.src, bufs.score_ws)
    return bufs


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
