"""GPU: kvs_score_merge at the shapes and in the launch configuration that bench.py and
the per-config timings time.

* C2: one Llama-3.1-8B layer at 32K (8 x 128 KV heads, 32 query heads, window 32, keep
  32 recent), a full round through the fused call with bf16 output, exactly as the bench
  step calls it, and again with fp32 output.  The bf16 output must be the round-to-
  nearest-even image of the fp32 output bit for bit; the fp32 output must equal the
  separate calls (kvs_score -> kvs_merge_weights -> kvs_merge_compact) bit for bit; two
  heads are compared with the oracle; then the bench's decode step over the bf16 merged
  cache is compared with the oracle on that cache.
* C3: one layer at 128K, partial round M = 38011 of 65536 pairs per head (selection
  between the passes, merge inside the second): bit for bit against the separate calls,
  one head against the oracle.
* C5: the second round (every count 2) of one layer at 128K through the fused call:
  bit for bit against the separate calls, one head against the oracle.
"""
import math

import numpy as np
import pytest
import torch

from oracle import kvs_oracle as O
from tests.parity import REL_TOL, check_round_slice, host, maxrel

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _same(a, b, what):
    assert torch.equal(a, b), f"{what}: {(a != b).sum().item()} elements differ"


def _fused(K, V, n, Qw, cfg, M, N, odt):
    from long_context_kv_kvslimmer_amd import pipeline
    bufs = pipeline.alloc_round(K, cfg.q_heads, cfg.window, cfg.n_sink, cfg.n_recent, M, n_slots=N, out_dtype=odt)
    pipeline.run_round_fused(K, V, n, Qw, cfg.q_heads, cfg.window, cfg.n_sink, cfg.n_recent, M, bufs, n_slots=N)
    return bufs


def _separate(K, V, n, Qw, cfg, M, N, odt):
    from long_context_kv_kvslimmer_amd import pipeline
    return pipeline.merge_round(K, V, n, Qw, cfg.q_heads, cfg.window, cfg.n_sink, cfg.n_recent, M, n_slots=N,
                                out_dtype=odt, want_flags=False)


def _same_round(a, b, P, T):
    for f in ("lse", "O", "g_self"):
        _same(getattr(a, f), getattr(b, f), f)
    _same(a.g_cross[..., :P], b.g_cross[..., :P], "g_cross")
    for f in ("K", "V", "n", "src"):
        _same(getattr(a, f)[:, :, :T], getattr(b, f)[:, :, :T], f)


def test_c2_full_round_fused_as_timed():
    from long_context_kv_kvslimmer_amd import configs, synth
    cfg = configs.C2
    N, M = cfg.n_slots, cfg.rounds[0]
    P = O.num_pairs(N, cfg.n_sink, cfg.n_recent)
    T = N - M
    assert M == P
    print("\n[C2 fused] full layer, bf16 and fp32 outputs", flush=True)
    K, V, _ = synth.make_cache(cfg, 0, 0, DEV)
    K, V = K[None].contiguous(), V[None].contiguous()
    Qw = synth.window_queries(cfg, 0, 0, 0, DEV)[None].contiguous()
    b16 = _fused(K, V, None, Qw, cfg, M, N, torch.bfloat16)
    b32 = _fused(K, V, None, Qw, cfg, M, N, torch.float32)
    sep = _separate(K, V, None, Qw, cfg, M, N, torch.float32)
    torch.cuda.synchronize()
    _same(b16.K[:, :, :T], b32.K[:, :, :T].to(torch.bfloat16), "bf16 K' = RNE(fp32 K')")
    _same(b16.V[:, :, :T], b32.V[:, :, :T].to(torch.bfloat16), "bf16 V' = RNE(fp32 V')")
    _same(b16.n[:, :, :T], b32.n[:, :, :T], "n'")
    _same(b16.src[:, :, :T], b32.src[:, :, :T], "src")
    for f in ("lse", "O", "g_self", "g_cross"):
        _same(getattr(b16, f), getattr(b32, f), f)
    _same_round(b32, sep, P, T)
    scale = 1 / math.sqrt(cfg.head_dim)
    for h in (0, 5):
        print(f"[C2 fused] oracle head {h}", flush=True)
        check_round_slice(b32, K, V, None, Qw, 0, h, N, cfg.n_sink, cfg.n_recent, M, scale, label=f"C2 fused h{h}",
                          with_cos=False)
    # the bench step's decode: one query per head over the bf16 merged cache
    from long_context_kv_kvslimmer_amd import pipeline
    q = synth.decode_query(cfg, 0, 0, 0, DEV)[None].contiguous()
    out = pipeline.decode(b16.K, b16.V, b16.n, q, n_slots=T)
    torch.cuda.synchronize()
    for hq in (0, 9, 22, 31):
        h = hq // cfg.group
        ref = O.decode(host(b16.K[0, h, :T]), host(b16.V[0, h, :T]), host(b16.n[0, h, :T]), host(q[0, hq]), scale)
        assert maxrel(host(out[0, hq]), ref) <= REL_TOL, f"C2 decode hq {hq}"


def test_c3_partial_round_fused_as_timed():
    from long_context_kv_kvslimmer_amd import configs, pipeline, synth
    cfg = configs.C3
    layer = 7
    N, M = cfg.n_slots, cfg.rounds[0]
    P = O.num_pairs(N, cfg.n_sink, cfg.n_recent)
    T = N - M
    assert 0 < M < P
    print("\n[C3 fused] layer 7, N=131072, M=38011", flush=True)
    K, V, _ = pipeline.config_cache(cfg, layer, DEV)
    Qw = torch.stack([synth.window_queries(cfg, layer, 0, 0, DEV)])
    f16 = _fused(K, V, None, Qw, cfg, M, N, torch.bfloat16)
    s16 = _separate(K, V, None, Qw, cfg, M, N, torch.bfloat16)
    torch.cuda.synchronize()
    _same_round(f16, s16, P, T)
    del s16
    f32 = _fused(K, V, None, Qw, cfg, M, N, torch.float32)
    torch.cuda.synchronize()
    _same(f16.K[:, :, :T], f32.K[:, :, :T].to(torch.bfloat16), "bf16 K' = RNE(fp32 K')")
    _same(f16.src[:, :, :T], f32.src[:, :, :T], "src")
    print("[C3 fused] oracle head 2", flush=True)
    check_round_slice(f32, K, V, None, Qw, 0, 2, N, cfg.n_sink, cfg.n_recent, M, 1 / math.sqrt(cfg.head_dim),
                      label="C3 fused h2", with_cos=False)


def test_c5_second_round_with_counts_fused():
    from long_context_kv_kvslimmer_amd import configs, pipeline, synth
    cfg = configs.C5
    layer = 3
    print("\n[C5 fused] layer 3, round 1 then round 2 (counts 2)", flush=True)
    K, V, _ = pipeline.config_cache(cfg, layer, DEV)
    N1, M1 = cfg.n_slots, cfg.rounds[0]
    Qw1 = torch.stack([synth.window_queries(cfg, layer, 0, 0, DEV)])
    r1 = _fused(K, V, None, Qw1, cfg, M1, N1, torch.bfloat16)
    N2, M2 = N1 - M1, cfg.rounds[1]
    P2 = O.num_pairs(N2, cfg.n_sink, cfg.n_recent)
    T2 = N2 - M2
    Qw2 = torch.stack([synth.window_queries(cfg, layer, 0, 1, DEV)])
    f16 = _fused(r1.K, r1.V, r1.n, Qw2, cfg, M2, N2, torch.bfloat16)
    s16 = _separate(r1.K, r1.V, r1.n, Qw2, cfg, M2, N2, torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.all(r1.n[:, :, :N2] == 2)
    _same_round(f16, s16, P2, T2)
    assert torch.all(f16.n[:, :, :T2] == 4)
    del s16
    f32 = _fused(r1.K, r1.V, r1.n, Qw2, cfg, M2, N2, torch.float32)
    torch.cuda.synchronize()
    _same(f16.K[:, :, :T2], f32.K[:, :, :T2].to(torch.bfloat16), "bf16 K' = RNE(fp32 K')")
    print("[C5 fused] oracle round 2, head 6", flush=True)
    r = check_round_slice(f32, r1.K, r1.V, r1.n, Qw2, 0, 6, N2, cfg.n_sink, cfg.n_recent, M2,
                          1 / math.sqrt(cfg.head_dim), label="C5 fused r2 h6", with_cos=False)
    assert np.all(r.n == 4)
