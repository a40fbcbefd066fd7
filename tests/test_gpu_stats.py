"""GPU: kvs_score_merge_stats, a whole round given the window statistics (lse, O) that
the prefill attention already computed.  Given the statistics kvs_score_merge computes
itself, every output must equal kvs_score_merge's bit for bit (full, partial and empty
rounds; the fused shapes and the separate-pass shapes); given the oracle's statistics,
the outputs must match the oracle's round on those statistics."""
import math
import zlib

import numpy as np
import pytest
import torch

from oracle import kvs_oracle as O
from tests.parity import REL_TOL, elemrel, host, maxrel
from tests.test_gpu_fused import CASES, RANDOM_CASES
from tests.test_gpu_parity import make_inputs

pytestmark = pytest.mark.gpu


def _same(a, b, what):
    assert torch.equal(a, b), f"{what}: {(a != b).sum().item()} elements differ"


@pytest.mark.parametrize("frac", [1.0, 0.29, 0.0])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_given_stats_match_score_merge(case, frac):
    from long_context_kv_kvslimmer_amd import pipeline
    name, B, Hkv, Hq, D, N, cap, W, S, R, dtype, counts, odt = case
    print(f"\n[stats] {name} frac {frac}", flush=True)
    K, V, n, Qw = make_inputs(zlib.crc32(name.encode()) % 10000, B, Hkv, Hq, D, N, cap, W, dtype, counts)
    P = O.num_pairs(N, S, R)
    M = int(round(frac * P))
    T = N - M
    ref = pipeline.alloc_round(K, Hq, W, S, R, M, n_slots=N, out_dtype=odt)
    pipeline.run_round_fused(K, V, n, Qw, Hq, W, S, R, M, ref, n_slots=N)
    got = pipeline.alloc_round(K, Hq, W, S, R, M, n_slots=N, out_dtype=odt)
    pipeline.run_round_given_stats(K, V, n, Qw, ref.lse, ref.O, Hq, W, S, R, M, got, n_slots=N)
    torch.cuda.synchronize()
    _compare_outputs(got, ref, P, T)


def _compare_outputs(got, ref, P, T):
    _same(got.g_self, ref.g_self, "g_self")
    _same(got.g_cross[..., :P], ref.g_cross[..., :P], "g_cross")
    _same(got.K[:, :, :T], ref.K[:, :, :T], "K_out")
    _same(got.V[:, :, :T], ref.V[:, :, :T], "V_out")
    _same(got.n[:, :, :T], ref.n[:, :, :T], "n_out")
    _same(got.src[:, :, :T], ref.src[:, :, :T], "src_out")


@pytest.mark.parametrize("case", RANDOM_CASES, ids=[c[0] for c in RANDOM_CASES])
def test_given_stats_random_shapes(case):
    """The seeded random shapes of the fused-call tests, through the given-statistics call."""
    from long_context_kv_kvslimmer_amd import pipeline
    name, B, Hkv, Hq, D, N, W, S, R, frac, counts, odt = case
    print(f"\n[stats random] {name} B={B}", flush=True)
    K, V, n, Qw = make_inputs(zlib.crc32(name.encode()) % 10000, B, Hkv, Hq, D, N, N, W, torch.bfloat16, counts)
    P = O.num_pairs(N, S, R)
    M = int(round(frac * P))
    ref = pipeline.alloc_round(K, Hq, W, S, R, M, n_slots=N, out_dtype=odt)
    pipeline.run_round_fused(K, V, n, Qw, Hq, W, S, R, M, ref, n_slots=N)
    got = pipeline.alloc_round(K, Hq, W, S, R, M, n_slots=N, out_dtype=odt)
    pipeline.run_round_given_stats(K, V, n, Qw, ref.lse, ref.O, Hq, W, S, R, M, got, n_slots=N)
    torch.cuda.synchronize()
    _compare_outputs(got, ref, P, N - M)


@pytest.mark.parametrize("frac", [1.0, 0.35])
def test_given_stats_against_oracle(frac):
    """The oracle's own statistics (rounded to fp32) go to both sides."""
    from long_context_kv_kvslimmer_amd import pipeline
    B, Hkv, Hq, D, N, W, S, R = 1, 2, 8, 128, 1001, 8, 3, 7
    G = Hq // Hkv
    K, V, n, Qw = make_inputs(777, B, Hkv, Hq, D, N, N, W, torch.bfloat16, True)
    P = O.num_pairs(N, S, R)
    M = int(round(frac * P))
    scale = 1 / math.sqrt(D)
    lse = torch.empty(B, Hq, W, dtype=torch.float32)
    Ow = torch.empty(B, Hq, W, D, dtype=torch.float32)
    sl = []
    for h in range(Hkv):
        Ks, Vs, ns = host(K[0, h]), host(V[0, h]), host(n[0, h]).astype(np.int64)
        Qs = host(Qw[0, h * G:(h + 1) * G]).reshape(-1, D)
        l, _, o = O.window_statistics(Ks, Vs, ns, Qs, scale)
        lse[0, h * G:(h + 1) * G] = torch.from_numpy(l.reshape(G, W)).float()
        Ow[0, h * G:(h + 1) * G] = torch.from_numpy(o.reshape(G, W, D)).float()
        sl.append((Ks, Vs, ns, Qs))
    bufs = pipeline.alloc_round(K, Hq, W, S, R, M, n_slots=N, out_dtype=torch.float32)
    pipeline.run_round_given_stats(K, V, n, Qw, lse.cuda(), Ow.cuda(), Hq, W, S, R, M, bufs, n_slots=N)
    torch.cuda.synchronize()
    T = N - M
    for h in range(Hkv):
        Ks, Vs, ns, Qs = sl[h]
        r = O.merge_round_given_stats(Ks, Vs, ns, Qs, host(lse[0, h * G:(h + 1) * G]).reshape(-1),
                                      host(Ow[0, h * G:(h + 1) * G]).reshape(-1, D), scale, S, R, M)
        assert elemrel(host(bufs.g_self[0, h]), r.g_self) <= REL_TOL, f"g_self h{h}"
        assert elemrel(host(bufs.g_cross[0, h, :P]), r.g_cross) <= REL_TOL, f"g_cross h{h}"
        assert np.array_equal(host(bufs.src[0, h, :T]).astype(np.int64), r.src), f"src h{h}"
        assert np.array_equal(host(bufs.n[0, h, :T]).astype(np.int64), r.n), f"n h{h}"
        assert maxrel(host(bufs.K[0, h, :T]), r.K) <= REL_TOL, f"K' h{h}"
        assert maxrel(host(bufs.V[0, h, :T]), r.V) <= REL_TOL, f"V' h{h}"
