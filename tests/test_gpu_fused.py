"""GPU: kvs_score_merge (a whole round in one call; for partial rounds the selection runs
between the scorer's passes, and the merge runs inside the second pass when the shape
allows) against kvs_score -> kvs_merge_weights -> kvs_merge_compact, bit for bit, and
against the oracle.  Shapes that the fused kernel does not take (fp32, more than 128
window queries per kv head) exercise the separate-pass path of the same call."""
import math
import zlib

import numpy as np
import pytest
import torch

from oracle import kvs_oracle as O
from tests.parity import check_round_slice
from tests.test_gpu_parity import make_inputs

pytestmark = pytest.mark.gpu

CASES = [
    # name, B, Hkv, Hq, D, N, cap, W, S, R, dtype, counts, out dtype
    ("c2-like", 1, 8, 32, 128, 4096, 4096, 32, 0, 32, torch.bfloat16, False, torch.bfloat16),
    ("odd-sinks-counts", 1, 2, 8, 128, 1001, 1001, 8, 3, 7, torch.bfloat16, True, torch.float32),
    ("d64-sinks", 1, 3, 6, 64, 1500, 1536, 4, 32, 32, torch.bfloat16, False, torch.float32),
    ("tiny-N3", 1, 1, 4, 128, 3, 3, 2, 0, 0, torch.bfloat16, False, torch.bfloat16),
    ("multi-chunk-counts", 1, 2, 8, 128, 40000, 40000, 16, 0, 32, torch.bfloat16, True, torch.bfloat16),
    ("batch2-d64", 2, 2, 4, 64, 2000, 2048, 16, 0, 0, torch.bfloat16, False, torch.bfloat16),
    ("two-pass-f32", 1, 1, 8, 128, 513, 520, 3, 1, 0, torch.float32, True, torch.float32),
    ("two-pass-gw256", 1, 1, 8, 128, 700, 700, 32, 0, 0, torch.bfloat16, False, torch.bfloat16),
]


def _same(a, b, what):
    assert torch.equal(a, b), f"{what}: {(a != b).sum().item()} elements differ"


def _compare(K, V, n, Qw, Hq, W, S, R, M, N, odt):
    from long_context_kv_kvslimmer_amd import pipeline
    P = O.num_pairs(N, S, R)
    T = N - M
    ref = pipeline.merge_round(K, V, n, Qw, Hq, W, S, R, M, n_slots=N, out_dtype=odt, want_flags=False)
    fused = pipeline.alloc_round(K, Hq, W, S, R, M, n_slots=N, out_dtype=odt)
    if M == P:
        pipeline.run_full_round_fused(K, V, n, Qw, Hq, W, S, R, fused, n_slots=N)
    else:
        pipeline.run_round_fused(K, V, n, Qw, Hq, W, S, R, M, fused, n_slots=N)
    torch.cuda.synchronize()
    _same(fused.lse, ref.lse, "lse")
    _same(fused.O, ref.O, "O")
    _same(fused.g_self, ref.g_self, "g_self")
    _same(fused.g_cross[..., :P], ref.g_cross[..., :P], "g_cross")
    _same(fused.K[:, :, :T], ref.K[:, :, :T], "K_out")
    _same(fused.V[:, :, :T], ref.V[:, :, :T], "V_out")
    _same(fused.n[:, :, :T], ref.n[:, :, :T], "n_out")
    _same(fused.src[:, :, :T], ref.src[:, :, :T], "src_out")
    return fused


@pytest.mark.parametrize("frac", [1.0, 0.29, 0.0])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_fused_round_matches_separate_calls(case, frac):
    name, B, Hkv, Hq, D, N, cap, W, S, R, dtype, counts, odt = case
    print(f"\n[fused] {name} frac {frac}", flush=True)
    K, V, n, Qw = make_inputs(zlib.crc32(name.encode()) % 10000, B, Hkv, Hq, D, N, cap, W, dtype, counts)
    M = int(round(frac * O.num_pairs(N, S, R)))
    _compare(K, V, n, Qw, Hq, W, S, R, M, N, odt)


def test_fused_partial_round_with_tie_runs():
    """Bit-identical pairs tie at the selection threshold; the cut falls inside a tie run."""
    K, V, n, Qw = make_inputs(11, 1, 2, 8, 128, 1024, 1024, 8, torch.bfloat16, True)
    for h in range(2):
        for p in range(0, 512, 3):          # every third pair: identical rows
            K[0, h, 2 * p + 1] = K[0, h, 2 * p]
    for M in (1, 100, 171, 172, 300):       # 171 pairs tie at cosine 1
        print(f"\n[fused ties] M={M}", flush=True)
        _compare(K, V, n, Qw, 8, 8, 0, 0, M, 1024, torch.bfloat16)


def test_fused_round_against_oracle():
    from long_context_kv_kvslimmer_amd import pipeline
    B, Hkv, Hq, D, N, W, S, R = 1, 2, 8, 128, 1001, 8, 3, 7
    K, V, n, Qw = make_inputs(4242, B, Hkv, Hq, D, N, N, W, torch.bfloat16, True)
    P = O.num_pairs(N, S, R)
    bufs = pipeline.alloc_round(K, Hq, W, S, R, P, n_slots=N, out_dtype=torch.float32, want_flags=False)
    pipeline.run_full_round_fused(K, V, n, Qw, Hq, W, S, R, bufs, n_slots=N)
    torch.cuda.synchronize()
    for h in range(Hkv):
        check_round_slice(bufs, K, V, n, Qw, 0, h, N, S, R, P, 1 / math.sqrt(D), label=f"fused h{h}", with_cos=False)
    # a partial round: the oracle's own selection decides the compaction it is compared with
    M = 173
    bufs = pipeline.alloc_round(K, Hq, W, S, R, M, n_slots=N, out_dtype=torch.float32, want_flags=False)
    pipeline.run_round_fused(K, V, n, Qw, Hq, W, S, R, M, bufs, n_slots=N)
    torch.cuda.synchronize()
    for h in range(Hkv):
        check_round_slice(bufs, K, V, n, Qw, 0, h, N, S, R, M, 1 / math.sqrt(D), label=f"fused partial h{h}",
                          with_cos=False)


def _random_cases(count, seed=2024):
    """Seeded shapes over the fused pass's edges: chunks of one to a few tiles, ragged
    ends, sinks and recent slots of any parity, counts on and off, every GQA ratio."""
    rs = np.random.RandomState(seed)
    out = []
    for i in range(count):
        D = int(rs.choice([64, 128]))
        Hkv = int(rs.randint(1, 4))
        G = int(rs.choice([1, 2, 4, 8]))
        W = int(rs.choice([1, 3, 8, 16, 32]))
        if G * W > 128:
            W = 128 // G
        N = int(rs.choice([5, 33, 64, 65, 97, 130, 600, 2049, 5000]))
        S = int(rs.randint(0, min(N, 40)))
        R = int(rs.randint(0, min(N - S, 40) + 1))
        frac = float(rs.choice([1.0, 0.5, 0.13, 0.0]))
        counts = bool(rs.randint(2))
        odt = torch.bfloat16 if rs.randint(2) else torch.float32
        out.append((f"rand{i}-d{D}-h{Hkv}-g{G}-w{W}-n{N}-s{S}-r{R}-f{frac}", 1 + int(rs.randint(2)), Hkv, G * Hkv, D,
                    N, W, S, R, frac, counts, odt))
    return out


RANDOM_CASES = _random_cases(24)


@pytest.mark.parametrize("case", RANDOM_CASES, ids=[c[0] for c in RANDOM_CASES])
def test_fused_random_shapes_match_separate_calls(case):
    name, B, Hkv, Hq, D, N, W, S, R, frac, counts, odt = case
    print(f"\n[fused random] {name} B={B}", flush=True)
    K, V, n, Qw = make_inputs(zlib.crc32(name.encode()) % 10000, B, Hkv, Hq, D, N, N, W, torch.bfloat16, counts)
    P = O.num_pairs(N, S, R)
    M = int(round(frac * P))
    fused = _compare(K, V, n, Qw, Hq, W, S, R, M, N, odt)
    # full and empty rounds (no selection to disagree on near a tie) also against the oracle
    if M in (0, P) and N <= 2049:
        for b, h in ((0, 0), (B - 1, Hkv - 1)):
            check_round_slice(fused, K, V, n, Qw, b, h, N, S, R, M, 1 / math.sqrt(D), label=f"{name} b{b} h{h}",
                              with_cos=False)


def test_three_query_blocks_are_deterministic():
    """384 window queries per kv head (three 128-query blocks): the pass-2 sums of the
    blocks are added in block order, so two runs give identical bits; the round (the
    fused call takes the separate-pass path here) is also checked against the oracle."""
    from long_context_kv_kvslimmer_amd import pipeline
    B, Hkv, Hq, D, N, W, S, R = 1, 2, 16, 128, 3001, 48, 2, 5
    K, V, n, Qw = make_inputs(777, B, Hkv, Hq, D, N, N, W, torch.bfloat16, True)
    P = O.num_pairs(N, S, R)
    for M in (P, 300):
        runs = []
        for _ in range(2):
            bufs = pipeline.alloc_round(K, Hq, W, S, R, M, n_slots=N, out_dtype=torch.float32, want_flags=False)
            pipeline.run_round_fused(K, V, n, Qw, Hq, W, S, R, M, bufs, n_slots=N)
            runs.append(bufs)
        torch.cuda.synchronize()
        a, b = runs
        for f in ("lse", "O", "g_self", "g_cross", "K", "V", "n", "src"):
            _same(getattr(a, f), getattr(b, f), f"run-to-run {f} (M={M})")
        for h in range(Hkv):
            check_round_slice(a, K, V, n, Qw, 0, h, N, S, R, M, 1 / math.sqrt(D), label=f"gw384 M{M} h{h}",
                              with_cos=False)


def test_layers_over_two_streams_match_one_stream():
    """pipeline.run_layers_fused: five independent layers, each a partial round then a full
    round on its output (counts 2 in the second), on one stream and alternating over two
    streams: every output of every round bit for bit the same (the rounds' oracle parity is
    checked by the tests above)."""
    from long_context_kv_kvslimmer_amd import kvslim as L
    from long_context_kv_kvslimmer_amd import pipeline
    B, Hkv, Hq, D, N, W, S, R = 1, 2, 8, 128, 2048, 16, 4, 16
    print("\n[layers] 5 layers x 2 rounds, one stream against two", flush=True)
    layers = []
    for layer in range(5):
        K, V, n, Qw = make_inputs(900 + layer, B, Hkv, Hq, D, N, N, W, torch.bfloat16, False)
        plan = []
        Ni, Ki, Vi, ni = N, K, V, None
        for r, frac in enumerate((0.3, 1.0)):
            P = L.num_pairs(Ni, S, R)
            M = int(round(frac * P))
            bufs = pipeline.alloc_round(Ki, Hq, W, S, R, M, n_slots=Ni)
            plan.append((Ki, Vi, ni, Qw, M, Ni, bufs))
            Ki, Vi, ni, Ni = bufs.K, bufs.V, bufs.n, Ni - M
        layers.append(plan)

    def snapshot():
        torch.cuda.synchronize()
        return [[(b.K[:, :, :Nr - M].clone(), b.V[:, :, :Nr - M].clone(), b.n[:, :, :Nr - M].clone(),
                  b.src[:, :, :Nr - M].clone(), b.g_self[:, :, :Nr].clone(), b.lse.clone(), b.O.clone())
                 for (_, _, _, _, M, Nr, b) in plan] for plan in layers]

    pipeline.run_layers_fused(layers, Hq, W, S, R, n_streams=1)
    one = snapshot()
    for plan in layers:   # clear every output so the second run must write them again
        for (_, _, _, _, _, _, b) in plan:
            for t in (b.K, b.V, b.n, b.src, b.g_self, b.lse, b.O):
                t.zero_()
    pipeline.run_layers_fused(layers, Hq, W, S, R, n_streams=2)
    two = snapshot()
    for li, (a_l, b_l) in enumerate(zip(one, two)):
        for r, (a_r, b_r) in enumerate(zip(a_l, b_l)):
            for name, x, y in zip(("K", "V", "n", "src", "g_self", "lse", "O"), a_r, b_r):
                _same(x, y, f"layer {li} round {r} {name}")
