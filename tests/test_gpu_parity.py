"""GPU parity: every output of the HIP path against the CPU oracle, through the C ABI.

Inputs are seeded and synthetic (AR(1) keys, iid N(0,1) values and queries); the
oracle receives host copies of the exact tensors the GPU gets.  Tolerances are
in tests/parity.py.
"""
import math
import zlib

import numpy as np
import pytest
import torch

from oracle import kvs_oracle as O
from tests.parity import REL_TOL, check_round_slice, host, maxrel

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _gen(seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return g


def make_inputs(seed, B, Hkv, Hq, D, N, cap, W, dtype, counts, rho=0.9):
    from long_context_kv_kvslimmer_amd import synth
    g = _gen(seed)
    K = torch.zeros(B, Hkv, cap, D, device=DEV, dtype=dtype)
    V = torch.zeros(B, Hkv, cap, D, device=DEV, dtype=dtype)
    for b in range(B):
        K[b, :, :N] = synth.ar1(Hkv, N, D, rho, g, DEV).to(dtype)
        V[b, :, :N] = torch.randn(Hkv, N, D, generator=g, device=DEV).to(dtype)
    n = None
    if counts:
        n = torch.randint(1, 5, (B, Hkv, cap), generator=g, device=DEV, dtype=torch.int32)
    Qw = torch.randn(B, Hq, W, D, generator=g, device=DEV).to(dtype)
    return K, V, n, Qw


CASES = [
    # name, B, Hkv, Hq, D, N, cap, W, S, R, merge fraction, dtype, counts
    ("d64-f32-g1", 1, 1, 1, 64, 300, 300, 16, 0, 0, 1.0, torch.float32, False),
    ("d128-bf16-g4-partial-counts", 2, 2, 8, 128, 777, 800, 8, 3, 5, 0.4, torch.bfloat16, True),
    ("d64-bf16-g2-sinks", 1, 3, 6, 64, 1500, 1536, 4, 32, 32, 0.7, torch.bfloat16, False),
    ("d128-f32-g8-counts", 1, 1, 8, 128, 513, 520, 3, 1, 0, 0.5, torch.float32, True),
    ("d128-bf16-none-merged", 1, 2, 8, 128, 200, 200, 4, 0, 0, 0.0, torch.bfloat16, False),
    ("d128-bf16-full-ragged", 1, 2, 8, 128, 1001, 1001, 5, 0, 7, 1.0, torch.bfloat16, True),
    ("tiny-N3", 1, 1, 4, 128, 3, 3, 2, 0, 0, 1.0, torch.bfloat16, False),
    ("no-pairs", 1, 1, 1, 64, 40, 40, 2, 32, 8, 0.0, torch.float32, False),
    ("single-slot", 1, 1, 1, 64, 1, 1, 2, 0, 0, 0.0, torch.float32, False),
    ("d64-f32-partial-g4", 1, 2, 8, 64, 4100, 4100, 8, 0, 32, 0.29, torch.float32, True),
    # 24 pass-1 splits over 256 window-query rows: the wave-per-row combine with every split in one round
    ("d64-bf16-24-splits", 1, 2, 8, 64, 24000, 24000, 32, 0, 16, 1.0, torch.bfloat16, False),
    # the largest window the calls accept: 65536 queries per head, 512 query blocks in pass 2
    ("max-window-bf16", 1, 1, 1, 64, 96, 96, 65536, 0, 0, 0.5, torch.bfloat16, False),
    ("max-window-f32-counts", 1, 1, 1, 128, 70, 72, 65536, 3, 1, 0.4, torch.float32, True),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_round_parity(case):
    from long_context_kv_kvslimmer_amd import pipeline
    name, B, Hkv, Hq, D, N, cap, W, S, R, frac, dtype, counts = case
    print(f"\n[parity] {name}", flush=True)
    K, V, n, Qw = make_inputs(zlib.crc32(name.encode()) % 10000, B, Hkv, Hq, D, N, cap, W, dtype, counts)
    P = O.num_pairs(N, S, R)
    M = int(round(frac * P))
    bufs = pipeline.merge_round(K, V, n, Qw, Hq, W, S, R, M, n_slots=N, out_dtype=torch.float32,
                                out_capacity=N - M + 3)
    torch.cuda.synchronize()
    for b in range(B):
        for h in range(Hkv):
            check_round_slice(bufs, K, V, n, Qw, b, h, N, S, R, M, 1 / math.sqrt(D), label=f"{name} b{b} h{h}")


def _random_partial_cases(count, seed=7):
    """Seeded partial rounds over small caches: the one-workgroup selection at several key
    counts per thread, sinks and recent slots of any parity, counts on and off."""
    rs = np.random.RandomState(seed)
    out = []
    for i in range(count):
        D = int(rs.choice([64, 128]))
        Hkv = int(rs.randint(1, 3))
        G = int(rs.choice([1, 2, 4]))
        W = int(rs.choice([2, 8, 16]))
        N = int(rs.choice([70, 257, 800, 1500, 3000]))
        S = int(rs.randint(0, 33))
        R = int(rs.randint(0, 33))
        frac = float(rs.choice([0.05, 0.3, 0.7, 0.95]))
        counts = bool(rs.randint(2))
        out.append((f"prand{i}-d{D}-h{Hkv}-g{G}-w{W}-n{N}-s{S}-r{R}-f{frac}", Hkv, G * Hkv, D, N, W, S, R, frac,
                    counts))
    return out


PARTIAL_RANDOM = _random_partial_cases(12)


@pytest.mark.parametrize("case", PARTIAL_RANDOM, ids=[c[0] for c in PARTIAL_RANDOM])
def test_round_parity_random_partial(case):
    """The separate calls (selection flags out) against the oracle on every slice, the
    selection bit-exact outside the tie margin."""
    from long_context_kv_kvslimmer_amd import pipeline
    name, Hkv, Hq, D, N, W, S, R, frac, counts = case
    print(f"\n[parity random] {name}", flush=True)
    K, V, n, Qw = make_inputs(zlib.crc32(name.encode()) % 10000, 1, Hkv, Hq, D, N, N, W, torch.bfloat16, counts)
    P = O.num_pairs(N, S, R)
    M = int(round(frac * P))
    bufs = pipeline.merge_round(K, V, n, Qw, Hq, W, S, R, M, n_slots=N, out_dtype=torch.float32)
    torch.cuda.synchronize()
    for h in range(Hkv):
        check_round_slice(bufs, K, V, n, Qw, 0, h, N, S, R, M, 1 / math.sqrt(D), label=f"{name} h{h}")


def test_bf16_output_is_rne_of_fp32_output_and_deterministic():
    from long_context_kv_kvslimmer_amd import pipeline
    K, V, n, Qw = make_inputs(7, 1, 2, 8, 128, 2048, 2048, 8, torch.bfloat16, True)
    P = O.num_pairs(2048, 0, 0)
    for M in (P, 700):
        a = pipeline.merge_round(K, V, n, Qw, 8, 8, 0, 0, M, out_dtype=torch.float32)
        b = pipeline.merge_round(K, V, n, Qw, 8, 8, 0, 0, M, out_dtype=torch.bfloat16)
        c = pipeline.merge_round(K, V, n, Qw, 8, 8, 0, 0, M, out_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        assert torch.equal(a.K.to(torch.bfloat16), b.K) and torch.equal(a.V.to(torch.bfloat16), b.V)
        assert torch.equal(a.n, b.n) and torch.equal(a.src, b.src)
        for x, y in ((b.K, c.K), (b.V, c.V), (b.g_self, c.g_self), (b.g_cross, c.g_cross), (b.cos, c.cos),
                     (b.lse, c.lse), (b.O, c.O)):
            assert torch.equal(x, y)


def test_selection_index_tie_break():
    """Pairs with bit-identical content tie exactly; the lower pair index wins."""
    from long_context_kv_kvslimmer_amd import pipeline
    K, V, n, Qw = make_inputs(11, 1, 1, 4, 128, 512, 512, 4, torch.bfloat16, False)
    src_pair = K[0, 0, 10:12].clone()
    tie_pairs = [5, 40, 41, 100, 200, 201, 255]
    for p in tie_pairs:
        K[0, 0, 2 * p:2 * p + 2] = src_pair
    # make the duplicated pair the most similar one: identical rows
    K[0, 0, 11] = K[0, 0, 10]
    for p in tie_pairs:
        K[0, 0, 2 * p + 1] = K[0, 0, 2 * p]
    for M in (2, 4, 6):
        bufs = pipeline.merge_round(K, V, n, Qw, 4, 4, 0, 0, M, out_dtype=torch.float32)
        torch.cuda.synchronize()
        sel = host(bufs.selected[0, 0]).astype(bool)
        ranked = sorted(set(tie_pairs))
        assert sel.sum() == M
        assert list(np.nonzero(sel)[0]) == ranked[:M]
        check_round_slice(bufs, K, V, n, Qw, 0, 0, 512, 0, 0, M, 1 / math.sqrt(128), label=f"ties M={M}")


@pytest.mark.parametrize("P", [150001, 20000, 16385, 16384, 4097, 4096, 1264, 65])
def test_selection_ties_against_brute_force(P):
    """Selection with long runs of bit-identical cosines at the threshold: the flags and the
    chunk offsets in the selection state equal a brute-force top-M with the lower index
    winning ties.  P = 150001, 20000 and 16385: many 4096-pair histogram workgroups (more
    than 1024 chunks for the first); 16384 and below: one workgroup per head, with 16 and 4
    keys per thread."""
    from long_context_kv_kvslimmer_amd import kvslim as L
    H = 3
    N = 2 * P + 1                                            # an odd leftover slot
    K = torch.empty(1, H, N, 64, dtype=torch.bfloat16, device=DEV)   # layout only; select reads cos
    rng = np.random.default_rng(7)
    cos = np.empty((H, P), np.float32)
    cos[0] = 0.875                                           # a single tie group
    cos[1] = rng.choice(np.float32([0.5, 0.625, 0.75, 0.8125, 0.875, 0.9375, 0.96875]), size=P)
    cos[2] = rng.uniform(0.6, 0.99, size=P).astype(np.float32)
    cos_t = torch.from_numpy(cos)[None].contiguous().to(DEV)
    cache = L.cache_desc(K, H)
    nch = (P + 63) // 64
    for M in sorted({m for m in (1, 512, 4097, 65537, P // 2, P - 1) if 1 <= m < P}):
        print(f"\n[select] P={P} M={M}", flush=True)
        rnd = L.round_desc(4, 0, 0, M, 0.125)
        st = torch.zeros(L.workspace_bytes(L.KVS_OP_SEL_STATE, cache, rnd), dtype=torch.uint8, device=DEV)
        selected = torch.empty(1, H, P, dtype=torch.uint8, device=DEV)
        L.kvs_merge_weights(cache, rnd, None, None, cos_t, None, selected, st)
        torch.cuda.synchronize()
        sel = host(selected)[0].astype(bool)
        sti = st.view(torch.int32).cpu().numpy()
        stride = sti.size // H
        for h in range(H):
            order = np.lexsort((np.arange(P), -cos[h].astype(np.float64)))
            ref = np.zeros(P, bool)
            ref[order[:M]] = True
            assert np.array_equal(sel[h], ref), f"flags h{h} M={M}"
            per_chunk = np.zeros(nch * 64, np.int64)
            per_chunk[:P] = ref
            excl = np.concatenate([[0], np.cumsum(per_chunk.reshape(nch, 64).sum(1))])
            offs = sti[h * stride + 4: h * stride + 4 + nch + 1]
            assert np.array_equal(offs, excl), f"offsets h{h} M={M}"


DECODE_CASES = [
    ("bf16-g4", 1, 8, 32, 128, 5000, 5100, torch.bfloat16, True),
    ("f32-g1-d64", 2, 1, 1, 64, 700, 700, torch.float32, False),
    ("bf16-g8-d64", 1, 2, 16, 64, 33, 40, torch.bfloat16, True),
    ("bf16-g2", 2, 3, 6, 128, 1, 8, torch.bfloat16, False),
    ("f32-g4", 1, 2, 8, 128, 300, 300, torch.float32, True),
    # several tiles per wave, so every ring buffer is refilled; chunks that are not whole tiles
    ("bf16-g4-long", 1, 8, 32, 128, 16400, 16400, torch.bfloat16, True),
    ("bf16-g4-d64-long", 1, 4, 16, 64, 40000, 40000, torch.bfloat16, False),
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=[c[0] for c in DECODE_CASES])
def test_decode_parity(case):
    from long_context_kv_kvslimmer_amd import pipeline
    name, B, Hkv, Hq, D, N, cap, dtype, counts = case
    print(f"\n[decode] {name}", flush=True)
    K, V, n, _ = make_inputs(zlib.crc32(name.encode()) % 1000, B, Hkv, Hq, D, N, cap, 1, dtype, counts)
    q = torch.randn(B, Hq, D, generator=_gen(3), device=DEV).to(dtype)
    out = pipeline.decode(K, V, n, q, n_slots=N)
    torch.cuda.synchronize()
    G = Hq // Hkv
    for b in range(B):
        for hq in range(Hq):
            h = hq // G
            ref = O.decode(host(K[b, h, :N]), host(V[b, h, :N]), None if n is None else host(n[b, h, :N]),
                           host(q[b, hq]), 1 / math.sqrt(D))
            assert maxrel(host(out[b, hq]), ref) <= REL_TOL, f"{name} b{b} hq{hq}"


def test_c1_config_round_and_decode():
    from long_context_kv_kvslimmer_amd import configs, pipeline, synth
    cfg = configs.C1
    K, V, last = synth.make_cache(cfg, 0, 0, DEV)
    K, V = K[None], V[None]
    Qw = synth.window_queries(cfg, 0, 0, 0, DEV)[None]
    M = cfg.rounds[0]
    bufs = pipeline.merge_round(K, V, None, Qw, cfg.q_heads, cfg.window, 0, 0, M, out_dtype=torch.float32)
    torch.cuda.synchronize()
    check_round_slice(bufs, K, V, None, Qw, 0, 0, cfg.n_slots, 0, 0, M, 1 / math.sqrt(cfg.head_dim), "C1")
    assert bufs.K.shape[2] == cfg.n_slots // 2
    q = synth.decode_query(cfg, 0, 0, 0, DEV)[None]
    out = pipeline.decode(bufs.K, bufs.V, bufs.n, q)
    torch.cuda.synchronize()
    ref = O.decode(host(bufs.K[0, 0]), host(bufs.V[0, 0]), host(bufs.n[0, 0]), host(q[0, 0]),
                   1 / math.sqrt(cfg.head_dim))
    assert maxrel(host(out[0, 0]), ref) <= REL_TOL


def test_c2_full_layer_sampled_heads():
    """Llama-3.1-8B layer at 32K, the launch configuration the benchmark times;
    two kv heads checked against the oracle, every head checked for invariants."""
    from long_context_kv_kvslimmer_amd import configs, pipeline, synth
    cfg = configs.C2
    K, V, _ = synth.make_cache(cfg, 0, 0, DEV)
    K, V = K[None], V[None]
    Qw = synth.window_queries(cfg, 0, 0, 0, DEV)[None]
    M = cfg.rounds[0]
    bufs = pipeline.merge_round(K, V, None, Qw, cfg.q_heads, cfg.window, cfg.n_sink, cfg.n_recent, M,
                                out_dtype=torch.float32)
    torch.cuda.synchronize()
    T = cfg.n_slots - M
    assert T == 16400
    nn = bufs.n.sum(dim=2)
    assert torch.all(nn == cfg.n_slots)
    src = bufs.src[0].long()
    assert torch.all(src[:, 1:] > src[:, :-1])
    for h in (0, 5):
        print(f"\n[C2] head {h}", flush=True)
        check_round_slice(bufs, K, V, None, Qw, 0, h, cfg.n_slots, cfg.n_sink, cfg.n_recent, M,
                          1 / math.sqrt(cfg.head_dim), label=f"C2 h{h}")


@pytest.mark.parametrize("vscale", [3000.0, 1e-4])
def test_value_range_of_the_f16_output_product(vscale):
    """The first scorer pass forms O from f16 probabilities and f16 values: values scaled
    up toward f16's largest normal and down into its subnormal range still give a round
    within the usual tolerance of the oracle (full and partial rounds, counts on)."""
    from long_context_kv_kvslimmer_amd import pipeline
    B, Hkv, Hq, D, N, W, S, R = 1, 2, 8, 128, 1200, 16, 2, 6
    K, V, n, Qw = make_inputs(5150, B, Hkv, Hq, D, N, N, W, torch.bfloat16, True)
    V = (V.float() * vscale).clamp(-60000.0, 60000.0).to(torch.bfloat16)
    print(f"\n[f16 range] scale {vscale}, max |V| {V.float().abs().max().item():.3g}", flush=True)
    P = O.num_pairs(N, S, R)
    for M in (P, 150):
        bufs = pipeline.merge_round(K, V, n, Qw, Hq, W, S, R, M, n_slots=N, out_dtype=torch.float32)
        torch.cuda.synchronize()
        for h in range(Hkv):
            check_round_slice(bufs, K, V, n, Qw, 0, h, N, S, R, M, 1 / math.sqrt(D), label=f"x{vscale} M{M} h{h}")
