"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks an oracle function against something that is not the oracle
itself: finite differences, brute-force minimisation, library routines,
closed forms, exact invariants, or numbers the pages print (tests/golden/).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import kvs_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


# ----------------------------------------------------------------- spectral --
def test_spectral_identity_random_w():
    """Σ_i c_i equals the cosine of the projected vectors (Eq. 8 identity)."""
    rng = _rng(1)
    for trial in range(20):
        W = rng.standard_normal((16, 8))
        x_t, x_t1 = rng.standard_normal(16), rng.standard_normal(16)
        c = O.spectral_mode_contributions(x_t, x_t1, W)
        y_t, y_t1 = x_t @ W, x_t1 @ W
        direct = float(y_t @ y_t1) / (np.linalg.norm(y_t) * np.linalg.norm(y_t1))
        assert abs(c.sum() - direct) < 1e-12
        assert abs(c.sum() - O.cosine(y_t, y_t1)) < 1e-12


def test_spectral_concentration_makes_neighbours_similar():
    """A rank-1-dominated W maps any two inputs to nearly parallel outputs."""
    rng = _rng(2)
    u = rng.standard_normal((16, 1))
    v = rng.standard_normal((1, 8))
    W = 10.0 * u @ v + 1e-3 * rng.standard_normal((16, 8))
    x_t, x_t1 = rng.standard_normal(16), rng.standard_normal(16)
    c = O.spectral_mode_contributions(x_t, x_t1, W)
    assert abs(abs(c.sum()) - 1.0) < 1e-3
    assert abs(abs(c[np.argmax(np.abs(c))]) - 1.0) < 1e-3   # one dominant mode


def test_cosine_special_cases():
    a = np.array([1.0, 2.0, -3.0])
    assert abs(O.cosine(a, a) - 1.0) < 1e-15
    assert abs(O.cosine(a, -2.5 * a) + 1.0) < 1e-15
    assert abs(O.cosine(np.array([1.0, 0.0]), np.array([0.0, 3.0]))) < 1e-15
    z = np.zeros(3)
    assert O.cosine(z, z) == 1.0
    assert O.cosine(z, a) == 0.0
    assert abs(O.cosine(a, 7.0 * a) - 1.0) < 1e-15


# ---------------------------------------------------------------- attention --
def test_attention_matches_torch_sdpa():
    rng = _rng(3)
    N, D = 37, 8
    K, V, q = rng.standard_normal((N, D)), rng.standard_normal((N, D)), rng.standard_normal(D)
    scale = 1 / math.sqrt(D)
    _, alpha, o = O.attention_forward(K, V, q, scale)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(q)[None, None, None], torch.tensor(K)[None, None], torch.tensor(V)[None, None])
    assert np.max(np.abs(o - ref[0, 0, 0].numpy())) < 1e-12
    assert abs(alpha.sum() - 1.0) < 1e-14


def test_attention_with_counts_equals_repeated_slots():
    """+ln n on a slot is the same as repeating that slot n times (reading O1)."""
    rng = _rng(4)
    N, D = 11, 6
    K, V, q = rng.standard_normal((N, D)), rng.standard_normal((N, D)), rng.standard_normal(D)
    n = rng.integers(1, 5, N)
    scale = 0.4
    _, _, o = O.attention_forward(K, V, q, scale, n)
    Kx = np.repeat(K, n, axis=0)
    Vx = np.repeat(V, n, axis=0)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(q)[None, None, None], torch.tensor(Kx)[None, None], torch.tensor(Vx)[None, None],
        scale=scale)
    assert np.max(np.abs(o - ref[0, 0, 0].numpy())) < 1e-12


def test_window_lse_matches_scipy_logsumexp():
    from scipy.special import logsumexp
    rng = _rng(5)
    N, D, GW = 50, 8, 6
    K, V, Q = rng.standard_normal((N, D)), rng.standard_normal((N, D)), rng.standard_normal((GW, D))
    n = rng.integers(1, 4, N)
    lse, alpha, Ow = O.window_statistics(K, V, n, Q, 0.3)
    for w in range(GW):
        assert abs(lse[w] - logsumexp(0.3 * (K @ Q[w]) + np.log(n))) < 1e-12
    assert np.allclose(alpha.sum(1), 1.0, atol=1e-14)


def test_softmax_jacobian_bound():
    """‖softmax(a) − softmax(b)‖₂ ≤ ½ ‖a − b‖₂ (KV-CoRE notes, §9.1)."""
    rng = _rng(6)
    K = np.eye(12)
    V = np.zeros((12, 1))
    for _ in range(200):
        a, b = 3 * rng.standard_normal(12), 3 * rng.standard_normal(12)
        _, pa, _ = O.attention_forward(K, V, a, 1.0)
        _, pb, _ = O.attention_forward(K, V, b, 1.0)
        assert np.linalg.norm(pa - pb) <= 0.5 * np.linalg.norm(a - b) + 1e-15


# --------------------------------------------------- gradient and Hessian --
def _loss(K, V, q, E, scale):
    _, _, o = O.attention_forward(K, V, q, scale)
    return float(E @ o)


def _setup(seed, N=7, D=4):
    rng = _rng(seed)
    K, V = rng.standard_normal((N, D)), rng.standard_normal((N, D))
    q, E = rng.standard_normal(D), rng.standard_normal(D)
    return K, V, q, E, 1 / math.sqrt(D)


def test_key_gradient_finite_difference():
    K, V, q, E, s = _setup(7)
    _, alpha, o = O.attention_forward(K, V, q, s)
    h = 1e-6
    for i in range(K.shape[0]):
        fd = np.zeros(K.shape[1])
        for a in range(K.shape[1]):
            Kp, Km = K.copy(), K.copy()
            Kp[i, a] += h
            Km[i, a] -= h
            fd[a] = (_loss(Kp, V, q, E, s) - _loss(Km, V, q, E, s)) / (2 * h)
        assert np.max(np.abs(fd - O.key_gradient(alpha, V, o, q, E, i, s))) < 1e-8


def _fd_hessian_block(K, V, q, E, s, i, j, h=1e-4):
    D = K.shape[1]
    H = np.zeros((D, D))
    for a in range(D):
        for b in range(D):
            def L(da, db):
                Kx = K.copy()
                Kx[i, a] += da
                Kx[j, b] += db
                return _loss(Kx, V, q, E, s)
            H[a, b] = (L(h, h) - L(h, -h) - L(-h, h) + L(-h, -h)) / (4 * h * h)
    return H


@pytest.mark.parametrize("i,j", [(2, 2), (2, 3), (3, 2), (0, 5), (6, 6)])
def test_hessian_blocks_finite_difference(i, j):
    """Exact Hessian blocks (1/d_k)[Eᵀ ∂s_i/∂e_j] q qᵀ against a 4-point FD of L."""
    K, V, q, E, s = _setup(8)
    _, alpha, o = O.attention_forward(K, V, q, s)
    fd = _fd_hessian_block(K, V, q, E, s, i, j)
    assert np.max(np.abs(fd - O.hessian_block(alpha, V, o, q, E, i, j, s))) < 1e-6


def test_c_vectors_are_the_pair_hessian_scalars():
    """c11, c22, c12 give h_mm, h_{m+1,m+1}, h_{m,m+1} (checked by FD), incl. c12's sign."""
    K, V, q, E, s = _setup(9)
    _, alpha, o = O.attention_forward(K, V, q, s)
    m = 3
    c11, c22, c12 = O.c_vectors(alpha, V, o, m)
    qq = s * s * np.outer(q, q)
    for c, (i, j) in ((c11, (m, m)), (c22, (m + 1, m + 1)), (c12, (m, m + 1))):
        fd = _fd_hessian_block(K, V, q, E, s, i, j)
        assert np.max(np.abs(fd - float(E @ c) * qq)) < 1e-6


def test_hessian_norm_sums_equal_literal_c_vector_norms():
    rng = _rng(10)
    N, D, GW, S = 13, 5, 4, 1
    K, V, Q = rng.standard_normal((N, D)), rng.standard_normal((N, D)), rng.standard_normal((GW, D))
    n = rng.integers(1, 3, N)
    P = O.num_pairs(N, S, 2)
    lse, alpha, Ow = O.window_statistics(K, V, n, Q, 0.5)
    g_self, g_cross = O.hessian_norm_sums(V, alpha, Ow, S, P)
    for p in range(P):
        m = S + 2 * p
        s11 = s22 = s12 = 0.0
        for w in range(GW):
            c11, c22, c12 = O.c_vectors(alpha[w], V, Ow[w], m)
            s11 += np.linalg.norm(c11)
            s22 += np.linalg.norm(c22)
            s12 += np.linalg.norm(c12)
        assert abs(g_self[m] - s11) < 1e-13
        assert abs(g_self[m + 1] - s22) < 1e-13
        assert abs(g_cross[p] - s12) < 1e-13


# --------------------------------------------------------- merge weights --
def test_hessian_weights_minimise_objective_brute_force():
    from scipy.optimize import minimize
    rng = _rng(11)
    for _ in range(10):
        D = 5
        k_m, k_m1 = rng.standard_normal(D), rng.standard_normal(D)
        g11, g22 = rng.uniform(0.5, 2.0, 2)
        g12 = rng.uniform(-0.4, 0.4)
        w0, w1 = O.hessian_weights(g11, g12, g22)
        k_star = w0 * k_m + w1 * k_m1
        res = minimize(lambda k: O.merge_objective(k, k_m, k_m1, g11, g12, g22),
                       rng.standard_normal(D), method="BFGS", options={"gtol": 1e-11})
        assert np.max(np.abs(res.x - k_star)) < 1e-5
        # central-difference gradient vanishes at k*
        h = 1e-6
        grad = [(O.merge_objective(k_star + h * e, k_m, k_m1, g11, g12, g22)
                 - O.merge_objective(k_star - h * e, k_m, k_m1, g11, g12, g22)) / (2 * h)
                for e in np.eye(D)]
        assert np.max(np.abs(grad)) < 1e-6
        assert abs(w0 + w1 - 1.0) < 1e-14


def test_forward_only_weights_minimise_objective_with_signed_norms():
    """With ĝ = (‖c11‖, −‖c12‖, ‖c22‖) the forward-only k* is the brute-force minimiser."""
    from scipy.optimize import minimize
    rng = _rng(12)
    N, D, GW = 9, 4, 3
    K, V, Q = rng.standard_normal((N, D)), rng.standard_normal((N, D)), rng.standard_normal((GW, D))
    _, alpha, Ow = O.window_statistics(K, V, None, Q, 0.5)
    g_self, g_cross = O.hessian_norm_sums(V, alpha, Ow, 0, O.num_pairs(N, 0, 0))
    for p in range(O.num_pairs(N, 0, 0)):
        m = 2 * p
        n11, n12, n22 = g_self[m], g_cross[p], g_self[m + 1]
        w0, w1, fb = O.forward_only_weights(n11, n12, n22)
        assert not fb
        k_star = w0 * K[m] + w1 * K[m + 1]
        res = minimize(lambda k: O.merge_objective(k, K[m], K[m + 1], n11, -n12, n22),
                       np.zeros(D), method="BFGS", options={"gtol": 1e-12})
        assert np.max(np.abs(res.x - k_star)) < 1e-5


def test_weight_special_cases():
    # no coupling: weights proportional to the self terms
    w0, w1, fb = O.forward_only_weights(3.0, 0.0, 1.0)
    assert (abs(w0 - 0.75) < 1e-15, abs(w1 - 0.25) < 1e-15, fb) == (True, True, False)
    # symmetric pair: plain average
    w0, w1, fb = O.forward_only_weights(2.0, 0.3, 2.0)
    assert abs(w0 - 0.5) < 1e-15 and abs(w1 - 0.5) < 1e-15 and not fb
    # degenerate denominator: fallback to the plain average
    assert O.forward_only_weights(1.0, 1.0, 1.0) == (0.5, 0.5, True)
    assert O.forward_only_weights(0.0, 0.0, 0.0) == (0.5, 0.5, True)
    assert O.forward_only_weights(float("nan"), 0.0, 1.0) == (0.5, 0.5, True)
    # sums to one whenever defined
    rng = _rng(13)
    for _ in range(100):
        a, b, c = rng.uniform(0, 1, 3)
        w0, w1, _ = O.forward_only_weights(a, b, c)
        assert abs(w0 + w1 - 1.0) < 1e-12


# -------------------------------------------------------------- selection --
def _brute_select(cos, M):
    P = len(cos)
    sel = np.zeros(P, bool)
    for p in range(P):
        better = sum(1 for q in range(P) if cos[q] > cos[p] or (cos[q] == cos[p] and q < p))
        sel[p] = better < M
    return sel


def test_select_pairs_brute_force_and_ties():
    rng = _rng(14)
    for _ in range(50):
        P = int(rng.integers(1, 12))
        cos = np.round(rng.uniform(-1, 1, P), 1)    # many exact ties
        for M in range(P + 1):
            assert np.array_equal(O.select_pairs(cos, M), _brute_select(cos, M))
    # crafted ties: equal pairs go to the lower index
    assert O.select_pairs(np.array([0.5, 0.9, 0.9, 0.9, 0.1]), 2).tolist() == [False, True, True, False, False]
    with pytest.raises(ValueError):
        O.select_pairs(np.zeros(3), 4)


def test_num_pairs():
    assert O.num_pairs(512, 0, 0) == 256
    assert O.num_pairs(32768, 0, 32) == 16368
    assert O.num_pairs(33, 32, 0) == 0
    assert O.num_pairs(10, 3, 2) == 2
    assert O.num_pairs(4, 3, 3) == 0


# ------------------------------------------------------------ merge round --
def _random_slice(seed, N=40, D=6, GW=5, counts=True):
    rng = _rng(seed)
    K = rng.standard_normal((N, D))
    V = rng.standard_normal((N, D))
    Q = rng.standard_normal((GW, D))
    n = rng.integers(1, 4, N) if counts else None
    return K, V, n, Q


@pytest.mark.parametrize("S,R,frac", [(0, 0, 1.0), (3, 5, 0.5), (2, 0, 0.0), (1, 1, 0.3)])
def test_merge_round_invariants(S, R, frac):
    K, V, n, Q = _random_slice(15 + S)
    N = K.shape[0]
    P = O.num_pairs(N, S, R)
    M = int(round(frac * P))
    r = O.merge_round(K, V, n, Q, 0.4, S, R, M)
    T = N - M
    assert r.K.shape == (T, K.shape[1]) and len(r.n) == T and len(r.src) == T
    assert np.all(np.diff(r.src) > 0)
    assert r.n.sum() == n.sum()                                    # Σ n conserved
    assert np.allclose((r.n[:, None] * r.V).sum(0), (n[:, None] * V).sum(0), atol=1e-12)
    assert r.selected.sum() == M
    # untouched slots are copied exactly; merged slots are the weighted keys
    for j, i in enumerate(r.src):
        p = (i - S) // 2
        if i >= S and (i - S) % 2 == 0 and p < P and r.selected[p]:
            assert np.allclose(r.K[j], r.w[p, 0] * K[i] + r.w[p, 1] * K[i + 1], atol=1e-14)
            assert r.n[j] == n[i] + n[i + 1]
        else:
            assert np.array_equal(r.K[j], K[i]) and np.array_equal(r.V[j], V[i]) and r.n[j] == n[i]
    # sinks and recent window are never merged
    assert np.array_equal(r.src[:S], np.arange(S))
    assert np.array_equal(r.src[T - R:], np.arange(N - R, N)) if R else True


def test_identical_adjacent_keys_merge_to_themselves():
    rng = _rng(16)
    N, D, GW = 16, 5, 3
    base = rng.standard_normal((N // 2, D))
    K = np.repeat(base, 2, axis=0)                 # k_{2p} == k_{2p+1}
    V = rng.standard_normal((N, D))
    Q = rng.standard_normal((GW, D))
    r = O.merge_round(K, V, None, Q, 0.5, 0, 0, N // 2)
    assert np.allclose(r.cos, 1.0, atol=1e-15)
    assert np.allclose(r.K, base, atol=1e-12)
    for p in range(N // 2):
        g11, g12, g22 = r.g_self[2 * p], -r.g_cross[p], r.g_self[2 * p + 1]
        assert abs(O.merge_objective(r.K[p], K[2 * p], K[2 * p + 1], g11, g12, g22)) < 1e-20
    # the merge is lossless here: decode outputs are unchanged
    for _ in range(5):
        q = rng.standard_normal(D)
        assert np.max(np.abs(O.decode(r.K, r.V, r.n, q, 0.5) - O.decode(K, V, None, q, 0.5))) < 1e-13


def test_value_merge_is_lossless_given_merged_keys():
    """Merged cache == expanded cache in which both positions carry k* and their own values."""
    K, V, n, Q = _random_slice(17, counts=True)
    N, D = K.shape
    r = O.merge_round(K, V, n, Q, 0.4, 2, 2, 12)
    Kx, Vx, nx = K.copy(), V.copy(), n.copy()
    for j, i in enumerate(r.src):
        p = (i - 2) // 2
        if i >= 2 and (i - 2) % 2 == 0 and p < len(r.selected) and r.selected[p]:
            Kx[i] = Kx[i + 1] = r.K[j]
    rng = _rng(18)
    for _ in range(10):
        q = 2 * rng.standard_normal(D)
        merged = O.decode(r.K, r.V, r.n, q, 0.4)
        expanded = O.decode(Kx, Vx, nx, q, 0.4)
        assert np.max(np.abs(merged - expanded)) < 1e-13


def test_handworked_round_golden():
    g = json.load(open(os.path.join(GOLDEN, "handworked_round.json")))
    K, V, Q = np.array(g["K"]), np.array(g["V"]), np.array(g["Qw"])
    ex = g["expected"]
    for M, key in ((1, "merge_1"), (2, "merge_2")):
        r = O.merge_round(K, V, None, Q, g["scale"], g["n_sink"], g["n_recent"], M)
        assert np.allclose(r.lse, ex["lse"], atol=1e-15)
        assert np.allclose(r.O, ex["O"], atol=1e-15)
        assert np.allclose(r.g_self, ex["g_self"], atol=1e-15)
        assert np.allclose(r.g_cross, ex["g_cross"], atol=1e-15)
        assert np.allclose(r.cos, ex["cos"], atol=1e-15)
        assert np.allclose(r.w, ex["w"], atol=1e-15)
        assert r.fallback.tolist() == ex["fallback"]
        e = ex[key]
        assert r.selected.tolist() == e["selected"]
        assert np.allclose(r.K, e["K"]) and np.allclose(r.V, e["V"])
        assert r.n.tolist() == e["n"] and r.src.tolist() == e["src"]


def test_three_rounds_reach_eight_fold_ratio():
    """Token count after three full 2x rounds is N/8 and src composes to the first slots."""
    K, V, _, Q = _random_slice(19, N=64, counts=False)
    n = None
    src = np.arange(64)
    for rnd in range(3):
        N = K.shape[0]
        r = O.merge_round(K, V, n, Q, 0.4, 0, 0, O.num_pairs(N, 0, 0))
        K, V, n = r.K, r.V, r.n
        src = O.compose_src(src, r.src)
    assert K.shape[0] == 8 and np.array_equal(n, np.full(8, 8))
    assert np.array_equal(src, np.arange(0, 64, 8))


def test_kv_bytes_golden():
    g = json.load(open(os.path.join(GOLDEN, "kv_bytes.json")))
    s = g["shape"]
    bpt = O.kv_bytes_per_token(s["layers"], s["kv_heads"], s["head_dim"], s["dtype_bytes"])
    assert bpt == g["bytes_per_token"]
    for ctx, gib in g["per_request_gib_approx"].items():
        assert round(bpt * int(ctx) / 2**30) == gib
    assert round(8 * 32768 * bpt / 2**30) == g["batch8_32k_gib_approx"]


# ------------------------------------------------------ chunked budget loop --
def _stream_inputs(seed, total, D, GW, chunk, rho=0.9):
    """AR(1) keys (similar neighbours), iid values, one window per chunk."""
    rng = _rng(seed)
    K = np.empty((total, D))
    K[0] = rng.standard_normal(D)
    for t in range(1, total):
        K[t] = rho * K[t - 1] + math.sqrt(1 - rho * rho) * rng.standard_normal(D)
    V = rng.standard_normal((total, D))
    Qs = [rng.standard_normal((GW, D)) for _ in range(-(-total // chunk))]
    return K, V, Qs


def test_stream_under_budget_copies_the_tokens():
    K, V, Qs = _stream_inputs(30, 90, 5, 3, 32)
    s = O.stream_prefill(K, V, Qs, 0.4, 4, 90, 32)
    assert s.rounds == []
    assert np.array_equal(s.K, K) and np.array_equal(s.V, V)
    assert np.array_equal(s.n, np.ones(90)) and np.array_equal(s.start, np.arange(90))


def test_stream_single_chunk_is_one_merge_round():
    K, V, Qs = _stream_inputs(31, 100, 5, 3, 100)
    s = O.stream_prefill(K, V, Qs, 0.4, 4, 60, 100)
    r = O.merge_round(K, V, None, Qs[0], 0.4, 4, 0, 40)
    assert len(s.rounds) == 1 and s.rounds[0][1:3] == (100, 40)
    assert np.allclose(s.K, r.K, atol=1e-14) and np.allclose(s.V, r.V, atol=1e-14)
    assert np.array_equal(s.n, r.n) and np.array_equal(s.start, r.src)


def test_stream_round_window_is_its_chunks_queries():
    """The first round runs on raw tokens only: its lse must be the log-sum-exp of the
    logits of the queries of the chunk that triggered it, over every slot held."""
    from scipy.special import logsumexp
    K, V, Qs = _stream_inputs(33, 160, 6, 3, 40)
    s = O.stream_prefill(K, V, Qs, 0.35, 2, 100, 40)
    c, N, M, r = s.rounds[0]
    assert (c, N, M) == (2, 120, 20)
    for w in range(3):
        assert abs(r.lse[w] - logsumexp(0.35 * K[:N] @ Qs[c][w])) < 1e-12


@pytest.mark.parametrize("total,budget,chunk,S", [(300, 64, 32, 4), (301, 64, 50, 0), (257, 40, 100, 8),
                                                  (200, 17, 16, 16)])
def test_stream_invariants(total, budget, chunk, S):
    D = 12
    K, V, Qs = _stream_inputs(32 + total, total, D, 4, chunk)
    s = O.stream_prefill(K, V, Qs, 0.3, S, budget, chunk)
    assert len(s.n) == min(total, budget)
    # rounds merge at most the excess over the budget, and the last round of a chunk
    # lands exactly on the budget; the cache never holds more than budget + chunk slots
    last = {}
    for c, N, M, r in s.rounds:
        assert 1 <= M <= min(N - budget, O.num_pairs(N, S, 0))
        assert len(r.n) == N - M and N <= budget + chunk
        last[c] = N - M
    assert all(v == budget for v in last.values())
    assert s.n.sum() == total
    # slots tile the token sequence in order
    assert np.array_equal(s.start, np.concatenate([[0], np.cumsum(s.n)[:-1]]))
    # the first tokens are kept verbatim
    assert np.array_equal(s.K[:S], K[:S]) and np.array_equal(s.V[:S], V[:S]) and np.all(s.n[:S] == 1)
    for j in range(len(s.n)):
        a, m = s.start[j], s.n[j]
        # lossless values: every slot holds the mean of the raw values it covers
        assert np.allclose(s.V[j], V[a:a + m].mean(axis=0), atol=1e-12)
        # merged keys are affine combinations of the raw keys they cover
        if m == 1:
            assert np.array_equal(s.K[j], K[a])
        elif m <= D - 1:
            X = (K[a + 1:a + m] - K[a]).T
            y = s.K[j] - K[a]
            coef = np.linalg.lstsq(X, y, rcond=None)[0]
            assert np.linalg.norm(X @ coef - y) < 1e-9 * (1 + np.linalg.norm(s.K[j]))


def test_stream_rejects_budget_not_above_sinks():
    K, V, Qs = _stream_inputs(34, 20, 4, 2, 8)
    with pytest.raises(ValueError):
        O.stream_prefill(K, V, Qs, 0.3, 8, 8, 8)


# ------------------------------------------------- round given the statistics --
def test_given_stats_equal_computed_stats():
    """Supplying the statistics the window attention computes reproduces the round."""
    K, V, n, Q = _random_slice(40, counts=True)
    for S, R, M in ((0, 0, 20), (2, 3, 7), (1, 0, 0)):
        ref = O.merge_round(K, V, n, Q, 0.4, S, R, M)
        r = O.merge_round_given_stats(K, V, n, Q, ref.lse, ref.O, 0.4, S, R, M)
        assert np.allclose(r.g_self, ref.g_self, rtol=1e-13, atol=0)
        assert np.allclose(r.g_cross, ref.g_cross, rtol=1e-13, atol=0)
        assert np.array_equal(r.selected, ref.selected) and np.array_equal(r.src, ref.src)
        assert np.allclose(r.K, ref.K, atol=1e-13) and np.array_equal(r.n, ref.n)


def test_given_stats_handworked():
    """N = 4 one-dimensional slots, one zero query: alpha = 1/4 for every slot whatever the
    keys, lse = ln 4.  With a supplied O = 10 (not the attention output 2.5), by hand:
    g_self[i] = 1/4 |1 - 1/2| |v_i - 10| = (9, 8, 7, 6) / 8 and
    g_cross[p] = 1/16 |v_m + v_{m+1} - 20| = (17, 13) / 16."""
    K = np.array([[0.3], [-1.2], [2.0], [0.7]])
    V = np.array([[1.0], [2.0], [3.0], [4.0]])
    Q = np.zeros((1, 1))
    r = O.merge_round_given_stats(K, V, None, Q, [math.log(4.0)], [[10.0]], 0.5, 0, 0, 1)
    assert np.allclose(r.g_self, [9 / 8, 8 / 8, 7 / 8, 6 / 8], rtol=1e-15)
    assert np.allclose(r.g_cross, [17 / 16, 13 / 16], rtol=1e-15)


# --------------------------------------------------- exact-gradient diagnostics --
def test_exact_scalars_are_the_hessian_blocks():
    """One window query: g_ij q qᵀ / d_k is the exact Hessian block (pinned by finite
    differences above), for the diagonal blocks and the cross block of every pair."""
    rng = _rng(50)
    N, D = 8, 5
    K, V = rng.standard_normal((N, D)), rng.standard_normal((N, D))
    q, E = rng.standard_normal(D), rng.standard_normal(D)
    s = 0.45
    _, alpha, o = O.attention_forward(K, V, q, s)
    lse = np.log(np.sum(np.exp(s * (K @ q))))
    d = O.exact_e_diagnostics(K, V, None, q[None], E[None], [lse], o[None], s, 0, 0)
    for p in range(N // 2):
        m = 2 * p
        for (i, j, g) in ((m, m, d["g_self_e"][m]), (m + 1, m + 1, d["g_self_e"][m + 1]), (m, m + 1, d["g_cross_e"][p])):
            H = O.hessian_block(alpha, V, o, q, E, i, j, s)
            assert np.allclose(g * s * s * np.outer(q, q), H, atol=1e-14, rtol=1e-12)


def test_exact_weights_equal_forward_only_when_angles_agree():
    """One dimension, one query, both values above the output and both attention weights
    below 1/2: cos(E, c11) = cos(E, c22) = -cos(E, c12) = sign(E), the pattern the
    forward-only weights assume, so the two closed forms give the same k*."""
    K = np.array([[0.2], [0.5], [-0.3], [0.1], [0.4], [-0.2]])
    V = np.array([[2.0], [3.0], [-1.0], [-2.0], [0.5], [0.4]])
    q = np.array([0.7])
    s = 1.0
    _, alpha, o = O.attention_forward(K, V, q, s)
    lse = np.log(np.sum(np.exp(s * (K @ q))))
    assert np.all(alpha < 0.5) and V[0, 0] > o[0] and V[1, 0] > o[0]
    for E in (1.7, -0.4):
        d = O.exact_e_diagnostics(K, V, None, q[None], np.array([[E]]), [lse], o[None], s, 0, 0)
        assert np.allclose(d["w_exact"][0], d["w_fwd"][0], atol=1e-12)
        assert abs(d["g_self_e"][0] / d["n_self_e"][0] - np.sign(E)) < 1e-12
        assert abs(d["g_cross_e"][0] / d["n_cross_e"][0] + np.sign(E)) < 1e-12
        assert d["loss_fwd"][0] == pytest.approx(d["loss_exact"][0], abs=1e-12)


def test_exact_diagnostics_invariants():
    """Effective cosines lie in [-1, 1]; the forward-only norm sums equal the round's;
    the exact k* is stationary for the exact model, so when it is convex it has the
    smaller loss."""
    K, V, n, Q = _random_slice(51, N=24, D=6, GW=4, counts=True)
    E = _rng(52).standard_normal((4, 6))
    ref = O.merge_round(K, V, n, Q, 0.4, 2, 2, 0)
    d = O.exact_e_diagnostics(K, V, n, Q, E, ref.lse, ref.O, 0.4, 2, 2)
    assert np.all(np.abs(d["g_self_e"]) <= d["n_self_e"] * (1 + 1e-12))
    assert np.all(np.abs(d["g_cross_e"]) <= d["n_cross_e"] * (1 + 1e-12))
    assert np.allclose(d["g_self"], ref.g_self, rtol=1e-12) and np.allclose(d["g_cross"], ref.g_cross, rtol=1e-12)
    for p in range(len(d["loss_exact"])):
        m = 2 + 2 * p
        g11, g12, g22 = d["g_self_e"][m], d["g_cross_e"][p], d["g_self_e"][m + 1]
        if g11 + 2 * g12 + g22 > 0 and g11 * g22 - g12 * g12 > 0:
            assert d["loss_exact"][p] <= d["loss_fwd"][p] + 1e-12


# ------------------------------------------------------- spectral contributions --
def test_spectral_contributions_match_the_pairwise_split():
    """Given the eigen-pairs of W Wᵀ from numpy.linalg.eigh, the sequence split equals the
    pairwise one for every adjacent pair, and its sum is the cosine of the projected keys;
    the d_k nonzero modes of the thin SVD give the same numbers."""
    rng = _rng(60)
    T, d, dk = 9, 12, 4
    X = rng.standard_normal((T, d))
    W = rng.standard_normal((d, dk))
    lam, U = np.linalg.eigh(W @ W.T)
    c, cs = O.spectral_contributions(X, U.T, lam)
    for t in range(T - 1):
        assert np.allclose(c[t], O.spectral_mode_contributions(X[t], X[t + 1], W), atol=1e-12)
        assert abs(cs[t] - O.cosine(X[t] @ W, X[t + 1] @ W)) < 1e-12
    Us, sig, _ = np.linalg.svd(W, full_matrices=False)
    c2, cs2 = O.spectral_contributions(X, Us.T, sig ** 2)
    assert np.allclose(cs2, cs, atol=1e-12)
    assert np.allclose(np.sort(c2, axis=1), np.sort(c[:, -dk:], axis=1), atol=1e-12)


def test_spectral_contributions_zero_token():
    X = np.array([[1.0, 0.0], [0.0, 0.0], [0.5, 0.5]])
    c, cs = O.spectral_contributions(X, np.eye(2), np.array([2.0, 1.0]))
    assert np.all(c[:2] == 0) and np.all(cs == 0)
