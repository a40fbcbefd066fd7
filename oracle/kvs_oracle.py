"""Plain fp64 CPU oracle for the KVSlimmer asymmetric KV-merge path.

TEST INFRASTRUCTURE ONLY.  This module is imported by ``tests/``, by
``__graft_entry__.smoke()`` and by the ``cpu_baseline`` leg of ``bench.py``;
nothing in the product package may import or call it.  It shares no code with
the HIP path: no kernels, no helpers, no constants.  Everything here is plain
NumPy in float64, written straight from the pages, slow on purpose so that a
reader can check every step against the formulas by eye.

Sources (cited by page title and section; the pages print no equation numbers
except the figure-2 caption's "Eq. 8"):

* [DD]  "论文专题讲解：KVSlimmer：非对称 KV 合并的数学与工程"
        (charles2530.github.io deep-dive).  Sections used:
        数学主线一 (spectral asymmetry), 数学主线二 (why a Hessian),
        数学主线三 (exact Hessian), 数学主线四 (forward-only weights),
        算一遍 (KV size arithmetic), 实验设置 (setting table),
        工程上怎么用 (sinks and recent window), 局限与边界 (uniform ratio,
        local adjacent merging).
* [ABS] KVSlimmer abstract, arXiv 2603.00907 (fugumt.com and
        thelatestinai.com pages), and the figure-2 caption there ("Eq. 8").
* [ASYM] AsymKV abstract ("Homogeneous Keys, Heterogeneous Values"), in the
        related-papers list of the fugumt.com page: keys are merged, values
        are compressed losslessly.

Readings of points the pages leave open are listed next to the function that
takes them, each with its label (O1, O2, ...).

Pinned functions (tests/test_oracle_pins.py): every public function below is
checked against something other than itself: finite differences, brute-force
minimisation, closed forms, textbook/library routines, exact invariants or the
numbers the pages print.  Parity unpinned (true to the pages only by argument):
the multi-query aggregation of the Hessian norms (reading O2), the pair
selection policy (O6/O7) and the degenerate-denominator thresholds (O10, and
O22 for the exact-gradient weights); each is marked "parity unpinned" below.
The chunked budget loop (O21) is pinned by its invariants only: the pages give
its settings, not its steps.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

F64 = np.float64

# Relative size below which the closed-form denominator is treated as
# degenerate and the plain average is used instead (reading O10).
DEGENERATE_REL = 1e-6


# ---------------------------------------------------------------------------
# 数学主线一: spectral view of adjacent similarity
# ---------------------------------------------------------------------------
def cosine(a: np.ndarray, b: np.ndarray) -> float:
    """Cosine similarity of two vectors, the quantity whose per-mode split is
    [DD] 数学主线一 (the cos(y_t, y_{t+1}) equation) and [ABS] figure-2 "Eq. 8".

    Reading O9 (pages silent): if either norm is zero the cosine is 1 when the
    two vectors are equal (both zero) and 0 otherwise.
    """
    a = np.asarray(a, F64)
    b = np.asarray(b, F64)
    na = math.sqrt(float(a @ a))
    nb = math.sqrt(float(b @ b))
    if na == 0.0 or nb == 0.0:
        return 1.0 if np.array_equal(a, b) else 0.0
    return float(a @ b) / (na * nb)


def spectral_mode_contributions(x_t: np.ndarray, x_t1: np.ndarray, W: np.ndarray) -> np.ndarray:
    """Per-mode contributions c_i to cos(y_t, y_{t+1}) for y = x W.

    [DD] 数学主线一: M = W Wᵀ = U Λ Uᵀ, p_{t,i} = x_t u_i,
    x_t M x_{t+1}ᵀ = Σ_i λ_i p_{t,i} p_{t+1,i}, and
    cos(y_t, y_{t+1}) = Σ_i λ_i p_{t,i} p_{t+1,i} /
                        (sqrt(Σ_i λ_i p_{t,i}²) sqrt(Σ_i λ_i p_{t+1,i}²)) = Σ_i c_i.
    Returns c (one entry per eigen-mode, ordered as numpy.linalg.eigh returns
    them).  The identity Σ c_i = cosine(x_t W, x_{t+1} W) is a pin.
    """
    x_t = np.asarray(x_t, F64)
    x_t1 = np.asarray(x_t1, F64)
    W = np.asarray(W, F64)
    M = W @ W.T
    lam, U = np.linalg.eigh(M)
    p_t = x_t @ U
    p_t1 = x_t1 @ U
    den = math.sqrt(float(np.sum(lam * p_t * p_t))) * math.sqrt(float(np.sum(lam * p_t1 * p_t1)))
    return lam * p_t * p_t1 / den


def spectral_contributions(X: np.ndarray, modes: np.ndarray, lam: np.ndarray):
    """The per-mode split of [DD] 数学主线一 for a whole token sequence, given the
    eigen-pairs of M = W Wᵀ: ``modes`` [r, d] holds the eigenvectors u_i as rows,
    ``lam`` [r] their eigenvalues (the modes with λ_i = 0 contribute nothing, so
    the r = d_k nonzero ones of a thin SVD W = U Σ Vᵀ, λ = σ², suffice).  For every
    adjacent pair (t, t+1): p_{t,i} = x_t u_i, and
    c[t, i] = λ_i p_{t,i} p_{t+1,i} / (sqrt(Σ_i λ_i p_{t,i}²) sqrt(Σ_i λ_i p_{t+1,i}²)),
    cos[t] = Σ_i c[t, i] = cos(x_t W, x_{t+1} W).  A zero norm gives c = 0 and
    cos = 0 (reading O23).  Returns (c [T−1, r], cos [T−1])."""
    X = np.asarray(X, F64)
    U = np.asarray(modes, F64)
    lam = np.asarray(lam, F64)
    Pm = X @ U.T
    ny = np.sqrt(np.sum(lam * Pm * Pm, axis=1))
    T = X.shape[0]
    c = np.zeros((max(T - 1, 0), U.shape[0]))
    for t in range(T - 1):
        den = ny[t] * ny[t + 1]
        if den > 0:
            c[t] = lam * Pm[t] * Pm[t + 1] / den
    return c, c.sum(axis=1)


# ---------------------------------------------------------------------------
# 数学主线三: single-query attention, gradient and exact Hessian blocks
# ---------------------------------------------------------------------------
def attention_forward(K: np.ndarray, V: np.ndarray, q: np.ndarray, scale: float,
                      n: np.ndarray | None = None):
    """Single-query softmax attention, [DD] 数学主线三 first equation:
    e_i = q k_iᵀ / sqrt(d_k), α = softmax(e), o = Σ_t α_t v_t.

    ``scale`` is 1/sqrt(d_k) (reading O5: d_k = head_dim).  With slot counts
    ``n`` (reading O1, see ``merge_values``) the logit of slot i gets + ln n_i
    and v_i is the slot's mean value; n = None means every slot holds one
    token.  Returns (e, alpha, o).
    """
    K = np.asarray(K, F64)
    V = np.asarray(V, F64)
    q = np.asarray(q, F64)
    e = scale * (K @ q)
    if n is not None:
        e = e + np.log(np.asarray(n, F64))
    mx = np.max(e)
    w = np.exp(e - mx)
    alpha = w / np.sum(w)
    o = alpha @ V
    return e, alpha, o


def key_gradient(alpha: np.ndarray, V: np.ndarray, o: np.ndarray, q: np.ndarray,
                 E: np.ndarray, i: int, scale: float) -> np.ndarray:
    """g_i = ∇_{k_i} L = (1/sqrt(d_k)) α_i [Eᵀ(v_i − o)] q, with E = ∂L/∂o
    ([DD] 数学主线三, key-gradient equation).  Test pin only: needs E."""
    V = np.asarray(V, F64)
    return scale * alpha[i] * float(np.asarray(E, F64) @ (V[i] - o)) * np.asarray(q, F64)


def ds_de(alpha: np.ndarray, V: np.ndarray, o: np.ndarray, i: int, j: int) -> np.ndarray:
    """∂s_i/∂e_j for s_i = α_i (v_i − o), [DD] 数学主线三:
    diagonal  ∂s_i/∂e_i = α_i (1 − 2α_i)(v_i − o);
    off-diag  ∂s_i/∂e_j = −α_i α_j (v_i + v_j − 2o), i ≠ j."""
    V = np.asarray(V, F64)
    if i == j:
        return alpha[i] * (1.0 - 2.0 * alpha[i]) * (V[i] - o)
    return -alpha[i] * alpha[j] * (V[i] + V[j] - 2.0 * o)


def hessian_block(alpha: np.ndarray, V: np.ndarray, o: np.ndarray, q: np.ndarray,
                  E: np.ndarray, i: int, j: int, scale: float) -> np.ndarray:
    """h_ij = ∂g_i/∂k_jᵀ = (1/d_k) [Eᵀ ∂s_i/∂e_j] q qᵀ ([DD] 数学主线三,
    unified Hessian-block form; scale² = 1/d_k).  Test pin only."""
    q = np.asarray(q, F64)
    return scale * scale * float(np.asarray(E, F64) @ ds_de(alpha, V, o, i, j)) * np.outer(q, q)


# ---------------------------------------------------------------------------
# 数学主线四: forward-only vectors and the closed-form key merge
# ---------------------------------------------------------------------------
def c_vectors(alpha: np.ndarray, V: np.ndarray, o: np.ndarray, m: int):
    """The three forward-only vectors of [DD] 数学主线四 for the pair (m, m+1):
    c11 = α_m (1 − 2α_m)(v_m − o), c22 = α_{m+1}(1 − 2α_{m+1})(v_{m+1} − o),
    c12 = −α_m α_{m+1} (v_m + v_{m+1} − 2o)."""
    V = np.asarray(V, F64)
    a0, a1 = alpha[m], alpha[m + 1]
    c11 = a0 * (1.0 - 2.0 * a0) * (V[m] - o)
    c22 = a1 * (1.0 - 2.0 * a1) * (V[m + 1] - o)
    c12 = -a0 * a1 * (V[m] + V[m + 1] - 2.0 * o)
    return c11, c22, c12


def merge_objective(k: np.ndarray, k_m: np.ndarray, k_m1: np.ndarray,
                    g11: float, g12: float, g22: float) -> float:
    """Second-order merge loss in the effective scalars g11, g12, g22
    ([DD] 数学主线二):
    g11 ‖k − k_m‖² + 2 g12 (k − k_m)ᵀ(k − k_{m+1}) + g22 ‖k − k_{m+1}‖²."""
    k = np.asarray(k, F64)
    d0 = k - np.asarray(k_m, F64)
    d1 = k - np.asarray(k_m1, F64)
    return float(g11 * (d0 @ d0) + 2.0 * g12 * (d0 @ d1) + g22 * (d1 @ d1))


def hessian_weights(g11: float, g12: float, g22: float):
    """Stationary point of ``merge_objective`` ([DD] 数学主线二, setting the
    derivative to zero): k* = [(g11+g12) k_m + (g12+g22) k_{m+1}] /
    (g11 + 2 g12 + g22).  Returns (w_m, w_{m+1}); [DD] 数学主线四 writes the
    same pair as the weights of k* = w_m k_m + w_{m+1} k_{m+1}."""
    den = g11 + 2.0 * g12 + g22
    return (g11 + g12) / den, (g12 + g22) / den


def forward_only_weights(n11: float, n12: float, n22: float):
    """Closed-form, forward-only weights of [DD] 数学主线四 (last equation):
    k* = (‖c11‖ − 2‖c12‖ + ‖c22‖)⁻¹ [(‖c11‖ − ‖c12‖) k_m + (‖c22‖ − ‖c12‖) k_{m+1}].

    Arguments are the (window-summed, reading O2) norms ‖c11‖, ‖c12‖, ‖c22‖.
    Reading O10 (pages silent on a vanishing or negative denominator): if
    A = n11 − 2 n12 + n22 is not finite or A <= 1e-6 (n11 + n22 + 2 n12) the
    plain average (½, ½) of [DD] 数学主线二 is used.  No clamping otherwise.
    Returns (w_m, w_{m+1}, used_fallback).  The threshold is parity unpinned.
    """
    A = n11 - 2.0 * n12 + n22
    scale = n11 + n22 + 2.0 * n12
    if not math.isfinite(A) or A <= DEGENERATE_REL * scale:
        return 0.5, 0.5, True
    return (n11 - n12) / A, (n22 - n12) / A, False


def merge_values(v_m: np.ndarray, v_m1: np.ndarray, n_m: int, n_m1: int):
    """Lossless value handling (reading O1).

    [DD] 数学主线一 and the 本页结论 summary say values are heterogeneous and
    must not follow the key-merge rule; [ASYM] compresses values losslessly.
    Once both positions share the merged key k*, they get identical logits, so
    one slot holding the count-weighted mean value and the count n_m + n_{m+1}
    (whose logit carries + ln n) gives exactly the attention output of the two
    separate values.  Returns (v̄*, n*)."""
    v_m = np.asarray(v_m, F64)
    v_m1 = np.asarray(v_m1, F64)
    n_tot = int(n_m) + int(n_m1)
    return (n_m * v_m + n_m1 * v_m1) / n_tot, n_tot


# ---------------------------------------------------------------------------
# Cache policy: candidate pairs and selection
# ---------------------------------------------------------------------------
def num_pairs(n_slots: int, n_sink: int, n_recent: int) -> int:
    """Aligned candidate pairs (S+2p, S+2p+1) inside [S, N−R) (reading O6:
    "adjacent" pairs of [DD] 数学主线二, disjoint so that one round is a
    matching; the sinks and recent window of [DD] 实验设置 / 工程上怎么用
    are never merged).  An odd leftover slot is kept."""
    return max(0, (n_slots - n_sink - n_recent) // 2)


def select_pairs(cos: np.ndarray, n_merge: int) -> np.ndarray:
    """Boolean flags of the n_merge pairs to merge in one round.

    Reading O7 (parity unpinned: the pages give only "homogeneous adjacent
    keys" and a uniform ratio, [DD] 局限与边界): the pairs with the highest
    adjacent-key cosine, ties to the lower pair index.  Implemented as a stable
    sort on −cos."""
    P = len(cos)
    if n_merge > P or n_merge < 0:
        raise ValueError("infeasible merge count")
    order = np.argsort(-np.asarray(cos, F64), kind="stable")
    sel = np.zeros(P, dtype=bool)
    sel[order[:n_merge]] = True
    return sel


# ---------------------------------------------------------------------------
# One merge round on one (batch, layer, kv-head) slice
# ---------------------------------------------------------------------------
@dataclass
class RoundResult:
    lse: np.ndarray        # [GW]
    O: np.ndarray          # [GW, D]
    g_self: np.ndarray     # [N]
    g_cross: np.ndarray    # [P]
    cos: np.ndarray        # [P]
    selected: np.ndarray   # [P] bool
    w: np.ndarray          # [P, 2]
    fallback: np.ndarray   # [P] bool
    K: np.ndarray          # [T, D]
    V: np.ndarray          # [T, D]
    n: np.ndarray          # [T] int64
    src: np.ndarray        # [T] int64
    extras: dict = field(default_factory=dict)


def window_statistics(K, V, n, Qw, scale):
    """Step 1: for every window query w (the W queries of each of the G query
    heads of this KV head, reading O3; no causal mask, reading O4), the
    attention of [DD] 数学主线三 over all N slots with the + ln n slot bias.
    Returns lse [GW], alpha [GW, N], O [GW, D]."""
    K = np.asarray(K, F64)
    V = np.asarray(V, F64)
    Qw = np.asarray(Qw, F64)
    GW = Qw.shape[0]
    N = K.shape[0]
    lse = np.empty(GW)
    alpha = np.empty((GW, N))
    O = np.empty((GW, V.shape[1]))
    for w in range(GW):
        e, a, o = attention_forward(K, V, Qw[w], scale, n)
        mx = np.max(e)
        lse[w] = mx + math.log(float(np.sum(np.exp(e - mx))))
        alpha[w] = a
        O[w] = o
    return lse, alpha, O


def hessian_norm_sums(V, alpha, O, n_sink, P):
    """Step 2 ([DD] 数学主线四 norms, aggregated over the window by reading
    O2, parity unpinned): g_self[i] = Σ_w ‖α_{w,i}(1 − 2α_{w,i})(v_i − o_w)‖,
    which is Σ_w ‖c11^{(w)}‖ when i is the first slot of a pair and
    Σ_w ‖c22^{(w)}‖ when it is the second; and, for the pair p with first slot
    m = S + 2p, g_cross[p] = Σ_w ‖c12^{(w)}‖.  Norms by direct subtraction."""
    V = np.asarray(V, F64)
    GW, N = alpha.shape
    g_self = np.zeros(N)
    g_cross = np.zeros(P)
    m = n_sink + 2 * np.arange(P)
    for w in range(GW):
        a = alpha[w]
        o = O[w]
        r = np.sqrt(np.sum((V - o) ** 2, axis=1))                 # ‖v_i − o_w‖
        g_self += np.abs(a * (1.0 - 2.0 * a)) * r
        if P:
            rc = np.sqrt(np.sum((V[m] + V[m + 1] - 2.0 * o) ** 2, axis=1))
            g_cross += a[m] * a[m + 1] * rc
    return g_self, g_cross


def merge_round(K, V, n, Qw, scale, n_sink, n_recent, n_merge) -> RoundResult:
    """One KVSlimmer merge round on one slice, steps 1-7 in page order.

    K, V: [N, D] (V holds slot mean values), n: [N] counts or None (all ones),
    Qw: [GW, D] window queries.  Output length T = N − n_merge.
    """
    K = np.asarray(K, F64)
    V = np.asarray(V, F64)
    N, D = K.shape
    nn = np.ones(N, dtype=np.int64) if n is None else np.asarray(n, dtype=np.int64)
    P = num_pairs(N, n_sink, n_recent)
    if not (0 <= n_merge <= P):
        raise ValueError("infeasible merge count")

    # 1. window attention statistics
    lse, alpha, O = window_statistics(K, V, None if n is None else nn, Qw, scale)
    return _round_steps_2_to_7(K, V, nn, lse, alpha, O, n_sink, P, n_merge)


def merge_round_given_stats(K, V, n, Qw, lse, O, scale, n_sink, n_recent, n_merge) -> RoundResult:
    """The same round when the window statistics come from elsewhere (the prefill
    attention that already computed them): lse [GW] and O [GW, D] are taken as given
    instead of step 1, and the attention weights follow from them by the definition of
    [DD] 数学主线三, α_{w,i} = exp(e_{w,i} − lse_w) with e = scale·q·k + ln n.  With the
    lse and O of ``window_statistics`` this is ``merge_round``."""
    K = np.asarray(K, F64)
    V = np.asarray(V, F64)
    Qw = np.asarray(Qw, F64)
    N, D = K.shape
    nn = np.ones(N, dtype=np.int64) if n is None else np.asarray(n, dtype=np.int64)
    P = num_pairs(N, n_sink, n_recent)
    if not (0 <= n_merge <= P):
        raise ValueError("infeasible merge count")
    lse = np.asarray(lse, F64)
    O = np.asarray(O, F64)
    alpha = np.empty((Qw.shape[0], N))
    for w in range(Qw.shape[0]):
        e = scale * (K @ Qw[w]) + np.log(nn.astype(F64))
        alpha[w] = np.exp(e - lse[w])
    return _round_steps_2_to_7(K, V, nn, lse, alpha, O, n_sink, P, n_merge)


def _round_steps_2_to_7(K, V, nn, lse, alpha, O, n_sink, P, n_merge) -> RoundResult:
    # 2. Hessian-norm sums
    g_self, g_cross = hessian_norm_sums(V, alpha, O, n_sink, P)
    # 3. adjacent-key similarity
    cos = np.array([cosine(K[n_sink + 2 * p], K[n_sink + 2 * p + 1]) for p in range(P)])
    # 4. selection
    selected = select_pairs(cos, n_merge)
    # 5. closed-form weights (for every candidate pair; only selected ones are used)
    w = np.empty((P, 2))
    fb = np.zeros(P, dtype=bool)
    for p in range(P):
        m = n_sink + 2 * p
        w0, w1, f = forward_only_weights(g_self[m], g_cross[p], g_self[m + 1])
        w[p] = (w0, w1)
        fb[p] = f
    # 6 + 7. merge and compaction
    Ko, Vo, no, so = compact(K, V, nn, w, selected, n_sink)
    return RoundResult(lse=lse, O=O, g_self=g_self, g_cross=g_cross, cos=cos,
                       selected=selected, w=w, fallback=fb, K=Ko, V=Vo, n=no, src=so,
                       extras={"alpha": alpha})


def compact(K, V, n, w, selected, n_sink):
    """Steps 6 and 7: walk the slots in order; the first slot i of a selected pair
    p emits the merged slot (k* = w_m k_m + w_{m+1} k_{m+1}, [DD] 数学主线四; the
    lossless value slot of ``merge_values``) with src = i and skips i + 1; every
    other slot is copied with src = i.  Output length N − (number selected)."""
    K = np.asarray(K, F64)
    V = np.asarray(V, F64)
    N, D = K.shape
    nn = np.asarray(n, dtype=np.int64)
    P = len(selected)
    out_k, out_v, out_n, out_src = [], [], [], []
    i = 0
    while i < N:
        p = (i - n_sink) // 2
        first_of_pair = (i >= n_sink and (i - n_sink) % 2 == 0 and p < P)
        if first_of_pair and selected[p]:
            k_star = w[p, 0] * K[i] + w[p, 1] * K[i + 1]
            v_star, n_star = merge_values(V[i], V[i + 1], nn[i], nn[i + 1])
            out_k.append(k_star)
            out_v.append(v_star)
            out_n.append(n_star)
            out_src.append(i)
            i += 2
        else:
            out_k.append(K[i])
            out_v.append(V[i])
            out_n.append(int(nn[i]))
            out_src.append(i)
            i += 1
    return (np.array(out_k).reshape(-1, D), np.array(out_v).reshape(-1, D),
            np.array(out_n, dtype=np.int64), np.array(out_src, dtype=np.int64))


def decode(K, V, n, q, scale) -> np.ndarray:
    """Decode attention over a (merged) cache: the attention of [DD] 数学主线三
    with the + ln n slot bias of reading O1; returns o = Σ_j α_j v̄_j."""
    _, _, o = attention_forward(K, V, q, scale, n)
    return o


def compose_src(prev_src: np.ndarray, src: np.ndarray) -> np.ndarray:
    """Map the src indices of a later round back to the original slots."""
    return np.asarray(prev_src)[np.asarray(src)]


# ---------------------------------------------------------------------------
# 数学主线三/四: exact-gradient scalars against the forward-only substitution
# ---------------------------------------------------------------------------
def exact_weights(g11: float, g12: float, g22: float):
    """``hessian_weights`` with the degenerate case handled (reading O22, pages
    silent; the threshold is parity unpinned): when g11 + 2 g12 + g22 is not
    finite or its magnitude is at most 1e-6 (|g11| + 2|g12| + |g22|), the plain
    average (½, ½).  An indefinite model keeps its stationary point (no
    clamping).  Returns (w_m, w_{m+1})."""
    den = g11 + 2.0 * g12 + g22
    scale = abs(g11) + 2.0 * abs(g12) + abs(g22)
    if not math.isfinite(den) or abs(den) <= DEGENERATE_REL * scale:
        return 0.5, 0.5
    return hessian_weights(g11, g12, g22)


def pair_loss(w0: float, w1: float, k_m, k_m1, g11: float, g12: float, g22: float) -> float:
    """``merge_objective`` at k = w0 k_m + w1 k_{m+1}."""
    k = w0 * np.asarray(k_m, F64) + w1 * np.asarray(k_m1, F64)
    return merge_objective(k, k_m, k_m1, g11, g12, g22)


def exact_e_diagnostics(K, V, n, Qw, E, lse, O, scale, n_sink, n_recent) -> dict:
    """Given an upstream gradient E_w = ∂L/∂o_w per window query, the exact
    scalars g_ij = E_wᵀ c_ij^{(w)} of [DD] 数学主线三 (the Hessian blocks are
    g_ij q qᵀ / d_k), summed over the window as the norms are (reading O2);
    their exact-weight k* (``exact_weights``, the stationary point of
    数学主线二); the forward-only k* of 数学主线四 from the norms; and the
    quantities that compare the two: Σ_w ‖E_w‖‖c^{(w)}‖ (so that g / that sum is
    a norm-weighted cos(E, c), whose pattern cos11 ≈ cos22 ≈ −cos12 is what the
    forward-only weights assume) and the exact second-order loss of each k*.

    Window statistics lse [GW], O [GW, D] as in ``merge_round_given_stats``.
    Per slot i (any slot: c_ii = α_i (1 − 2α_i)(v_i − o_w)): g_self_e, n_self_e,
    g_self (the forward-only norm sum).  Per candidate pair p: g_cross_e, n_cross_e,
    g_cross, w_exact [P, 2], w_fwd [P, 2], loss_exact, loss_fwd."""
    K = np.asarray(K, F64)
    V = np.asarray(V, F64)
    Qw = np.asarray(Qw, F64)
    E = np.asarray(E, F64)
    lse = np.asarray(lse, F64)
    O = np.asarray(O, F64)
    N, D = K.shape
    nn = np.ones(N, dtype=np.int64) if n is None else np.asarray(n, dtype=np.int64)
    P = num_pairs(N, n_sink, n_recent)
    g_self_e, n_self_e, g_self = np.zeros(N), np.zeros(N), np.zeros(N)
    g_cross_e, n_cross_e, g_cross = np.zeros(P), np.zeros(P), np.zeros(P)
    for w in range(Qw.shape[0]):
        e = scale * (K @ Qw[w]) + np.log(nn.astype(F64))
        alpha = np.exp(e - lse[w])
        en = math.sqrt(float(E[w] @ E[w]))
        for i in range(N):
            c = alpha[i] * (1.0 - 2.0 * alpha[i]) * (V[i] - O[w])
            g_self_e[i] += float(E[w] @ c)
            g_self[i] += math.sqrt(float(c @ c))
            n_self_e[i] += en * math.sqrt(float(c @ c))
        for p in range(P):
            _, _, c12 = c_vectors(alpha, V, O[w], n_sink + 2 * p)
            g_cross_e[p] += float(E[w] @ c12)
            g_cross[p] += math.sqrt(float(c12 @ c12))
            n_cross_e[p] += en * math.sqrt(float(c12 @ c12))
    w_exact = np.empty((P, 2))
    w_fwd = np.empty((P, 2))
    loss_exact = np.empty(P)
    loss_fwd = np.empty(P)
    for p in range(P):
        m = n_sink + 2 * p
        g11, g12, g22 = g_self_e[m], g_cross_e[p], g_self_e[m + 1]
        w_exact[p] = exact_weights(g11, g12, g22)
        w_fwd[p] = forward_only_weights(g_self[m], g_cross[p], g_self[m + 1])[:2]
        loss_exact[p] = pair_loss(w_exact[p, 0], w_exact[p, 1], K[m], K[m + 1], g11, g12, g22)
        loss_fwd[p] = pair_loss(w_fwd[p, 0], w_fwd[p, 1], K[m], K[m + 1], g11, g12, g22)
    return {"g_self_e": g_self_e, "n_self_e": n_self_e, "g_self": g_self, "g_cross_e": g_cross_e,
            "n_cross_e": n_cross_e, "g_cross": g_cross, "w_exact": w_exact, "w_fwd": w_fwd,
            "loss_exact": loss_exact, "loss_fwd": loss_fwd}


# ---------------------------------------------------------------------------
# 实验设置: chunked prefill under a fixed cache budget
# ---------------------------------------------------------------------------
@dataclass
class StreamResult:
    K: np.ndarray          # [T, D] final cache keys
    V: np.ndarray          # [T, D] final slot mean values
    n: np.ndarray          # [T] counts
    start: np.ndarray      # [T] first original token position each slot covers
    rounds: list           # (chunk index, N before the round, M, RoundResult)


def stream_prefill(K, V, Qw_chunks, scale, n_sink, budget, chunk) -> StreamResult:
    """The evaluation regime of [DD] 实验设置 (a fixed cache budget, the prompt
    prefilled in fixed-size chunks, the first tokens kept): reading O21.

    The raw tokens K, V [total, D] arrive in chunks of ``chunk`` (the last one
    may be shorter).  After a chunk is appended the cache holds N slots; while
    N > budget one merge round runs with M = min(N − budget, P) pairs,
    P = num_pairs(N, n_sink, 0): the first n_sink slots never merge and no
    recent window is protected (the pages name none in this setting).  The
    round's observation window is Qw_chunks[c] ([GW, D]), the last queries of
    chunk c.  Requires budget > n_sink, so that every round has a pair to merge.
    """
    K = np.asarray(K, F64)
    V = np.asarray(V, F64)
    total, D = K.shape
    if chunk < 1 or n_sink < 0 or budget <= n_sink:
        raise ValueError("need chunk >= 1 and budget > n_sink >= 0")
    cK, cV = np.empty((0, D)), np.empty((0, D))
    cn = np.empty(0, dtype=np.int64)
    start = np.empty(0, dtype=np.int64)
    rounds = []
    for c, c0 in enumerate(range(0, total, chunk)):
        c1 = min(total, c0 + chunk)
        cK = np.vstack([cK, K[c0:c1]])
        cV = np.vstack([cV, V[c0:c1]])
        cn = np.concatenate([cn, np.ones(c1 - c0, dtype=np.int64)])
        start = np.concatenate([start, np.arange(c0, c1, dtype=np.int64)])
        while len(cn) > budget:
            N = len(cn)
            M = min(N - budget, num_pairs(N, n_sink, 0))
            r = merge_round(cK, cV, cn, Qw_chunks[c], scale, n_sink, 0, M)
            rounds.append((c, N, M, r))
            cK, cV, cn = r.K, r.V, r.n
            start = start[r.src]
    return StreamResult(K=cK, V=cV, n=cn, start=start, rounds=rounds)


# ---------------------------------------------------------------------------
# 算一遍: KV bytes
# ---------------------------------------------------------------------------
def kv_bytes_per_token(layers: int, kv_heads: int, head_dim: int, dtype_bytes: int) -> int:
    """[DD] 算一遍: layers × 2 (K and V) × kv_heads × head_dim × bytes."""
    return layers * 2 * kv_heads * head_dim * dtype_bytes
