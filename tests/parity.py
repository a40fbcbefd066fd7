"""Helpers for GPU-vs-oracle parity tests: slicing, running the oracle per
(batch, kv-head) slice on host copies of the GPU inputs, and comparisons.

Tolerances (written here once, used by every parity test):
* floating outputs: per output vector, max|x - ref| / max|ref| <= 2e-3, the bound
  the merged keys and decode outputs must meet (inputs bf16, fp32 accumulation);
* the Hessian-norm sums g_self and g_cross: element by element, |x - ref| <= 2e-3 |ref|
  (elements below 1e-6 of their head's largest are held to 2e-9 of that largest);
* cosine: absolute 1e-6 (fp32 dot products of 128 terms);
* integer outputs (counts, compaction indices, selection flags): bit-exact, with
  selection compared only on pairs whose oracle cosine is at least 1e-6 away from
  the selection threshold.
"""
from __future__ import annotations

import numpy as np
import torch

from oracle import kvs_oracle as O

REL_TOL = 2e-3
STAT_FLOOR = 1e-6
COS_TOL = 1e-6
MARGIN = 1e-6


def maxrel(x, ref) -> float:
    """max over vectors (last axis) of max|x - ref| / max|ref|."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    if x.size == 0:
        return 0.0
    x = x.reshape(-1, x.shape[-1]) if x.ndim > 1 else x.reshape(1, -1)
    ref = ref.reshape(x.shape)
    err = np.max(np.abs(x - ref), axis=1)
    scale = np.max(np.abs(ref), axis=1)
    scale = np.where(scale > 0, scale, 1.0)
    return float(np.max(err / scale))


def elemrel(x, ref, mag=None, floor=STAT_FLOOR) -> float:
    """max over elements of |x - ref| / max(|mag|, floor * max|mag|), mag = ref by default.

    For sums of non-negative terms (the Hessian-norm sums g_self, g_cross) mag is the
    reference itself, so every element is held to the relative bound; for signed sums whose
    terms can cancel, mag is the sum of the terms' magnitudes.  The floor (a fraction of
    the largest element of the same head) only matters for elements that are negligible
    within their head, where fp32 underflow of exp2 is allowed."""
    x = np.asarray(x, np.float64).reshape(-1)
    ref = np.asarray(ref, np.float64).reshape(-1)
    if x.size == 0:
        return 0.0
    m = np.abs(ref if mag is None else np.asarray(mag, np.float64).reshape(-1))
    top = float(np.max(m))
    if top == 0.0:
        return float(np.max(np.abs(x - ref)))
    return float(np.max(np.abs(x - ref) / np.maximum(m, floor * top)))


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy() if t.is_floating_point() else t.detach().cpu().numpy()


def slice_inputs(K, V, n, Qw, b, h, N):
    """Host fp64 copies of one (b, kv-head) slice; Qw rows of the G query heads."""
    G = Qw.shape[1] // K.shape[1]
    Ks = host(K[b, h, :N])
    Vs = host(V[b, h, :N])
    ns = None if n is None else host(n[b, h, :N]).astype(np.int64)
    Qs = host(Qw[b, h * G:(h + 1) * G]).reshape(-1, K.shape[-1])
    return Ks, Vs, ns, Qs


def selection_from_src(src: np.ndarray, S: int, P: int) -> np.ndarray:
    """Selection flags read back from a compacted slice: pair p (first slot m = S + 2p)
    merged iff slot m starts an output slot and slot m + 1 does not."""
    m = S + 2 * np.arange(P)
    return np.isin(m, src) & ~np.isin(m + 1, src)


def selection_threshold(cos: np.ndarray, M: int) -> float | None:
    if M == 0 or M == len(cos):
        return None
    order = np.argsort(-cos, kind="stable")
    return float(cos[order[M - 1]])


def check_round_slice(bufs, K, V, n, Qw, b, h, N, S, R, M, scale, label="", with_cos=True):
    """Compare every output of one GPU round on slice (b, h) with the oracle.
    Returns the oracle result (with the GPU selection applied where it differs
    only inside the tie margin)."""
    Ks, Vs, ns, Qs = slice_inputs(K, V, n, Qw, b, h, N)
    G = Qw.shape[1] // K.shape[1]
    W = Qw.shape[2]
    r = O.merge_round(Ks, Vs, ns, Qs, scale, S, R, M)
    P = len(r.cos)
    T = N - M
    lse = host(bufs.lse[b, h * G:(h + 1) * G]).reshape(-1)
    Ow = host(bufs.O[b, h * G:(h + 1) * G]).reshape(G * W, -1)
    assert np.max(np.abs(lse - r.lse)) < 1e-4 * max(1.0, np.max(np.abs(r.lse))), f"{label} lse"
    assert maxrel(Ow, r.O) <= REL_TOL, f"{label} O {maxrel(Ow, r.O)}"
    gs = host(bufs.g_self[b, h, :N])
    assert elemrel(gs, r.g_self) <= REL_TOL, f"{label} g_self {elemrel(gs, r.g_self)}"
    if P:
        gc = host(bufs.g_cross[b, h, :P])
        assert elemrel(gc, r.g_cross) <= REL_TOL, f"{label} g_cross {elemrel(gc, r.g_cross)}"
        if with_cos:
            cs = host(bufs.cos[b, h, :P])
            assert np.max(np.abs(cs - r.cos)) <= COS_TOL, f"{label} cos {np.max(np.abs(cs - r.cos))}"
    # selection (bit-exact outside the tie margin); a call that writes no flags (the fused
    # round) shows its selection in the compaction sources
    sel = r.selected
    gflags = None
    if bufs.selected is not None and P:
        gflags = host(bufs.selected[b, h, :P]).astype(bool)
    elif P and 0 < M < P:
        gflags = selection_from_src(host(bufs.src[b, h, :T]).astype(np.int64), S, P)
    if gflags is not None:
        gsel = gflags
        assert int(gsel.sum()) == M, f"{label} selected count"
        tau = selection_threshold(r.cos, M)
        if tau is None:
            assert np.array_equal(gsel, sel), f"{label} selection"
        else:
            far = np.abs(r.cos - tau) >= MARGIN
            assert np.array_equal(gsel[far], sel[far]), f"{label} selection outside margin"
            sel = gsel
    if bufs.w is not None and P:
        gw = host(bufs.w[b, h, :P])
        # weights compared away from the degenerate-denominator switch
        A = r.g_self[S + 2 * np.arange(P)] - 2 * r.g_cross + r.g_self[S + 2 * np.arange(P) + 1]
        sc = r.g_self[S + 2 * np.arange(P)] + 2 * r.g_cross + r.g_self[S + 2 * np.arange(P) + 1]
        ok = np.abs(A - 1e-6 * sc) > 1e-3 * np.abs(sc)
        assert maxrel(gw[ok], r.w[ok]) <= REL_TOL, f"{label} weights"
    # compaction with the (possibly margin-adjusted) selection
    Kc, Vc, nc, srcc = O.compact(Ks, Vs, ns if ns is not None else np.ones(N, np.int64), r.w, sel, S)
    assert Kc.shape[0] == T
    Kg = host(bufs.K[b, h, :T])
    Vg = host(bufs.V[b, h, :T])
    assert np.array_equal(host(bufs.src[b, h, :T]).astype(np.int64), srcc), f"{label} src"
    assert np.array_equal(host(bufs.n[b, h, :T]).astype(np.int64), nc), f"{label} n"
    assert maxrel(Kg, Kc) <= REL_TOL, f"{label} K' {maxrel(Kg, Kc)}"
    assert maxrel(Vg, Vc) <= REL_TOL, f"{label} V' {maxrel(Vg, Vc)}"
    return r
