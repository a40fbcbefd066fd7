"""ctypes binding of libkvslim.so (C ABI in include/kvslim.h).

Argument marshalling only: tensors are passed as device pointers, shapes as the
kvs_cache / kvs_round structs, and the current torch stream as the HIP stream.
Every step of the path runs in the library's HIP kernels; if the library is
missing this module raises at import time, so nothing falls back to another path.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# KVSLIM_LIBRARY names another build of the same library (for instance one with the host
# code under AddressSanitizer); the in-tree build is the default.
LIB_PATH = os.environ.get("KVSLIM_LIBRARY") or os.path.join(_PKG, "libkvslim.so")

KVS_OK, KVS_ERR_NULL, KVS_ERR_SHAPE, KVS_ERR_DTYPE, KVS_ERR_STRIDE, KVS_ERR_ALIGN, \
    KVS_ERR_INFEASIBLE, KVS_ERR_WORKSPACE, KVS_ERR_HIP = range(9)
KVS_BF16, KVS_F32 = 0, 1
KVS_OP_SCORE, KVS_OP_SELECT, KVS_OP_SEL_STATE, KVS_OP_DECODE, KVS_OP_SCORE_MERGE, KVS_OP_STATS_MERGE = range(6)

EXPORTS = ("kvs_num_pairs", "kvs_workspace_bytes", "kvs_score", "kvs_score_merge", "kvs_merge_weights", "kvs_merge_compact",
           "kvs_append", "kvs_score_merge_stats", "kvs_exact_e_diag", "kvs_spectral_modes",
           "kvs_decode_attn", "kvs_decode_attn_static", "kvs_marks_begin", "kvs_marks_end", "kvs_mark_name", "kvs_mark_ms", "kvs_status_str",
           "kvs_last_error", "kvs_version")


class KvsCache(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("n_slots", ctypes.c_int64), ("stride_b", ctypes.c_int64),
                ("stride_h", ctypes.c_int64)]


class KvsRound(ctypes.Structure):
    _fields_ = [("window", ctypes.c_int32), ("n_sink", ctypes.c_int64), ("n_recent", ctypes.c_int64),
                ("n_merge", ctypes.c_int64), ("sm_scale", ctypes.c_float)]


class KvsError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{status_str(status)}: {msg}")
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m long_context_kv_kvslimmer_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
    C, R = ctypes.POINTER(KvsCache), ctypes.POINTER(KvsRound)
    sig = {
        "kvs_num_pairs": (I64, [I64, I64, I64]),
        "kvs_workspace_bytes": (SZ, [ctypes.c_int, C, R]),
        "kvs_score": (ctypes.c_int, [C, ctypes.c_int, P, P, P, P, R, P, P, P, P, P, P, SZ, P]),
        "kvs_score_merge": (ctypes.c_int, [C, ctypes.c_int, P, P, P, P, R, P, P, P, P, C, ctypes.c_int, P, P, P, P, P,
                                            SZ, P]),
        "kvs_merge_weights": (ctypes.c_int, [C, R, P, P, P, P, P, P, SZ, P, SZ, P]),
        "kvs_merge_compact": (ctypes.c_int, [C, ctypes.c_int, P, P, P, P, P, R, P, C, ctypes.c_int, P, P, P, P, P]),
        "kvs_decode_attn": (ctypes.c_int, [C, ctypes.c_int, P, P, P, P, F, P, P, SZ, P]),
        "kvs_decode_attn_static": (ctypes.c_int, [C, ctypes.c_int, P, P, P, P, F, P, P]),
        "kvs_append": (ctypes.c_int, [C, ctypes.c_int, P, P, P, I64, C, P, P, I64, I64, P]),
        "kvs_exact_e_diag": (ctypes.c_int, [C, ctypes.c_int, P, P, P, P, R, P, P, P, P, P, P]),
        "kvs_spectral_modes": (ctypes.c_int, [ctypes.c_int, P, I64, I32, P, P, I32, P, P, P, P]),
        "kvs_score_merge_stats": (ctypes.c_int, [C, ctypes.c_int, P, P, P, P, R, P, P, P, P, C, ctypes.c_int, P, P,
                                                  P, P, P, SZ, P]),
        "kvs_marks_begin": (ctypes.c_int, [I32, ctypes.c_char_p]),
        "kvs_marks_end": (I32, []),
        "kvs_mark_name": (ctypes.c_char_p, [I32]),
        "kvs_mark_ms": (F, [I32]),
        "kvs_status_str": (ctypes.c_char_p, [ctypes.c_int]),
        "kvs_last_error": (ctypes.c_char_p, []),
        "kvs_version": (I32, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()


def status_str(s: int) -> str:
    return _lib.kvs_status_str(s).decode()


def last_error() -> str:
    return _lib.kvs_last_error().decode()


def version() -> int:
    return _lib.kvs_version()


class KernelMarks:
    """Time the library's kernel launches inside a `with` block: HIP events recorded by the
    library right before and after each launch (only those labelled `label`, if given),
    on that launch's stream.  After the block `.times()` gives [(label, ms), ...]."""

    def __init__(self, max_launches: int = 64, label: str | None = None):
        self.max_launches = max_launches
        self.label = label
        self.n = 0

    def __enter__(self):
        _check(_lib.kvs_marks_begin(self.max_launches, None if self.label is None else self.label.encode()))
        return self

    def __exit__(self, *exc):
        self.n = _lib.kvs_marks_end()
        return False

    def times(self):
        out = []
        for k in range(self.n):
            ms = _lib.kvs_mark_ms(k)
            if ms < 0:
                raise KvsError(KVS_ERR_HIP, f"timing mark {k} failed")
            out.append((_lib.kvs_mark_name(k).decode(), ms))
        return out


def _check(s: int):
    if s != KVS_OK:
        raise KvsError(s, last_error())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream) if torch.cuda.is_available() else None


def dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return KVS_BF16
    if t.dtype == torch.float32:
        return KVS_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def cache_desc(K: torch.Tensor, n_q_heads: int, n_slots: int | None = None) -> KvsCache:
    """Describe K (or V) of shape [B, H_kv, capacity, D] (rows contiguous) holding n_slots slots."""
    if K.dim() != 4 or K.stride(3) != 1 or K.stride(2) != K.shape[3]:
        raise ValueError("cache tensors must be [B, H_kv, capacity, D] with contiguous rows")
    B, H, cap, D = K.shape
    n = cap if n_slots is None else n_slots
    if n > cap:
        raise ValueError("n_slots exceeds capacity")
    return KvsCache(B, H, n_q_heads, D, n, K.stride(0), K.stride(1))


def round_desc(window: int, n_sink: int, n_recent: int, n_merge: int, sm_scale: float) -> KvsRound:
    return KvsRound(window, n_sink, n_recent, n_merge, sm_scale)


def num_pairs(n_slots: int, n_sink: int, n_recent: int) -> int:
    return _lib.kvs_num_pairs(n_slots, n_sink, n_recent)


def workspace_bytes(op: int, cache: KvsCache, rnd: KvsRound | None) -> int:
    return _lib.kvs_workspace_bytes(op, ctypes.byref(cache), ctypes.byref(rnd) if rnd is not None else None)


def _same_layout(K, V):
    if K.shape != V.shape or K.stride() != V.stride() or K.dtype != V.dtype:
        raise ValueError("K and V must share shape, strides and dtype")


def kvs_score(cache: KvsCache, K, V, n, Qw, rnd: KvsRound, lse, O, g_self, g_cross, cos, workspace):
    _same_layout(K, V)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.kvs_score(ctypes.byref(cache), dtype_code(K), _ptr(K), _ptr(V), _ptr(n), _ptr(Qw),
                          ctypes.byref(rnd), _ptr(lse), _ptr(O), _ptr(g_self), _ptr(g_cross), _ptr(cos),
                          _ptr(workspace), ws_bytes, _stream()))


def kvs_score_merge(cache: KvsCache, K, V, n, Qw, rnd: KvsRound, lse, O, g_self, g_cross,
                    out: KvsCache, K_out, V_out, n_out, src_out, workspace):
    _same_layout(K, V)
    if K_out.dtype != V_out.dtype:
        raise ValueError("K_out and V_out must share a dtype")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.kvs_score_merge(ctypes.byref(cache), dtype_code(K), _ptr(K), _ptr(V), _ptr(n), _ptr(Qw),
                                ctypes.byref(rnd), _ptr(lse), _ptr(O), _ptr(g_self), _ptr(g_cross),
                                ctypes.byref(out), dtype_code(K_out), _ptr(K_out), _ptr(V_out), _ptr(n_out),
                                _ptr(src_out), _ptr(workspace), ws_bytes, _stream()))


def kvs_score_merge_stats(cache: KvsCache, K, V, n, Qw, rnd: KvsRound, lse, O, g_self, g_cross,
                          out: KvsCache, K_out, V_out, n_out, src_out, workspace):
    _same_layout(K, V)
    if K_out.dtype != V_out.dtype:
        raise ValueError("K_out and V_out must share a dtype")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.kvs_score_merge_stats(ctypes.byref(cache), dtype_code(K), _ptr(K), _ptr(V), _ptr(n), _ptr(Qw),
                                      ctypes.byref(rnd), _ptr(lse), _ptr(O), _ptr(g_self), _ptr(g_cross),
                                      ctypes.byref(out), dtype_code(K_out), _ptr(K_out), _ptr(V_out), _ptr(n_out),
                                      _ptr(src_out), _ptr(workspace), ws_bytes, _stream()))


def kvs_merge_weights(cache: KvsCache, rnd: KvsRound, g_self, g_cross, cos, w, selected, sel_state):
    sb = 0 if sel_state is None else sel_state.numel() * sel_state.element_size()
    _check(_lib.kvs_merge_weights(ctypes.byref(cache), ctypes.byref(rnd), _ptr(g_self), _ptr(g_cross), _ptr(cos),
                                  _ptr(w), _ptr(selected), _ptr(sel_state), sb, None, 0, _stream()))


def kvs_merge_compact(cache: KvsCache, K, V, n, g_self, g_cross, rnd: KvsRound, sel_state,
                      out: KvsCache, K_out, V_out, n_out, src_out):
    _same_layout(K, V)
    if K_out.dtype != V_out.dtype:
        raise ValueError("K_out and V_out must share a dtype")
    _check(_lib.kvs_merge_compact(ctypes.byref(cache), dtype_code(K), _ptr(K), _ptr(V), _ptr(n), _ptr(g_self),
                                  _ptr(g_cross), ctypes.byref(rnd), _ptr(sel_state), ctypes.byref(out),
                                  dtype_code(K_out), _ptr(K_out), _ptr(V_out), _ptr(n_out), _ptr(src_out),
                                  _stream()))


def kvs_decode_attn(cache: KvsCache, K, V, n, q, sm_scale: float, out, workspace):
    _same_layout(K, V)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.kvs_decode_attn(ctypes.byref(cache), dtype_code(K), _ptr(K), _ptr(V), _ptr(n), _ptr(q),
                                ctypes.c_float(sm_scale), _ptr(out), _ptr(workspace), ws_bytes, _stream()))


def kvs_decode_attn_static(cache: KvsCache, K, V, n, q, sm_scale: float, out):
    """kvs_decode_attn with the library's static scratch instead of a workspace."""
    _same_layout(K, V)
    _check(_lib.kvs_decode_attn_static(ctypes.byref(cache), dtype_code(K), _ptr(K), _ptr(V), _ptr(n), _ptr(q),
                                       ctypes.c_float(sm_scale), _ptr(out), _stream()))


def kvs_append(cache: KvsCache, K, V, n, at: int, src: KvsCache, K_new, V_new, from_: int, count: int):
    """Copy rows [from_, from_ + count) of K_new/V_new into rows [at, at + count) of K/V, counts 1."""
    _same_layout(K, V)
    _same_layout(K_new, V_new)
    if K.dtype != K_new.dtype:
        raise ValueError("cache and source must share a dtype")
    _check(_lib.kvs_append(ctypes.byref(cache), dtype_code(K), _ptr(K), _ptr(V), _ptr(n), at, ctypes.byref(src),
                           _ptr(K_new), _ptr(V_new), from_, count, _stream()))


def kvs_exact_e_diag(cache: KvsCache, K, V, n, Qw, rnd: KvsRound, E, lse, O, slot_out, pair_out):
    _same_layout(K, V)
    _check(_lib.kvs_exact_e_diag(ctypes.byref(cache), dtype_code(K), _ptr(K), _ptr(V), _ptr(n), _ptr(Qw),
                                 ctypes.byref(rnd), _ptr(E), _ptr(lse), _ptr(O), _ptr(slot_out), _ptr(pair_out),
                                 _stream()))


def kvs_spectral_modes(X, modes, eigvals, proj, contrib, cos):
    """X [T, d] and modes [r, d] bf16 (rows contiguous), eigvals [r] fp32; writes proj [T, r],
    contrib [T - 1, r] (may be None) and cos [T - 1]."""
    if X.dim() != 2 or modes.dim() != 2 or X.stride(1) != 1 or modes.stride(1) != 1 or \
            X.stride(0) != X.shape[1] or modes.stride(0) != modes.shape[1] or X.shape[1] != modes.shape[1]:
        raise ValueError("X [T, d] and modes [r, d] must be contiguous with the same d")
    _check(_lib.kvs_spectral_modes(dtype_code(X), _ptr(X), X.shape[0], X.shape[1], _ptr(modes), _ptr(eigvals),
                                   modes.shape[0], _ptr(proj), _ptr(contrib), _ptr(cos), _stream()))
