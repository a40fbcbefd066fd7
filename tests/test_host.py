"""Host-side checks of the C-ABI library: it loads, exports every declared
symbol, sizes workspaces, and rejects bad arguments before launching anything.
No call here reaches a kernel, so these run without a GPU."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvslim.h")
LIB = os.path.join(ROOT, "long_context_kv_kvslimmer_amd", "libkvslim.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libkvslim.so not built")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvs_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    lib = ctypes.CDLL(LIB)
    names = _declared()
    assert len(names) >= 9
    for name in names:
        assert hasattr(lib, name), name
    from long_context_kv_kvslimmer_amd import kvslim as L
    assert set(L.EXPORTS) == set(names)


@pytest.fixture(scope="module")
def L():
    from long_context_kv_kvslimmer_amd import kvslim
    return kvslim


def test_num_pairs(L):
    assert L.num_pairs(512, 0, 0) == 256
    assert L.num_pairs(32768, 0, 32) == 16368
    assert L.num_pairs(131072, 0, 0) == 65536
    assert L.num_pairs(33, 32, 0) == 0
    assert L.num_pairs(10, 3, 2) == 2
    assert L.num_pairs(-1, 0, 0) == 0
    assert L.version() == 100


def _cache(B=1, H=8, Hq=32, D=128, N=32768, sb=None, sh=None):
    from long_context_kv_kvslimmer_amd import kvslim as L
    sh = N * D if sh is None else sh
    sb = H * sh if sb is None else sb
    return L.KvsCache(B, H, Hq, D, N, sb, sh)


def test_workspace_sizes(L):
    c = _cache()
    r = L.round_desc(32, 0, 32, 16368, 128 ** -0.5)
    assert L.workspace_bytes(L.KVS_OP_SCORE, c, r) > 0
    assert L.workspace_bytes(L.KVS_OP_SELECT, c, r) == 0
    # selection state per (b, h): header + one offset per 64-pair chunk + total (padded to
    # 4 ints), then four 256-bin digit histograms and two counts per chunk
    P = 16368
    chunks = (P + 63) // 64
    per = (((4 + chunks + 1) + 3) // 4 * 4 + 4 * 256 + 2 * chunks + 3) // 4 * 4
    assert L.workspace_bytes(L.KVS_OP_SEL_STATE, c, r) == 8 * per * 4
    assert L.workspace_bytes(L.KVS_OP_DECODE, c, None) > 0
    bad = _cache(D=96)
    assert L.workspace_bytes(L.KVS_OP_SCORE, bad, r) == 0


FAKE = ctypes.c_void_p(4096)   # aligned, never dereferenced: every call below fails validation


def _score(L, c, r, dtype=0, K=FAKE, V=FAKE, Qw=FAKE, lse=FAKE, O=FAKE, gs=FAKE, gc=FAKE, ws=FAKE, wsb=1 << 30):
    return L._lib.kvs_score(ctypes.byref(c) if c is not None else None, dtype, K, V, None, Qw,
                            ctypes.byref(r) if r is not None else None, lse, O, gs, gc, None, ws, wsb, None)


def test_score_validation(L):
    r = L.round_desc(32, 0, 32, 16368, 0.1)
    assert _score(L, None, r) == L.KVS_ERR_NULL
    assert _score(L, _cache(), None) == L.KVS_ERR_NULL
    assert _score(L, _cache(D=96), r) == L.KVS_ERR_SHAPE
    assert _score(L, _cache(Hq=30), r) == L.KVS_ERR_SHAPE
    assert _score(L, _cache(sh=32768 * 128 + 1), r) == L.KVS_ERR_STRIDE
    assert _score(L, _cache(), r, dtype=7) == L.KVS_ERR_DTYPE
    assert _score(L, _cache(), r, K=None) == L.KVS_ERR_NULL
    assert _score(L, _cache(), r, gc=None) == L.KVS_ERR_NULL
    assert _score(L, _cache(), r, K=ctypes.c_void_p(4100)) == L.KVS_ERR_ALIGN
    assert _score(L, _cache(), r, wsb=16) == L.KVS_ERR_WORKSPACE
    assert _score(L, _cache(), L.round_desc(32, 0, 32, 16369, 0.1)) == L.KVS_ERR_INFEASIBLE
    assert _score(L, _cache(), L.round_desc(32, 0, 32, -1, 0.1)) == L.KVS_ERR_INFEASIBLE
    assert _score(L, _cache(), L.round_desc(0, 0, 32, 10, 0.1)) == L.KVS_ERR_SHAPE
    assert _score(L, _cache(), L.round_desc(65537, 0, 32, 10, 0.1)) == L.KVS_ERR_SHAPE
    assert _score(L, _cache(N=0), L.round_desc(32, 0, 0, 0, 0.1)) == L.KVS_ERR_SHAPE
    assert _score(L, _cache(), L.round_desc(32, 0, 32, 10, float("nan"))) == L.KVS_ERR_SHAPE
    assert "n_merge" in L.last_error() or "sm_scale" in L.last_error()


def test_cache_size_limits(L):
    # B * H_q <= 2^20 and B * H_kv * N <= 2^36: checked before anything is sized or launched
    r = L.round_desc(32, 0, 0, 0, 0.1)
    assert _score(L, _cache(B=(1 << 15) + 1, H=8, Hq=32, N=64), r) == L.KVS_ERR_SHAPE
    assert "n_q_heads" in L.last_error()
    assert _score(L, _cache(B=1 << 10, H=1 << 10, Hq=1 << 10, N=(1 << 16) + 1), r) == L.KVS_ERR_SHAPE
    assert "n_slots" in L.last_error()
    assert _score(L, _cache(N=(1 << 31)), r) == L.KVS_ERR_SHAPE
    # at the limits exactly the shape is accepted (the workspace query sizes it)
    assert L.workspace_bytes(L.KVS_OP_DECODE, _cache(B=1 << 15, H=8, Hq=32, N=1 << 18), None) > 0
    assert L.workspace_bytes(L.KVS_OP_DECODE, _cache(B=(1 << 15) + 1, H=8, Hq=32, N=64), None) == 0
    assert L.workspace_bytes(L.KVS_OP_DECODE, _cache(B=1, H=1 << 6, Hq=1 << 6, N=(1 << 31) - 1), None) == 0


def test_merge_weights_validation(L):
    c = _cache()
    r = L.round_desc(32, 0, 32, 100, 0.1)
    f = L._lib.kvs_merge_weights
    assert f(ctypes.byref(c), ctypes.byref(r), FAKE, FAKE, FAKE, None, None, None, 0, None, 0, None) == L.KVS_ERR_NULL
    # a partial round needs the cosine
    assert f(ctypes.byref(c), ctypes.byref(r), FAKE, FAKE, None, None, None, FAKE, 1 << 30, None, 0,
             None) == L.KVS_ERR_NULL
    assert f(ctypes.byref(c), ctypes.byref(r), FAKE, FAKE, FAKE, None, None, FAKE, 16, None, 0,
             None) == L.KVS_ERR_WORKSPACE


def test_merge_compact_validation(L):
    c = _cache()
    r = L.round_desc(32, 0, 32, 16368, 0.1)
    f = L._lib.kvs_merge_compact
    good_out = _cache(N=32768 - 16368, sh=(32768 - 16368) * 128)
    wrong_len = _cache(N=32768 - 16367, sh=(32768 - 16368) * 128)
    wrong_dim = L.KvsCache(1, 8, 32, 64, 32768 - 16368, 8 * 16400 * 64, 16400 * 64)

    def call(out, sel=None, K=FAKE, rr=r, dt=0):
        return f(ctypes.byref(c), 0, K, FAKE, None, FAKE, FAKE, ctypes.byref(rr), sel,
                 ctypes.byref(out) if out is not None else None, dt, FAKE, FAKE, FAKE, FAKE, None)
    assert call(None) == L.KVS_ERR_NULL
    assert call(wrong_len) == L.KVS_ERR_SHAPE
    assert call(wrong_dim) == L.KVS_ERR_SHAPE
    assert call(good_out, K=None) == L.KVS_ERR_NULL
    assert call(good_out, K=ctypes.c_void_p(4104)) == L.KVS_ERR_ALIGN
    assert call(good_out, dt=5) == L.KVS_ERR_DTYPE
    partial = L.round_desc(32, 0, 32, 100, 0.1)
    part_out = _cache(N=32768 - 100, sh=(32768 - 100) * 128)
    assert call(part_out, sel=None, rr=partial) == L.KVS_ERR_NULL     # partial round needs sel_state


def test_decode_validation(L):
    f = L._lib.kvs_decode_attn
    c = _cache()
    assert f(ctypes.byref(c), 0, FAKE, FAKE, None, FAKE, 0.1, FAKE, FAKE, 16, None) == L.KVS_ERR_WORKSPACE
    assert f(ctypes.byref(_cache(Hq=24)), 0, FAKE, FAKE, None, FAKE, 0.1, FAKE, FAKE, 1 << 30,
             None) == L.KVS_ERR_SHAPE   # group 3
    assert f(ctypes.byref(_cache(N=0)), 0, FAKE, FAKE, None, FAKE, 0.1, FAKE, FAKE, 1 << 30,
             None) == L.KVS_ERR_SHAPE
    assert f(ctypes.byref(c), 0, FAKE, FAKE, None, None, 0.1, FAKE, FAKE, 1 << 30, None) == L.KVS_ERR_NULL


def test_status_strings(L):
    for s in range(9):
        assert L.status_str(s).startswith("KVS_")


def test_timing_marks_validation(L):
    lib = L._lib
    assert lib.kvs_marks_begin(0, None) == L.KVS_ERR_SHAPE
    assert lib.kvs_marks_begin(1 << 17, None) == L.KVS_ERR_SHAPE
    assert lib.kvs_marks_begin(4, b"x" * 64) == L.KVS_ERR_SHAPE
    # nothing was marked: no names, no durations
    assert lib.kvs_marks_end() == 0
    assert lib.kvs_mark_name(0) == b""
    assert lib.kvs_mark_ms(0) == -1.0


def test_score_merge_validation(L):
    f = L._lib.kvs_score_merge
    c = L.KvsCache(1, 2, 8, 128, 1000, 2 * 1000 * 128, 1000 * 128)
    o = L.KvsCache(1, 2, 8, 128, 500, 2 * 500 * 128, 500 * 128)
    r_partial = L.round_desc(8, 0, 0, 100, 0.1)
    args = [FAKE, FAKE, None, FAKE]
    # out must hold N - M slots
    assert f(ctypes.byref(c), L.KVS_BF16, *args, ctypes.byref(r_partial), FAKE, FAKE, FAKE, FAKE, ctypes.byref(o),
             L.KVS_BF16, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == L.KVS_ERR_SHAPE
    # a partial round needs room for the cosine and the selection state as well
    o900 = L.KvsCache(1, 2, 8, 128, 900, 2 * 900 * 128, 900 * 128)
    ws_score = L.workspace_bytes(L.KVS_OP_SCORE, c, r_partial)
    ws_part = L.workspace_bytes(L.KVS_OP_SCORE_MERGE, c, r_partial)
    assert ws_part >= ws_score + 2 * 500 * 4
    assert f(ctypes.byref(c), L.KVS_BF16, *args, ctypes.byref(r_partial), FAKE, FAKE, FAKE, FAKE, ctypes.byref(o900),
             L.KVS_BF16, FAKE, FAKE, FAKE, FAKE, FAKE, 16, None) == L.KVS_ERR_WORKSPACE
    r_all = L.round_desc(8, 0, 0, 500, 0.1)
    r_none = L.round_desc(8, 0, 0, 0, 0.1)
    assert L.workspace_bytes(L.KVS_OP_SCORE_MERGE, c, r_all) == L.workspace_bytes(L.KVS_OP_SCORE, c, r_all)
    assert L.workspace_bytes(L.KVS_OP_SCORE_MERGE, c, r_none) == L.workspace_bytes(L.KVS_OP_SCORE, c, r_none)
    r_full = L.round_desc(8, 0, 0, 500, 0.1)
    bad_out = L.KvsCache(1, 2, 8, 128, 499, 2 * 500 * 128, 500 * 128)
    assert f(ctypes.byref(c), L.KVS_BF16, *args, ctypes.byref(r_full), FAKE, FAKE, FAKE, FAKE, ctypes.byref(bad_out),
             L.KVS_BF16, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == L.KVS_ERR_SHAPE
    assert f(ctypes.byref(c), L.KVS_BF16, *args, ctypes.byref(r_full), FAKE, FAKE, FAKE, FAKE, ctypes.byref(o),
             L.KVS_BF16, FAKE, FAKE, None, FAKE, FAKE, 1 << 30, None) == L.KVS_ERR_NULL
    assert f(ctypes.byref(c), L.KVS_BF16, *args, ctypes.byref(r_full), FAKE, FAKE, FAKE, FAKE, ctypes.byref(o),
             L.KVS_BF16, FAKE, FAKE, FAKE, FAKE, FAKE, 16, None) == L.KVS_ERR_WORKSPACE


def test_append_validation(L):
    f = L._lib.kvs_append
    c = L.KvsCache(1, 2, 8, 128, 200, 2 * 200 * 128, 200 * 128)
    src = L.KvsCache(1, 2, 8, 128, 50, 2 * 50 * 128, 50 * 128)
    other = L.KvsCache(1, 4, 8, 128, 50, 4 * 50 * 128, 50 * 128)

    def call(at, frm, count, s=src, K=FAKE, dt=L.KVS_BF16):
        return f(ctypes.byref(c), dt, K, FAKE, None, at, ctypes.byref(s), FAKE, FAKE, frm, count, None)
    assert call(190, 0, 11) == L.KVS_ERR_SHAPE        # past the cache's rows
    assert call(0, 45, 6) == L.KVS_ERR_SHAPE          # past the source's rows
    assert call(0, 0, 5, s=other) == L.KVS_ERR_SHAPE  # different head count
    assert call(-1, 0, 5) == L.KVS_ERR_SHAPE
    assert call(0, 0, 5, K=None) == L.KVS_ERR_NULL
    assert call(0, 0, 5, K=ctypes.c_void_p(4104)) == L.KVS_ERR_ALIGN
    assert call(0, 0, 5, dt=9) == L.KVS_ERR_DTYPE
    assert call(200, 50, 0) == L.KVS_OK               # nothing to write: no launch


def test_score_merge_stats_validation(L):
    f = L._lib.kvs_score_merge_stats
    c = L.KvsCache(1, 2, 8, 128, 1000, 2 * 1000 * 128, 1000 * 128)
    r = L.round_desc(8, 0, 0, 100, 0.1)
    o900 = L.KvsCache(1, 2, 8, 128, 900, 2 * 900 * 128, 900 * 128)
    o500 = L.KvsCache(1, 2, 8, 128, 500, 2 * 500 * 128, 500 * 128)

    def call(out, lse=FAKE, O=FAKE, ws=1 << 30):
        return f(ctypes.byref(c), L.KVS_BF16, FAKE, FAKE, None, FAKE, ctypes.byref(r), lse, O, FAKE, FAKE,
                 ctypes.byref(out), L.KVS_BF16, FAKE, FAKE, FAKE, FAKE, FAKE, ws, None)
    assert call(o500) == L.KVS_ERR_SHAPE                  # out must hold N - M slots
    assert call(o900, lse=None) == L.KVS_ERR_NULL
    assert call(o900, O=ctypes.c_void_p(4100)) == L.KVS_ERR_ALIGN
    assert call(o900, ws=16) == L.KVS_ERR_WORKSPACE
    assert L.workspace_bytes(L.KVS_OP_STATS_MERGE, c, r) > 0


def test_exact_e_diag_validation(L):
    f = L._lib.kvs_exact_e_diag
    r = L.round_desc(8, 0, 0, 0, 0.1)

    def call(c, E=FAKE, pair=FAKE):
        return f(ctypes.byref(c), L.KVS_BF16, FAKE, FAKE, None, FAKE, ctypes.byref(r), E, FAKE, FAKE, FAKE, pair,
                 None)
    assert call(_cache(D=96)) == L.KVS_ERR_SHAPE
    assert call(_cache(), E=None) == L.KVS_ERR_NULL
    assert call(_cache(), pair=None) == L.KVS_ERR_NULL      # P > 0 needs the pair outputs
    assert call(_cache(N=0)) == L.KVS_ERR_SHAPE


def test_spectral_modes_validation(L):
    f = L._lib.kvs_spectral_modes

    def call(dt=L.KVS_BF16, X=FAKE, T=100, d=256, r=16, modes=FAKE, cos=FAKE):
        return f(dt, X, T, d, modes, FAKE, r, FAKE, None, cos, None)
    assert call(dt=L.KVS_F32) == L.KVS_ERR_DTYPE
    assert call(d=96) == L.KVS_ERR_SHAPE                    # d_model a multiple of 64
    assert call(r=0) == L.KVS_ERR_SHAPE
    assert call(T=0) == L.KVS_ERR_SHAPE
    assert call(X=None) == L.KVS_ERR_NULL
    assert call(cos=None) == L.KVS_ERR_NULL
    assert call(modes=ctypes.c_void_p(4104)) == L.KVS_ERR_ALIGN


def test_static_decode_rejects_shapes_beyond_its_scratch(L):
    """kvs_decode_attn_static refuses, before touching the GPU, shapes whose split records
    would not fit the library's static scratch."""
    big = _cache(B=8, H=8, Hq=32, D=128, N=65536)
    assert L.workspace_bytes(L.KVS_OP_DECODE, big, None) > (8 << 20)
    st = L._lib.kvs_decode_attn_static(ctypes.byref(big), 1, FAKE, FAKE, None, FAKE, ctypes.c_float(0.1), FAKE,
                                       None)
    assert st == 7 and "static" in L.last_error()
    st = L._lib.kvs_decode_attn_static(ctypes.byref(big), 1, None, FAKE, None, FAKE, ctypes.c_float(0.1), FAKE, None)
    assert st == 1
    bad = _cache(Hq=24)
    st = L._lib.kvs_decode_attn_static(ctypes.byref(bad), 0, FAKE, FAKE, None, FAKE, ctypes.c_float(0.1), FAKE, None)
    assert st == 2
