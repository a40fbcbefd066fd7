"""GPU: kvs_exact_e_diag (exact-gradient scalars, both closed-form weight pairs and the
exact second-order loss of each merged key) against the oracle's exact_e_diagnostics on
the same inputs, with the oracle's own window statistics (rounded to fp32) given to both."""
import math
import zlib

import numpy as np
import pytest
import torch

from oracle import kvs_oracle as O
from tests.parity import REL_TOL, elemrel, host, maxrel
from tests.test_gpu_parity import make_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"

CASES = [
    # name, B, Hkv, Hq, D, N, W, S, R, dtype, counts
    ("f32-d64-g1-counts", 1, 1, 1, 64, 200, 8, 2, 3, torch.float32, True),
    ("bf16-d128-g4", 1, 2, 8, 128, 300, 8, 0, 0, torch.bfloat16, False),
    ("bf16-d64-g2-odd-counts", 2, 1, 2, 64, 129, 16, 1, 0, torch.bfloat16, True),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_exact_e_diag_against_oracle(case):
    from long_context_kv_kvslimmer_amd import pipeline
    name, B, Hkv, Hq, D, N, W, S, R, dtype, counts = case
    print(f"\n[diag] {name}", flush=True)
    G = Hq // Hkv
    K, V, n, Qw = make_inputs(zlib.crc32(name.encode()) % 10000, B, Hkv, Hq, D, N, N, W, dtype, counts)
    g = torch.Generator().manual_seed(9)
    E = torch.randn(B, Hq, W, D, generator=g, dtype=torch.float32)
    scale = 1 / math.sqrt(D)
    lse = torch.empty(B, Hq, W, dtype=torch.float32)
    Ow = torch.empty(B, Hq, W, D, dtype=torch.float32)
    sl = {}
    for b in range(B):
        for h in range(Hkv):
            Ks, Vs = host(K[b, h, :N]), host(V[b, h, :N])
            ns = None if n is None else host(n[b, h, :N]).astype(np.int64)
            Qs = host(Qw[b, h * G:(h + 1) * G]).reshape(-1, D)
            l, _, o = O.window_statistics(Ks, Vs, ns, Qs, scale)
            lse[b, h * G:(h + 1) * G] = torch.from_numpy(l.reshape(G, W)).float()
            Ow[b, h * G:(h + 1) * G] = torch.from_numpy(o.reshape(G, W, D)).float()
            sl[(b, h)] = (Ks, Vs, ns, Qs)
    slot, pair = pipeline.exact_e_diag(K, V, n, Qw, E.to(DEV), lse.to(DEV), Ow.to(DEV), Hq, W, S, R, n_slots=N)
    torch.cuda.synchronize()
    P = O.num_pairs(N, S, R)
    for (b, h), (Ks, Vs, ns, Qs) in sl.items():
        d = O.exact_e_diagnostics(Ks, Vs, ns, Qs, host(E[b, h * G:(h + 1) * G]).reshape(-1, D),
                                  host(lse[b, h * G:(h + 1) * G]).reshape(-1),
                                  host(Ow[b, h * G:(h + 1) * G]).reshape(-1, D), scale, S, R)
        so, po = host(slot[b, h]), host(pair[b, h])
        # element by element: the signed exact scalars against the sum of their terms'
        # magnitudes (sum |E| |c|), the norm sums against themselves
        for col, key, mag in ((0, "g_self_e", "n_self_e"), (1, "n_self_e", None), (2, "g_self", None)):
            e = elemrel(so[:, col], d[key], None if mag is None else d[mag])
            assert e <= REL_TOL, f"{name} b{b} h{h} {key} {e}"
        for col, key, mag in ((0, "g_cross_e", "n_cross_e"), (1, "n_cross_e", None), (2, "g_cross", None)):
            e = elemrel(po[:, col], d[key], None if mag is None else d[mag])
            assert e <= REL_TOL, f"{name} b{b} h{h} {key} {e}"
        m = S + 2 * np.arange(P)
        g11, g12, g22 = d["g_self_e"][m], d["g_cross_e"], d["g_self_e"][m + 1]
        den, sc = g11 + 2 * g12 + g22, np.abs(g11) + 2 * np.abs(g12) + np.abs(g22)
        ok_e = np.abs(den) > 1e-2 * sc                       # away from the degenerate switch
        A = d["g_self"][m] - 2 * d["g_cross"] + d["g_self"][m + 1]
        scf = d["g_self"][m] + 2 * d["g_cross"] + d["g_self"][m + 1]
        ok_f = np.abs(A - 1e-6 * scf) > 1e-3 * np.abs(scf)
        assert ok_e.sum() > P // 2
        assert maxrel(po[ok_e, 3:5], d["w_exact"][ok_e]) <= REL_TOL, f"{name} exact weights"
        assert maxrel(po[ok_f, 5:7], d["w_fwd"][ok_f]) <= REL_TOL, f"{name} forward-only weights"
        both = ok_e & ok_f
        assert maxrel(po[both, 7], d["loss_exact"][both]) <= REL_TOL, f"{name} exact loss"
        assert maxrel(po[both, 8], d["loss_fwd"][both]) <= REL_TOL, f"{name} forward-only loss"
