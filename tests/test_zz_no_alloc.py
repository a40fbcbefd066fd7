"""GPU: kvs_decode_attn_static (the decode with the library's static scratch, for callers
that cannot allocate) against kvs_decode_attn with a caller workspace, bit for bit, over
several calls in a row whose inputs shrink and grow again (the scratch keeps the last
call's records), and against the oracle on sampled heads."""
import math

import numpy as np
import pytest
import torch

from oracle import kvs_oracle as O
from tests.parity import REL_TOL, host, maxrel

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _inputs(seed, B, Hkv, Hq, D, N, dtype, counts):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    K = torch.randn(B, Hkv, N, D, generator=g, device=DEV).to(dtype)
    V = torch.randn(B, Hkv, N, D, generator=g, device=DEV).to(dtype)
    q = torch.randn(B, Hq, D, generator=g, device=DEV).to(dtype)
    n = torch.randint(1, 5, (B, Hkv, N), generator=g, device=DEV, dtype=torch.int32) if counts else None
    return K, V, n, q


CALLS = [
    # B, Hkv, Hq, D, N, dtype, counts
    (1, 8, 32, 128, 40000, torch.bfloat16, True),
    (1, 2, 8, 64, 3001, torch.bfloat16, False),      # smaller than the call before
    (2, 2, 4, 128, 5000, torch.float32, True),
    (1, 1, 8, 128, 77, torch.bfloat16, True),        # a single split
    (1, 8, 32, 128, 32800, torch.bfloat16, False),
]


def test_static_scratch_decode_matches_workspace_decode():
    from long_context_kv_kvslimmer_amd import kvslim as L
    for i, (B, Hkv, Hq, D, N, dtype, counts) in enumerate(CALLS):
        print(f"\n[static decode] call {i}: B={B} Hkv={Hkv} Hq={Hq} D={D} N={N} {dtype} counts={counts}", flush=True)
        K, V, n, q = _inputs(100 + i, B, Hkv, Hq, D, N, dtype, counts)
        cache = L.cache_desc(K, Hq, N)
        scale = 1.0 / math.sqrt(D)
        ws = torch.empty(max(L.workspace_bytes(L.KVS_OP_DECODE, cache, None), 16), dtype=torch.uint8, device=DEV)
        ref = torch.empty(B, Hq, D, dtype=torch.float32, device=DEV)
        got = torch.full((B, Hq, D), float("nan"), dtype=torch.float32, device=DEV)
        L.kvs_decode_attn(cache, K, V, n, q, scale, ref, ws)
        L.kvs_decode_attn_static(cache, K, V, n, q, scale, got)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), f"call {i}: {(got != ref).sum().item()} elements differ"
        for b, hq in ((0, 0), (B - 1, Hq - 1)):
            h = hq // (Hq // Hkv)
            ns = None if n is None else host(n[b, h])
            r = O.decode(host(K[b, h]), host(V[b, h]), ns, host(q[b, hq]), scale)
            assert maxrel(host(got[b, hq]), r) <= REL_TOL, f"call {i} b{b} hq{hq}"
        assert np.isfinite(host(got)).all()
