"""Seeded synthetic inputs shared by the HIP path and the CPU oracle.

This module holds no arithmetic of the merge method: it only draws keys,
values and queries.  Keys are an AR(1) process across tokens (homogeneous
neighbours), optionally rotated by per-head-phase rotary embeddings; values
and queries are iid N(0, 1) (heterogeneous).  Every draw comes from a
``torch.Generator`` seeded from ``numpy.random.SeedSequence`` over
(config, layer, batch, round, kind), so a tensor is reproducible on its own.
The oracle receives host copies of the very tensors the GPU gets.
"""
from __future__ import annotations

import math

import numpy as np
import torch

KIND = {"K": 0, "V": 1, "Qw": 2, "Qdec": 3, "rho": 4, "phi": 5, "Knew": 6, "Vnew": 7}
TORCH_DTYPE = {"fp32": torch.float32, "bf16": torch.bfloat16}


def seed_for(cfg_idx: int, layer: int, batch: int, rnd: int, kind: str) -> int:
    ss = np.random.SeedSequence([0x4B56, cfg_idx, layer, batch, rnd, KIND[kind]])
    return int(ss.generate_state(1, dtype=np.uint64)[0] & np.uint64(0x7FFFFFFFFFFFFFFF))


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def ar1(n_heads: int, n_tokens: int, dim: int, rho: float, gen: torch.Generator, device,
        block: int = 256, start: torch.Tensor | None = None) -> torch.Tensor:
    """fp32 [H, N, D]: k_0 ~ N(0, I/(1-rho^2)) (or rho*start + eps_0 when
    continuing a sequence), k_t = rho k_{t-1} + eps_t, eps ~ N(0, I).
    Evaluated in 256-step blocks with a lower-triangular Toeplitz matmul."""
    eps = torch.randn(n_heads, n_tokens, dim, generator=gen, device=device, dtype=torch.float32)
    if start is None:
        eps[:, 0] *= 1.0 / math.sqrt(1.0 - rho * rho)
        carry = torch.zeros(n_heads, dim, device=device, dtype=torch.float32)
    else:
        carry = start.to(device=device, dtype=torch.float32)
    t = torch.arange(block, device=device, dtype=torch.float64)
    diff = t[:, None] - t[None, :]
    L = torch.where(diff >= 0, rho ** diff.clamp(min=0), torch.zeros((), dtype=torch.float64, device=device))
    L = L.to(torch.float32).expand(n_heads, block, block).contiguous()
    pw = (rho ** (t + 1)).to(torch.float32)
    out = torch.empty_like(eps)
    for b0 in range(0, n_tokens, block):
        e = eps[:, b0:b0 + block]
        nb = e.shape[1]
        y = torch.bmm(L[:, :nb, :nb].contiguous(), e.contiguous()) + pw[:nb, None] * carry[:, None, :]
        out[:, b0:b0 + nb] = y
        carry = y[:, -1]
    return out


def rope(x: torch.Tensor, pos0: int, theta: float, phase: torch.Tensor) -> torch.Tensor:
    """Rotate-half rotary embedding of fp32 [H, N, D] at positions pos0.. with a
    per-head phase [H, D/2] added to every angle."""
    H, N, D = x.shape
    half = D // 2
    dev = x.device
    pos = torch.arange(pos0, pos0 + N, device=dev, dtype=torch.float64)
    freq = theta ** (-2.0 * torch.arange(half, device=dev, dtype=torch.float64) / D)
    out = torch.empty_like(x)
    for h in range(H):
        ang = pos[:, None] * freq[None, :] + phase[h].to(torch.float64)[None, :]
        c, s = torch.cos(ang).float(), torch.sin(ang).float()
        x1, x2 = x[h, :, :half], x[h, :, half:]
        out[h, :, :half] = x1 * c - x2 * s
        out[h, :, half:] = x1 * s + x2 * c
    return out


def layer_rho(cfg, layer: int) -> float:
    lo, hi = cfg.rho
    if lo == hi:
        return float(lo)
    g = np.random.default_rng(seed_for(cfg.idx, layer, 0, 0, "rho"))
    return float(g.uniform(lo, hi))


def make_cache(cfg, layer: int, batch: int, device, n_tokens: int | None = None):
    """Raw cache of one (layer, batch item): K, V [H_kv, N, D] in the config
    dtype, plus the last pre-rotary fp32 key per head [H_kv, D] (where a decode
    continuation of the AR(1) process starts)."""
    N = cfg.n_slots if n_tokens is None else n_tokens
    H, D = cfg.kv_heads, cfg.head_dim
    rho = layer_rho(cfg, layer)
    k = ar1(H, N, D, rho, _gen(seed_for(cfg.idx, layer, batch, 0, "K"), device), device)
    last = k[:, -1].clone()
    if cfg.rope_theta is not None:
        phase = torch.rand(H, D // 2, generator=_gen(seed_for(cfg.idx, layer, batch, 0, "phi"), device),
                           device=device, dtype=torch.float32) * (2 * math.pi)
        k = rope(k, 0, cfg.rope_theta, phase)
    v = torch.randn(H, N, D, generator=_gen(seed_for(cfg.idx, layer, batch, 0, "V"), device),
                    device=device, dtype=torch.float32)
    dt = TORCH_DTYPE[cfg.dtype]
    return k.to(dt).contiguous(), v.to(dt).contiguous(), last


def window_queries(cfg, layer: int, batch: int, rnd: int, device) -> torch.Tensor:
    """Observation-window queries [H_q, W, D], iid N(0, 1), redrawn per round
    when the config says so."""
    r = rnd if cfg.redraw_window else 0
    q = torch.randn(cfg.q_heads, cfg.window, cfg.head_dim,
                    generator=_gen(seed_for(cfg.idx, layer, batch, r, "Qw"), device),
                    device=device, dtype=torch.float32)
    return q.to(TORCH_DTYPE[cfg.dtype]).contiguous()


def decode_query(cfg, layer: int, batch: int, step: int, device) -> torch.Tensor:
    """Decode query [H_q, D], iid N(0, 1)."""
    q = torch.randn(cfg.q_heads, cfg.head_dim,
                    generator=_gen(seed_for(cfg.idx, layer, batch, 1000 + step, "Qdec"), device),
                    device=device, dtype=torch.float32)
    return q.to(TORCH_DTYPE[cfg.dtype]).contiguous()


def decode_tokens(cfg, layer: int, batch: int, last_raw: torch.Tensor, steps: int, device):
    """Keys and values appended during decode: the AR(1) sequence continued
    from the last pre-merge raw key, rotated at positions N.., values N(0,1).
    Returns K_new, V_new [H_kv, steps, D] in the config dtype."""
    H, D = cfg.kv_heads, cfg.head_dim
    rho = layer_rho(cfg, layer)
    k = ar1(H, steps, D, rho, _gen(seed_for(cfg.idx, layer, batch, 0, "Knew"), device), device,
            start=last_raw.to(device))
    if cfg.rope_theta is not None:
        phase = torch.rand(H, D // 2, generator=_gen(seed_for(cfg.idx, layer, batch, 0, "phi"), device),
                           device=device, dtype=torch.float32) * (2 * math.pi)
        k = rope(k, cfg.n_slots, cfg.rope_theta, phase)
    v = torch.randn(H, steps, D, generator=_gen(seed_for(cfg.idx, layer, batch, 0, "Vnew"), device),
                    device=device, dtype=torch.float32)
    dt = TORCH_DTYPE[cfg.dtype]
    return k.to(dt).contiguous(), v.to(dt).contiguous()
