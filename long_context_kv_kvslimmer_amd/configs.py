"""The seeded synthetic workloads the merge path is checked and measured on.

Shapes follow the Llama-3.1-8B KV layout the KVSlimmer deep-dive
(charles2530.github.io, section 算一遍) uses for its byte count: 32 layers,
8 KV heads, head_dim 128, bf16; the Mistral-7B cache has the same KV shape.
"""
from __future__ import annotations

from dataclasses import dataclass


@dataclass(frozen=True)
class Config:
    idx: int
    name: str
    batch: int
    layers: int
    kv_heads: int
    q_heads: int
    head_dim: int
    n_slots: int
    dtype: str                 # "fp32" | "bf16"
    window: int                # observation-window queries per query head
    n_sink: int
    n_recent: int
    rounds: tuple              # merges per round (per batch, layer, kv-head)
    rho: tuple                 # (lo, hi): per-layer AR(1) coefficient ~ U[lo, hi]; lo == hi fixed
    rope_theta: float | None   # None: no rotary embedding on the synthetic keys
    decode_steps: int = 0
    redraw_window: bool = True  # fresh window queries every round
    budget: int = 0            # > 0: chunked prefill under this cache budget (slots per head)
    chunk: int = 0             # tokens appended per chunk in that regime

    @property
    def group(self) -> int:
        return self.q_heads // self.kv_heads

    def slots_after(self, r: int) -> int:
        """Slots per (batch, layer, head) after ``r`` rounds."""
        return self.n_slots - sum(self.rounds[:r])


C1 = Config(1, "tiny-fp32", batch=1, layers=1, kv_heads=1, q_heads=1, head_dim=64, n_slots=512,
            dtype="fp32", window=16, n_sink=0, n_recent=0, rounds=(256,), rho=(0.9, 0.9),
            rope_theta=None)
C2 = Config(2, "llama8b-layer-32k", batch=1, layers=1, kv_heads=8, q_heads=32, head_dim=128,
            n_slots=32768, dtype="bf16", window=32, n_sink=0, n_recent=32, rounds=(16368,),
            rho=(0.9, 0.9), rope_theta=5.0e5)
C3 = Config(3, "llama8b-32L-128k-29pct", batch=1, layers=32, kv_heads=8, q_heads=32, head_dim=128,
            n_slots=131072, dtype="bf16", window=32, n_sink=0, n_recent=0, rounds=(38011,),
            rho=(0.7, 0.95), rope_theta=5.0e5)
C4 = Config(4, "mistral7b-b8-32k-3x2", batch=8, layers=32, kv_heads=8, q_heads=32, head_dim=128,
            n_slots=32768, dtype="bf16", window=32, n_sink=0, n_recent=0, rounds=(16384, 8192, 4096),
            rho=(0.9, 0.9), rope_theta=1.0e6)
C5 = Config(5, "llama8b-128k-4x-decode", batch=1, layers=32, kv_heads=8, q_heads=32, head_dim=128,
            n_slots=131072, dtype="bf16", window=32, n_sink=0, n_recent=0, rounds=(65536, 32768),
            rho=(0.9, 0.9), rope_theta=5.0e5, decode_steps=128)

# The evaluation regime of the deep-dive's 实验设置: the prompt is prefilled in chunks of
# 512 tokens into a cache of at most 2048 slots per head, the first 32 tokens never merge.
# All 32 layers of the model are folded into the batch dimension, so one round per chunk
# covers the whole model.
C6 = Config(6, "llama8b-32L-stream-32k-budget2048-chunk512", batch=1, layers=32, kv_heads=8, q_heads=32,
            head_dim=128, n_slots=32768, dtype="bf16", window=32, n_sink=32, n_recent=0, rounds=(),
            rho=(0.7, 0.95), rope_theta=5.0e5, budget=2048, chunk=512)

CONFIGS = {c.idx: c for c in (C1, C2, C3, C4, C5, C6)}
