"""Seeded LoRA adapters for the routed experts (input generation only).

Each routed expert e gets four bf16 matrices, each from its own stream of
the layer's seed with index e, N(0, sigma) like the layer's weights:
  a13 [rank, H]    shrink of the gate/up projection
  b13 [2I, rank]   expand of the gate/up projection
  a2  [rank, I]    shrink of the down projection
  b2  [H, rank]    expand of the down projection
B is drawn nonzero (an adapter after training; LoRA starts B at zero, which
would make the update vanish).  The scale multiplies the update as given.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor

import numpy as np

from . import MoEConfig, _threads, normal_bf16

S_LORA_A13, S_LORA_B13, S_LORA_A2, S_LORA_B2 = range(10, 14)

# Adapter of rank 64 over a router with top-10: rank 64 // 10 = 6 per
# expert; alpha 32 over r 64.
DEFAULT_RANK = 6
DEFAULT_SCALE = 0.5


def lora_adapters(cfg: MoEConfig, rank: int = DEFAULT_RANK, scale: float = DEFAULT_SCALE,
                  sigma: float | None = None) -> dict:
    E, H, I = cfg.experts, cfg.hidden, cfg.inter
    sig = cfg.w_sigma if sigma is None else sigma
    out = {
        "a13": np.empty((E, rank, H), np.uint16),
        "b13": np.empty((E, 2 * I, rank), np.uint16),
        "a2": np.empty((E, rank, I), np.uint16),
        "b2": np.empty((E, H, rank), np.uint16),
        "rank": rank,
        "scale": float(scale),
    }

    def gen(e):
        out["a13"][e] = normal_bf16(cfg.seed, S_LORA_A13, e, (rank, H), sig)
        out["b13"][e] = normal_bf16(cfg.seed, S_LORA_B13, e, (2 * I, rank), sig)
        out["a2"][e] = normal_bf16(cfg.seed, S_LORA_A2, e, (rank, I), sig)
        out["b2"][e] = normal_bf16(cfg.seed, S_LORA_B2, e, (H, rank), sig)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(gen, range(E)))
    return out
