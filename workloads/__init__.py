"""Seeded synthetic inputs for the routed MoE layer.

This module only draws random numbers and lays them out.  It holds none of
the layer's arithmetic (no projection, selection, permutation or expert
math), so the CPU oracle and the HIP path can both consume it without
sharing any computation.

Shapes follow the layer the RL-Kernel pull request 557 page measures (one
Qwen3-Next MoE layer: 512 routed experts, top-10, a shared expert; see its
"What" and "Prior art & reuse decision" sections) and the SkyRL pull
request 2513 page ("What": 512 routed experts, top-10, shared expert).
The pages never print hidden or intermediate sizes, so those come from the
workload table below.  The pages measure on real checkpoint weights, which
are not available; seeded N(0, sigma) tensors of the same shape stand in.

Generator: numpy PCG64 seeded with the entropy triple (seed, stream,
index), standard normal in float32, scaled by sigma; bf16 tensors are the
round-to-nearest-even truncation of that float32 value, stored as uint16
bit patterns.  Every tensor has its own stream, so a tensor never depends on
the shapes of the others, and each expert's weights have their own index.
"""
from __future__ import annotations

import dataclasses
import hashlib
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

# stream ids (one per tensor family)
S_X, S_WR, S_W13, S_W2, S_WS13, S_WS2, S_WSG, S_BIAS, S_DOUT, S_COMPANION = range(10)


@dataclasses.dataclass(frozen=True)
class MoEConfig:
    name: str
    tokens: int
    hidden: int
    experts: int = 512
    top_k: int = 10
    inter: int = 512
    shared_inter: int = 512
    seed: int = 0
    x_sigma: float = 1.0
    w_sigma: float = 0.02
    # Zipf exponent of the per-expert router bias (0 = no bias)
    zipf_s: float = 0.0
    # temperature that scales the Zipf log-ranks into logit units
    zipf_tau: float = 0.0
    # number of lowest-ranked experts the bias switches off entirely
    zipf_off: int = 0
    backward: bool = False

    @property
    def routes(self) -> int:
        return self.tokens * self.top_k


# tau for the skewed workload is calibrated by
# tests/golden/calibrate_skew.py (it calls only the oracle's router): the
# smallest tau on a 0.05 grid for which the busiest expert receives more than
# 2000 routes at 16384 tokens, with the 100 lowest-ranked experts switched off.
SKEW_TAU = 0.15
SKEW_OFF = 100

CONFIGS = {
    "tiny": MoEConfig("tiny", tokens=256, hidden=512, inter=128, shared_inter=128),
    "moe1k": MoEConfig("moe1k", tokens=1024, hidden=2048),
    "moe8k": MoEConfig("moe8k", tokens=8192, hidden=2048),
    "skew16k": MoEConfig("skew16k", tokens=16384, hidden=2048, zipf_s=1.2,
                         zipf_tau=SKEW_TAU, zipf_off=SKEW_OFF),
    "bwd4k": MoEConfig("bwd4k", tokens=4096, hidden=2048, backward=True),
}


def _rng(seed: int, stream: int, index: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64([seed, stream, index]))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest even), returned as uint16 bit patterns.

    Input values are finite normals, so no NaN handling is needed."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def normal_f32(seed: int, stream: int, index: int, shape, sigma: float) -> np.ndarray:
    a = _rng(seed, stream, index).standard_normal(int(np.prod(shape)), dtype=np.float32)
    if sigma != 1.0:
        a *= np.float32(sigma)
    return a.reshape(shape)


def normal_bf16(seed: int, stream: int, index: int, shape, sigma: float) -> np.ndarray:
    return f32_to_bf16_bits(normal_f32(seed, stream, index, shape, sigma))


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def expert_weights(cfg: MoEConfig, first: int = 0, count: int | None = None):
    """W13 [count, 2I, H] and W2 [count, H, I] as bf16 bits for experts
    first .. first+count-1 (rows 0..I-1 of W13 are the gate, I..2I-1 up)."""
    E, H, I = cfg.experts, cfg.hidden, cfg.inter
    count = E - first if count is None else count
    w13 = np.empty((count, 2 * I, H), np.uint16)
    w2 = np.empty((count, H, I), np.uint16)

    def gen(j):
        e = first + j
        w13[j] = normal_bf16(cfg.seed, S_W13, e, (2 * I, H), cfg.w_sigma)
        w2[j] = normal_bf16(cfg.seed, S_W2, e, (H, I), cfg.w_sigma)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(gen, range(count)))
    return w13, w2


def zipf_bias(cfg: MoEConfig) -> np.ndarray | None:
    """Per-expert router bias b_e = -tau * s * ln(rank_e) (float32), where
    rank is a seeded permutation of 1..E.  Adding b to the logits multiplies
    expert e's softmax weight by rank_e^(-s*tau), a Zipf(s) skew whose
    strength tau sets.  The zipf_off lowest-ranked experts get a bias of
    -64 (far beyond the logits' spread), so they receive no route: a
    log-rank bias alone is too flat in its tail to empty experts without
    piling nearly every token onto the head."""
    if cfg.zipf_s == 0.0:
        return None
    rank = _rng(cfg.seed, S_BIAS).permutation(cfg.experts) + 1
    b = -cfg.zipf_tau * cfg.zipf_s * np.log(rank.astype(np.float64))
    if cfg.zipf_off:
        b[rank > cfg.experts - cfg.zipf_off] = -64.0
    return b.astype(np.float32)


def tokens(cfg: MoEConfig, count: int | None = None, stream: int = S_X, index: int = 0):
    """x [count, H] bf16 bits (count defaults to cfg.tokens)."""
    T = cfg.tokens if count is None else count
    return normal_bf16(cfg.seed, stream, index, (T, cfg.hidden), cfg.x_sigma)


def grad_out(cfg: MoEConfig, count: int | None = None):
    """dOut [T, H] bf16 bits, N(0, 1), on its own stream."""
    T = cfg.tokens if count is None else count
    return normal_bf16(cfg.seed, S_DOUT, 0, (T, cfg.hidden), 1.0)


def make_layer(cfg: MoEConfig, with_experts: bool = True) -> dict:
    """All weights of one layer as numpy arrays (bf16 as uint16 bits).

    Keys: w_router [E,H] f32, router_bias [E] f32 or None, w13 [E,2I,H],
    w2 [E,H,I], ws13 [2Is,H], ws2 [H,Is], w_sgate [H]."""
    E, H, I, Is = cfg.experts, cfg.hidden, cfg.inter, cfg.shared_inter
    layer = {
        "w_router": normal_f32(cfg.seed, S_WR, 0, (E, H), cfg.w_sigma),
        "router_bias": zipf_bias(cfg),
        "ws13": normal_bf16(cfg.seed, S_WS13, 0, (2 * Is, H), cfg.w_sigma) if Is else None,
        "ws2": normal_bf16(cfg.seed, S_WS2, 0, (H, Is), cfg.w_sigma) if Is else None,
        "w_sgate": normal_bf16(cfg.seed, S_WSG, 0, (H,), cfg.w_sigma) if Is else None,
    }
    if with_experts:
        layer["w13"], layer["w2"] = expert_weights(cfg)
    return layer


def digest(a: np.ndarray | None) -> str:
    if a is None:
        return "none"
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()[:16]
