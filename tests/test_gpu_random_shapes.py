"""Seeded random shapes within the supported ranges, each through the GPU
forward and backward against the FP64 oracle on every token and every
gradient: T in 1..300, E a multiple of 64 up to 1024, K 1..16, H a multiple
of 256 up to 1024, I and Is multiples of 128 up to 512 (Is may be 0).  The
forward is held to the layer's rule (routes exact, fp32 ties forced); the
backward to the same rule against the oracle fed the GPU's saved fp32
forward values (the kernels' own error) and, where that fed oracle itself
meets the rule, against the plain oracle too."""
import numpy as np
import pytest

import workloads as W
from tests.gpu_util import check_forward, dev_bits, dev_weights, gpu_forward, say
from tests.test_gpu_backward import full_backward_check

pytestmark = pytest.mark.gpu


def random_shapes(n=10, seed=2026):
    rng = np.random.default_rng(seed)
    shapes = []
    for _ in range(n):
        E = int(rng.integers(1, 17)) * 64
        shapes.append(dict(tokens=int(rng.integers(1, 301)), hidden=int(rng.integers(1, 5)) * 256, experts=E,
                           top_k=int(rng.integers(1, min(16, E) + 1)), inter=int(rng.integers(1, 5)) * 128,
                           shared_inter=int(rng.choice([0, 128, 256, 384, 512]))))
    return shapes


@pytest.mark.parametrize("shape", random_shapes(), ids=lambda s: "T{tokens}-H{hidden}-E{experts}-K{top_k}-I{inter}-S{shared_inter}".format(**s))
def test_random_shape_forward_and_backward(shape):
    cfg = W.MoEConfig(name="random", **shape)
    layer = W.make_layer(cfg)
    x = W.tokens(cfg)
    say(f"case: random shape {shape}")
    g = gpu_forward(cfg, dev_weights(layer), dev_bits(x)).host()
    check_forward(cfg, layer, x, g)
    full_backward_check(cfg, layer, x, W.grad_out(cfg))
