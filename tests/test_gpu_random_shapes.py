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


@pytest.mark.parametrize("shape", random_shapes()[:5], ids=lambda s: "T{tokens}-H{hidden}-E{experts}-K{top_k}-I{inter}-S{shared_inter}".format(**s))
def test_random_shape_mx_and_lora(shape):
    """The same random shapes with block-scaled FP8 expert weights (bit for
    bit the bf16 forward on the represented weights) and with LoRA adapters
    of a random rank (forward and every gradient against the oracle)."""
    import workloads.lora as WL
    import workloads.mx as MX
    from tests.test_gpu_lora_backward import full_check
    from tests.test_gpu_mx import gpu_forward_mx, mx_weights, represented_bits
    cfg = W.MoEConfig(name="random", **shape)
    layer = W.make_layer(cfg)
    x = W.tokens(cfg)
    xd = dev_bits(x)
    say(f"case: random shape {shape}, MX weights")
    mxl = MX.mx_layer(layer)
    rep = dict(layer)
    for k in ("w13", "w2", "ws13", "ws2"):
        if mxl[k] is not None:
            rep[k] = represented_bits(*mxl[k])
    g_mx = gpu_forward_mx(cfg, mx_weights(layer, mxl), xd)
    g_bf = gpu_forward(cfg, dev_weights(rep), xd).host()
    for k in ("idx", "sorted_route", "gates", "y", "s", "out32", "out16"):
        if g_bf[k] is None:
            assert g_mx[k] is None, k
            continue
        assert np.array_equal(np.asarray(g_mx[k]).view(np.uint8), np.asarray(g_bf[k]).view(np.uint8)), k
    rank = int(np.random.default_rng(shape["tokens"]).integers(1, 17))
    say(f"case: random shape {shape}, LoRA rank {rank}")
    full_check(cfg, layer, WL.lora_adapters(cfg, rank), x, W.grad_out(cfg))
