"""Worst-case routing through the C ABI: every token's K routes go to the same
K experts, in a per-token slot order, given as replayed routes.

The layer's routing step (top-k, then the renormalised gates) is replaced by
caller-supplied ids; the gates are the renormalised softmax of the router's
own logits over those ids, computed by the oracle.  Each of the K experts then
holds T routes while every other expert is empty: the up projection's
balanced tiles, the down projection's row tiles, the backward's row tiles and
the weight-gradient segments all run at their maximum count for one expert,
and the weight gradients take the path for segments too long to stage their
token ids on chip.  Checks:

  - the permutation is the oracle's counting sort, bit for bit;
  - the 256-token and the 4096-token layer (hidden 2048, intermediate 512):
    route rows, output and every gradient against the oracle in full (cheap
    here, with only K experts holding routes), zero weight gradients for the
    empty experts, and at 4096 tokens the output and dX of sampled tokens
    bit-identical to a small batch of those tokens with the same routes (the
    contract's batch invariance at maximum load);
  - the 8192-token layer: route rows and output in full.

At 4096 tokens the router gradient of a loaded expert is a sum of 4096
terms that largely cancel; the fp32 forward values alone (the oracle fed
them) already move it beyond the layer's rule, so that one check takes
assert_grad_close's split, as the hidden-16384 edge shape does.
"""
import numpy as np
import pytest
import torch

import mixture_experts_layer_counting_amd as m
import oracle as O
import workloads as W
from tests.gpu_util import (DEV, assert_close, bf16_rne_bits, dev_bits, dev_weights, dims_of, fed_forward,
                            load_cfg, say)
from tests.test_gpu_backward import GRADS, assert_grad_close

pytestmark = pytest.mark.gpu


def concentrated_routes(T, E, K, seed):
    """K fixed expert ids (the first and last expert among them), each token
    taking all of them in its own seeded slot order."""
    rng = np.random.default_rng(seed)
    fixed = np.concatenate([[0, E - 1], rng.choice(np.arange(1, E - 1), K - 2, replace=False)])
    order = np.argsort(rng.random((T, K)), axis=1)
    return fixed[order].astype(np.int32)


def replay_forward(cfg, w, xd, idx, gates, training=False, ws=None):
    """moe_permute -> moe_grouped_ffn -> moe_combine on caller routes."""
    d = dims_of(cfg, int(xd.shape[0]))
    if ws is None:
        ws = m.alloc_workspace(d, m.MOE_OP_BACKWARD if training else m.MOE_OP_FORWARD, DEV)
    routes = m.alloc_routes(d, DEV, logits=False)
    saved = m.alloc_saved(d, DEV, training)
    routes.topk_idx.copy_(torch.from_numpy(np.ascontiguousarray(idx, np.int32)))
    routes.topk_gate.copy_(torch.from_numpy(np.ascontiguousarray(gates, np.float32)))
    out32 = torch.empty(d.tokens, d.hidden, dtype=torch.float32, device=DEV)
    out16 = torch.empty(d.tokens, d.hidden, dtype=torch.int16, device=DEV)
    m.check(m.moe_permute(d, routes, ws), "moe_permute")
    m.check(m.moe_grouped_ffn(d, xd, w, routes, saved, ws), "moe_grouped_ffn")
    m.check(m.moe_combine(d, routes, saved, out32, out16), "moe_combine")
    torch.cuda.synchronize()
    assert m.moe_last_device_error(ws) == m.MOE_OK
    return routes, saved, out32, out16, ws


def replay_backward(cfg, w, xd, routes, saved, dout_d, ws):
    d = dims_of(cfg, int(xd.shape[0]))
    grads = m.alloc_grads(d, DEV)
    dx32 = torch.empty(d.tokens, d.hidden, dtype=torch.float32, device=DEV)
    dx16 = torch.empty(d.tokens, d.hidden, dtype=torch.int16, device=DEV)
    m.check(m.moe_backward(d, w, xd, routes, saved, dout_d, dx32, dx16, grads, ws), "moe_backward")
    torch.cuda.synchronize()
    assert m.moe_last_device_error(ws) == m.MOE_OK
    return dx32, dx16, grads


def check_permutation(routes, idx, E):
    off, srt, pos = O.permute_routes(idx, E)
    assert np.array_equal(routes.expert_offsets.cpu().numpy(), off)
    assert np.array_equal(routes.sorted_route.cpu().numpy(), srt)
    assert np.array_equal(routes.route_pos.cpu().numpy(), pos)


def u32(t):
    return t.contiguous().view(torch.int32)


def full_check(cfg, layer, x, idx):
    """Forward and backward on replayed routes, every output and gradient
    compared with the oracle in full (cheap here: only K experts have
    routes).  Returns the device tensors for further checks."""
    logits = O.router_logits(x, layer["w_router"], layer.get("router_bias"))
    g32 = O.route_gates(logits, idx).astype(np.float32)
    w = dev_weights(layer)
    xd = dev_bits(x)
    routes, saved, out32, out16, ws = replay_forward(cfg, w, xd, idx, g32, training=True)
    check_permutation(routes, idx, cfg.experts)
    # the oracle is run on the fp32 gates the kernels were given
    ref = O.forward(layer, x, cfg.top_k, forced_idx=idx)
    ref["gates"] = g32.astype(np.float64)
    ref["out"] = O.combine(ref["y"], ref["gates"], ref.get("s"), ref.get("sg"))
    assert_close(saved.y.cpu().numpy(), ref["y"], "route rows Y")
    assert_close(out32.cpu().numpy(), ref["out"], "out_f32")
    assert np.array_equal(out16.cpu().numpy().view(np.uint16), bf16_rne_bits(out32.cpu().numpy()))
    dout = W.grad_out(cfg)
    dx32, dx16, gr = replay_backward(cfg, w, xd, routes, saved, dev_bits(dout), ws)
    bref = O.backward(layer, x, ref, dout)
    fed = O.backward(layer, x, fed_forward(layer, x, idx, g32, saved.gu.cpu().numpy(),
                                           routes.route_pos.cpu().numpy(), saved.shared_gu.cpu().numpy(),
                                           saved.shared_gate.cpu().numpy()), dout)
    dx = dx32.cpu().numpy()
    assert_grad_close(dx, bref["dx"], fed["dx"], "dX")
    assert np.array_equal(dx16.cpu().numpy().view(np.uint16), bf16_rne_bits(dx))
    for key in GRADS:
        assert_grad_close(getattr(gr, key).cpu().numpy(), bref[key], fed[key], key)
    # experts without routes get exact zero weight gradients
    empty = torch.from_numpy(np.setdiff1d(np.arange(cfg.experts), np.unique(idx))).to(DEV)
    for key in ("d_w13", "d_w2", "d_w_router"):
        assert not getattr(gr, key)[empty].any(), f"{key} of an expert without routes is not zero"
    return w, g32, dout, out32, dx32


def test_tiny_concentrated_full():
    cfg, layer, x = load_cfg("tiny")
    say("case: tiny, all routes on 10 experts, forward + backward in full")
    full_check(cfg, layer, x, concentrated_routes(cfg.tokens, cfg.experts, cfg.top_k, seed=31))


def test_bwd4k_concentrated_full_and_batch_invariant():
    cfg, layer, x = load_cfg("bwd4k")
    T, K = cfg.tokens, cfg.top_k
    say(f"case: bwd4k, all {T * K} routes on 10 experts ({T} routes each), forward + backward in full")
    idx = concentrated_routes(T, cfg.experts, K, seed=32)
    w, g32, dout, out32, dx32 = full_check(cfg, layer, x, idx)
    rng = np.random.default_rng(12)
    tok = np.unique(np.concatenate([[0, 1, 95, 96, 127, 128, 2047, T - 1], rng.choice(T, 24, replace=False)]))
    say(f"  {len(tok)} sampled tokens alone, same routes: output and dX bit for bit")
    xs = dev_bits(x[tok])
    r2, s2, o2, _, ws2 = replay_forward(cfg, w, xs, idx[tok], g32[tok], training=True)
    dx2 = replay_backward(cfg, w, xs, r2, s2, dev_bits(dout[tok]), ws2)[0]
    tdev = torch.from_numpy(tok).to(DEV)
    assert torch.equal(u32(o2), u32(out32[tdev])), "output of the sampled tokens depends on the batch"
    assert torch.equal(u32(dx2), u32(dx32[tdev])), "dX of the sampled tokens depends on the batch"


def test_moe8k_concentrated_forward_full():
    cfg, layer, x = load_cfg("moe8k")
    T, K = cfg.tokens, cfg.top_k
    say(f"case: moe8k, all {T * K} routes on 10 experts, forward in full")
    idx = concentrated_routes(T, cfg.experts, K, seed=33)
    logits = O.router_logits(x, layer["w_router"], layer.get("router_bias"))
    g32 = O.route_gates(logits, idx).astype(np.float32)
    w = dev_weights(layer)
    routes, saved, out32, _, _ = replay_forward(cfg, w, dev_bits(x), idx, g32)
    check_permutation(routes, idx, cfg.experts)
    ref = O.forward(layer, x, K, forced_idx=idx)
    assert_close(saved.y.cpu().numpy(), ref["y"], "route rows Y")
    assert_close(out32.cpu().numpy(), O.combine(ref["y"], g32.astype(np.float64), ref.get("s"), ref.get("sg")),
                 "out_f32")
