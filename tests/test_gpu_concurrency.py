"""Calls on different streams with their own workspaces and outputs share no
state: two forwards (different layers' sizes, different inputs) and two
backwards enqueued on two streams at once, without waiting between them,
give the bits the same calls give one after another."""
import pytest
import torch

import mixture_experts_layer_counting_amd as m
import workloads as W
from tests.gpu_util import DEV, dev_bits, dev_weights, dims_of, gpu_forward, load_cfg, say

pytestmark = pytest.mark.gpu


def bits(t):
    return t.contiguous().view(torch.int32)


def test_concurrent_forwards_on_two_streams():
    cfg, layer, x = load_cfg("moe1k")
    w = dev_weights(layer)
    xs = [dev_bits(x), dev_bits(W.tokens(cfg, 700, stream=W.S_COMPANION, index=27))]
    ref = [gpu_forward(cfg, w, xi) for xi in xs]
    streams = [torch.cuda.Stream() for _ in xs]
    outs = []
    torch.cuda.synchronize()
    say("case: moe1k (1024 and 700 tokens), two streams at once")
    for xi, st in zip(xs, streams):
        d = dims_of(cfg, int(xi.shape[0]))
        r, sv = m.alloc_routes(d, DEV), m.alloc_saved(d, DEV)
        o32 = torch.empty(d.tokens, d.hidden, dtype=torch.float32, device=DEV)
        o16 = torch.empty(d.tokens, d.hidden, dtype=torch.int16, device=DEV)
        ws = m.alloc_workspace(d, m.MOE_OP_FORWARD, DEV)
        st.wait_stream(torch.cuda.current_stream())  # allocations are ordered first
        outs.append((r, sv, o32, o16, ws))
    for (r, sv, o32, o16, ws), xi, st in zip(outs, xs, streams):
        d = dims_of(cfg, int(xi.shape[0]))
        for _ in range(3):  # repeated, so that the two streams' kernels interleave
            m.check(m.moe_forward(d, w, xi, r, sv, o32, o16, ws, st), "moe_forward")
    torch.cuda.synchronize()
    for (r, sv, o32, o16, ws), want in zip(outs, ref):
        assert torch.equal(r.topk_idx, want.routes.topk_idx)
        assert torch.equal(bits(sv.y), bits(want.saved.y))
        assert torch.equal(bits(o32), bits(want.out32))
        assert torch.equal(o16, want.out16)
        assert m.moe_last_device_error(ws) == m.MOE_OK


def test_concurrent_backwards_on_two_streams():
    cfg, layer, x = load_cfg("tiny")
    w = dev_weights(layer)
    d = dims_of(cfg)
    xd = dev_bits(x)
    fwd = gpu_forward(cfg, w, xd, training=True)
    douts = [dev_bits(W.grad_out(cfg)), dev_bits(W.normal_bf16(cfg.seed, W.S_COMPANION, 28, (cfg.tokens, cfg.hidden), 1.0))]

    def alloc():
        return (torch.empty(d.tokens, d.hidden, dtype=torch.float32, device=DEV), m.alloc_grads(d, DEV),
                m.alloc_workspace(d, m.MOE_OP_BACKWARD, DEV))

    ref = []
    for do in douts:
        dx, g, ws = alloc()
        m.check(m.moe_backward(d, w, xd, fwd.routes, fwd.saved, do, dx, None, g, ws), "moe_backward")
        torch.cuda.synchronize()
        ref.append((dx, g))
    streams = [torch.cuda.Stream() for _ in douts]
    outs = [alloc() for _ in douts]
    for st in streams:
        st.wait_stream(torch.cuda.current_stream())
    say("case: tiny backward, two upstream gradients on two streams at once")
    for (dx, g, ws), do, st in zip(outs, douts, streams):
        for _ in range(3):
            m.check(m.moe_backward(d, w, xd, fwd.routes, fwd.saved, do, dx, None, g, ws, st), "moe_backward")
    torch.cuda.synchronize()
    for (dx, g, ws), (rdx, rg) in zip(outs, ref):
        assert torch.equal(bits(dx), bits(rdx))
        for k in ("d_w_router", "d_w13", "d_w2", "d_ws13", "d_ws2", "d_w_sgate"):
            if getattr(g, k) is not None:
                assert torch.equal(bits(getattr(g, k)), bits(getattr(rg, k))), k
        assert m.moe_last_device_error(ws) == m.MOE_OK
