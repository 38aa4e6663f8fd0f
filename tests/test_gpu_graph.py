"""The forward and the backward under HIP graph capture: captured once,
replayed several times with other eager work and synchronisations between
the replays, every replay bit-identical to an eager call (the library
enqueues only kernel launches on the caller's stream: no memset, no
allocation, no host sync).  Also for moe_forward_noalloc, whose callers are
the ones that capture, for the LoRA backward, for the forwards with FP8
expert weights and with LoRA adapters, and for the four stage calls
captured as one graph."""
import pytest
import torch

import mixture_experts_layer_counting_amd as m
import workloads as W
from tests.gpu_util import DEV, dev_bits, dev_weights, dims_of, gpu_forward, load_cfg, say

pytestmark = pytest.mark.gpu


def bits(t):
    return t.contiguous().view(torch.int32)


@pytest.mark.parametrize("name,noalloc", [("tiny", False), ("moe1k", False), ("moe1k", True)])
def test_forward_graph_replays_match_eager(name, noalloc):
    cfg, layer, x = load_cfg(name)
    w = dev_weights(layer)
    xd = dev_bits(x)
    other = dev_bits(W.tokens(cfg, stream=W.S_COMPANION, index=21))
    d = dims_of(cfg)
    routes = m.alloc_routes(d, DEV)
    saved = m.alloc_saved(d, DEV)
    out32 = torch.empty(d.tokens, d.hidden, dtype=torch.float32, device=DEV)
    out16 = torch.empty(d.tokens, d.hidden, dtype=torch.int16, device=DEV)
    ws = m.alloc_workspace(d, m.MOE_OP_FORWARD, DEV)
    xin = xd.clone()

    def fwd(stream):
        if noalloc:
            return m.moe_forward_noalloc(d, w, xin, routes, saved, out32, out16, stream)
        return m.moe_forward(d, w, xin, routes, saved, out32, out16, ws, stream)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        m.check(fwd(s), "warm-up")  # also looks up the no-alloc array before capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    say(f"case: {name}, capture {'moe_forward_noalloc' if noalloc else 'moe_forward'}")
    with torch.cuda.graph(graph, stream=s):
        m.check(fwd(torch.cuda.current_stream()), "captured forward")
    ref = gpu_forward(cfg, w, xd)
    ref_other = gpu_forward(cfg, w, other)
    for i in range(4):
        xin.copy_(other if i % 2 else xd)
        out32.zero_()
        graph.replay()
        torch.cuda.synchronize()
        want = ref_other if i % 2 else ref
        assert torch.equal(routes.topk_idx, want.routes.topk_idx), f"replay {i}: routes"
        assert torch.equal(bits(saved.y), bits(want.saved.y)), f"replay {i}: route rows"
        assert torch.equal(bits(out32), bits(want.out32)), f"replay {i}: out_f32"
        assert torch.equal(out16, want.out16), f"replay {i}: out_bf16"
        # eager work between replays
        gpu_forward(cfg, w, other if i % 2 else xd)


GRADS = ("d_w_router", "d_w13", "d_w2", "d_ws13", "d_ws2", "d_w_sgate")


@pytest.mark.parametrize("lora", [False, True])
def test_backward_graph_replays_match_eager(lora):
    """moe_backward (and moe_backward_lora) captured once on the tiny layer
    and replayed four times with a different upstream gradient on every
    other replay and eager backwards between the replays: every replay's dX
    and weight (and adapter) gradients equal an eager backward's bits."""
    import workloads.lora as WL
    cfg, layer, x = load_cfg("tiny")
    w = dev_weights(layer)
    xd = dev_bits(x)
    d = dims_of(cfg)
    ws = m.alloc_workspace(d, m.MOE_OP_BACKWARD_LORA, DEV)
    lo = None
    if lora:
        ad = WL.lora_adapters(cfg)
        lo = m.Lora(rank=ad["rank"], scale=ad["scale"], a13=dev_bits(ad["a13"]), b13=dev_bits(ad["b13"]),
                    a2=dev_bits(ad["a2"]), b2=dev_bits(ad["b2"]))
    routes = m.alloc_routes(d, DEV)
    saved = m.alloc_saved(d, DEV, training=True)
    out16 = torch.empty(d.tokens, d.hidden, dtype=torch.int16, device=DEV)
    if lora:
        m.check(m.moe_forward_lora(d, w, lo, xd, routes, saved, None, out16, ws), "moe_forward_lora")
    else:
        m.check(m.moe_forward(d, w, xd, routes, saved, None, out16, ws), "moe_forward")
    dout_a = dev_bits(W.grad_out(cfg))
    dout_b = dev_bits(W.normal_bf16(cfg.seed, W.S_COMPANION, 22, (cfg.tokens, cfg.hidden), 1.0))
    din = dout_a.clone()

    def alloc():
        g = m.alloc_grads(d, DEV)
        lg = m.alloc_lora_grads(d, lo.rank, DEV) if lora else None
        return torch.empty(d.tokens, d.hidden, dtype=torch.float32, device=DEV), g, lg

    def bwd(dout, dx, g, lg, stream):
        if lora:
            return m.moe_backward_lora(d, w, lo, xd, routes, saved, dout, dx, None, g, lg, ws, stream)
        return m.moe_backward(d, w, xd, routes, saved, dout, dx, None, g, ws, stream)

    def eager(dout):
        dx, g, lg = alloc()
        m.check(bwd(dout, dx, g, lg, None), "eager backward")
        torch.cuda.synchronize()
        return dx, g, lg

    ref = {0: eager(dout_a), 1: eager(dout_b)}
    dx, g, lg = alloc()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        m.check(bwd(din, dx, g, lg, s), "warm-up")
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    say(f"case: tiny, capture {'moe_backward_lora' if lora else 'moe_backward'}")
    with torch.cuda.graph(graph, stream=s):
        m.check(bwd(din, dx, g, lg, torch.cuda.current_stream()), "captured backward")
    for i in range(4):
        din.copy_(dout_b if i % 2 else dout_a)
        dx.zero_()
        graph.replay()
        torch.cuda.synchronize()
        rdx, rg, rlg = ref[i % 2]
        assert torch.equal(bits(dx), bits(rdx)), f"replay {i}: dX"
        for k in GRADS:
            if getattr(g, k) is not None:
                assert torch.equal(bits(getattr(g, k)), bits(getattr(rg, k))), f"replay {i}: {k}"
        if lora:
            for k in ("d_a13", "d_b13", "d_a2", "d_b2"):
                assert torch.equal(bits(getattr(lg, k)), bits(getattr(rlg, k))), f"replay {i}: {k}"
        eager(dout_a if i % 2 else dout_b)
    assert m.moe_last_device_error(ws) == m.MOE_OK


def test_backward_side_streams_graph_replays_match_eager():
    """moe_backward_side captured on a stream: its fork and join events pull
    the two side streams into the capture; four replays with alternating
    upstream gradients equal eager moe_backward bit for bit."""
    cfg, layer, x = load_cfg("tiny")
    w = dev_weights(layer)
    xd = dev_bits(x)
    d = dims_of(cfg)
    ws = m.alloc_workspace(d, m.MOE_OP_BACKWARD, DEV)
    routes = m.alloc_routes(d, DEV)
    saved = m.alloc_saved(d, DEV, training=True)
    out16 = torch.empty(d.tokens, d.hidden, dtype=torch.int16, device=DEV)
    m.check(m.moe_forward(d, w, xd, routes, saved, None, out16, ws), "moe_forward")
    dout_a = dev_bits(W.grad_out(cfg))
    dout_b = dev_bits(W.normal_bf16(cfg.seed, W.S_COMPANION, 23, (cfg.tokens, cfg.hidden), 1.0))
    din = dout_a.clone()

    def eager(dout):
        g = m.alloc_grads(d, DEV)
        dx = torch.empty(d.tokens, d.hidden, dtype=torch.float32, device=DEV)
        m.check(m.moe_backward(d, w, xd, routes, saved, dout, dx, None, g, ws), "eager backward")
        torch.cuda.synchronize()
        return dx, g

    ref = {0: eager(dout_a), 1: eager(dout_b)}
    side = m.SideStreams(DEV)
    g = m.alloc_grads(d, DEV)
    dx = torch.empty(d.tokens, d.hidden, dtype=torch.float32, device=DEV)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        m.check(m.moe_backward_side(d, w, xd, routes, saved, din, dx, None, g, ws, side, s), "warm-up")
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    say("case: tiny, capture moe_backward_side")
    with torch.cuda.graph(graph, stream=s):
        m.check(m.moe_backward_side(d, w, xd, routes, saved, din, dx, None, g, ws, side,
                                    torch.cuda.current_stream()), "captured backward")
    for i in range(4):
        din.copy_(dout_b if i % 2 else dout_a)
        dx.zero_()
        graph.replay()
        torch.cuda.synchronize()
        rdx, rg = ref[i % 2]
        assert torch.equal(bits(dx), bits(rdx)), f"replay {i}: dX"
        for k in GRADS:
            if getattr(g, k) is not None:
                assert torch.equal(bits(getattr(g, k)), bits(getattr(rg, k))), f"replay {i}: {k}"
        eager(dout_a if i % 2 else dout_b)


def test_forward_side_streams_graph_replays_match_eager():
    """moe_forward_side captured: the fork event pulls the shared expert's
    side stream into the capture and the join brings it back before the
    combine; four replays on alternating inputs equal eager forwards."""
    cfg, layer, x = load_cfg("moe1k")
    w = dev_weights(layer)
    xd = dev_bits(x)
    other = dev_bits(W.tokens(cfg, stream=W.S_COMPANION, index=24))
    d = dims_of(cfg)
    routes = m.alloc_routes(d, DEV)
    saved = m.alloc_saved(d, DEV)
    out32 = torch.empty(d.tokens, d.hidden, dtype=torch.float32, device=DEV)
    out16 = torch.empty(d.tokens, d.hidden, dtype=torch.int16, device=DEV)
    ws = m.alloc_workspace(d, m.MOE_OP_FORWARD, DEV)
    side = m.SideStreams(DEV)
    xin = xd.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        m.check(m.moe_forward_side(d, w, xin, routes, saved, out32, out16, ws, side, s), "warm-up")
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    say("case: moe1k, capture moe_forward_side")
    with torch.cuda.graph(graph, stream=s):
        m.check(m.moe_forward_side(d, w, xin, routes, saved, out32, out16, ws, side,
                                   torch.cuda.current_stream()), "captured forward")
    ref = gpu_forward(cfg, w, xd)
    ref_other = gpu_forward(cfg, w, other)
    for i in range(4):
        xin.copy_(other if i % 2 else xd)
        out32.zero_()
        graph.replay()
        torch.cuda.synchronize()
        want = ref_other if i % 2 else ref
        assert torch.equal(routes.topk_idx, want.routes.topk_idx), f"replay {i}: routes"
        assert torch.equal(bits(saved.shared_y), bits(want.saved.shared_y)), f"replay {i}: shared rows"
        assert torch.equal(bits(out32), bits(want.out32)), f"replay {i}: out_f32"
        assert torch.equal(out16, want.out16), f"replay {i}: out_bf16"
        gpu_forward(cfg, w, other if i % 2 else xd)


@pytest.mark.parametrize("variant", ["mx", "lora"])
def test_mx_and_lora_forward_graph_replays_match_eager(variant):
    """moe_forward_mx (block-scaled FP8 expert weights) and moe_forward_lora
    captured once on the 256-token layer and replayed four times on
    alternating inputs, with eager forwards between the replays: every
    replay equals an eager call bit for bit."""
    import workloads.lora as WL
    import workloads.mx as MX
    from tests.test_gpu_mx import mx_weights
    cfg, layer, x = load_cfg("tiny")
    xd = dev_bits(x)
    other = dev_bits(W.tokens(cfg, stream=W.S_COMPANION, index=25))
    d = dims_of(cfg)
    if variant == "mx":
        wm = mx_weights(layer, MX.mx_layer(layer))
        ws = m.alloc_workspace(d, m.MOE_OP_FORWARD, DEV)

        def fwd(xin, routes, saved, out32, out16, stream):
            return m.moe_forward_mx(d, wm, xin, routes, saved, out32, out16, ws, stream)
    else:
        w = dev_weights(layer)
        ad = WL.lora_adapters(cfg)
        lo = m.Lora(rank=ad["rank"], scale=ad["scale"], a13=dev_bits(ad["a13"]), b13=dev_bits(ad["b13"]),
                    a2=dev_bits(ad["a2"]), b2=dev_bits(ad["b2"]))
        ws = m.alloc_workspace(d, m.MOE_OP_FORWARD_LORA, DEV)

        def fwd(xin, routes, saved, out32, out16, stream):
            return m.moe_forward_lora(d, w, lo, xin, routes, saved, out32, out16, ws, stream)

    def alloc():
        return (m.alloc_routes(d, DEV), m.alloc_saved(d, DEV),
                torch.empty(d.tokens, d.hidden, dtype=torch.float32, device=DEV),
                torch.empty(d.tokens, d.hidden, dtype=torch.int16, device=DEV))

    def eager(xin):
        r, sv, o32, o16 = alloc()
        m.check(fwd(xin, r, sv, o32, o16, None), "eager forward")
        torch.cuda.synchronize()
        return r, sv, o32, o16

    ref = {0: eager(xd), 1: eager(other)}
    xin = xd.clone()
    routes, saved, out32, out16 = alloc()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        m.check(fwd(xin, routes, saved, out32, out16, s), "warm-up")
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    say(f"case: tiny, capture moe_forward_{variant}")
    with torch.cuda.graph(graph, stream=s):
        m.check(fwd(xin, routes, saved, out32, out16, torch.cuda.current_stream()), "captured forward")
    for i in range(4):
        xin.copy_(other if i % 2 else xd)
        out32.zero_()
        graph.replay()
        torch.cuda.synchronize()
        wr, wsv, w32, w16 = ref[i % 2]
        assert torch.equal(routes.topk_idx, wr.topk_idx), f"replay {i}: routes"
        assert torch.equal(bits(saved.y), bits(wsv.y)), f"replay {i}: route rows"
        assert torch.equal(bits(out32), bits(w32)), f"replay {i}: out_f32"
        assert torch.equal(out16, w16), f"replay {i}: out_bf16"
        eager(xd if i % 2 else other)


def test_staged_calls_graph_replays_match_forward():
    """The four stage calls (moe_route, moe_permute, moe_grouped_ffn,
    moe_combine) captured as one graph on the 1024-token layer: four replays
    on alternating inputs equal moe_forward's bits."""
    cfg, layer, x = load_cfg("moe1k")
    w = dev_weights(layer)
    xd = dev_bits(x)
    other = dev_bits(W.tokens(cfg, stream=W.S_COMPANION, index=26))
    d = dims_of(cfg)
    ws = m.alloc_workspace(d, m.MOE_OP_FORWARD, DEV)
    routes = m.alloc_routes(d, DEV)
    saved = m.alloc_saved(d, DEV)
    out32 = torch.empty(d.tokens, d.hidden, dtype=torch.float32, device=DEV)
    out16 = torch.empty(d.tokens, d.hidden, dtype=torch.int16, device=DEV)
    xin = xd.clone()

    def staged(stream):
        m.check(m.moe_route(d, xin, w, routes, ws, stream), "moe_route")
        m.check(m.moe_permute(d, routes, ws, stream), "moe_permute")
        m.check(m.moe_grouped_ffn(d, xin, w, routes, saved, ws, stream), "moe_grouped_ffn")
        m.check(m.moe_combine(d, routes, saved, out32, out16, stream), "moe_combine")

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        staged(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    say("case: moe1k, capture moe_route + moe_permute + moe_grouped_ffn + moe_combine")
    with torch.cuda.graph(graph, stream=s):
        staged(torch.cuda.current_stream())
    ref = gpu_forward(cfg, w, xd)
    ref_other = gpu_forward(cfg, w, other)
    for i in range(4):
        xin.copy_(other if i % 2 else xd)
        out32.zero_()
        graph.replay()
        torch.cuda.synchronize()
        want = ref_other if i % 2 else ref
        assert torch.equal(routes.topk_idx, want.routes.topk_idx), f"replay {i}: routes"
        assert torch.equal(bits(out32), bits(want.out32)), f"replay {i}: out_f32"
        assert torch.equal(out16, want.out16), f"replay {i}: out_bf16"
        gpu_forward(cfg, w, other if i % 2 else xd)
    assert m.moe_last_device_error(ws) == m.MOE_OK
