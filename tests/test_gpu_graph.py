"""The forward under HIP graph capture: captured once, replayed several
times with other eager work and synchronisations between the replays, every
replay bit-identical to an eager forward (the library enqueues only kernel
launches on the caller's stream: no memset, no allocation, no host sync).
Also for moe_forward_noalloc, whose callers are the ones that capture."""
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
