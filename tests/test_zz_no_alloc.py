"""moe_forward_noalloc (workspace in the library's own device array) against
moe_forward (caller workspace) through the C ABI: two calls in a row, the
second with a smaller batch, bit for bit on every output; and the host-side
refusal of a batch whose workspace exceeds the array."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_counting_amd as m
from tests.gpu_util import DEV, dev_bits, dev_weights, dims_of, gpu_forward, load_cfg, say

pytestmark = pytest.mark.gpu


def noalloc_forward(cfg, w, xd):
    d = dims_of(cfg, int(xd.shape[0]))
    routes = m.alloc_routes(d, DEV)
    saved = m.alloc_saved(d, DEV)
    out32 = torch.empty(d.tokens, d.hidden, dtype=torch.float32, device=DEV)
    out16 = torch.empty(d.tokens, d.hidden, dtype=torch.int16, device=DEV)
    m.check(m.moe_forward_noalloc(d, w, xd, routes, saved, out32, out16), "moe_forward_noalloc")
    torch.cuda.synchronize()
    return routes, saved, out32, out16


def same(a, b):
    return torch.equal(a.contiguous().view(torch.int32), b.contiguous().view(torch.int32))


@pytest.mark.parametrize("name,sizes", [("moe1k", (1024, 300)), ("tiny", (256, 37))])
def test_noalloc_forward_equals_forward(name, sizes):
    cfg, layer, x = load_cfg(name)
    w = dev_weights(layer)
    for T in sizes:
        say(f"case: {name}, {T} tokens, moe_forward_noalloc vs moe_forward")
        xd = dev_bits(x[:T])
        ref = gpu_forward(cfg, w, xd)
        routes, saved, out32, out16 = noalloc_forward(cfg, w, xd)
        assert torch.equal(routes.topk_idx, ref.routes.topk_idx)
        assert same(routes.topk_gate, ref.routes.topk_gate)
        assert same(routes.logits, ref.routes.logits)
        assert torch.equal(routes.expert_offsets, ref.routes.expert_offsets)
        assert torch.equal(routes.sorted_route, ref.routes.sorted_route)
        assert torch.equal(routes.route_pos, ref.routes.route_pos)
        assert same(saved.y, ref.saved.y)
        assert same(saved.shared_y, ref.saved.shared_y)
        assert same(saved.shared_gate, ref.saved.shared_gate)
        assert same(out32, ref.out32)
        assert torch.equal(out16, ref.out16)


def test_noalloc_refuses_a_batch_beyond_its_array():
    cfg, layer, x = load_cfg("tiny")
    d = m.Dims(4096, 2048, 512, 10, 512, 512)
    assert m.moe_workspace_bytes(d, m.MOE_OP_FORWARD) > m.NOALLOC_SCRATCH_BYTES
    w = dev_weights(layer)
    # rejected on the host before any pointer is read
    assert m.moe_forward_noalloc(d, w, None, m.Routes(), m.Saved(), None, None) == m.MOE_E_WORKSPACE
