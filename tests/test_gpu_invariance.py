"""Batch invariance and determinism of the GPU forward, raw bits.

The pages' invariance gate (RL-Kernel pull request 557, "Prior art & reuse
decision": probe tokens alone vs inside batches of several sizes at the
first, middle and last position; EP4 gate cases: full == chunked, reordered
tokens, training forward == no-grad; repeated launches) is reproduced on one
GPU: every comparison here is on raw bits, GPU against GPU.
"""
import numpy as np
import pytest
import torch

import mixture_experts_layer_counting_amd as m
import workloads as W
from tests.gpu_util import DEV, dev_bits, dev_weights, dims_of, gpu_forward, load_cfg, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def layer1k():
    cfg, layer, x = load_cfg("moe1k")
    return cfg, dev_weights(layer), x


def bits32(t):
    return t.contiguous().view(torch.int32)


def probe_rows(cfg, g, pos):
    """Per-token outputs of the tokens at positions `pos` of a forward."""
    K = cfg.top_k
    pos_t = torch.as_tensor(pos, device=DEV, dtype=torch.int64)
    rows = (pos_t[:, None] * K + torch.arange(K, device=DEV)[None, :]).reshape(-1)
    return dict(idx=g.routes.topk_idx[pos_t].clone(), gate=bits32(g.routes.topk_gate[pos_t]).clone(),
                logit=bits32(g.routes.logits[pos_t]).clone(), y=bits32(g.saved.y[rows]).clone(),
                out=bits32(g.out32[pos_t]).clone(), s=bits32(g.saved.shared_y[pos_t]).clone())


def same(a, b, what):
    for k in a:
        assert torch.equal(a[k], b[k]), f"{what}: '{k}' differs"


def test_probe_tokens_alone_vs_in_batches(layer1k):
    cfg, w, _ = layer1k
    probes = dev_bits(W.tokens(cfg, 8, stream=W.S_COMPANION, index=1))
    filler = dev_bits(W.tokens(cfg, 8192, stream=W.S_COMPANION, index=2))
    ref = probe_rows(cfg, gpu_forward(cfg, w, probes), list(range(8)))
    sizes = sorted({8, 9, 16, 31, 32, 33, 63, 64, 65, 100, 127, 128, 129, 255, 256, 257, 511, 512, 1023, 1024,
                    2048, 4095, 4096, 8192})
    for B in sizes:
        for where in ("first", "middle", "last"):
            start = {"first": 0, "middle": (B - 8) // 2, "last": B - 8}[where]
            x = filler[:B].clone()
            x[start:start + 8] = probes
            say(f"case: batch {B}, probes at {where} ({start})")
            g = gpu_forward(cfg, w, x)
            same(ref, probe_rows(cfg, g, list(range(start, start + 8))), f"batch {B} {where}")


def test_single_token_across_every_batch_size(layer1k):
    """One probe token, alone and at the last position of batches of every
    size 1..1024 and every 61st size up to 8192 (the permutation, tile split
    and grid all change with the batch; the token's bits must not)."""
    cfg, w, _ = layer1k
    probe = dev_bits(W.tokens(cfg, 1, stream=W.S_COMPANION, index=3))
    filler = dev_bits(W.tokens(cfg, 8192, stream=W.S_COMPANION, index=4))
    ref = probe_rows(cfg, gpu_forward(cfg, w, probe), [0])
    sizes = list(range(1, 1025)) + list(range(1025, 8193, 61)) + [8192]
    d = dims_of(cfg, 8192)
    ws = m.alloc_workspace(d, m.MOE_OP_FORWARD, DEV)
    say(f"case: single probe token across {len(sizes)} batch sizes")
    for B in sizes:
        x = filler[:B].clone()
        x[B - 1] = probe[0]
        g = gpu_forward(cfg, w, x, ws=ws)
        same(ref, probe_rows(cfg, g, [B - 1]), f"batch {B}")


def test_repeated_runs_are_bitwise_identical(layer1k):
    cfg, w, x = layer1k
    xd = dev_bits(x)
    say("case: 20 repeated forwards, 1024 tokens")
    first = gpu_forward(cfg, w, xd)
    keep = [first.routes.topk_idx, bits32(first.routes.topk_gate), first.routes.sorted_route,
            bits32(first.saved.y), bits32(first.out32), first.out16]
    s2 = torch.cuda.Stream()
    for i in range(19):
        if i == 10:
            with torch.cuda.stream(s2):
                g = gpu_forward(cfg, w, xd, stream=s2)
        else:
            g = gpu_forward(cfg, w, xd)
        now = [g.routes.topk_idx, bits32(g.routes.topk_gate), g.routes.sorted_route, bits32(g.saved.y),
               bits32(g.out32), g.out16]
        for a, b in zip(keep, now):
            assert torch.equal(a, b), f"run {i + 1} differs"


def test_full_equals_chunked_and_reordered(layer1k):
    cfg, w, x = layer1k
    xd = dev_bits(x)
    full = gpu_forward(cfg, w, xd)
    say("case: full batch vs 4 chunks of 256")
    for c in range(4):
        part = gpu_forward(cfg, w, xd[c * 256:(c + 1) * 256].clone())
        sl = slice(c * 256, (c + 1) * 256)
        assert torch.equal(bits32(part.out32), bits32(full.out32[sl]))
        assert torch.equal(part.routes.topk_idx, full.routes.topk_idx[sl])
    say("case: reordered tokens")
    perm = torch.randperm(cfg.tokens, generator=torch.Generator().manual_seed(3)).to(DEV)
    rev = gpu_forward(cfg, w, xd[perm].contiguous())
    assert torch.equal(bits32(rev.out32), bits32(full.out32[perm]))
    assert torch.equal(rev.routes.topk_idx, full.routes.topk_idx[perm])


def test_training_forward_equals_inference_forward(layer1k):
    cfg, w, x = layer1k
    xd = dev_bits(x)
    say("case: forward saving gate/up (training) vs not")
    a = gpu_forward(cfg, w, xd, training=False)
    b = gpu_forward(cfg, w, xd, training=True)
    assert torch.equal(bits32(a.out32), bits32(b.out32))
    assert torch.equal(bits32(a.saved.y), bits32(b.saved.y))
