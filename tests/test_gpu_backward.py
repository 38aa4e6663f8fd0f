"""GPU parity of the backward against the FP64 oracle, through the C ABI,
plus its determinism and the batch invariance of the input gradient.

The input gradient dX, a per-token quantity, is compared with the per-token
rule |gpu - ref| <= 5e-5 + 1e-3 |ref|.  A weight gradient sums n per-token
terms over the batch; its absolute floor grows as sqrt(n)
(tests/gpu_util.assert_close_sum), n = the routes summed into it (an
expert's route count, or T for the shared expert and its gate).  The
relative part is taken against the sum of the terms' absolute values (sum
over routes of |dGU| |x| for dW13, |dy| |act| for dW2, |dl| |x| for the
router, |dz| |x| for the shared gate): each term carries a small relative
error (the bf16 hi/lo operands, fp32 forward outputs), and terms of both
signs cancel in the sum while their errors do not.  The small
layer is compared in full; the 4096-token layer on sampled tokens (dX rows),
sampled experts (their dW13, dW2 and router rows, from those experts' own
routes) and the shared expert's weight gradients in full.
"""
import numpy as np
import pytest
import torch

import mixture_experts_layer_counting_amd as m
import oracle as O
import workloads as W
from tests.gpu_util import (DEV, assert_close, assert_close_sum, bf16_rne_bits, compare_routes, dev_bits,
                            dev_weights, dims_of, expert_term_scales, gate_term_scale, gpu_forward, load_cfg,
                            router_term_scale, say, shared_term_scales)

pytestmark = pytest.mark.gpu


def gpu_backward(cfg, w, xd, g, dout_d, ws=None):
    d = dims_of(cfg, int(xd.shape[0]))
    grads = m.alloc_grads(d, DEV)
    dx32 = torch.empty(d.tokens, d.hidden, dtype=torch.float32, device=DEV)
    dx16 = torch.empty(d.tokens, d.hidden, dtype=torch.int16, device=DEV)
    if ws is None:
        ws = m.alloc_workspace(d, m.MOE_OP_BACKWARD, DEV)
    m.check(m.moe_backward(d, w, xd, g.routes, g.saved, dout_d, dx32, dx16, grads, ws), "moe_backward")
    torch.cuda.synchronize()
    return dx32, dx16, grads


def full_backward_check(cfg, layer, x, dout):
    w = dev_weights(layer)
    xd = dev_bits(x)
    g = gpu_forward(cfg, w, xd, training=True)
    idx = g.routes.topk_idx.cpu().numpy()
    ref_f = O.forward(layer, x, cfg.top_k)
    ties = compare_routes(idx, ref_f["idx"], ref_f["logits"])
    if ties:
        say(f"  {len(ties)} tokens with router ties: oracle uses the GPU routes")
        ref_f = O.forward(layer, x, cfg.top_k, forced_idx=idx)
    ref = O.backward(layer, x, ref_f, dout)
    dx32, dx16, gr = gpu_backward(cfg, w, xd, g, dev_bits(dout))
    assert_close(dx32.cpu().numpy(), ref["dx"], "dX")
    assert np.array_equal(dx16.cpu().numpy().view(np.uint16), bf16_rne_bits(dx32.cpu().numpy()))
    load = np.bincount(idx.reshape(-1), minlength=cfg.experts)
    scales = {"d_w_router": router_term_scale(x, ref_f["idx"], ref["dl"], cfg.experts),
              "d_w13": np.zeros(layer["w13"].shape), "d_w2": np.zeros(layer["w2"].shape)}
    for e in np.nonzero(load)[0]:
        scales["d_w13"][e], scales["d_w2"][e] = expert_term_scales(layer, x, dout, ref_f["idx"], ref_f["gates"],
                                                                  ref_f["gu"], int(e))
    for name, key in (("dW_router", "d_w_router"), ("dW13", "d_w13"), ("dW2", "d_w2")):
        got = getattr(gr, key).cpu().numpy().astype(np.float64)
        err = np.abs(got - ref[key])
        floor = 5e-5 * np.sqrt(np.maximum(1, load)).reshape(-1, *([1] * (got.ndim - 1)))
        scale = np.maximum(np.abs(ref[key]), scales[key])
        ratio = err / (floor + 1e-3 * scale)
        strict = err / (5e-5 + 1e-3 * np.abs(ref[key]))
        say(f"  {name}: max-abs {err.max():.3e}, worst err/tol {ratio.max():.3f} (sum rule), "
            f"{strict.max():.3f} (per-token rule)")
        assert ratio.max() <= 1.0, f"{name}: {(ratio > 1).sum()} elements outside tolerance"
    if cfg.shared_inter:
        s13, s2 = shared_term_scales(layer, x, dout, ref_f["sg"], ref_f["sgu"])
        assert_close_sum(gr.d_ws13.cpu().numpy(), ref["d_ws13"], "dWs13", cfg.tokens, s13)
        assert_close_sum(gr.d_ws2.cpu().numpy(), ref["d_ws2"], "dWs2", cfg.tokens, s2)
        assert_close_sum(gr.d_w_sgate.cpu().numpy(), ref["d_w_sgate"], "dw_sgate", cfg.tokens,
                         gate_term_scale(x, ref["dz"]))


def test_tiny_backward_full():
    cfg, layer, x = load_cfg("tiny")
    say("case: tiny backward, every gradient in full")
    full_backward_check(cfg, layer, x, W.grad_out(cfg))


@pytest.mark.parametrize("shape", [
    dict(tokens=100, hidden=256, experts=192, top_k=6, inter=128, shared_inter=0),
    dict(tokens=77, hidden=256, experts=64, top_k=16, inter=256, shared_inter=128),
    dict(tokens=33, hidden=512, experts=128, top_k=2, inter=128, shared_inter=384),
    dict(tokens=24, hidden=16384, experts=64, top_k=2, inter=128, shared_inter=128),
    dict(tokens=40, hidden=256, experts=64, top_k=4, inter=4096, shared_inter=0),
    dict(tokens=1, hidden=512, experts=512, top_k=10, inter=512, shared_inter=512),
])
def test_backward_shape_edge_cases(shape):
    cfg = W.MoEConfig(name="edge", **shape)
    layer = W.make_layer(cfg)
    say(f"case: backward edge shape {shape}")
    full_backward_check(cfg, layer, W.tokens(cfg), W.grad_out(cfg))


def test_bwd4k_sampled():
    cfg, layer, x = load_cfg("bwd4k")
    w = dev_weights(layer)
    xd = dev_bits(x)
    dout = W.grad_out(cfg)
    say("case: bwd4k forward + backward on GPU")
    g = gpu_forward(cfg, w, xd, training=True)
    dx32, dx16, gr = gpu_backward(cfg, w, xd, g, dev_bits(dout))
    idx = g.routes.topk_idx.cpu().numpy()
    rng = np.random.default_rng(11)
    # dX rows of sampled tokens: the oracle backward of the token subset
    tok = np.unique(np.concatenate([[0, 1, 63, 64, 2047, cfg.tokens - 1], rng.choice(cfg.tokens, 26, replace=False)]))
    say(f"  oracle backward on {len(tok)} sampled tokens")
    fs = O.forward(layer, x[tok], cfg.top_k, forced_idx=idx[tok])
    compare_routes(idx[tok], O.select_routes(fs["logits"], cfg.top_k), fs["logits"])
    bs = O.backward(layer, x[tok], fs, dout[tok])
    assert_close(dx32.cpu().numpy()[tok], bs["dx"], "dX (sampled tokens)")
    # sampled experts: their weight gradients from their own routes
    experts = [0, 17, 255, 511] + list(rng.choice(cfg.experts, 4, replace=False))
    dw13 = gr.d_w13.cpu().numpy()
    dw2 = gr.d_w2.cpu().numpy()
    dwr = gr.d_w_router.cpu().numpy()
    for e in experts:
        te = np.unique(np.nonzero((idx == e).any(axis=1))[0])
        fe = O.forward(layer, x[te], cfg.top_k, forced_idx=idx[te])
        rows = np.nonzero(fe["idx"].reshape(-1) == e)[0]
        r13, r2 = O.expert_weight_grads(layer, x[te], dout[te], fe["idx"], fe["gates"], fe["gu"][rows], int(e))
        s13, s2 = expert_term_scales(layer, x[te], dout[te], fe["idx"], fe["gates"], fe["gu"], int(e))
        assert_close_sum(dw13[e], r13, f"dW13[{e}]", len(te), s13)
        assert_close_sum(dw2[e], r2, f"dW2[{e}]", len(te), s2)
        be = O.backward(layer, x[te], fe, dout[te])
        assert_close_sum(dwr[e], be["d_w_router"][e], f"dW_router[{e}]", len(te),
                         router_term_scale(x[te], fe["idx"], be["dl"], cfg.experts)[e])
    say("  oracle shared-expert gradients over all tokens")
    sh = O.shared_expert_grads(layer, x, dout)
    _, s_sg, s_sgu = O.shared_expert(x, layer["ws13"], layer["ws2"], layer["w_sgate"])
    s13, s2 = shared_term_scales(layer, x, dout, s_sg, s_sgu)
    assert_close_sum(gr.d_ws13.cpu().numpy(), sh["d_ws13"], "dWs13", cfg.tokens, s13)
    assert_close_sum(gr.d_ws2.cpu().numpy(), sh["d_ws2"], "dWs2", cfg.tokens, s2)
    assert_close_sum(gr.d_w_sgate.cpu().numpy(), sh["d_w_sgate"], "dw_sgate", cfg.tokens,
                     gate_term_scale(x, sh["dz"]))


def test_backward_deterministic_and_dx_batch_invariant():
    cfg, layer, x = load_cfg("tiny")
    w = dev_weights(layer)
    xd = dev_bits(x)
    dout = dev_bits(W.grad_out(cfg))
    say("case: tiny backward twice, then dX of 8 probe tokens alone vs in the batch")
    g = gpu_forward(cfg, w, xd, training=True)
    a = gpu_backward(cfg, w, xd, g, dout)
    b = gpu_backward(cfg, w, xd, g, dout)
    for t1, t2 in [(a[0], b[0])] + [(getattr(a[2], k), getattr(b[2], k)) for k in
                                     ("d_w_router", "d_w13", "d_w2", "d_ws13", "d_ws2", "d_w_sgate")]:
        assert torch.equal(t1.view(torch.int32), t2.view(torch.int32))
    for start in (0, 100, 248):
        sl = slice(start, start + 8)
        gs = gpu_forward(cfg, w, xd[sl].clone(), training=True)
        p = gpu_backward(cfg, w, xd[sl].clone(), gs, dout[sl].clone())
        assert torch.equal(p[0].view(torch.int32), a[0][sl].view(torch.int32)), f"dX rows at {start} differ"
