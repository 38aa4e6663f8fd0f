"""GPU parity of the backward with LoRA adapters on the routed experts
(moe_backward_lora) against the FP64 oracle, through the C ABI.

The adapters are the seeded ones of the LoRA forward tests (rank 6 =
64 // 10, scale 0.5, N(0, 0.02) factors, B nonzero).  Checks:
  * every gradient -- dX, the base weight gradients and the four adapter
    gradients dA13, dB13, dA2, dB2 -- against the oracle's backward with the
    same adapters under the layer's rule |gpu - ref| <= 5e-5 + 1e-3 |ref|
    (split as in the plain backward's tests only where the method's fp32
    forward values alone exceed it), in full on small layers (ranks 1, 6,
    16; no shared expert; ragged tokens; a single token through the
    unrolled hidden-2048 kernels) and on sampled tokens and experts of the
    4096-token layer;
  * the adapter gradients also against the oracle fed the GPU's own fp32
    forward values, by relative Frobenius error (the kernels' own error);
  * adapters with zero expand matrices: base gradients and dX equal to
    moe_backward's values, dA13 = dA2 = 0;
  * two backwards give the same bits; dX rows of a sub-batch equal the
    full batch's.
"""
import numpy as np
import pytest
import torch

import mixture_experts_layer_counting_amd as m
import oracle as O
import workloads as W
import workloads.lora as WL
from tests.gpu_util import (DEV, GpuForward, assert_close, bf16_rne_bits, compare_routes, dev_bits, dev_weights,
                            dims_of, fed_forward, gpu_forward, load_cfg, say, strict_ratio)
from tests.test_gpu_backward import GRADS, assert_grad_close, gpu_backward

pytestmark = pytest.mark.gpu

LGRADS = ("d_a13", "d_b13", "d_a2", "d_b2")

EDGE = {
    "edge_noshared": dict(tokens=100, hidden=256, experts=192, top_k=6, inter=128, shared_inter=0),
    "edge_t1": dict(tokens=1, hidden=2048, experts=64, top_k=10, inter=512, shared_inter=512),
    "edge_k16": dict(tokens=77, hidden=256, experts=64, top_k=16, inter=256, shared_inter=128),
}


def load_any(name):
    if name in EDGE:
        cfg = W.MoEConfig(name=name, **EDGE[name])
        return cfg, W.make_layer(cfg), W.tokens(cfg)
    return load_cfg(name)


def dev_lora(ad) -> m.Lora:
    return m.Lora(rank=ad["rank"], scale=ad["scale"], a13=dev_bits(ad["a13"]), b13=dev_bits(ad["b13"]),
                  a2=dev_bits(ad["a2"]), b2=dev_bits(ad["b2"]))


def forward_lora_training(cfg, w, lo, xd, ws=None) -> GpuForward:
    d = dims_of(cfg, int(xd.shape[0]))
    routes = m.alloc_routes(d, DEV)
    saved = m.alloc_saved(d, DEV, training=True)
    out32 = torch.empty(d.tokens, d.hidden, dtype=torch.float32, device=DEV)
    out16 = torch.empty(d.tokens, d.hidden, dtype=torch.int16, device=DEV)
    if ws is None:
        ws = m.alloc_workspace(d, m.MOE_OP_BACKWARD_LORA, DEV)
    m.check(m.moe_forward_lora(d, w, lo, xd, routes, saved, out32, out16, ws), "moe_forward_lora")
    torch.cuda.synchronize()
    assert m.moe_last_device_error(ws) == m.MOE_OK
    return GpuForward(routes, saved, out32, out16)


def backward_lora(cfg, w, lo, xd, g, dout_d, ws=None):
    d = dims_of(cfg, int(xd.shape[0]))
    grads = m.alloc_grads(d, DEV)
    lg = m.alloc_lora_grads(d, lo.rank, DEV)
    dx32 = torch.empty(d.tokens, d.hidden, dtype=torch.float32, device=DEV)
    dx16 = torch.empty(d.tokens, d.hidden, dtype=torch.int16, device=DEV)
    if ws is None:
        ws = m.alloc_workspace(d, m.MOE_OP_BACKWARD_LORA, DEV)
    m.check(m.moe_backward_lora(d, w, lo, xd, g.routes, g.saved, dout_d, dx32, dx16, grads, lg, ws),
            "moe_backward_lora")
    torch.cuda.synchronize()
    assert m.moe_last_device_error(ws) == m.MOE_OK
    return dx32, dx16, grads, lg


def rel_fro(got, ref):
    ref = np.asarray(ref, np.float64)
    return float(np.linalg.norm(np.asarray(got, np.float64) - ref) / max(np.linalg.norm(ref), 1e-300))


def check_lora_grad(got, ref, fed, what):
    say(f"  {what}: max |ref| {np.max(np.abs(ref)):.3e}, relative Frobenius error vs the fed oracle "
        f"{rel_fro(got, fed):.2e}")
    assert_grad_close(got, ref, fed, what)
    assert rel_fro(got, fed) <= 1e-4, f"{what}: relative Frobenius error vs the fed oracle"


def full_check(cfg, layer, ad, x, dout):
    w, lo, xd = dev_weights(layer), dev_lora(ad), dev_bits(x)
    g = forward_lora_training(cfg, w, lo, xd)
    h = g.host()
    idx = h["idx"]
    ref_f = O.forward(layer, x, cfg.top_k, lora=ad)
    if compare_routes(idx, ref_f["idx"], ref_f["logits"]):
        say("  router ties: the oracle uses the GPU routes")
        ref_f = O.forward(layer, x, cfg.top_k, forced_idx=idx, lora=ad)
    ref = O.backward(layer, x, ref_f, dout, lora=ad)
    fed = O.backward(layer, x, fed_forward(layer, x, idx, h["gates"], h["gu"], h["route_pos"], h["sgu"], h["sg"],
                                           lora=ad), dout, lora=ad)
    dx32, dx16, gr, lg = backward_lora(cfg, w, lo, xd, g, dev_bits(dout))
    dx = dx32.cpu().numpy()
    assert_grad_close(dx, ref["dx"], fed["dx"], "dX")
    assert np.array_equal(dx16.cpu().numpy().view(np.uint16), bf16_rne_bits(dx))
    for key in GRADS:
        if key in ref:
            assert_grad_close(getattr(gr, key).cpu().numpy(), ref[key], fed[key], key)
    for key in LGRADS:
        check_lora_grad(getattr(lg, key).cpu().numpy(), ref[key], fed[key], key)
    # the adapters move the gradients well beyond the rule
    plain = O.backward(layer, x, O.forward(layer, x, cfg.top_k, forced_idx=idx), dout)
    assert strict_ratio(plain["dx"], ref["dx"]) > 1.0


@pytest.mark.parametrize("name,rank", [("tiny", 6), ("tiny", 1), ("tiny", 16), ("edge_noshared", 6),
                                       ("edge_t1", 6), ("edge_k16", 6)])
def test_lora_backward_matches_oracle(name, rank):
    cfg, layer, x = load_any(name)
    ad = WL.lora_adapters(cfg, rank)
    say(f"case: {name}, rank {rank}, moe_backward_lora vs oracle, every gradient in full")
    full_check(cfg, layer, ad, x, W.grad_out(cfg))


def test_lora_backward_bwd4k_sampled():
    cfg, layer, x = load_cfg("bwd4k")
    ad = WL.lora_adapters(cfg)
    w, lo, xd = dev_weights(layer), dev_lora(ad), dev_bits(x)
    dout = W.grad_out(cfg)
    say("case: bwd4k LoRA forward + backward on GPU")
    g = forward_lora_training(cfg, w, lo, xd)
    h = g.host()
    dx32, _, gr, lg = backward_lora(cfg, w, lo, xd, g, dev_bits(dout))
    idx = h["idx"]
    rng = np.random.default_rng(12)
    tok = np.unique(np.concatenate([[0, 127, 128, cfg.tokens - 1], rng.choice(cfg.tokens, 24, replace=False)]))
    say(f"  oracle LoRA backward on {len(tok)} sampled tokens")
    fs = O.forward(layer, x[tok], cfg.top_k, forced_idx=idx[tok], lora=ad)
    compare_routes(idx[tok], O.select_routes(fs["logits"], cfg.top_k), fs["logits"])
    bs = O.backward(layer, x[tok], fs, dout[tok], lora=ad)
    assert_close(dx32.cpu().numpy()[tok], bs["dx"], "dX (sampled tokens)")
    host = {k: getattr(gr, k).cpu().numpy() for k in ("d_w13", "d_w2", "d_w_router")}
    host.update({k: getattr(lg, k).cpu().numpy() for k in LGRADS})
    for e in [0, 255, 511] + list(rng.choice(cfg.experts, 3, replace=False)):
        te = np.unique(np.nonzero((idx == e).any(axis=1))[0])
        say(f"  expert {e}: oracle LoRA backward of its {len(te)} tokens")
        fe = O.forward(layer, x[te], cfg.top_k, forced_idx=idx[te], lora=ad)
        be = O.backward(layer, x[te], fe, dout[te], lora=ad)
        for key in ("d_w13", "d_w2", "d_w_router") + LGRADS:
            assert_close(host[key][e], be[key][e], f"{key}[{e}]")


def test_lora_backward_with_zero_expand_gives_the_plain_gradients():
    cfg, layer, x = load_cfg("tiny")
    ad = WL.lora_adapters(cfg)
    ad["b13"][:] = 0
    ad["b2"][:] = 0
    w, lo, xd = dev_weights(layer), dev_lora(ad), dev_bits(x)
    dout = W.grad_out(cfg)
    dd = dev_bits(dout)
    say("case: tiny, zero expand matrices: moe_backward_lora vs moe_backward")
    g = forward_lora_training(cfg, w, lo, xd)
    dx, _, gr, lg = backward_lora(cfg, w, lo, xd, g, dd)
    pdx, _, pgr = gpu_backward(cfg, w, xd, g, dd)
    # equal values (a zero update may turn an exact -0 into +0)
    assert torch.equal(dx, pdx), "dX"
    for k in GRADS:
        if getattr(gr, k) is not None:
            assert torch.equal(getattr(gr, k), getattr(pgr, k)), k
    assert not lg.d_a13.any() and not lg.d_a2.any()
    # dB13 and dB2 do not vanish: the oracle's
    h = g.host()
    f = O.forward(layer, x, cfg.top_k, forced_idx=h["idx"], lora=ad)
    ref = O.backward(layer, x, f, dout, lora=ad)
    assert_close(lg.d_b13.cpu().numpy(), ref["d_b13"], "dB13")
    assert_close(lg.d_b2.cpu().numpy(), ref["d_b2"], "dB2")


def bits(t):
    return t.contiguous().view(torch.int32)


def test_lora_backward_deterministic_and_dx_batch_invariant():
    cfg, layer, x = load_cfg("tiny")
    ad = WL.lora_adapters(cfg)
    w, lo, xd = dev_weights(layer), dev_lora(ad), dev_bits(x)
    dd = dev_bits(W.grad_out(cfg))
    say("case: tiny LoRA backward twice, then dX of 8 probe tokens alone vs in the batch")
    g = forward_lora_training(cfg, w, lo, xd)
    a = backward_lora(cfg, w, lo, xd, g, dd)
    b = backward_lora(cfg, w, lo, xd, g, dd)
    assert torch.equal(bits(a[0]), bits(b[0])), "dX"
    for k in GRADS:
        if getattr(a[2], k) is not None:
            assert torch.equal(bits(getattr(a[2], k)), bits(getattr(b[2], k))), k
    for k in LGRADS:
        assert torch.equal(bits(getattr(a[3], k)), bits(getattr(b[3], k))), k
    for start in (0, 100, 248):
        sl = slice(start, start + 8)
        gs = forward_lora_training(cfg, w, lo, xd[sl].clone())
        p = backward_lora(cfg, w, lo, xd[sl].clone(), gs, dd[sl].clone())
        assert torch.equal(bits(p[0]), bits(a[0][sl])), f"dX rows at {start} differ"


@pytest.mark.parametrize("name", ["tiny", "bwd4k"])
def test_lora_backward_side_streams_equal(name):
    """moe_backward_lora_side gives moe_backward_lora's bits for every
    gradient, adapter gradients included."""
    cfg, layer, x = load_any(name)
    ad = WL.lora_adapters(cfg)
    w, lo, xd = dev_weights(layer), dev_lora(ad), dev_bits(x)
    dd = dev_bits(W.grad_out(cfg))
    say(f"case: {name}, moe_backward_lora_side vs moe_backward_lora")
    g = forward_lora_training(cfg, w, lo, xd)
    ref = backward_lora(cfg, w, lo, xd, g, dd)
    d = dims_of(cfg)
    side = m.SideStreams(DEV)
    ws = m.alloc_workspace(d, m.MOE_OP_BACKWARD_LORA, DEV)
    grads = m.alloc_grads(d, DEV)
    lg = m.alloc_lora_grads(d, lo.rank, DEV)
    dx32 = torch.empty(d.tokens, d.hidden, dtype=torch.float32, device=DEV)
    m.check(m.moe_backward_lora_side(d, w, lo, xd, g.routes, g.saved, dd, dx32, None, grads, lg, ws, side),
            "moe_backward_lora_side")
    torch.cuda.synchronize()
    assert m.moe_last_device_error(ws) == m.MOE_OK
    assert torch.equal(bits(dx32), bits(ref[0])), "dX"
    for k in GRADS:
        if getattr(grads, k) is not None:
            assert torch.equal(bits(getattr(grads, k)), bits(getattr(ref[2], k))), k
    for k in LGRADS:
        assert torch.equal(bits(getattr(lg, k)), bits(getattr(ref[3], k))), k
