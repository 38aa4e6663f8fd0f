"""Helpers shared by the GPU tests: device copies of seeded layers, calls
through the C ABI, and the comparison rules against the FP64 oracle.

Comparison rules:
  * expert ids: ordered lists, bit-exact, except where the two disputed
    experts' exact logits lie closer than 1e-6 (a tie of the fp32 router);
    such tokens are counted and re-checked with the GPU's routes forced;
  * permutation: bit-exact with the oracle's counting sort of the GPU ids;
  * floating outputs: |gpu - ref| <= 5e-5 + 1e-3 |ref| elementwise;
  * bf16 output: exactly the round-to-nearest-even of the GPU's fp32 output.
"""
from __future__ import annotations

import dataclasses
import sys

import numpy as np
import torch

import mixture_experts_layer_counting_amd as m
import oracle as O
import workloads as W

ATOL, RTOL = 5e-5, 1e-3
TIE_GAP = 1e-6
DEV = torch.device("cuda:0")


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def dev_bits(a):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV)


def dev_f32(a):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def dims_of(cfg, tokens=None) -> m.Dims:
    return m.Dims(cfg.tokens if tokens is None else tokens, cfg.hidden, cfg.experts, cfg.top_k, cfg.inter,
                  cfg.shared_inter)


def dev_weights(layer) -> m.Weights:
    return m.Weights(w_router=dev_f32(layer["w_router"]), w13=dev_bits(layer["w13"]), w2=dev_bits(layer["w2"]),
                     router_bias=dev_f32(layer["router_bias"]), ws13=dev_bits(layer["ws13"]),
                     ws2=dev_bits(layer["ws2"]), w_sgate=dev_bits(layer["w_sgate"]))


@dataclasses.dataclass
class GpuForward:
    routes: m.Routes
    saved: m.Saved
    out32: torch.Tensor
    out16: torch.Tensor

    def host(self):
        r, s = self.routes, self.saved
        h = lambda t: None if t is None else t.cpu().numpy()
        return dict(idx=h(r.topk_idx), gates=h(r.topk_gate), logits=h(r.logits), offsets=h(r.expert_offsets),
                    sorted_route=h(r.sorted_route), route_pos=h(r.route_pos), y=h(s.y), gu=h(s.gu),
                    s=h(s.shared_y), sg=h(s.shared_gate), sgu=h(s.shared_gu), out32=h(self.out32),
                    out16=h(self.out16).view(np.uint16))


def gpu_forward(cfg, w: m.Weights, x_dev, training=False, ws=None, stream=None) -> GpuForward:
    d = dims_of(cfg, int(x_dev.shape[0]))
    routes = m.alloc_routes(d, DEV)
    saved = m.alloc_saved(d, DEV, training)
    out32 = torch.empty(d.tokens, d.hidden, dtype=torch.float32, device=DEV)
    out16 = torch.empty(d.tokens, d.hidden, dtype=torch.int16, device=DEV)
    if ws is None:
        ws = m.alloc_workspace(d, m.MOE_OP_BACKWARD if training else m.MOE_OP_FORWARD, DEV)
    m.check(m.moe_forward(d, w, x_dev, routes, saved, out32, out16, ws, stream), "moe_forward")
    torch.cuda.synchronize()
    return GpuForward(routes, saved, out32, out16)


def bf16_rne_bits(a32: np.ndarray) -> np.ndarray:
    u = np.ascontiguousarray(a32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def assert_close(got, ref, what, atol=ATOL, rtol=RTOL):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    err = np.abs(got - ref)
    tol = atol + rtol * np.abs(ref)
    bad = err > tol
    big = np.abs(ref) > 1e-3
    rel = (err[big] / np.abs(ref[big])).max() if big.any() else 0.0
    say(f"  {what}: max-abs {err.max():.3e}, max-rel(|ref|>1e-3) {rel:.3e}, worst err/tol {(err / tol).max():.3f}")
    assert not bad.any(), f"{what}: {bad.sum()} of {bad.size} elements outside tolerance, max-abs {err.max():.3e}"
    return err.max()


def fed_forward(layer, x_bits, idx, gates, gu_sorted, route_pos, sgu=None, sg=None, lora=None):
    """An oracle forward dict holding the GPU's saved fp32 forward values --
    gate/up pre-activations, route gates, shared gate -- (exact in float64),
    with Y and S recomputed from them in float64.

    Those fp32 values are rounding points of the method (the forward keeps
    its fp32 accumulators and fp32 gates, and the backward starts from
    them).  Feeding them to the oracle's backward isolates what these
    rounding points alone cost: the distance of this oracle from the plain
    one is inherent to the method, the distance of the GPU from this oracle
    is the backward kernels' own error.  With `lora` (the adapters of the
    forward) Y carries the down adapter's update."""
    K = idx.shape[1]
    x64 = O.bf16_to_f64(x_bits)
    gu = np.asarray(gu_sorted, np.float64)[np.asarray(route_pos)]
    inter = gu.shape[1] // 2
    y = np.zeros((idx.size, x64.shape[1]))
    flat = idx.reshape(-1)
    for e in np.unique(flat):
        rows = np.nonzero(flat == e)[0]
        act = O.silu(gu[rows, :inter]) * gu[rows, inter:]
        y[rows] = act @ O.bf16_to_f64(layer["w2"][e]).T
        if lora is not None:
            z2 = act @ O.bf16_to_f64(lora["a2"][e]).T
            y[rows] += float(lora["scale"]) * (z2 @ O.bf16_to_f64(lora["b2"][e]).T)
    f = dict(idx=idx, gates=np.asarray(gates, np.float64), gu=gu, y=y)
    if sgu is not None:
        s_gu = np.asarray(sgu, np.float64)
        i_s = s_gu.shape[1] // 2
        f.update(sgu=s_gu, sg=np.asarray(sg, np.float64),
                 s=(O.silu(s_gu[:, :i_s]) * s_gu[:, i_s:]) @ O.bf16_to_f64(layer["ws2"]).T)
    return f


def strict_ratio(got, ref):
    """Worst |got - ref| / (5e-5 + 1e-3 |ref|) over all elements."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return float((np.abs(got - ref) / (ATOL + RTOL * np.abs(ref))).max()) if ref.size else 0.0


def tie_census(logits64, top_k):
    """Tokens whose exact logits hold a near-tie (gap < 1e-6) that decides
    the route list: between the top_k-th and (top_k+1)-th largest (which
    experts are selected) or between two selected ones (their slot order).
    Returns (boundary ties, in-order ties)."""
    srt = -np.sort(-np.asarray(logits64), axis=1)[:, :top_k + 1]
    gaps = srt[:, :-1] - srt[:, 1:]
    boundary = int((gaps[:, top_k - 1] < TIE_GAP).sum())
    inorder = int((gaps[:, :top_k - 1] < TIE_GAP).any(axis=1).sum())
    return boundary, inorder


def p8_expected_ties(tokens, hidden, experts, top_k, w_sigma=0.02):
    """Expected boundary near-ties per batch from the closed form: the gap
    between consecutive order statistics at the selection threshold is
    about exponential with rate rho = E phi(z) / sigma_l, z = Phi^-1(1 -
    (K + 1/2) / E), sigma_l = w_sigma sqrt(H) (unit-variance tokens)."""
    from scipy.stats import norm
    z = norm.ppf(1.0 - (top_k + 0.5) / experts)
    rho = experts * norm.pdf(z) / (w_sigma * np.sqrt(hidden))
    return tokens * (1.0 - np.exp(-rho * TIE_GAP))


def compare_routes(idx_gpu, idx_ref, logits64, logits_gpu=None):
    """Ordered expert lists equal except for fp32 router ties; returns the
    tokens with a tie (their gap is checked on the exact logits, and the
    GPU's own fp32 gap is reported when its logits are given)."""
    diff = np.nonzero((idx_gpu != idx_ref).any(axis=1))[0]
    ties = []
    for t in diff:
        for k in np.nonzero(idx_gpu[t] != idx_ref[t])[0]:
            eg, eo = int(idx_gpu[t, k]), int(idx_ref[t, k])
            assert 0 <= eg < logits64.shape[1], f"token {t} slot {k}: expert id {eg} out of range"
            gap = abs(logits64[t, eg] - logits64[t, eo])
            assert gap < TIE_GAP, f"token {t} slot {k}: gpu {eg} vs oracle {eo}, exact logit gap {gap:.3e}"
            g32 = "" if logits_gpu is None else \
                f", GPU fp32 gap {abs(float(logits_gpu[t, eg]) - float(logits_gpu[t, eo])):.3e}"
            say(f"  tie: token {t} slot {k}: gpu expert {eg}, oracle {eo}, exact gap {gap:.3e}{g32}")
        ties.append(int(t))
    return ties


def check_permutation(g, E):
    off, srt, pos = O.permute_routes(g["idx"], E)
    assert np.array_equal(g["offsets"], off), "expert_offsets differ from the oracle's counting sort"
    assert np.array_equal(g["sorted_route"], srt), "sorted_route differs from the oracle's counting sort"
    assert np.array_equal(g["route_pos"], pos), "route_pos differs from the oracle's counting sort"


def check_forward(cfg, layer, x_bits, g, tokens=None, check_perm=True):
    """Full comparison of a GPU forward (host dict g) with the oracle on a
    token subset (all tokens by default)."""
    T, K = x_bits.shape[0], cfg.top_k
    tok = np.arange(T) if tokens is None else np.asarray(tokens)
    ref = O.forward(layer, x_bits, K, tokens=tok)
    ties = compare_routes(g["idx"][tok], ref["idx"], ref["logits"])
    say(f"  routes: {len(tok)} tokens compared, {len(ties)} with fp32 ties")
    if ties:
        ref = O.forward(layer, x_bits, K, tokens=tok, forced_idx=g["idx"])
    if check_perm:
        check_permutation(g, cfg.experts)
    rows = (tok[:, None] * K + np.arange(K)[None, :]).reshape(-1)
    assert_close(g["gates"][tok], ref["gates"], "gates", atol=1e-6, rtol=1e-5)
    if g["logits"] is not None:
        assert_close(g["logits"][tok], ref["logits"], "logits", atol=2e-6, rtol=2e-7)
    assert_close(g["y"][rows], ref["y"], "route rows Y")
    if cfg.shared_inter:
        assert_close(g["s"][tok], ref["s"], "shared expert S")
        assert_close(g["sg"][tok], ref["sg"], "shared gate", atol=1e-6, rtol=1e-5)
    assert_close(g["out32"][tok], ref["out"], "out_f32")
    assert np.array_equal(g["out16"], bf16_rne_bits(g["out32"])), "out_bf16 is not the RNE of out_f32"
    return ref, ties


def load_cfg(name, with_experts=True):
    cfg = W.CONFIGS[name]
    say(f"generating layer '{name}' (T={cfg.tokens}, H={cfg.hidden}, E={cfg.experts}, I={cfg.inter})")
    return cfg, W.make_layer(cfg, with_experts), W.tokens(cfg)
