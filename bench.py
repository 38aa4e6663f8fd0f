#!/usr/bin/env python3
"""Forward (and backward) throughput of the routed 512-expert top-10 MoE
layer on one MI355X.

One step = one whole forward pass (router, top-k, permutation, grouped
SwiGLU expert GEMMs with the shared expert, combine) over one batch of
seeded synthetic tokens, through the C ABI, inputs already resident in HBM.
The headline workload is the 1024-token layer (hidden 2048, 512 experts
top-10, expert and shared intermediate 512).

Timing protocol (the RL-Kernel pull request 557 page, "Latency" paragraph:
warm-up, then the median of 20 forward calls and of 5 forward + backward
calls), with the caches handled: W untimed warm-up calls, then K timed calls,
each bracketed by HIP events on the kernels' stream, with a 1 GiB scratch
write between calls so that no call finds the previous one's bytes in L2 or
the 256 MB MALL (followed by a 1 GiB read, so that the write's dirty lines
are written back before the call rather than during it).  ms_per_step is the median call; p10/p90 beside it; the
wall clock of the whole timed loop (evictions included) and a back-to-back
run without evictions are reported too.

Prints ONE JSON line.  Besides the headline it carries
  configs       every forward workload (tiny flushed and warm, 1K, 8K, the
                skewed 16K) with its roofline fractions;
  roofline      the dominant kernel (ffn_up at 1K) against the HBM peak,
                timed live with HIP events recorded by moe_forward_profiled
                on the stream the kernels run on;
  backward      the 4096-token backward: 5 forward + backward calls and K
                backward-only calls;
  cpu_baseline  the FP64 oracle timed on this host on bounded token samples
                of all five workloads.

usage: python bench.py [--gpus 1] [--steps 20] [--warmup 3]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time


def _blas_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    cap = os.environ.get("OMP_NUM_THREADS")
    return max(1, min(n, int(cap))) if cap and cap.isdigit() else n


# the oracle's BLAS threads are pinned before numpy is first imported
for _v in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
    os.environ[_v] = str(_blas_threads())

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0        # MI355X HBM3E, GB/s
PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, TFLOP/s
METRIC = "MoE-layer fwd tokens/sec at 1K & 8K tokens; % bf16 MFMA peak / % HBM GB/s"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "ffn_up_moe1k_traffic.txt")
FFN_SOURCE = os.path.join(ROOT, "mixture_experts_layer_counting_amd", "csrc", "ffn_kernels.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# HIP events through the runtime's C API (the library's stream is torch's
# current stream, so the events sit on the same stream as the kernels)
# ---------------------------------------------------------------------------
class Hip:
    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        # full signatures: an undeclared argument would be passed as a 32-bit int
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventCreate.restype = ctypes.c_int
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventElapsedTime.restype = ctypes.c_int

    def event(self):
        e = ctypes.c_void_p()
        if self.lib.hipEventCreate(ctypes.byref(e)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return e

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        if self.lib.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value


# ---------------------------------------------------------------------------
# algorithmic work (no redundant bytes counted: every weight byte of a touched
# expert once, activations/x once, the method's fp32 route rows Y once each way)
# ---------------------------------------------------------------------------
def ffn_up_bytes(cfg, touched):
    H, I, Is, T, R = cfg.hidden, cfg.inter, cfg.shared_inter, cfg.tokens, cfg.routes
    return (touched * 2 * I * H * 2 + (2 * Is * H * 2 if Is else 0) + T * H * 2
            + (R * I + T * Is) * 2 * 2)


def ffn_down_bytes(cfg, touched):
    H, I, Is, T, R = cfg.hidden, cfg.inter, cfg.shared_inter, cfg.tokens, cfg.routes
    return (touched * H * I * 2 + (H * Is * 2 if Is else 0) + (R * I + T * Is) * 2 * 2
            + (R + T) * H * 4)


def layer_work(cfg, touched):
    H, I, Is, T, R, E = cfg.hidden, cfg.inter, cfg.shared_inter, cfg.tokens, cfg.routes, cfg.experts
    flop = 2 * (R * 3 * I * H + T * 3 * Is * H)
    byts = (touched * 3 * I * H * 2 + 3 * Is * H * 2 + E * H * 4 + H * 2 + T * H * 2
            + R * H * 4 * 2 + T * H * 2)
    return flop, byts


def traffic_from_profile(workload: str):
    """Measured HBM bytes per ffn_up launch from the committed counter
    summary, or None if the summary is missing, the kernel source changed
    since the counters were taken, or the timed workload is not the one the
    counters were taken on (moe1k)."""
    if workload != "moe1k" or not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        if ":" in line:
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    src = hashlib.sha256(open(FFN_SOURCE, "rb").read()).hexdigest()[:16]
    if kv.get("ffn_kernels_sha256_16") != src or "traffic_bytes_per_launch" not in kv:
        return None
    return float(kv["traffic_bytes_per_launch"])


# ---------------------------------------------------------------------------
def device_layer(layer, cfg=None):
    """The layer's weights in device memory; with `cfg`, also the router
    weight's three bf16 planes, split once here (moe_split_router) as a
    deployment splits its constant router weight at load time."""
    import torch
    dev = torch.device("cuda:0")
    bits = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)
    f32 = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)
    import mixture_experts_layer_counting_amd as m
    w = m.Weights(w_router=f32(layer["w_router"]), w13=bits(layer["w13"]), w2=bits(layer["w2"]),
                  router_bias=f32(layer["router_bias"]), ws13=bits(layer["ws13"]), ws2=bits(layer["ws2"]),
                  w_sgate=bits(layer["w_sgate"]))
    if cfg is not None:
        d = m.Dims(cfg.tokens, cfg.hidden, cfg.experts, cfg.top_k, cfg.inter, cfg.shared_inter)
        w.w_router_planes = m.split_router(d, w.w_router)
    return w


class Evictor:
    """Between timed calls: a 1 GiB fill (more than L2, 4 MB per XCD, and
    the 256 MB MALL hold), then a 1 GiB read of another buffer, which pushes
    the fill's dirty lines out before the timed call, so that the call
    neither finds its own bytes in a cache nor pays for write-backs that
    are not its own."""

    def __init__(self, mib=1024):
        import torch
        n = mib * (1 << 20) // 4
        self.wbuf = torch.empty(n, dtype=torch.float32, device="cuda:0")
        self.rbuf = torch.ones(n, dtype=torch.float32, device="cuda:0")
        self.sink = torch.empty((), dtype=torch.float32, device="cuda:0")
        self.n = 0

    def __call__(self):
        import torch
        self.n += 1
        self.wbuf.fill_(float(self.n & 0xff))
        torch.sum(self.rbuf, dim=0, out=self.sink)


def stats(ms):
    a = np.asarray(ms, np.float64)
    return {"median_ms": float(np.median(a)), "p10_ms": float(np.percentile(a, 10)),
            "p90_ms": float(np.percentile(a, 90)), "mean_ms": float(a.mean()), "calls": int(a.size)}


def forward_inputs(cfg, w):
    import torch
    import mixture_experts_layer_counting_amd as m
    import workloads as W
    dev = torch.device("cuda:0")
    x = torch.from_numpy(W.tokens(cfg).view(np.int16)).to(dev)
    d = m.Dims(cfg.tokens, cfg.hidden, cfg.experts, cfg.top_k, cfg.inter, cfg.shared_inter)
    return dict(d=d, x=x, routes=m.alloc_routes(d, dev, logits=False), saved=m.alloc_saved(d, dev),
                out16=torch.empty(d.tokens, d.hidden, dtype=torch.int16, device=dev),
                ws=m.alloc_workspace(d, m.MOE_OP_FORWARD, dev))


def run_config(cfg, w, steps, warmup, hip, evict, breakdown=True, side=True):
    """Time `steps` forwards of `cfg`, each bracketed by HIP events on the
    kernels' stream with an eviction write before it (the events around
    ffn_up give the roofline kernel's duration in the same calls); then a
    back-to-back run of `steps` forwards without evictions (wall clock), and,
    untimed, one pass with an event before every kernel for the per-kernel
    breakdown.  Returns the measurements."""
    import torch
    import mixture_experts_layer_counting_amd as m
    f = forward_inputs(cfg, w)
    d, x, routes, saved, out16, ws = f["d"], f["x"], f["routes"], f["saved"], f["out16"], f["ws"]
    names = m.forward_kernel_names(d)
    nk = len(names)
    assert nk == m.moe_forward_kernel_count(d)
    iu = names.index("ffn_up")
    stream = torch.cuda.current_stream()
    evs = []
    for _ in range(steps):
        arr = (ctypes.c_void_p * (nk + 1))()
        for k in {0, iu, iu + 1, nk}:
            arr[k] = hip.event()
        evs.append(arr)

    def fwd():
        m.check(m.moe_forward(d, w, x, routes, saved, None, out16, ws, stream), "moe_forward")

    for _ in range(warmup):
        fwd()
    torch.cuda.synchronize()
    # timed region: exactly `steps` forwards, an eviction write before each
    t0 = time.perf_counter()
    for i in range(steps):
        evict()
        m.check(m.moe_forward_profiled(d, w, x, routes, saved, None, out16, ws, evs[i], stream),
                "moe_forward_profiled")
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    call_ms = [hip.elapsed_ms(evs[i][0], evs[i][nk]) for i in range(steps)]
    up_ms = [hip.elapsed_ms(evs[i][iu], evs[i][iu + 1]) for i in range(steps)]
    # back to back, no evictions, wall clock
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fwd()
    torch.cuda.synchronize()
    b2b = (time.perf_counter() - t0) / steps * 1e3
    per_kernel = {}
    if breakdown:
        # untimed: an event before every kernel (each marker adds its own gap)
        mk = [(ctypes.c_void_p * (nk + 1))(*[hip.event() for _ in range(nk + 1)]) for _ in range(3)]
        for i in range(3):
            evict()
            m.check(m.moe_forward_profiled(d, w, x, routes, saved, None, out16, ws, mk[i], stream),
                    "moe_forward_profiled")
        torch.cuda.synchronize()
        per_kernel = {n: float(np.median([hip.elapsed_ms(mk[i][k], mk[i][k + 1]) for i in range(3)]))
                      for k, n in enumerate(names)}
    assert m.moe_last_device_error(ws) == m.MOE_OK
    # the same forwards with the shared expert on a side stream (moe_forward_side)
    streams = m.SideStreams(torch.device("cuda:0")) if side else None

    def fwd_side():
        m.check(m.moe_forward_side(d, w, x, routes, saved, None, out16, ws, streams, stream), "moe_forward_side")

    for _ in range(warmup if side else 0):
        fwd_side()
    torch.cuda.synchronize()
    side_ms = []
    for _ in range(steps if side else 0):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        evict()
        e0.record(stream)
        fwd_side()
        e1.record(stream)
        torch.cuda.synchronize()
        side_ms.append(e0.elapsed_time(e1))
    assert m.moe_last_device_error(ws) == m.MOE_OK
    touched = int((np.diff(routes.expert_offsets.cpu().numpy()) > 0).sum())
    load = np.diff(routes.expert_offsets.cpu().numpy())
    return dict(call=stats(call_ms), up=stats(up_ms), wall_ms=wall / steps * 1e3, b2b_ms=b2b,
                per_kernel=per_kernel, touched=touched, max_load=int(load.max()),
                empty=int((load == 0).sum()), side=stats(side_ms) if side_ms else None)


def summarize(cfg, r):
    ms = r["call"]["median_ms"]
    flop, byts = layer_work(cfg, r["touched"])
    t_mfma = flop / (PEAK_BF16_TFLOPS * 1e12)
    t_hbm = byts / (PEAK_HBM_GBS * 1e9)
    t_roof = max(t_mfma, t_hbm)
    out = dict(
        workload=f"{cfg.name}: {cfg.tokens} tokens, hidden {cfg.hidden}, {cfg.experts} experts top-{cfg.top_k}, "
                 f"expert inter {cfg.inter}, shared inter {cfg.shared_inter}"
                 + (f", router bias Zipf s={cfg.zipf_s} (tau {cfg.zipf_tau}, {cfg.zipf_off} experts off)"
                    if cfg.zipf_s else ""),
        tokens_per_s=cfg.tokens / (ms / 1e3),
        ms_per_step=ms, p10_ms=r["call"]["p10_ms"], p90_ms=r["call"]["p90_ms"],
        wall_ms_per_step_incl_eviction=r["wall_ms"], back_to_back_ms_per_step=r["b2b_ms"],
        ffn_up_ms=r["up"]["mean_ms"], ffn_up_median_ms=r["up"]["median_ms"],
        kernel_ms_marked=r["per_kernel"],
        touched_experts=r["touched"], max_expert_routes=r["max_load"], empty_experts=r["empty"],
        layer_roofline=dict(
            flop=flop, bytes=byts, t_roof_ms=t_roof * 1e3, t_mfma_ms=t_mfma * 1e3, t_hbm_ms=t_hbm * 1e3,
            bound="mfma" if t_mfma > t_hbm else "hbm",
            frac=t_roof / (ms / 1e3),
            hbm_frac=byts / (ms / 1e3) / (PEAK_HBM_GBS * 1e9),
            mfma_frac=flop / (ms / 1e3) / (PEAK_BF16_TFLOPS * 1e12),
            mfma_frac_cap=t_mfma / t_roof),
    )
    sm = r["side"]["median_ms"] if r["side"] else None
    out["side_streams"] = None if sm is None else dict(what="moe_forward_side: the shared expert's GEMMs on a side stream beside "
                                    "the routing and the routed GEMMs (same protocol, bit-identical output)",
                               ms_per_step=sm, p10_ms=r["side"]["p10_ms"], p90_ms=r["side"]["p90_ms"],
                               tokens_per_s=cfg.tokens / (sm / 1e3), layer_roofline_frac=t_roof / (sm / 1e3))
    if r["per_kernel"]:
        out["ffn_up_gbs"] = ffn_up_bytes(cfg, r["touched"]) / (r["up"]["mean_ms"] / 1e3) / 1e9
        out["ffn_down_gbs"] = ffn_down_bytes(cfg, r["touched"]) / (r["per_kernel"]["ffn_down"] / 1e3) / 1e9
    return out


def expert_share(m, cfg, w, x, share):
    """One GPU's share of an expert-parallel layout over `share` GPUs: the
    dims, weights and permutation of experts [0, E/share) with their routes
    of this batch (from the full layer's routing on the GPU), in ascending
    route id per expert -- what that GPU's grouped FFN receives after the
    exchange.  No shared expert (it is not expert-sharded)."""
    import torch
    dev = x.device
    d = m.Dims(cfg.tokens, cfg.hidden, cfg.experts, cfg.top_k, cfg.inter, cfg.shared_inter)
    routes = m.alloc_routes(d, dev, logits=False)
    ws = m.alloc_workspace(d, m.MOE_OP_FORWARD, dev)
    m.check(m.moe_route(d, x, w, routes, ws), "moe_route")
    m.check(m.moe_permute(d, routes, ws), "moe_permute")
    torch.cuda.synchronize()
    el = cfg.experts // share
    dl = m.Dims(cfg.tokens, cfg.hidden, el, cfg.top_k, cfg.inter, 0)
    rl = m.alloc_routes(dl, dev, logits=False)
    rl.expert_offsets.copy_(routes.expert_offsets[:el + 1])
    n_local = int(routes.expert_offsets[el].item())
    rl.sorted_route.fill_(-1)
    rl.sorted_route[:n_local].copy_(routes.sorted_route[:n_local])
    wl = m.Weights(w_router=w.w_router, w13=w.w13, w2=w.w2, router_bias=w.router_bias)
    return dl, wl, rl, routes, n_local


def run_ep_share(cfg, w, steps, warmup, share):
    """Grouped FFN (up + down) of one GPU's expert share, HIP-event timed on
    the kernels' stream."""
    import torch
    import mixture_experts_layer_counting_amd as m
    import workloads as W
    dev = torch.device("cuda:0")
    x = torch.from_numpy(W.tokens(cfg).view(np.int16)).to(dev)
    dl, wl, rl, _, n_local = expert_share(m, cfg, w, x, share)
    saved = m.alloc_saved(dl, dev)
    ws = m.alloc_workspace(dl, m.MOE_OP_FFN, dev)
    stream = torch.cuda.current_stream()

    def ffn():
        m.check(m.moe_grouped_ffn(dl, x, wl, rl, saved, ws, stream), "moe_grouped_ffn")

    for _ in range(warmup):
        ffn()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(steps):
        ffn()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    touched = int((np.diff(rl.expert_offsets.cpu().numpy()) > 0).sum())
    H, I = cfg.hidden, cfg.inter
    # touched local experts' weights once, their x rows gathered once per
    # route, act hi/lo written and read once, fp32 route rows written once
    byts = touched * 3 * I * H * 2 + n_local * H * 2 + n_local * I * 4 * 2 + n_local * H * 4
    return {"workload": f"{cfg.name}: experts [0, {dl.experts}) of {cfg.experts} (one GPU of {share}) "
                        f"with their {n_local} routes, grouped FFN only",
            "ms": ms, "routes": n_local, "bytes": byts,
            "hbm_frac": byts / (ms / 1e3) / (PEAK_HBM_GBS * 1e9)}


def run_mx(cfg, layer, steps, warmup):
    """The forward with block-scaled FP8 expert weights (the layer's bf16
    expert weights encoded to OCP MX E4M3 + E8M0 scales per 32 elements),
    HIP-event timed on the kernels' stream over `steps` forwards."""
    import torch
    import mixture_experts_layer_counting_amd as m
    import workloads as W
    import workloads.mx as MX
    dev = torch.device("cuda:0")
    mxl = MX.mx_layer(layer)
    u8 = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a, np.uint8)).to(dev)
    f32 = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)
    bits = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)
    g = lambda k, i: None if mxl[k] is None else u8(mxl[k][i])
    wm = m.WeightsMx(w_router=f32(layer["w_router"]), router_bias=f32(layer["router_bias"]),
                     w13_q=g("w13", 0), w13_s=g("w13", 1), w2_q=g("w2", 0), w2_s=g("w2", 1),
                     ws13_q=g("ws13", 0), ws13_s=g("ws13", 1), ws2_q=g("ws2", 0), ws2_s=g("ws2", 1),
                     w_sgate=bits(layer["w_sgate"]))
    del mxl
    x = torch.from_numpy(W.tokens(cfg).view(np.int16)).to(dev)
    d = m.Dims(cfg.tokens, cfg.hidden, cfg.experts, cfg.top_k, cfg.inter, cfg.shared_inter)
    wm.w_router_planes = m.split_router(d, wm.w_router)  # once, as at weight load
    routes = m.alloc_routes(d, dev, logits=False)
    saved = m.alloc_saved(d, dev)
    out16 = torch.empty(d.tokens, d.hidden, dtype=torch.int16, device=dev)
    ws = m.alloc_workspace(d, m.MOE_OP_FORWARD, dev)
    stream = torch.cuda.current_stream()

    def fwd():
        m.check(m.moe_forward_mx(d, wm, x, routes, saved, None, out16, ws, stream), "moe_forward_mx")

    for _ in range(warmup):
        fwd()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(steps):
        fwd()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    assert m.moe_last_device_error(ws) == m.MOE_OK
    touched = int((np.diff(routes.expert_offsets.cpu().numpy()) > 0).sum())
    H, I, Is, T, R, E = cfg.hidden, cfg.inter, cfg.shared_inter, cfg.tokens, cfg.routes, cfg.experts
    # as the bf16 layer's bytes with one byte per expert weight plus one
    # scale byte per 32
    wb = 1 + 1 / 32
    byts = (touched * 3 * I * H * wb + 3 * Is * H * wb + E * H * 4 + H * 2 + T * H * 2
            + R * H * 4 * 2 + T * H * 2)
    return {"workload": f"{cfg.name}: {T} tokens, expert weights block-scaled FP8 (OCP MX E4M3, "
                        f"32-element E8M0 scales)", "dtype": "bf16 activations, fp8-e4m3 expert weights",
            "ms": ms, "tokens_per_s": T / (ms / 1e3), "bytes": byts,
            "hbm_frac": byts / (ms / 1e3) / (PEAK_HBM_GBS * 1e9)}


def run_lora(cfg, w, steps, warmup):
    """The forward with LoRA adapters on every routed expert (seeded, rank
    64 // 10 = 6), HIP-event timed on the kernels' stream over `steps`
    forwards, with the plain forward timed the same way beside it."""
    import torch
    import mixture_experts_layer_counting_amd as m
    import workloads as W
    import workloads.lora as WL
    dev = torch.device("cuda:0")
    ad = WL.lora_adapters(cfg)
    bits = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)
    lo = m.Lora(rank=ad["rank"], scale=ad["scale"], a13=bits(ad["a13"]), b13=bits(ad["b13"]),
                a2=bits(ad["a2"]), b2=bits(ad["b2"]))
    x = torch.from_numpy(W.tokens(cfg).view(np.int16)).to(dev)
    d = m.Dims(cfg.tokens, cfg.hidden, cfg.experts, cfg.top_k, cfg.inter, cfg.shared_inter)
    routes = m.alloc_routes(d, dev, logits=False)
    saved = m.alloc_saved(d, dev)
    out16 = torch.empty(d.tokens, d.hidden, dtype=torch.int16, device=dev)
    ws = m.alloc_workspace(d, m.MOE_OP_FORWARD_LORA, dev)
    stream = torch.cuda.current_stream()

    def timed(fn):
        for _ in range(warmup):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    ms = timed(lambda: m.check(m.moe_forward_lora(d, w, lo, x, routes, saved, None, out16, ws, stream),
                               "moe_forward_lora"))
    assert m.moe_last_device_error(ws) == m.MOE_OK
    ms_plain = timed(lambda: m.check(m.moe_forward(d, w, x, routes, saved, None, out16, ws, stream),
                                     "moe_forward"))
    return {"workload": f"{cfg.name}: {cfg.tokens} tokens, LoRA adapters of rank {ad['rank']} on all "
                        f"{cfg.experts} routed experts", "ms": ms, "tokens_per_s": cfg.tokens / (ms / 1e3),
            "plain_forward_ms": ms_plain, "adapter_bytes": sum(int(ad[k].nbytes) for k in ("a13", "b13", "a2", "b2"))}


def run_backward(cfg, w, steps, warmup, evict, fb_calls=5, lora=True, side=True):
    """`fb_calls` forward (training mode) + backward calls, then `steps`
    backward-only calls of the same batch, each HIP-event timed on the
    kernels' stream with an eviction write before it.  With `lora`, also
    `steps` backward calls of the layer with seeded LoRA adapters on every
    routed expert (after one training-mode LoRA forward), timed the same
    way."""
    import torch
    import mixture_experts_layer_counting_amd as m
    import workloads as W
    dev = torch.device("cuda:0")
    x = torch.from_numpy(W.tokens(cfg).view(np.int16)).to(dev)
    dout = torch.from_numpy(W.grad_out(cfg).view(np.int16)).to(dev)
    d = m.Dims(cfg.tokens, cfg.hidden, cfg.experts, cfg.top_k, cfg.inter, cfg.shared_inter)
    ws = m.alloc_workspace(d, m.MOE_OP_BACKWARD_LORA if lora else m.MOE_OP_BACKWARD, dev)
    routes = m.alloc_routes(d, dev, logits=False)
    saved = m.alloc_saved(d, dev, training=True)
    out16 = torch.empty(d.tokens, d.hidden, dtype=torch.int16, device=dev)
    grads = m.alloc_grads(d, dev)
    dx32 = torch.empty(d.tokens, d.hidden, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def fwd():
        m.check(m.moe_forward(d, w, x, routes, saved, None, out16, ws, stream), "moe_forward")

    def bwd():
        m.check(m.moe_backward(d, w, x, routes, saved, dout, dx32, None, grads, ws, stream), "moe_backward")

    def timed(fn, n):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        for e0, e1 in ev:
            evict()
            e0.record(stream)
            fn()
            e1.record(stream)
        torch.cuda.synchronize()
        return stats([e0.elapsed_time(e1) for e0, e1 in ev])

    fb = timed(lambda: (fwd(), bwd()), fb_calls)
    bo = timed(bwd, steps)
    assert m.moe_last_device_error(ws) == m.MOE_OK
    bs = None
    if side:
        streams = m.SideStreams(dev)
        bs = timed(lambda: m.check(m.moe_backward_side(d, w, x, routes, saved, dout, dx32, None, grads, ws,
                                                       streams, stream), "moe_backward_side"), steps)
        assert m.moe_last_device_error(ws) == m.MOE_OK
    lb = None
    if lora:
        import workloads.lora as WL
        ad = WL.lora_adapters(cfg)
        bits = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)
        lo = m.Lora(rank=ad["rank"], scale=ad["scale"], a13=bits(ad["a13"]), b13=bits(ad["b13"]),
                    a2=bits(ad["a2"]), b2=bits(ad["b2"]))
        lg = m.alloc_lora_grads(d, lo.rank, dev)
        m.check(m.moe_forward_lora(d, w, lo, x, routes, saved, None, out16, ws, stream), "moe_forward_lora")
        lbs = timed(lambda: m.check(m.moe_backward_lora(d, w, lo, x, routes, saved, dout, dx32, None, grads, lg,
                                                        ws, stream), "moe_backward_lora"), steps)
        assert m.moe_last_device_error(ws) == m.MOE_OK
        lss = None
        if side:
            streams_l = m.SideStreams(dev)
            lss = timed(lambda: m.check(m.moe_backward_lora_side(d, w, lo, x, routes, saved, dout, dx32, None, grads,
                                                                 lg, ws, streams_l, stream),
                                        "moe_backward_lora_side"), steps)
            assert m.moe_last_device_error(ws) == m.MOE_OK
        lb = {"workload": f"{cfg.name}: backward with LoRA adapters of rank {ad['rank']} on all {cfg.experts} "
                          f"routed experts (adapter gradients included)",
              "ms": lbs["median_ms"], "p10_ms": lbs["p10_ms"], "p90_ms": lbs["p90_ms"], "calls": lbs["calls"],
              "tokens_per_s": cfg.tokens / (lbs["median_ms"] / 1e3),
              "over_plain_ms": lbs["median_ms"] - bo["median_ms"],
              "side_streams_ms": lss["median_ms"] if lss else None}
    touched = int((np.diff(routes.expert_offsets.cpu().numpy()) > 0).sum())
    H, I, Is, T, R, E = cfg.hidden, cfg.inter, cfg.shared_inter, cfg.tokens, cfg.routes, cfg.experts
    # algorithmic bytes: weights read, fp32 weight gradients written, per-route
    # and per-token activations read once (gate/up, x, dOut), dx route rows
    # written and read once, dX written
    byts = (touched * 3 * I * H * 2 + 3 * Is * H * 2 + E * H * 4 + touched * 3 * I * H * 4 + 3 * Is * H * 4
            + E * H * 4 + R * 2 * I * 4 + T * 2 * Is * 4 + T * H * 4 + 2 * T * H * 2
            + R * H * 4 * 2 + T * H * 4)
    flop = 2 * 2 * (R * 3 * I * H + T * 3 * Is * H)
    ms = bo["median_ms"]
    t_roof = max(flop / (PEAK_BF16_TFLOPS * 1e12), byts / (PEAK_HBM_GBS * 1e9))
    return {"workload": f"{cfg.name}: {T} tokens backward (hidden {H}, {E} experts top-{cfg.top_k}, "
                        f"inter {I}, shared {Is})",
            "ms": ms, "p10_ms": bo["p10_ms"], "p90_ms": bo["p90_ms"], "calls": bo["calls"],
            "tokens_per_s": T / (ms / 1e3),
            "fwd_bwd_ms": fb["median_ms"], "fwd_bwd_p10_ms": fb["p10_ms"], "fwd_bwd_p90_ms": fb["p90_ms"],
            "fwd_bwd_calls": fb["calls"], "fwd_bwd_tokens_per_s": T / (fb["median_ms"] / 1e3),
            "bytes": byts, "flop": flop, "t_roof_ms": t_roof * 1e3, "roofline_frac": t_roof / (ms / 1e3),
            "hbm_frac": byts / (ms / 1e3) / (PEAK_HBM_GBS * 1e9),
            "mfma_frac": flop / (ms / 1e3) / (PEAK_BF16_TFLOPS * 1e12), "lora": lb,
            "side_streams": None if bs is None else {
                "what": "moe_backward_side: dW13 and dW2 on two caller-owned streams beside dx",
                "ms": bs["median_ms"], "p10_ms": bs["p10_ms"], "p90_ms": bs["p90_ms"],
                "calls": bs["calls"], "tokens_per_s": T / (bs["median_ms"] / 1e3)}}


def gpu_info():
    """Identity of the timed GPU (torch's view of the HIP device)."""
    import torch
    p = torch.cuda.get_device_properties(0)
    return {"name": p.name, "arch": getattr(p, "gcnArchName", "unknown"),
            "compute_units": p.multi_processor_count, "memory_gib": round(p.total_memory / 2**30, 1)}


def achieved_peaks():
    """What this machine reaches, beside the vendor peaks, with the library's
    measurement probes (include/moe_probes.h): a 4 GiB streaming read, a
    2 GiB streaming copy (read + write bytes) and back-to-back bf16 MFMAs on
    independent accumulators; each the median of 5 HIP-event-timed runs
    after a warm-up."""
    import torch
    import mixture_experts_layer_counting_amd as m
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()

    def timed(fn, n=5):
        fn()
        ms = []
        for _ in range(n):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ms.append(e0.elapsed_time(e1))
        return float(np.median(ms))

    sink = torch.zeros(64, dtype=torch.float32, device=dev)
    a = torch.ones((1 << 30,), dtype=torch.float32, device=dev)
    read_ms = timed(lambda: m.check(m.moe_probe_read(a, 1 << 32, sink, stream), "moe_probe_read"))
    b = torch.empty((1 << 29,), dtype=torch.float32, device=dev)
    copy_ms = timed(lambda: m.check(m.moe_probe_copy(b, a, 1 << 31, stream), "moe_probe_copy"))
    del a, b
    iters = 8192
    mfma_ms = timed(lambda: m.check(m.moe_probe_mfma(sink, iters, stream), "moe_probe_mfma"))
    torch.cuda.empty_cache()
    flop = iters * 1024 * 4 * 8 * 32768
    return {"read_gbs": (1 << 32) / (read_ms / 1e3) / 1e9, "copy_gbs": (1 << 32) / (copy_ms / 1e3) / 1e9,
            "bf16_mfma_tflops": flop / (mfma_ms / 1e3) / 1e12,
            "how": "moe_probe_read (4 GiB), moe_probe_copy (2 GiB, read + write bytes), moe_probe_mfma "
                   "(32x32x16 bf16, 8 independent accumulators per wave); median of 5 after a warm-up"}


def host_info():
    """CPU model, BLAS library and thread count of this host."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:  # pragma: no cover
        pass
    blas, threads = "unknown", 1
    try:
        from threadpoolctl import threadpool_info
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if info:
            blas = f"{info[0].get('internal_api')} {info[0].get('version')}"
            threads = int(info[0].get("num_threads", 1))
    except Exception:  # pragma: no cover
        pass
    return model, blas, threads


def cpu_baseline(layers, sample=32, bwd_sample=16, tiny_calls=20):
    """The FP64 oracle as it stands, timed on this host: for each workload one
    warm-up call and the median of 3 calls (the tiny one: `tiny_calls`),
    excluding data generation, on the workload's first `sample` tokens (the
    whole batch for the tiny one; `bwd_sample` for the backward workload,
    whose oracle allocates the dense fp64 weight gradients of every expert);
    forward for the forward workloads,
    forward + backward for the backward one.  Reported as tokens/s."""
    import oracle as O
    import workloads as W
    model, blas, threads = host_info()
    per = {}
    for name, layer in layers.items():
        cfg = W.CONFIGS[name]
        n = cfg.tokens if name == "tiny" else min(bwd_sample if cfg.backward else sample, cfg.tokens)
        x = W.tokens(cfg)[:n]
        if cfg.backward:
            dout = W.grad_out(cfg)[:n]
            fn = lambda: O.backward(layer, x, O.forward(layer, x, cfg.top_k), dout)
        else:
            fn = lambda: O.forward(layer, x, cfg.top_k)
        fn()
        times = []
        for _ in range(tiny_calls if name == "tiny" else 3):
            t0 = time.perf_counter()
            fn()
            times.append(time.perf_counter() - t0)
        med = float(np.median(times))
        per[name] = {"tokens_per_s": n / med, "median_s": med, "tokens": n, "calls": len(times),
                     "what": "forward + backward" if cfg.backward else "forward"}
        log(f"bench: cpu oracle {name}: {n / med:.1f} tokens/s")
    head = per["moe1k"]
    return {"value": head["tokens_per_s"], "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"oracle (numpy float64) on the first {head['tokens']} tokens of the moe1k workload, "
                      f"median of {head['calls']} calls after one warm-up; every workload in per_config",
            "cpu_model": model, "blas": blas, "per_config": per}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="moe1k")
    ap.add_argument("--configs", default="tiny,moe8k,skew16k",
                    help="further forward workloads to report (comma separated), or 'none'")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--backward", default="bwd4k", help="workload of the backward timing, or 'none'")
    ap.add_argument("--ep-share", type=int, default=8,
                    help="also time the grouped FFN on one GPU's share of this many expert-parallel GPUs (0: off)")
    ap.add_argument("--mx", type=int, default=1,
                    help="also time the forward with block-scaled FP8 expert weights (0: off)")
    ap.add_argument("--lora", type=int, default=1,
                    help="also time the forward with LoRA adapters on the routed experts (0: off)")
    ap.add_argument("--no-evict", action="store_true", help="time without the eviction writes (profiling runs)")
    ap.add_argument("--no-peaks", action="store_true", help="skip the achieved-peak probes")
    ap.add_argument("--no-side", action="store_true",
                    help="skip the side-stream variants (profiling runs: their shared-only launches share kernel names)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also launch one plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library runs the whole layer on a single MI355X "
              "with all experts resident and has no multi-GPU path", file=sys.stderr)
        sys.exit(2)

    import torch
    import mixture_experts_layer_counting_amd as m
    import workloads as W
    m.load_library()
    hip = Hip()
    cfg = W.CONFIGS[args.config]
    extra = [] if args.configs == "none" else [c for c in args.configs.split(",") if c and c != cfg.name]
    # host layers: the 2048-hidden workloads share one set of weights (the
    # skewed one adds its router bias)
    host = {}

    def host_layer(c):
        key = (c.hidden, c.inter, c.shared_inter, c.experts, c.seed)
        if key not in host:
            log(f"bench: generating the weights of {c.name}")
            host[key] = W.make_layer(c)
        base = host[key]
        return base if c.zipf_s == 0.0 else dict(base, router_bias=W.zipf_bias(c))

    dev_cache = {}

    def dev_layer(c):
        key = (c.hidden, c.inter, c.shared_inter, c.experts, c.seed)
        if key not in dev_cache:
            dev_cache[key] = device_layer(host_layer(c), c)
        w = dev_cache[key]
        if c.zipf_s == 0.0:
            return w
        b = torch.from_numpy(np.ascontiguousarray(W.zipf_bias(c), np.float32)).to("cuda:0")
        return m.Weights(w_router=w.w_router, w13=w.w13, w2=w.w2, router_bias=b, ws13=w.ws13, ws2=w.ws2,
                         w_sgate=w.w_sgate, w_router_planes=w.w_router_planes)

    w = dev_layer(cfg)
    evict = (lambda: None) if args.no_evict else Evictor()
    torch.cuda.synchronize()

    if args.copy_probe_mib:
        n = args.copy_probe_mib * (1 << 20) // 4
        a = torch.empty(n, dtype=torch.float32, device="cuda:0").fill_(1.0)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    log(f"bench: {cfg.name} warmup {args.warmup}, steps {args.steps}")
    main_r = run_config(cfg, w, args.steps, args.warmup, hip, evict, side=not args.no_side)
    main_s = summarize(cfg, main_r)
    log(f"bench: {cfg.name} median {main_s['ms_per_step']:.3f} ms (p10 {main_s['p10_ms']:.3f}, "
        f"p90 {main_s['p90_ms']:.3f}), back to back {main_s['back_to_back_ms_per_step']:.3f} ms, "
        + (f"side streams {main_s['side_streams']['ms_per_step']:.3f} ms, " if main_s["side_streams"] else "") +
        f"kernels {main_s['kernel_ms_marked']}")

    configs = {cfg.name: main_s}
    for name in extra:
        c2 = W.CONFIGS[name]
        log(f"bench: {c2.name} warmup {args.warmup}, steps {args.steps}")
        r2 = run_config(c2, dev_layer(c2), args.steps, args.warmup, hip, evict, side=not args.no_side)
        configs[c2.name] = summarize(c2, r2)
        if name == "tiny":
            # the tiny layer's weights fit in the MALL: its warm number beside the flushed one
            configs[c2.name]["warm_ms_per_step"] = configs[c2.name]["back_to_back_ms_per_step"]
        ss = configs[c2.name]["side_streams"]
        log(f"bench: {c2.name} median {configs[c2.name]['ms_per_step']:.3f} ms"
            + (f" (side streams {ss['ms_per_step']:.3f})" if ss else "")
            + f", roofline {configs[c2.name]['layer_roofline']['frac']:.3f}")

    ep_share = None
    if args.ep_share > 1:
        log(f"bench: grouped FFN on one of {args.ep_share} expert shares")
        ep_share = run_ep_share(cfg, w, args.steps, args.warmup, args.ep_share)
        log(f"bench: expert share {ep_share['ms']:.3f} ms")

    mx = None
    if args.mx:
        log(f"bench: {cfg.name} with block-scaled FP8 expert weights")
        mx = run_mx(cfg, host_layer(cfg), args.steps, args.warmup)
        log(f"bench: {cfg.name} mx {mx['ms']:.3f} ms/step")

    lora = None
    if args.lora:
        log(f"bench: {cfg.name} with LoRA adapters")
        lora = run_lora(cfg, w, args.steps, args.warmup)
        log(f"bench: {cfg.name} lora {lora['ms']:.3f} ms/step (plain {lora['plain_forward_ms']:.3f})")

    backward = None
    if args.backward != "none":
        cb = W.CONFIGS[args.backward]
        log(f"bench: backward {cb.name}")
        backward = run_backward(cb, dev_layer(cb), args.steps, 1, evict, lora=bool(args.lora), side=not args.no_side)
        log(f"bench: backward {backward['ms']:.3f} ms"
            + (f" (side streams {backward['side_streams']['ms']:.3f} ms)" if backward["side_streams"] else "")
            + f", forward + backward {backward['fwd_bwd_ms']:.3f} ms"
            + (f", LoRA backward {backward['lora']['ms']:.3f} ms" if backward["lora"] else ""))

    cpu = None
    if not args.no_cpu_baseline:
        log("bench: cpu baseline (oracle)")
        names = [cfg.name] + extra + ([args.backward] if args.backward != "none" else [])
        if "moe1k" not in names:
            names.append("moe1k")
        cpu = cpu_baseline({n: host_layer(W.CONFIGS[n]) for n in dict.fromkeys(names)})

    peaks = None
    if not args.no_peaks:
        log("bench: achieved peaks (read stream, copy, bf16 MFMA)")
        peaks = achieved_peaks()
        log(f"bench: achieved read {peaks['read_gbs']:.0f} GB/s, copy {peaks['copy_gbs']:.0f} GB/s, "
            f"bf16 MFMA {peaks['bf16_mfma_tflops']:.0f} TFLOP/s")

    up_ms = main_s["ffn_up_ms"]
    up_bytes = ffn_up_bytes(cfg, main_r["touched"])
    achieved = up_bytes / (up_ms / 1e3) / 1e9
    traffic = traffic_from_profile(cfg.name)
    line = {
        "metric": METRIC,
        "value": main_s["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_s["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) tokens, N(0,0.02) weights; no checkpoint)",
        "config": {"workload": main_s["workload"], "tokens": cfg.tokens, "hidden": cfg.hidden,
                   "experts": cfg.experts, "top_k": cfg.top_k, "inter": cfg.inter,
                   "shared_inter": cfg.shared_inter,
                   "router_weight": "fp32, split once into its exact bf16 planes at weight load (moe_split_router)"},
        "timing": {"protocol": ("median of the timed calls, each bracketed by HIP events on the kernels' "
                                "stream after a 1 GiB eviction write and a 1 GiB read" if not args.no_evict else
                                "median of the timed calls, HIP events, no eviction writes"),
                   "p10_ms": main_s["p10_ms"], "p90_ms": main_s["p90_ms"],
                   "wall_ms_per_step_incl_eviction": main_s["wall_ms_per_step_incl_eviction"],
                   "back_to_back_ms_per_step": main_s["back_to_back_ms_per_step"]},
        "roofline": {"kernel": "ffn_up", "bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS, "traffic": traffic,
                     "algorithmic_bytes": up_bytes, "avg_ms": up_ms,
                     "median_ms": main_s["ffn_up_median_ms"],
                     "frac_of_achieved_read": achieved / peaks["read_gbs"] if peaks else None},
        "gpu": gpu_info(),
        "achieved_peaks": peaks,
        "layer_roofline": main_s["layer_roofline"],
        "cpu_baseline": cpu,
        "configs": configs,
        "ep_share": ep_share,
        "mx_weights": mx,
        "lora": lora,
        "backward": backward,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
