#!/usr/bin/env python3
"""Forward throughput of the routed 512-expert top-10 MoE layer on one MI355X.

One step = one whole forward pass (router, top-k, permutation, grouped
SwiGLU expert GEMMs with the shared expert, combine) over one batch of
seeded synthetic tokens, through the C ABI, inputs already resident in HBM.
The headline workload is the 1024-token layer (hidden 2048, 512 experts
top-10, expert and shared intermediate 512); the 8192-token layer is reported
alongside under "secondary".

Prints ONE JSON line.  Besides the throughput it carries
  roofline      the dominant kernel (ffn_up) against the HBM peak, timed live
                with HIP events recorded by moe_forward_profiled on the
                stream the kernels run on, over the timed steps;
  layer_roofline the whole forward against max(FLOP/MFMA peak, bytes/HBM peak);
  cpu_baseline  the FP64 oracle timed on this host on a bounded token sample.

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


def traffic_from_profile():
    """Measured HBM bytes per ffn_up launch from the committed counter
    summary, or None if the summary is missing or the kernel source changed
    since the counters were taken."""
    if not os.path.exists(TRAFFIC_FILE):
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
def device_layer(layer):
    import torch
    dev = torch.device("cuda:0")
    bits = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)
    f32 = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)
    import mixture_experts_layer_counting_amd as m
    return m.Weights(w_router=f32(layer["w_router"]), w13=bits(layer["w13"]), w2=bits(layer["w2"]),
                     router_bias=f32(layer["router_bias"]), ws13=bits(layer["ws13"]), ws2=bits(layer["ws2"]),
                     w_sgate=bits(layer["w_sgate"]))


def run_config(cfg, w, steps, warmup, hip):
    """Time `steps` profiled forwards; returns a dict of measurements."""
    import torch
    import mixture_experts_layer_counting_amd as m
    import workloads as W
    dev = torch.device("cuda:0")
    x = torch.from_numpy(W.tokens(cfg).view(np.int16)).to(dev)
    d = m.Dims(cfg.tokens, cfg.hidden, cfg.experts, cfg.top_k, cfg.inter, cfg.shared_inter)
    routes = m.alloc_routes(d, dev, logits=False)
    saved = m.alloc_saved(d, dev)
    out16 = torch.empty(d.tokens, d.hidden, dtype=torch.int16, device=dev)
    ws = m.alloc_workspace(d, m.MOE_OP_FORWARD, dev)
    names = m.forward_kernel_names(d)
    nk = len(names)
    assert nk == m.moe_forward_kernel_count(d)
    iu = names.index("ffn_up")
    # timed region: events only around ffn_up (the roofline kernel), so the
    # step time carries no per-kernel marker overhead
    up_evs = []
    for _ in range(steps):
        arr = (ctypes.c_void_p * (nk + 1))()
        arr[iu], arr[iu + 1] = hip.event(), hip.event()
        up_evs.append(arr)
    stream = torch.cuda.current_stream()

    def fwd():
        m.check(m.moe_forward(d, w, x, routes, saved, None, out16, ws, stream), "moe_forward")

    for _ in range(warmup):
        fwd()
    torch.cuda.synchronize()
    # timed region: exactly `steps` forwards
    t0 = time.perf_counter()
    for i in range(steps):
        m.check(m.moe_forward_profiled(d, w, x, routes, saved, None, out16, ws, up_evs[i], stream),
                "moe_forward_profiled")
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    up_ms = [hip.elapsed_ms(up_evs[i][iu], up_evs[i][iu + 1]) for i in range(steps)]
    # untimed: the same number of forwards with an event before every kernel,
    # for the per-kernel breakdown (the markers add their own gaps)
    evs = [(ctypes.c_void_p * (nk + 1))(*[hip.event() for _ in range(nk + 1)]) for _ in range(steps)]
    for i in range(steps):
        m.check(m.moe_forward_profiled(d, w, x, routes, saved, None, out16, ws, evs[i], stream),
                "moe_forward_profiled")
    torch.cuda.synchronize()
    per_kernel = {n: [] for n in names}
    for i in range(steps):
        for k, n in enumerate(names):
            per_kernel[n].append(hip.elapsed_ms(evs[i][k], evs[i][k + 1]))
    assert m.moe_last_device_error(ws) == m.MOE_OK
    touched = int((np.diff(routes.expert_offsets.cpu().numpy()) > 0).sum())
    return dict(wall=wall, up_ms=float(np.mean(up_ms)),
                per_kernel={n: float(np.mean(v)) for n, v in per_kernel.items()}, touched=touched)


def summarize(cfg, r, steps):
    ms = r["wall"] / steps * 1e3
    up_ms = r["up_ms"]
    up_bytes = ffn_up_bytes(cfg, r["touched"])
    dn_bytes = ffn_down_bytes(cfg, r["touched"])
    flop, byts = layer_work(cfg, r["touched"])
    t_roof = max(flop / (PEAK_BF16_TFLOPS * 1e12), byts / (PEAK_HBM_GBS * 1e9))
    return dict(
        tokens_per_s=cfg.tokens / (ms / 1e3),
        ms_per_step=ms,
        ffn_up_ms=up_ms,
        kernel_ms=r["per_kernel"],
        touched_experts=r["touched"],
        ffn_up_gbs=up_bytes / (up_ms / 1e3) / 1e9,
        ffn_down_gbs=dn_bytes / (r["per_kernel"]["ffn_down"] / 1e3) / 1e9,
        layer_roofline=dict(
            flop=flop, bytes=byts, t_roof_ms=t_roof * 1e3,
            bound="mfma" if flop / (PEAK_BF16_TFLOPS * 1e12) > byts / (PEAK_HBM_GBS * 1e9) else "hbm",
            frac=t_roof / (ms / 1e3),
            hbm_frac=byts / (ms / 1e3) / (PEAK_HBM_GBS * 1e9),
            mfma_frac=flop / (ms / 1e3) / (PEAK_BF16_TFLOPS * 1e12)),
    )


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


def run_backward(cfg, steps, warmup):
    """Forward (training mode) once, then `steps` timed backward passes of
    the same batch (HIP-event timed on the kernels' stream)."""
    import torch
    import mixture_experts_layer_counting_amd as m
    import workloads as W
    dev = torch.device("cuda:0")
    w = device_layer(W.make_layer(cfg))
    x = torch.from_numpy(W.tokens(cfg).view(np.int16)).to(dev)
    dout = torch.from_numpy(W.grad_out(cfg).view(np.int16)).to(dev)
    d = m.Dims(cfg.tokens, cfg.hidden, cfg.experts, cfg.top_k, cfg.inter, cfg.shared_inter)
    ws = m.alloc_workspace(d, m.MOE_OP_BACKWARD, dev)
    routes = m.alloc_routes(d, dev, logits=False)
    saved = m.alloc_saved(d, dev, training=True)
    out16 = torch.empty(d.tokens, d.hidden, dtype=torch.int16, device=dev)
    m.check(m.moe_forward(d, w, x, routes, saved, None, out16, ws), "moe_forward")
    grads = m.alloc_grads(d, dev)
    dx32 = torch.empty(d.tokens, d.hidden, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def bwd():
        m.check(m.moe_backward(d, w, x, routes, saved, dout, dx32, None, grads, ws, stream), "moe_backward")

    for _ in range(warmup):
        bwd()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(steps):
        bwd()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    touched = int((np.diff(routes.expert_offsets.cpu().numpy()) > 0).sum())
    H, I, Is, T, R, E = cfg.hidden, cfg.inter, cfg.shared_inter, cfg.tokens, cfg.routes, cfg.experts
    # algorithmic bytes: weights read, fp32 weight gradients written, per-route
    # and per-token activations read once (Y, gate/up, x, dOut), dx route rows
    # written and read once, dX written
    byts = (touched * 3 * I * H * 2 + 3 * Is * H * 2 + E * H * 4 + touched * 3 * I * H * 4 + 3 * Is * H * 4
            + E * H * 4 + R * H * 4 + R * 2 * I * 4 + T * 2 * Is * 4 + T * H * 4 + 2 * T * H * 2
            + R * H * 4 * 2 + T * H * 4)
    flop = 2 * 2 * (R * 3 * I * H + T * 3 * Is * H)
    t_roof = max(flop / (PEAK_BF16_TFLOPS * 1e12), byts / (PEAK_HBM_GBS * 1e9))
    return {"workload": f"{cfg.name}: {T} tokens backward", "ms": ms, "tokens_per_s": T / (ms / 1e3),
            "bytes": byts, "flop": flop, "t_roof_ms": t_roof * 1e3, "roofline_frac": t_roof / (ms / 1e3),
            "hbm_frac": byts / (ms / 1e3) / (PEAK_HBM_GBS * 1e9)}


def cpu_baseline(cfg, layer, budget_s=12.0):
    """The FP64 oracle as it stands, on the first tokens of the same workload,
    64 at a time until `budget_s` seconds have passed."""
    import oracle as O
    import workloads as W
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    x = W.tokens(cfg)
    done, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < budget_s and done < cfg.tokens:
        tok = np.arange(done, min(done + 64, cfg.tokens))
        O.forward(layer, x, cfg.top_k, tokens=tok)
        done += len(tok)
    el = time.perf_counter() - t0
    return {"value": done / el, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"oracle forward (numpy float64) on tokens 0..{done - 1} of the {cfg.name} workload, "
                      f"{el:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="moe1k")
    ap.add_argument("--secondary", default="moe8k", help="second workload to report, or 'none'")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--backward", default="bwd4k", help="workload of the backward timing, or 'none'")
    ap.add_argument("--ep-share", type=int, default=8,
                    help="also time the grouped FFN on one GPU's share of this many expert-parallel GPUs (0: off)")
    ap.add_argument("--mx", type=int, default=1,
                    help="also time the forward with block-scaled FP8 expert weights (0: off)")
    ap.add_argument("--lora", type=int, default=1,
                    help="also time the forward with LoRA adapters on the routed experts (0: off)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also launch one plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build runs the whole layer on a single MI355X "
              "with all experts resident and has no multi-GPU path", file=sys.stderr)
        sys.exit(2)

    import torch
    import mixture_experts_layer_counting_amd as m
    import workloads as W
    m.load_library()
    hip = Hip()
    cfg = W.CONFIGS[args.config]
    log(f"bench: generating {cfg.name} weights")
    layer = W.make_layer(cfg)
    w = device_layer(layer)
    torch.cuda.synchronize()

    if args.copy_probe_mib:
        n = args.copy_probe_mib * (1 << 20) // 4
        a = torch.empty(n, dtype=torch.float32, device="cuda:0").fill_(1.0)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    log(f"bench: {cfg.name} warmup {args.warmup}, steps {args.steps}")
    main_r = run_config(cfg, w, args.steps, args.warmup, hip)
    main_s = summarize(cfg, main_r, args.steps)
    log(f"bench: {cfg.name} {main_s['ms_per_step']:.3f} ms/step, kernels {main_s['kernel_ms']}")

    secondary = {}
    if args.secondary != "none":
        c2 = W.CONFIGS[args.secondary]
        same_weights = (c2.hidden, c2.inter, c2.shared_inter, c2.experts, c2.seed, c2.zipf_s) == \
                       (cfg.hidden, cfg.inter, cfg.shared_inter, cfg.experts, cfg.seed, cfg.zipf_s)
        w2 = w if same_weights else device_layer(W.make_layer(c2))
        log(f"bench: {c2.name} warmup {args.warmup}, steps {args.steps}")
        r2 = run_config(c2, w2, args.steps, args.warmup, hip)
        secondary[c2.name] = summarize(c2, r2, args.steps)
        log(f"bench: {c2.name} {secondary[c2.name]['ms_per_step']:.3f} ms/step")

    ep_share = None
    if args.ep_share > 1:
        log(f"bench: grouped FFN on one of {args.ep_share} expert shares")
        ep_share = run_ep_share(cfg, w, args.steps, args.warmup, args.ep_share)
        log(f"bench: expert share {ep_share['ms']:.3f} ms")

    mx = None
    if args.mx:
        log(f"bench: {cfg.name} with block-scaled FP8 expert weights")
        mx = run_mx(cfg, layer, args.steps, args.warmup)
        log(f"bench: {cfg.name} mx {mx['ms']:.3f} ms/step")

    lora = None
    if args.lora:
        log(f"bench: {cfg.name} with LoRA adapters")
        lora = run_lora(cfg, w, args.steps, args.warmup)
        log(f"bench: {cfg.name} lora {lora['ms']:.3f} ms/step (plain {lora['plain_forward_ms']:.3f})")

    backward = None
    if args.backward != "none":
        log(f"bench: backward {args.backward}")
        backward = run_backward(W.CONFIGS[args.backward], max(3, args.steps // 4), 1)
        log(f"bench: backward {backward['ms']:.3f} ms")

    cpu = None
    if not args.no_cpu_baseline:
        log("bench: cpu baseline (oracle)")
        cpu = cpu_baseline(cfg, layer)

    up_ms = main_s["ffn_up_ms"]
    up_bytes = ffn_up_bytes(cfg, main_r["touched"])
    achieved = up_bytes / (up_ms / 1e3) / 1e9
    traffic = traffic_from_profile()
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
        "config": {"workload": f"{cfg.name}: {cfg.tokens} tokens, hidden {cfg.hidden}, {cfg.experts} experts "
                               f"top-{cfg.top_k}, expert inter {cfg.inter}, shared inter {cfg.shared_inter}",
                   "tokens": cfg.tokens, "hidden": cfg.hidden, "experts": cfg.experts, "top_k": cfg.top_k,
                   "inter": cfg.inter, "shared_inter": cfg.shared_inter},
        "roofline": {"kernel": "ffn_up", "bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS, "traffic": traffic,
                     "algorithmic_bytes": up_bytes, "avg_ms": up_ms},
        "layer_roofline": main_s["layer_roofline"],
        "kernel_ms_marked": main_s["kernel_ms"],
        "ffn_down_gbs": main_s["ffn_down_gbs"],
        "cpu_baseline": cpu,
        "secondary": secondary,
        "ep_share": ep_share,
        "mx_weights": mx,
        "lora": lora,
        "backward": backward,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
