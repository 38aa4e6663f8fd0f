"""Host-side checks of the C ABI (no GPU needed, nothing is launched).

The library must load, export every entry point the headers in include/
declare (the layer's boundary and the measurement probes), size its workspace, and reject bad arguments with the documented
status before anything is enqueued (fail closed).  Validation runs before
the device check, so these calls return without touching a GPU; fake but
aligned addresses are fine because nothing dereferences them.
"""
import glob
import os
import re

import pytest

import mixture_experts_layer_counting_amd as m

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_mi355x.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(m.LIB_PATH):
        from mixture_experts_layer_counting_amd._build import build
        build()
    return m.load_library()


def declared_functions(headers=None):
    names = set()
    for h in headers or sorted(glob.glob(os.path.join(ROOT, "include", "*.h"))):
        names |= set(re.findall(r"^[a-z][\w ]*?\**\s*\**(moe_\w+)\(", open(h).read(), flags=re.M))
    return sorted(names)


def test_header_declares_the_boundary():
    names = declared_functions([HEADER])
    for n in ("moe_route", "moe_permute", "moe_grouped_ffn", "moe_combine", "moe_forward", "moe_backward",
              "moe_workspace_bytes", "moe_status_str", "moe_abi_version", "moe_last_device_error"):
        assert n in names, n


def test_library_exports_every_declared_symbol(lib):
    declared = declared_functions()
    assert "moe_probe_read" in declared and "moe_backward_lora" in declared
    for n in declared:
        assert hasattr(lib, n), f"{n} declared in a header but not exported"
    # the binding lists every declared entry point, and nothing else
    assert set(declared) == set(m.EXPORTS), set(declared) ^ set(m.EXPORTS)
    assert m.moe_abi_version() == m.ABI_VERSION


def test_status_strings(lib):
    for s in range(9):
        assert m.moe_status_str(s) and m.moe_status_str(s) != "unknown status"
    assert m.moe_status_str(99) == "unknown status"


def test_workspace_sizes(lib):
    d = m.Dims(1024, 2048)
    fwd = m.moe_workspace_bytes(d, m.MOE_OP_FORWARD)
    assert fwd > 0
    assert m.moe_workspace_bytes(d, m.MOE_OP_BACKWARD) >= fwd
    # grows with tokens; zero for invalid dims or op
    assert m.moe_workspace_bytes(m.Dims(8192, 2048), m.MOE_OP_FORWARD) > fwd
    assert m.moe_workspace_bytes(m.Dims(1024, 2000), m.MOE_OP_FORWARD) == 0
    assert m.moe_workspace_bytes(d, 17) == 0


# fake, 256-byte aligned, non-overlapping device addresses
class Fake:
    def __init__(self):
        self.next = 1 << 40

    def __call__(self, nbytes):
        a = self.next
        self.next += (nbytes + 4095) // 4096 * 4096 + 4096
        return a


def full_args(d: m.Dims):
    f = Fake()
    T, H, E, K, I, Is = d.tokens, d.hidden, d.experts, d.top_k, d.inter, d.shared_inter
    w = m.Weights(w_router=f(E * H * 4), w13=f(E * 2 * I * H * 2), w2=f(E * H * I * 2), router_bias=None,
                  ws13=f(2 * Is * H * 2), ws2=f(H * Is * 2), w_sgate=f(H * 2))
    r = m.Routes(topk_idx=f(T * K * 4), topk_gate=f(T * K * 4), logits=f(T * E * 4), expert_offsets=f((E + 1) * 4),
                 sorted_route=f(T * K * 4), route_pos=f(T * K * 4))
    s = m.Saved(y=f(T * K * H * 4), gu=None, shared_y=f(T * H * 4), shared_gate=f(T * 4), shared_gu=None)
    x = f(T * H * 2)
    o32, o16 = f(T * H * 4), f(T * H * 2)
    nws = m.moe_workspace_bytes(d, m.MOE_OP_FORWARD)
    ws = (f(nws), nws)
    return w, r, s, x, o32, o16, ws, f


def fwd(d, w, r, s, x, o32, o16, ws):
    return m.moe_forward(d, w, x, r, s, o32, o16, ws, stream=0)


def test_forward_validation_fails_closed(lib):
    d = m.Dims(64, 512, 512, 10, 128, 128)
    w, r, s, x, o32, o16, ws, f = full_args(d)
    assert fwd(m.Dims(64, 500, 512, 10, 128, 128), w, r, s, x, o32, o16, ws) == m.MOE_E_SHAPE
    assert fwd(m.Dims(64, 512, 500, 10, 128, 128), w, r, s, x, o32, o16, ws) == m.MOE_E_SHAPE
    assert fwd(m.Dims(64, 512, 512, 17, 128, 128), w, r, s, x, o32, o16, ws) == m.MOE_E_SHAPE
    assert fwd(m.Dims(64, 512, 512, 10, 96, 128), w, r, s, x, o32, o16, ws) == m.MOE_E_SHAPE
    assert fwd(m.Dims(-1, 512, 512, 10, 128, 128), w, r, s, x, o32, o16, ws) == m.MOE_E_SHAPE
    assert fwd(m.Dims(1 << 28, 512, 512, 10, 128, 128), w, r, s, x, o32, o16, ws) == m.MOE_E_SHAPE
    assert fwd(d, w, r, s, None, o32, o16, ws) == m.MOE_E_NULL
    assert fwd(d, w, r, s, x, None, None, ws) == m.MOE_E_NULL
    w2 = m.Weights(**{**w.__dict__, "w13": None})
    assert fwd(d, w2, r, s, x, o32, o16, ws) == m.MOE_E_NULL
    w3 = m.Weights(**{**w.__dict__, "w2": w.w2 + 2})
    assert fwd(d, w3, r, s, x, o32, o16, ws) == m.MOE_E_ALIGN
    # an output aliasing an input
    r2 = m.Routes(**{**r.__dict__, "topk_gate": x})
    assert fwd(d, w, r2, s, x, o32, o16, ws) == m.MOE_E_ALIAS
    s2 = m.Saved(**{**s.__dict__, "y": o32})
    assert fwd(d, w, r, s2, x, o32, o16, ws) == m.MOE_E_ALIAS
    # workspace missing / too small / misaligned
    assert fwd(d, w, r, s, x, o32, o16, (ws[0], ws[1] - 1)) == m.MOE_E_WORKSPACE
    assert fwd(d, w, r, s, x, o32, o16, None) == m.MOE_E_WORKSPACE
    assert fwd(d, w, r, s, x, o32, o16, (ws[0] + 16, ws[1])) == m.MOE_E_ALIGN
    # T == 0 is a no-op, whatever the pointers
    assert fwd(m.Dims(0, 512, 512, 10, 128, 128), w, r, s, None, None, None, None) == m.MOE_OK


def test_stage_validation_fails_closed(lib):
    d = m.Dims(64, 512, 512, 10, 128, 128)
    w, r, s, x, o32, o16, ws, f = full_args(d)
    assert m.moe_route(d, None, w, r, ws, stream=0) == m.MOE_E_NULL
    assert m.moe_permute(d, m.Routes(topk_idx=r.topk_idx), ws, stream=0) == m.MOE_E_NULL
    assert m.moe_grouped_ffn(d, x, w, r, m.Saved(), ws, stream=0) == m.MOE_E_NULL
    assert m.moe_combine(d, r, s, None, None, stream=0) == m.MOE_E_NULL
    assert m.moe_combine(d, r, m.Saved(**{**s.__dict__, "shared_y": None}), o32, None, stream=0) == m.MOE_E_NULL
    assert m.moe_combine(d, r, s, s.y, None, stream=0) == m.MOE_E_ALIAS
    assert m.moe_last_device_error(None, stream=0) == m.MOE_E_WORKSPACE


def test_valid_arguments_reach_the_device_check(lib):
    """With every argument valid the only remaining check is the gfx950
    device; without a GPU it fails there, so still nothing is launched."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present: valid fake pointers would be launched")
    d = m.Dims(64, 512, 512, 10, 128, 128)
    w, r, s, x, o32, o16, ws, f = full_args(d)
    assert fwd(d, w, r, s, x, o32, o16, ws) == m.MOE_E_DEVICE


def test_mx_forward_validation_fails_closed(lib):
    """moe_forward_mx checks dims, every code and scale buffer and the
    workspace on the host before anything is launched."""
    d = m.Dims(64, 512, 512, 10, 128, 128)
    w, r, s, x, o32, o16, ws, f = full_args(d)
    E, H, I, Is = d.experts, d.hidden, d.inter, d.shared_inter
    wm = m.WeightsMx(w_router=w.w_router, w13_q=f(E * 2 * I * H), w13_s=f(E * 2 * I * H // 32),
                     w2_q=f(E * H * I), w2_s=f(E * H * I // 32), ws13_q=f(2 * Is * H), ws13_s=f(2 * Is * H // 32),
                     ws2_q=f(H * Is), ws2_s=f(H * Is // 32), w_sgate=w.w_sgate)
    mx = lambda dd, ww, xx=x, wss=ws: m.moe_forward_mx(dd, ww, xx, r, s, o32, o16, wss, stream=0)
    assert mx(m.Dims(64, 500, 512, 10, 128, 128), wm) == m.MOE_E_SHAPE
    assert mx(d, wm, xx=None) == m.MOE_E_NULL
    assert mx(d, m.WeightsMx(**{**wm.__dict__, "w13_s": None})) == m.MOE_E_NULL
    assert mx(d, m.WeightsMx(**{**wm.__dict__, "w2_q": wm.w2_q + 4})) == m.MOE_E_ALIGN
    assert mx(d, m.WeightsMx(**{**wm.__dict__, "ws2_s": None})) == m.MOE_E_NULL
    assert mx(d, wm, wss=(ws[0], ws[1] - 1)) == m.MOE_E_WORKSPACE
    assert mx(m.Dims(0, 512, 512, 10, 128, 128), wm, xx=None, wss=None) == m.MOE_OK
    import torch
    if not torch.cuda.is_available():
        assert mx(d, wm) == m.MOE_E_DEVICE


def test_lora_forward_validation_fails_closed(lib):
    """moe_forward_lora checks the rank, every adapter matrix (presence,
    alignment, overlap with outputs) and its larger workspace on the host
    before anything is launched."""
    d = m.Dims(64, 512, 512, 10, 128, 128)
    w, r, s, x, o32, o16, ws, f = full_args(d)
    E, H, I, rk = d.experts, d.hidden, d.inter, 6
    lo = m.Lora(rank=rk, scale=0.5, a13=f(E * rk * H * 2), b13=f(E * 2 * I * rk * 2), a2=f(E * rk * I * 2),
                b2=f(E * H * rk * 2))
    nws = m.moe_workspace_bytes(d, m.MOE_OP_FORWARD_LORA)
    assert nws > m.moe_workspace_bytes(d, m.MOE_OP_FORWARD)
    wsl = (f(nws), nws)
    call = lambda ll, wss=wsl, dd=d, ss=s: m.moe_forward_lora(dd, w, ll, x, r, ss, o32, o16, wss, stream=0)
    assert call(m.Lora(**{**lo.__dict__, "rank": 0})) == m.MOE_E_SHAPE
    assert call(m.Lora(**{**lo.__dict__, "rank": 17})) == m.MOE_E_SHAPE
    assert call(m.Lora(**{**lo.__dict__, "b2": None})) == m.MOE_E_NULL
    assert call(m.Lora(**{**lo.__dict__, "a13": lo.a13 + 2})) == m.MOE_E_ALIGN
    # an adapter matrix that overlaps an output
    assert call(m.Lora(**{**lo.__dict__, "a2": s.y})) == m.MOE_E_ALIAS
    # a workspace sized for the plain forward is too small
    assert call(lo, wss=ws) == m.MOE_E_WORKSPACE
    # the grouped-FFN stage checks the same adapters and workspace
    ffn = lambda ll, wss=wsl: m.moe_grouped_ffn_lora(d, x, w, ll, r, s, wss, stream=0)
    assert ffn(m.Lora(**{**lo.__dict__, "rank": 0})) == m.MOE_E_SHAPE
    assert ffn(m.Lora(**{**lo.__dict__, "a13": None})) == m.MOE_E_NULL
    assert ffn(lo, wss=ws) == m.MOE_E_WORKSPACE
    assert call(lo, dd=m.Dims(0, 512, 512, 10, 128, 128)) == m.MOE_OK
    import torch
    if not torch.cuda.is_available():
        assert call(lo) == m.MOE_E_DEVICE


def backward_args(d: m.Dims):
    w, r, s, x, o32, o16, ws, f = full_args(d)
    T, H, E, K, I, Is = d.tokens, d.hidden, d.experts, d.top_k, d.inter, d.shared_inter
    s.gu = f(T * K * 2 * I * 4)
    s.shared_gu = f(T * 2 * Is * 4)
    g = m.Grads(d_w_router=f(E * H * 4), d_w13=f(E * 2 * I * H * 4), d_w2=f(E * H * I * 4),
                d_ws13=f(2 * Is * H * 4), d_ws2=f(H * Is * 4), d_w_sgate=f(H * 4))
    dout, dx32, dx16 = f(T * H * 2), f(T * H * 4), f(T * H * 2)
    nws = m.moe_workspace_bytes(d, m.MOE_OP_BACKWARD)
    return w, r, s, x, g, dout, dx32, dx16, (f(nws), nws), ws


def test_backward_validation_fails_closed(lib):
    """moe_backward checks dims, the saved forward tensors it needs (gate/up
    values, the shared gate), every gradient buffer (presence, alignment,
    overlap) and its own larger workspace on the host before anything is
    launched; the saved route rows are not read and may be NULL."""
    d = m.Dims(64, 512, 512, 10, 128, 128)
    w, r, s, x, g, dout, dx32, dx16, wsb, wsf = backward_args(d)
    bwd = lambda dd=d, ss=s, gg=g, dd32=dx32, ww=wsb, do=dout: m.moe_backward(dd, w, x, r, ss, do, dd32, dx16, gg,
                                                                            ww, stream=0)
    assert bwd(dd=m.Dims(64, 500, 512, 10, 128, 128)) == m.MOE_E_SHAPE
    assert bwd(dd=m.Dims(64, 512, 512, 10, 100, 128)) == m.MOE_E_SHAPE
    assert bwd(do=None) == m.MOE_E_NULL
    assert bwd(dd32=None) == m.MOE_E_NULL
    assert bwd(ss=m.Saved(**{**s.__dict__, "gu": None})) == m.MOE_E_NULL
    assert bwd(ss=m.Saved(**{**s.__dict__, "shared_gu": None})) == m.MOE_E_NULL
    assert bwd(ss=m.Saved(**{**s.__dict__, "shared_gate": None})) == m.MOE_E_NULL
    assert bwd(gg=m.Grads(**{**g.__dict__, "d_w13": None})) == m.MOE_E_NULL
    assert bwd(gg=m.Grads(**{**g.__dict__, "d_w_sgate": None})) == m.MOE_E_NULL
    assert bwd(gg=m.Grads(**{**g.__dict__, "d_w2": g.d_w2 + 8})) == m.MOE_E_ALIGN
    # a gradient aliasing an input, or another gradient
    assert bwd(gg=m.Grads(**{**g.__dict__, "d_w_router": x})) == m.MOE_E_ALIAS
    assert bwd(gg=m.Grads(**{**g.__dict__, "d_ws2": g.d_ws13})) == m.MOE_E_ALIAS
    assert bwd(dd32=s.gu) == m.MOE_E_ALIAS
    # the forward's workspace is too small for the backward
    assert bwd(ww=wsf) == m.MOE_E_WORKSPACE
    assert bwd(ww=None) == m.MOE_E_WORKSPACE
    # T == 0 is a no-op
    assert bwd(dd=m.Dims(0, 512, 512, 10, 128, 128)) == m.MOE_OK
    import torch
    if not torch.cuda.is_available():
        # the route rows are not needed: valid otherwise, it stops at the device check
        assert bwd(ss=m.Saved(**{**s.__dict__, "y": None, "shared_y": None})) == m.MOE_E_DEVICE
        assert bwd() == m.MOE_E_DEVICE


def test_lora_backward_validation_fails_closed(lib):
    """moe_backward_lora checks everything moe_backward checks, plus the
    rank, the adapters, the adapter-gradient buffers (presence, alignment,
    overlap) and its own larger workspace, before anything is launched."""
    d = m.Dims(64, 512, 512, 10, 128, 128)
    w, r, s, x, g, dout, dx32, dx16, wsb, wsf = backward_args(d)
    f = Fake()
    f.next = 1 << 44  # clear of the addresses backward_args handed out
    E, H, I, rk = d.experts, d.hidden, d.inter, 6
    lo = m.Lora(rank=rk, scale=0.5, a13=f(E * rk * H * 2), b13=f(E * 2 * I * rk * 2), a2=f(E * rk * I * 2),
                b2=f(E * H * rk * 2))
    lg = m.LoraGrads(d_a13=f(E * rk * H * 4), d_b13=f(E * 2 * I * rk * 4), d_a2=f(E * rk * I * 4),
                     d_b2=f(E * H * rk * 4))
    nws = m.moe_workspace_bytes(d, m.MOE_OP_BACKWARD_LORA)
    assert nws > m.moe_workspace_bytes(d, m.MOE_OP_BACKWARD)
    wsl = (f(nws), nws)

    def call(ll=lo, lgg=lg, wss=wsl, dd=d, gg=g, ss=s):
        return m.moe_backward_lora(dd, w, ll, x, r, ss, dout, dx32, dx16, gg, lgg, wss, stream=0)

    assert call(dd=m.Dims(64, 500, 512, 10, 128, 128)) == m.MOE_E_SHAPE
    assert call(ll=None) == m.MOE_E_NULL
    assert call(lgg=None) == m.MOE_E_NULL
    assert call(ll=m.Lora(**{**lo.__dict__, "rank": 0})) == m.MOE_E_SHAPE
    assert call(ll=m.Lora(**{**lo.__dict__, "rank": 17})) == m.MOE_E_SHAPE
    assert call(ll=m.Lora(**{**lo.__dict__, "b13": None})) == m.MOE_E_NULL
    assert call(lgg=m.LoraGrads(**{**lg.__dict__, "d_b2": None})) == m.MOE_E_NULL
    assert call(lgg=m.LoraGrads(**{**lg.__dict__, "d_a2": lg.d_a2 + 4})) == m.MOE_E_ALIGN
    # an adapter gradient overlapping an adapter, a base gradient or another adapter gradient
    assert call(lgg=m.LoraGrads(**{**lg.__dict__, "d_a13": lo.a13})) == m.MOE_E_ALIAS
    assert call(lgg=m.LoraGrads(**{**lg.__dict__, "d_b13": g.d_w13})) == m.MOE_E_ALIAS
    assert call(lgg=m.LoraGrads(**{**lg.__dict__, "d_b2": lg.d_a2})) == m.MOE_E_ALIAS
    # the plain backward's workspace is too small
    assert call(wss=wsb) == m.MOE_E_WORKSPACE
    assert call(ss=m.Saved(**{**s.__dict__, "gu": None})) == m.MOE_E_NULL
    assert call(dd=m.Dims(0, 512, 512, 10, 128, 128)) == m.MOE_OK
    import torch
    if not torch.cuda.is_available():
        assert call() == m.MOE_E_DEVICE


def test_split_router_and_caller_planes_validation(lib):
    """moe_split_router checks dims, both buffers (presence, alignment,
    overlap) and the device; a forward given pre-split router planes checks
    them like any other input (alignment, overlap with an output)."""
    d = m.Dims(64, 512, 512, 10, 128, 128)
    w, r, s, x, o32, o16, ws, f = full_args(d)
    E, H = d.experts, d.hidden
    planes = f(3 * E * H * 2)
    split = lambda dd=d, wr=w.w_router, pl=planes: m.moe_split_router(dd, wr, pl, stream=0)
    assert split(dd=m.Dims(64, 500, 512, 10, 128, 128)) == m.MOE_E_SHAPE
    assert split(wr=None) == m.MOE_E_NULL
    assert split(pl=None) == m.MOE_E_NULL
    assert split(pl=planes + 8) == m.MOE_E_ALIGN
    assert split(pl=w.w_router + 4096) == m.MOE_E_ALIAS
    wp = m.Weights(**{**w.__dict__, "w_router_planes": planes})
    assert fwd(d, m.Weights(**{**wp.__dict__, "w_router_planes": planes + 2}), r, s, x, o32, o16, ws) == m.MOE_E_ALIGN
    assert fwd(d, m.Weights(**{**wp.__dict__, "w_router_planes": o32}), r, s, x, o32, o16, ws) == m.MOE_E_ALIAS
    import torch
    if not torch.cuda.is_available():
        assert split() == m.MOE_E_DEVICE
        assert fwd(d, wp, r, s, x, o32, o16, ws) == m.MOE_E_DEVICE


def test_noalloc_forward_refuses_what_its_array_cannot_hold(lib):
    """moe_forward_noalloc needs no workspace argument; dims whose forward
    workspace exceeds its array are refused on the host, invalid dims too."""
    big = m.Dims(4096, 2048, 512, 10, 512, 512)
    assert m.moe_workspace_bytes(big, m.MOE_OP_FORWARD) > m.NOALLOC_SCRATCH_BYTES
    d = m.Dims(64, 512, 512, 10, 128, 128)
    w, r, s, x, o32, o16, ws, f = full_args(d)
    assert m.moe_forward_noalloc(big, w, x, r, s, o32, o16, stream=0) == m.MOE_E_WORKSPACE
    assert m.moe_forward_noalloc(m.Dims(64, 500, 512, 10, 128, 128), w, x, r, s, o32, o16, stream=0) == m.MOE_E_SHAPE
    assert m.moe_forward_noalloc(m.Dims(0, 512, 512, 10, 128, 128), w, None, r, s, None, None, stream=0) == m.MOE_OK
    import torch
    if not torch.cuda.is_available():
        # dims it can hold: the device's array is looked up first, so without a GPU it stops there
        assert m.moe_forward_noalloc(d, w, None, r, s, o32, o16, stream=0) == m.MOE_E_DEVICE


def test_probe_validation(lib):
    """The measurement probes check their arguments before launching."""
    f = Fake()
    buf, sink = f(1 << 20), f(256)
    assert m.moe_probe_read(None, 1 << 20, sink, stream=0) == m.MOE_E_NULL
    assert m.moe_probe_read(buf, 0, sink, stream=0) == m.MOE_E_SHAPE
    assert m.moe_probe_read(buf, 1000, sink, stream=0) == m.MOE_E_SHAPE
    assert m.moe_probe_read(buf + 8, 1 << 20, sink, stream=0) == m.MOE_E_ALIGN
    assert m.moe_probe_copy(buf + 4096, buf, 1 << 16, stream=0) == m.MOE_E_ALIAS
    assert m.moe_probe_mfma(sink, 0, stream=0) == m.MOE_E_SHAPE
    assert m.moe_probe_mfma(None, 10, stream=0) == m.MOE_E_NULL
    import torch
    if not torch.cuda.is_available():
        assert m.moe_probe_read(buf, 1 << 20, sink, stream=0) == m.MOE_E_DEVICE
        assert m.moe_probe_mfma(sink, 10, stream=0) == m.MOE_E_DEVICE


def test_backward_side_validation(lib):
    """moe_backward_side checks everything moe_backward checks, plus its side
    streams and events (present, distinct from each other and from the
    call's stream), before anything is enqueued."""
    d = m.Dims(64, 512, 512, 10, 128, 128)
    w, r, s, x, g, dout, dx32, dx16, wsb, wsf = backward_args(d)

    class Side:
        def __init__(self, side=(0x1000, 0x2000), fork=0x3000, join=(0x4000, 0x5000)):
            self.v = (side, fork, join)

        def c(self):
            (a, b), f, (j0, j1) = self.v
            return m.MoeSideStreams((m._VP * 2)(a, b), f, (m._VP * 2)(j0, j1))

    call = lambda side, stream=0x9000, dd=d: m.moe_backward_side(dd, w, x, r, s, dout, dx32, dx16, g, wsb, side,
                                                                 stream=stream)
    assert call(None) == m.MOE_E_NULL
    assert call(Side(side=(0x1000, 0))) == m.MOE_E_NULL
    assert call(Side(join=(0x4000, 0))) == m.MOE_E_NULL
    assert call(Side(side=(0x1000, 0x1000))) == m.MOE_E_ALIAS
    assert call(Side(), stream=0x2000) == m.MOE_E_ALIAS
    assert call(Side(fork=0x4000)) == m.MOE_E_ALIAS
    assert call(Side(), dd=m.Dims(64, 500, 512, 10, 128, 128)) == m.MOE_E_SHAPE
    assert call(Side(), dd=m.Dims(0, 512, 512, 10, 128, 128)) == m.MOE_OK
    assert m.moe_backward_side(d, w, x, r, s, dout, dx32, dx16, g, wsf, Side(), stream=0x9000) == m.MOE_E_WORKSPACE
    import torch
    if not torch.cuda.is_available():
        assert call(Side()) == m.MOE_E_DEVICE


def test_forward_side_validation(lib):
    """moe_forward_side checks moe_forward's arguments and the side streams
    and events before anything is enqueued."""
    d = m.Dims(64, 512, 512, 10, 128, 128)
    w, r, s, x, o32, o16, ws, f = full_args(d)
    mk = lambda side=(0x1000, 0x2000), fork=0x3000, join=(0x4000, 0x5000): type(
        "S", (), {"c": lambda self: m.MoeSideStreams((m._VP * 2)(*side), fork, (m._VP * 2)(*join))})()
    call = lambda side, stream=0x9000, dd=d: m.moe_forward_side(dd, w, x, r, s, o32, o16, ws, side, stream=stream)
    assert call(None) == m.MOE_E_NULL
    assert call(mk(side=(0, 0x2000))) == m.MOE_E_NULL
    assert call(mk(side=(0x1000, 0x1000))) == m.MOE_E_ALIAS
    assert call(mk(), stream=0x1000) == m.MOE_E_ALIAS
    assert call(mk(join=(0x4000, 0x4000))) == m.MOE_E_ALIAS
    assert call(mk(), dd=m.Dims(64, 500, 512, 10, 128, 128)) == m.MOE_E_SHAPE
    assert call(mk(), dd=m.Dims(0, 512, 512, 10, 128, 128)) == m.MOE_OK
    assert m.moe_forward_side(d, w, x, r, s, None, None, ws, mk(), stream=0x9000) == m.MOE_E_NULL
    import torch
    if not torch.cuda.is_available():
        assert call(mk()) == m.MOE_E_DEVICE
