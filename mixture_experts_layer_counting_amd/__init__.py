"""Python binding of libmoe_mi355x.so, the gfx950 routed-MoE library.

Argument marshalling only: every step of the layer runs in the library's
HIP kernels.  torch supplies device memory (torch.empty) and the current
stream; nothing here computes any part of the layer, and there is no CPU
fallback -- importing works without a GPU, but every compute call needs the
built library and a gfx950 device.

The entry points mirror include/moe_mi355x.h one to one (EXPORTS lists
them) and return the library's status code.  `Layer` is a convenience holder that
allocates outputs and raises MoEError on a non-zero status.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_mi355x.so")

MOE_OK, MOE_E_NULL, MOE_E_SHAPE, MOE_E_UNSUPPORTED, MOE_E_ALIGN = 0, 1, 2, 3, 4
MOE_E_WORKSPACE, MOE_E_DEVICE, MOE_E_LAUNCH, MOE_E_ALIAS = 5, 6, 7, 8
(MOE_OP_ROUTE, MOE_OP_PERMUTE, MOE_OP_FFN, MOE_OP_FORWARD, MOE_OP_BACKWARD, MOE_OP_FORWARD_LORA,
 MOE_OP_BACKWARD_LORA) = range(7)
NOALLOC_SCRATCH_BYTES = 64 << 20  # MOE_NOALLOC_SCRATCH_BYTES
ABI_VERSION = 2


class MoEError(RuntimeError):
    pass


class MoeDims(ctypes.Structure):
    _fields_ = [("tokens", ctypes.c_int64), ("hidden", ctypes.c_int32), ("experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("inter", ctypes.c_int32), ("shared_inter", ctypes.c_int32)]


_VP = ctypes.c_void_p


class MoeWeights(ctypes.Structure):
    _fields_ = [(n, _VP) for n in ("w_router", "router_bias", "w13", "w2", "ws13", "ws2", "w_sgate",
                                   "w_router_planes")]


class MoeWeightsMx(ctypes.Structure):
    _fields_ = [(n, _VP) for n in ("w_router", "router_bias", "w13_q", "w13_s", "w2_q", "w2_s", "ws13_q",
                                   "ws13_s", "ws2_q", "ws2_s", "w_sgate", "w_router_planes")]


class MoeLora(ctypes.Structure):
    _fields_ = [("rank", ctypes.c_int32), ("scale", ctypes.c_float)] + \
        [(n, _VP) for n in ("a13", "b13", "a2", "b2")]


class MoeRoutes(ctypes.Structure):
    _fields_ = [(n, _VP) for n in ("topk_idx", "topk_gate", "logits", "expert_offsets", "sorted_route",
                                   "route_pos")]


class MoeSaved(ctypes.Structure):
    _fields_ = [(n, _VP) for n in ("y", "gu", "shared_y", "shared_gate", "shared_gu")]


class MoeGrads(ctypes.Structure):
    _fields_ = [(n, _VP) for n in ("d_w_router", "d_w13", "d_w2", "d_ws13", "d_ws2", "d_w_sgate")]


class MoeSideStreams(ctypes.Structure):
    _fields_ = [("side", _VP * 2), ("fork", _VP), ("join", _VP * 2)]


class MoeLoraGrads(ctypes.Structure):
    _fields_ = [(n, _VP) for n in ("d_a13", "d_b13", "d_a2", "d_b2")]


EXPORTS = ("moe_abi_version", "moe_status_str", "moe_workspace_bytes", "moe_route", "moe_permute",
           "moe_grouped_ffn", "moe_combine", "moe_forward", "moe_backward", "moe_last_device_error",
           "moe_forward_profiled", "moe_forward_kernel_count", "moe_forward_kernel_name", "moe_forward_mx",
           "moe_forward_lora", "moe_grouped_ffn_lora", "moe_forward_noalloc", "moe_backward_lora",
           "moe_split_router", "moe_probe_read", "moe_probe_copy", "moe_probe_mfma", "moe_backward_side",
           "moe_forward_side", "moe_backward_lora_side")

_lib = None


def load_library():
    """Load the built library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise MoEError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    lib.moe_abi_version.restype = ctypes.c_int
    lib.moe_abi_version.argtypes = []
    lib.moe_status_str.restype = ctypes.c_char_p
    lib.moe_status_str.argtypes = [ctypes.c_int]
    lib.moe_workspace_bytes.restype = ctypes.c_size_t
    lib.moe_workspace_bytes.argtypes = [P(MoeDims), ctypes.c_int]
    ws = [_VP, ctypes.c_size_t, _VP]
    lib.moe_route.restype = ctypes.c_int
    lib.moe_route.argtypes = [P(MoeDims), _VP, P(MoeWeights), P(MoeRoutes), *ws]
    lib.moe_permute.restype = ctypes.c_int
    lib.moe_permute.argtypes = [P(MoeDims), P(MoeRoutes), *ws]
    lib.moe_grouped_ffn.restype = ctypes.c_int
    lib.moe_grouped_ffn.argtypes = [P(MoeDims), _VP, P(MoeWeights), P(MoeRoutes), P(MoeSaved), *ws]
    lib.moe_combine.restype = ctypes.c_int
    lib.moe_combine.argtypes = [P(MoeDims), P(MoeRoutes), P(MoeSaved), _VP, _VP, _VP]
    lib.moe_forward.restype = ctypes.c_int
    lib.moe_forward.argtypes = [P(MoeDims), P(MoeWeights), _VP, P(MoeRoutes), P(MoeSaved), _VP, _VP, *ws]
    lib.moe_forward_mx.restype = ctypes.c_int
    lib.moe_forward_mx.argtypes = [P(MoeDims), P(MoeWeightsMx), _VP, P(MoeRoutes), P(MoeSaved), _VP, _VP,
                                   *ws]
    lib.moe_forward_lora.restype = ctypes.c_int
    lib.moe_forward_lora.argtypes = [P(MoeDims), P(MoeWeights), P(MoeLora), _VP, P(MoeRoutes), P(MoeSaved),
                                     _VP, _VP, *ws]
    lib.moe_grouped_ffn_lora.restype = ctypes.c_int
    lib.moe_grouped_ffn_lora.argtypes = [P(MoeDims), _VP, P(MoeWeights), P(MoeLora), P(MoeRoutes), P(MoeSaved),
                                         *ws]
    lib.moe_backward.restype = ctypes.c_int
    lib.moe_backward.argtypes = [P(MoeDims), P(MoeWeights), _VP, P(MoeRoutes), P(MoeSaved), _VP, _VP, _VP,
                                 P(MoeGrads), *ws]
    for name, args in (("moe_probe_read", [_VP, ctypes.c_size_t, _VP, _VP]),
                       ("moe_probe_copy", [_VP, _VP, ctypes.c_size_t, _VP]),
                       ("moe_probe_mfma", [_VP, ctypes.c_int, _VP])):
        getattr(lib, name).restype = ctypes.c_int
        getattr(lib, name).argtypes = args
    lib.moe_forward_side.restype = ctypes.c_int
    lib.moe_forward_side.argtypes = [P(MoeDims), P(MoeWeights), _VP, P(MoeRoutes), P(MoeSaved), _VP, _VP, *ws,
                                     P(MoeSideStreams)]
    lib.moe_backward_lora_side.restype = ctypes.c_int
    lib.moe_backward_lora_side.argtypes = [P(MoeDims), P(MoeWeights), P(MoeLora), _VP, P(MoeRoutes), P(MoeSaved),
                                           _VP, _VP, _VP, P(MoeGrads), P(MoeLoraGrads), *ws, P(MoeSideStreams)]
    lib.moe_backward_side.restype = ctypes.c_int
    lib.moe_backward_side.argtypes = [P(MoeDims), P(MoeWeights), _VP, P(MoeRoutes), P(MoeSaved), _VP, _VP, _VP,
                                      P(MoeGrads), *ws, P(MoeSideStreams)]
    lib.moe_split_router.restype = ctypes.c_int
    lib.moe_split_router.argtypes = [P(MoeDims), _VP, _VP, _VP]
    lib.moe_backward_lora.restype = ctypes.c_int
    lib.moe_backward_lora.argtypes = [P(MoeDims), P(MoeWeights), P(MoeLora), _VP, P(MoeRoutes), P(MoeSaved),
                                      _VP, _VP, _VP, P(MoeGrads), P(MoeLoraGrads), *ws]
    lib.moe_forward_profiled.restype = ctypes.c_int
    lib.moe_forward_profiled.argtypes = [P(MoeDims), P(MoeWeights), _VP, P(MoeRoutes), P(MoeSaved), _VP, _VP,
                                         _VP, ctypes.c_size_t, _VP, ctypes.c_int, _VP]
    lib.moe_forward_kernel_count.restype = ctypes.c_int
    lib.moe_forward_kernel_count.argtypes = [P(MoeDims)]
    lib.moe_forward_kernel_name.restype = ctypes.c_char_p
    lib.moe_forward_kernel_name.argtypes = [P(MoeDims), ctypes.c_int]
    lib.moe_last_device_error.restype = ctypes.c_int
    lib.moe_last_device_error.argtypes = [_VP, _VP]
    lib.moe_forward_noalloc.restype = ctypes.c_int
    lib.moe_forward_noalloc.argtypes = [P(MoeDims), P(MoeWeights), _VP, P(MoeRoutes), P(MoeSaved), _VP, _VP, _VP]
    if lib.moe_abi_version() != ABI_VERSION:
        raise MoEError(f"ABI version mismatch: library {lib.moe_abi_version()}, binding {ABI_VERSION}")
    _lib = lib
    return lib


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------
def _ptr(t):
    """Device address of a tensor (None -> NULL).  Plain ints pass through
    (used by host-only validation tests)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


@dataclasses.dataclass
class Dims:
    tokens: int
    hidden: int
    experts: int = 512
    top_k: int = 10
    inter: int = 512
    shared_inter: int = 512

    def c(self) -> MoeDims:
        return MoeDims(self.tokens, self.hidden, self.experts, self.top_k, self.inter, self.shared_inter)


@dataclasses.dataclass
class Weights:
    w_router: object
    w13: object
    w2: object
    router_bias: object = None
    ws13: object = None
    ws2: object = None
    w_sgate: object = None
    w_router_planes: object = None  # [3, E, H] bf16 from moe_split_router, or None

    def c(self) -> MoeWeights:
        return MoeWeights(*(_ptr(getattr(self, n)) for n, _ in MoeWeights._fields_))


@dataclasses.dataclass
class WeightsMx:
    """Block-scaled FP8 expert weights: E4M3 codes and E8M0 scale codes (one
    per 32 elements along each row) as uint8 tensors."""
    w_router: object
    w13_q: object
    w13_s: object
    w2_q: object
    w2_s: object
    router_bias: object = None
    ws13_q: object = None
    ws13_s: object = None
    ws2_q: object = None
    ws2_s: object = None
    w_sgate: object = None
    w_router_planes: object = None

    def c(self) -> MoeWeightsMx:
        return MoeWeightsMx(*(_ptr(getattr(self, n)) for n, _ in MoeWeightsMx._fields_))


@dataclasses.dataclass
class Lora:
    """LoRA adapters of the routed experts (bf16 tensors): a13 [E,rank,H],
    b13 [E,2I,rank], a2 [E,rank,I], b2 [E,H,rank]; the update's scale."""
    rank: int
    scale: float
    a13: object
    b13: object
    a2: object
    b2: object

    def c(self) -> MoeLora:
        return MoeLora(int(self.rank), float(self.scale), _ptr(self.a13), _ptr(self.b13), _ptr(self.a2),
                       _ptr(self.b2))


@dataclasses.dataclass
class Routes:
    topk_idx: object = None
    topk_gate: object = None
    logits: object = None
    expert_offsets: object = None
    sorted_route: object = None
    route_pos: object = None

    def c(self) -> MoeRoutes:
        return MoeRoutes(*(_ptr(getattr(self, n)) for n, _ in MoeRoutes._fields_))


@dataclasses.dataclass
class Saved:
    y: object = None
    gu: object = None
    shared_y: object = None
    shared_gate: object = None
    shared_gu: object = None

    def c(self) -> MoeSaved:
        return MoeSaved(*(_ptr(getattr(self, n)) for n, _ in MoeSaved._fields_))


@dataclasses.dataclass
class Grads:
    d_w_router: object = None
    d_w13: object = None
    d_w2: object = None
    d_ws13: object = None
    d_ws2: object = None
    d_w_sgate: object = None

    def c(self) -> MoeGrads:
        return MoeGrads(*(_ptr(getattr(self, n)) for n, _ in MoeGrads._fields_))


@dataclasses.dataclass
class LoraGrads:
    """Adapter gradients (fp32): d_a13 [E,rank,H], d_b13 [E,2I,rank],
    d_a2 [E,rank,I], d_b2 [E,H,rank]."""
    d_a13: object = None
    d_b13: object = None
    d_a2: object = None
    d_b2: object = None

    def c(self) -> MoeLoraGrads:
        return MoeLoraGrads(*(_ptr(getattr(self, n)) for n, _ in MoeLoraGrads._fields_))


def _ws(ws):
    if ws is None:
        return None, 0
    if isinstance(ws, tuple):
        return ws
    return ws.data_ptr(), ws.numel() * ws.element_size()


# ---------------------------------------------------------------------------
# entry points (same names as the C ABI; return the status code)
# ---------------------------------------------------------------------------
def moe_abi_version() -> int:
    return load_library().moe_abi_version()


def moe_status_str(status: int) -> str:
    return load_library().moe_status_str(status).decode()


def moe_workspace_bytes(dims: Dims, op: int) -> int:
    return load_library().moe_workspace_bytes(ctypes.byref(dims.c()), op)


def moe_route(dims, x, weights, routes, ws, stream=None) -> int:
    p, n = _ws(ws)
    return load_library().moe_route(ctypes.byref(dims.c()), _ptr(x), ctypes.byref(weights.c()),
                                    ctypes.byref(routes.c()), p, n, _stream(stream))


def moe_permute(dims, routes, ws, stream=None) -> int:
    p, n = _ws(ws)
    return load_library().moe_permute(ctypes.byref(dims.c()), ctypes.byref(routes.c()), p, n, _stream(stream))


def moe_grouped_ffn(dims, x, weights, routes, saved, ws, stream=None) -> int:
    p, n = _ws(ws)
    return load_library().moe_grouped_ffn(ctypes.byref(dims.c()), _ptr(x), ctypes.byref(weights.c()),
                                          ctypes.byref(routes.c()), ctypes.byref(saved.c()), p, n,
                                          _stream(stream))


def moe_combine(dims, routes, saved, out_f32=None, out_bf16=None, stream=None) -> int:
    return load_library().moe_combine(ctypes.byref(dims.c()), ctypes.byref(routes.c()), ctypes.byref(saved.c()),
                                      _ptr(out_f32), _ptr(out_bf16), _stream(stream))


def moe_forward(dims, weights, x, routes, saved, out_f32, out_bf16, ws, stream=None) -> int:
    p, n = _ws(ws)
    return load_library().moe_forward(ctypes.byref(dims.c()), ctypes.byref(weights.c()), _ptr(x),
                                      ctypes.byref(routes.c()), ctypes.byref(saved.c()), _ptr(out_f32),
                                      _ptr(out_bf16), p, n, _stream(stream))


def moe_forward_noalloc(dims, weights, x, routes, saved, out_f32, out_bf16, stream=None) -> int:
    return load_library().moe_forward_noalloc(ctypes.byref(dims.c()), ctypes.byref(weights.c()), _ptr(x),
                                              ctypes.byref(routes.c()), ctypes.byref(saved.c()), _ptr(out_f32),
                                              _ptr(out_bf16), _stream(stream))


def moe_forward_mx(dims, weights_mx, x, routes, saved, out_f32, out_bf16, ws, stream=None) -> int:
    p, n = _ws(ws)
    return load_library().moe_forward_mx(ctypes.byref(dims.c()), ctypes.byref(weights_mx.c()), _ptr(x),
                                         ctypes.byref(routes.c()), ctypes.byref(saved.c()), _ptr(out_f32),
                                         _ptr(out_bf16), p, n, _stream(stream))


def moe_forward_lora(dims, weights, lora, x, routes, saved, out_f32, out_bf16, ws, stream=None) -> int:
    p, n = _ws(ws)
    return load_library().moe_forward_lora(ctypes.byref(dims.c()), ctypes.byref(weights.c()),
                                           ctypes.byref(lora.c()), _ptr(x), ctypes.byref(routes.c()),
                                           ctypes.byref(saved.c()), _ptr(out_f32), _ptr(out_bf16), p, n,
                                           _stream(stream))


def moe_grouped_ffn_lora(dims, x, weights, lora, routes, saved, ws, stream=None) -> int:
    p, n = _ws(ws)
    return load_library().moe_grouped_ffn_lora(ctypes.byref(dims.c()), _ptr(x), ctypes.byref(weights.c()),
                                               ctypes.byref(lora.c()), ctypes.byref(routes.c()),
                                               ctypes.byref(saved.c()), p, n, _stream(stream))


def moe_backward(dims, weights, x, routes, saved, d_out, d_x_f32, d_x_bf16, grads, ws, stream=None) -> int:
    p, n = _ws(ws)
    return load_library().moe_backward(ctypes.byref(dims.c()), ctypes.byref(weights.c()), _ptr(x),
                                       ctypes.byref(routes.c()), ctypes.byref(saved.c()), _ptr(d_out),
                                       _ptr(d_x_f32), _ptr(d_x_bf16), ctypes.byref(grads.c()), p, n,
                                       _stream(stream))


class SideStreams:
    """Two side streams (torch, default priority) and three HIP events (no
    timing) owned by the caller, for moe_backward_side."""

    def __init__(self, device=None):
        import torch
        self.streams = [torch.cuda.Stream(device=device) for _ in range(2)]
        self._hip = ctypes.CDLL("libamdhip64.so")
        self._hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(_VP), ctypes.c_uint]
        self._hip.hipEventCreateWithFlags.restype = ctypes.c_int
        self._hip.hipEventDestroy.argtypes = [_VP]
        self.events = []
        for _ in range(3):
            e = _VP()
            if self._hip.hipEventCreateWithFlags(ctypes.byref(e), 0x2) != 0:  # hipEventDisableTiming
                raise MoEError("hipEventCreateWithFlags failed")
            self.events.append(e)

    def c(self) -> MoeSideStreams:
        s = [_VP(st.cuda_stream) for st in self.streams]
        return MoeSideStreams((_VP * 2)(s[0], s[1]), self.events[0], (_VP * 2)(self.events[1], self.events[2]))

    def __del__(self):
        for e in getattr(self, "events", []):
            self._hip.hipEventDestroy(e)


def moe_forward_side(dims, weights, x, routes, saved, out_f32, out_bf16, ws, side, stream=None) -> int:
    p, n = _ws(ws)
    sc = ctypes.byref(side.c()) if side is not None else None
    return load_library().moe_forward_side(ctypes.byref(dims.c()), ctypes.byref(weights.c()), _ptr(x),
                                           ctypes.byref(routes.c()), ctypes.byref(saved.c()), _ptr(out_f32),
                                           _ptr(out_bf16), p, n, _stream(stream), sc)


def moe_backward_lora_side(dims, weights, lora, x, routes, saved, d_out, d_x_f32, d_x_bf16, grads, lora_grads, ws,
                           side, stream=None) -> int:
    p, n = _ws(ws)
    lg = ctypes.byref(lora_grads.c()) if lora_grads is not None else None
    lc = ctypes.byref(lora.c()) if lora is not None else None
    sc = ctypes.byref(side.c()) if side is not None else None
    return load_library().moe_backward_lora_side(ctypes.byref(dims.c()), ctypes.byref(weights.c()), lc, _ptr(x),
                                                 ctypes.byref(routes.c()), ctypes.byref(saved.c()), _ptr(d_out),
                                                 _ptr(d_x_f32), _ptr(d_x_bf16), ctypes.byref(grads.c()), lg, p, n,
                                                 _stream(stream), sc)


def moe_backward_side(dims, weights, x, routes, saved, d_out, d_x_f32, d_x_bf16, grads, ws, side,
                      stream=None) -> int:
    p, n = _ws(ws)
    sc = ctypes.byref(side.c()) if side is not None else None
    return load_library().moe_backward_side(ctypes.byref(dims.c()), ctypes.byref(weights.c()), _ptr(x),
                                            ctypes.byref(routes.c()), ctypes.byref(saved.c()), _ptr(d_out),
                                            _ptr(d_x_f32), _ptr(d_x_bf16), ctypes.byref(grads.c()), p, n,
                                            _stream(stream), sc)


def moe_split_router(dims, w_router, planes, stream=None) -> int:
    return load_library().moe_split_router(ctypes.byref(dims.c()), _ptr(w_router), _ptr(planes), _stream(stream))


def moe_probe_read(buf, nbytes, sink, stream=None) -> int:
    """Measurement probe (include/moe_probes.h): stream `nbytes` of `buf`."""
    return load_library().moe_probe_read(_ptr(buf), nbytes, _ptr(sink), _stream(stream))


def moe_probe_copy(dst, src, nbytes, stream=None) -> int:
    return load_library().moe_probe_copy(_ptr(dst), _ptr(src), nbytes, _stream(stream))


def moe_probe_mfma(sink, iters, stream=None) -> int:
    return load_library().moe_probe_mfma(_ptr(sink), iters, _stream(stream))


def split_router(dims, w_router, device=None):
    """The router weight's three bf16 planes [3, E, H] (moe_split_router), to
    pass as Weights.w_router_planes."""
    import torch
    planes = torch.empty(3, dims.experts, dims.hidden, dtype=torch.int16,
                         device=device if device is not None else w_router.device)
    check(moe_split_router(dims, w_router, planes), "moe_split_router")
    return planes


def moe_backward_lora(dims, weights, lora, x, routes, saved, d_out, d_x_f32, d_x_bf16, grads, lora_grads, ws,
                      stream=None) -> int:
    p, n = _ws(ws)
    lg = ctypes.byref(lora_grads.c()) if lora_grads is not None else None
    lc = ctypes.byref(lora.c()) if lora is not None else None
    return load_library().moe_backward_lora(ctypes.byref(dims.c()), ctypes.byref(weights.c()), lc, _ptr(x),
                                            ctypes.byref(routes.c()), ctypes.byref(saved.c()), _ptr(d_out),
                                            _ptr(d_x_f32), _ptr(d_x_bf16), ctypes.byref(grads.c()), lg, p, n,
                                            _stream(stream))


def moe_forward_profiled(dims, weights, x, routes, saved, out_f32, out_bf16, ws, events, stream=None) -> int:
    """events: a ctypes array of hipEvent_t handles (see forward_kernel_names)."""
    p, n = _ws(ws)
    return load_library().moe_forward_profiled(ctypes.byref(dims.c()), ctypes.byref(weights.c()), _ptr(x),
                                               ctypes.byref(routes.c()), ctypes.byref(saved.c()), _ptr(out_f32),
                                               _ptr(out_bf16), p, n, events, len(events), _stream(stream))


def moe_forward_kernel_count(dims) -> int:
    return load_library().moe_forward_kernel_count(ctypes.byref(dims.c()))


def forward_kernel_names(dims):
    """Kernel names of moe_forward in launch order (from the library)."""
    lib = load_library()
    n = lib.moe_forward_kernel_count(ctypes.byref(dims.c()))
    return [lib.moe_forward_kernel_name(ctypes.byref(dims.c()), i).decode() for i in range(n)]


def moe_last_device_error(ws, stream=None) -> int:
    p, _ = _ws(ws)
    return load_library().moe_last_device_error(p, _stream(stream))


def check(status: int, what: str = "call"):
    if status != MOE_OK:
        raise MoEError(f"{what}: {moe_status_str(status)} (status {status})")


# ---------------------------------------------------------------------------
# allocation helpers (torch.empty only)
# ---------------------------------------------------------------------------
def alloc_routes(dims: Dims, device, logits: bool = True) -> Routes:
    import torch
    T, K, E = dims.tokens, dims.top_k, dims.experts
    e = lambda *s, dt=torch.int32: torch.empty(*s, dtype=dt, device=device)
    return Routes(topk_idx=e(T, K), topk_gate=e(T, K, dt=torch.float32),
                  logits=e(T, E, dt=torch.float32) if logits else None,
                  expert_offsets=e(E + 1), sorted_route=e(T * K), route_pos=e(T * K))


def alloc_saved(dims: Dims, device, training: bool = False) -> Saved:
    import torch
    T, K, H, I, Is = dims.tokens, dims.top_k, dims.hidden, dims.inter, dims.shared_inter
    f = lambda *s: torch.empty(*s, dtype=torch.float32, device=device)
    return Saved(y=f(T * K, H), gu=f(T * K, 2 * I) if training else None,
                 shared_y=f(T, H) if Is else None, shared_gate=f(T) if Is else None,
                 shared_gu=f(T, 2 * Is) if (Is and training) else None)


def alloc_grads(dims: Dims, device) -> Grads:
    import torch
    E, H, I, Is = dims.experts, dims.hidden, dims.inter, dims.shared_inter
    f = lambda *s: torch.empty(*s, dtype=torch.float32, device=device)
    return Grads(d_w_router=f(E, H), d_w13=f(E, 2 * I, H), d_w2=f(E, H, I),
                 d_ws13=f(2 * Is, H) if Is else None, d_ws2=f(H, Is) if Is else None,
                 d_w_sgate=f(H) if Is else None)


def alloc_lora_grads(dims: Dims, rank: int, device) -> LoraGrads:
    import torch
    E, H, I = dims.experts, dims.hidden, dims.inter
    f = lambda *s: torch.empty(*s, dtype=torch.float32, device=device)
    return LoraGrads(d_a13=f(E, rank, H), d_b13=f(E, 2 * I, rank), d_a2=f(E, rank, I), d_b2=f(E, H, rank))


def alloc_workspace(dims: Dims, op: int, device):
    import torch
    n = moe_workspace_bytes(dims, op)
    if n == 0:
        raise MoEError("invalid dims for workspace")
    return torch.empty(n, dtype=torch.uint8, device=device)


class Layer:
    """Device-resident weights of one layer plus convenience calls."""

    def __init__(self, dims: Dims, weights: Weights):
        self.dims = dims
        self.weights = weights

    def forward(self, x, training: bool = False, want_f32: bool = True, want_bf16: bool = True,
                ws=None, stream=None):
        import torch
        d = dataclasses.replace(self.dims, tokens=int(x.shape[0]))
        dev = x.device
        routes = alloc_routes(d, dev)
        saved = alloc_saved(d, dev, training)
        out32 = torch.empty(d.tokens, d.hidden, dtype=torch.float32, device=dev) if want_f32 else None
        out16 = torch.empty(d.tokens, d.hidden, dtype=torch.int16, device=dev) if want_bf16 else None
        if ws is None:
            ws = alloc_workspace(d, MOE_OP_BACKWARD if training else MOE_OP_FORWARD, dev)
        check(moe_forward(d, self.weights, x, routes, saved, out32, out16, ws, stream), "moe_forward")
        return routes, saved, out32, out16

    def backward(self, x, routes, saved, d_out, ws=None, want_bf16: bool = False, stream=None):
        """Gradients for upstream gradient d_out (bf16 bits); needs the
        routes and saved tensors of a training-mode forward."""
        import torch
        d = dataclasses.replace(self.dims, tokens=int(x.shape[0]))
        dev = x.device
        grads = alloc_grads(d, dev)
        dx32 = torch.empty(d.tokens, d.hidden, dtype=torch.float32, device=dev)
        dx16 = torch.empty(d.tokens, d.hidden, dtype=torch.int16, device=dev) if want_bf16 else None
        if ws is None:
            ws = alloc_workspace(d, MOE_OP_BACKWARD, dev)
        check(moe_backward(d, self.weights, x, routes, saved, d_out, dx32, dx16, grads, ws, stream),
              "moe_backward")
        return dx32, dx16, grads
