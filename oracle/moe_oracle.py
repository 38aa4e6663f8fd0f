"""Plain FP64 CPU oracle of the routed MoE layer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py use it.  It shares no code with the HIP
library (no kernels, headers, helpers, tables or pre/post-processing); the
only thing both sides consume is the seeded input generator in workloads/.

What it computes is the plain definition of the layer described on the
RL-Kernel pull request 557 page (Qwen3-Next EP4 logprob parity), in the
commit message of its stack entry "MoE route/combine contract with a
batch-invariant grouped expert GEMM" (bullets Routing, Experts, Combine,
Backward), with the model shape of the SkyRL pull request 2513 page
("What": 512 routed experts, top-10, one shared expert).  Every value is
carried in float64; bf16 and fp32 inputs convert to float64 exactly, so the
only rounding is float64's own.  There are no mirrored rounding points:
the GPU path's fp32/bf16 rounding is checked against these exact values
with a tolerance.

Readings taken where the pages leave a step open (each is listed in the
design notes):
  * expert activation is SwiGLU: act = silu(gate) * up, gate = first I rows
    of W13 (the contract names only gate_up and down projections);
  * the shared expert is a SwiGLU FFN scaled by sigmoid(w_sg . x) and
    added after the ten routed terms (the pages name a shared expert and a
    shared-expert gate, not their formula);
  * route selection is decided on the fp32 value of each logit (the pages'
    router precision), stable descending, ties to the lower expert id; the
    gates themselves are computed from the exact logits;
  * inside an expert's segment routes keep ascending route id
    (r = token * top_k + slot);
  * LoRA adapters (ROLL pull request 502 page: grouped expert LoRA of rank
    r // top_k, deterministic shrink) attach to the routed experts' two
    projections only, with the textbook update scale * B (A v); the scale
    is an input (the pages do not say whether alpha is divided by r or by
    the expert rank).

Parity pins: every public function here is pinned by tests/test_oracle_pins.py
against brute force, closed forms, special cases, finite differences or an
independent autograd; none is "parity unpinned" except the pages' own
max-abs figure on their real checkpoint, which cannot be reproduced without
that checkpoint.
"""
from __future__ import annotations

import numpy as np

F64 = np.float64


# --------------------------------------------------------------------------
# input decoding (exact)
# --------------------------------------------------------------------------
def bf16_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly.

    Floating-point arrays pass through as float64 unchanged, so the same
    functions serve the finite-difference pins, which perturb weights
    continuously."""
    a = np.asarray(bits)
    if a.dtype != np.uint16:
        return a.astype(F64)
    u = a.astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(F64)


def f64_to_bf16_bits(a) -> np.ndarray:
    """Round float64 to the nearest bf16 (ties to even) via the exact fp32
    value nearest to it, then bf16.  Used only to report the distance of a
    bf16 output from the exact one."""
    f = np.asarray(a, F64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def e4m3_to_f64(codes) -> np.ndarray:
    """OCP FP8 E4M3 element codes -> float64, exactly (OCP Microscaling
    Formats v1.0, element type E4M3: 1 sign bit, 4 exponent bits with bias 7,
    3 mantissa bits; exponent field 0 is subnormal, m x 2^-9; the codes with
    all exponent and mantissa bits set are NaN; no infinities)."""
    c = np.asarray(codes, np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(F64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.ldexp(1.0, e - 7))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


def e8m0_to_f64(codes) -> np.ndarray:
    """OCP E8M0 scale codes -> 2^(code - 127); code 255 is NaN."""
    c = np.asarray(codes, np.uint8).astype(np.int64)
    return np.where(c == 255, np.nan, np.ldexp(1.0, c - 127))


def mx_to_f64(codes, scale_codes, block: int = 32) -> np.ndarray:
    """Block-scaled FP8 weights -> float64: element i of a row times the scale
    of its block of `block` consecutive elements along the last axis."""
    v = e4m3_to_f64(codes)
    sc = e8m0_to_f64(scale_codes)
    return v * np.repeat(sc, block, axis=-1)


def silu(z):
    return z / (1.0 + np.exp(-z))


def sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


# --------------------------------------------------------------------------
# forward
# --------------------------------------------------------------------------
def router_logits(x_bits, w_router, bias=None) -> np.ndarray:
    """Router projection l[t,e] = sum_h x[t,h] W_r[e,h] (+ b[e]), exact.

    Contract "Routing" bullet: an FP32 router (the weights stay fp32)."""
    l = bf16_to_f64(x_bits) @ np.asarray(w_router).astype(F64).T
    if bias is not None:
        l = l + np.asarray(bias).astype(F64)[None, :]
    return l


def select_routes(logits, top_k: int) -> np.ndarray:
    """Top-k expert ids per token, slot 0 the largest.

    Contract "Routing" bullet: stable descending order, ties to the lower
    expert id.  The comparison is taken on the fp32 value of each logit,
    the router's own precision.  numpy's stable argsort of the negated
    fp32 keys keeps equal keys in ascending expert id."""
    key = np.asarray(logits, F64).astype(np.float32)
    order = np.argsort(-key, axis=1, kind="stable")
    return order[:, :top_k].astype(np.int32)


def route_gates(logits, idx) -> np.ndarray:
    """Renormalised gates g[t,k] = softmax over the selected logits.

    Contract "Routing" bullet: softmax over all experts, then FP32
    renormalisation of the selected ten; the full softmax restricted to the
    selected set and renormalised equals the softmax of the selected
    logits, which is what is computed here (shifted by the slot-0 logit)."""
    sel = np.take_along_axis(np.asarray(logits, F64), idx.astype(np.int64), axis=1)
    w = np.exp(sel - sel[:, :1])
    return w / w.sum(axis=1, keepdims=True)


def permute_routes(idx, experts: int):
    """Counting sort of route ids r = t*K + k by expert, stable in r.

    Returns (expert_offsets [E+1] int64, sorted_route [R] int64,
    route_pos [R] int64 with route_pos[sorted_route[p]] = p).  The pages call
    this dispatch step a local selection of each expert's routes (section
    "What" of the EP4 description)."""
    flat = np.asarray(idx).reshape(-1).astype(np.int64)
    counts = np.bincount(flat, minlength=experts)
    offsets = np.zeros(experts + 1, np.int64)
    offsets[1:] = np.cumsum(counts)
    sorted_route = np.argsort(flat, kind="stable").astype(np.int64)
    route_pos = np.empty_like(sorted_route)
    route_pos[sorted_route] = np.arange(flat.size, dtype=np.int64)
    return offsets, sorted_route, route_pos


def expert_lora_rank(r: int, top_k: int) -> int:
    """Rank of each routed expert's adapter for a LoRA of rank r (ROLL pull
    request 502 page, "What this changes", grouped expert LoRA rank bullet:
    the adapter rank is divided by the router's top-k, integer division)."""
    return r // top_k


def lora_delta(rows, a_bits, b_bits, scale: float):
    """LoRA update of one linear map y = rows W^T on a block of rows:
    scale * (rows A^T) B^T with A [rank, in] (the shrink) and B [out, rank]
    (the expand), both bf16 bits (Hu et al., LoRA, section 4.1: h = W0 x +
    B A x, scaled by alpha / r; the scale is the caller's)."""
    a = bf16_to_f64(a_bits)
    b = bf16_to_f64(b_bits)
    return scale * ((rows @ a.T) @ b.T)


def swiglu_expert(xrows, w13_bits, w2_bits, lora=None):
    """One SwiGLU expert on a block of rows (float64).

    gu = x W13^T (first I columns gate, last I up), act = silu(gate)*up,
    y = act W2^T.  `lora` = (a13, b13, a2, b2, scale) adds a LoRA update to
    both projections: gu += scale (x A13^T) B13^T, y += scale (act A2^T)
    B2^T.  Returns (y, gu)."""
    w13 = bf16_to_f64(w13_bits)
    w2 = bf16_to_f64(w2_bits)
    inter = w13.shape[0] // 2
    gu = xrows @ w13.T
    if lora is not None:
        gu = gu + lora_delta(xrows, lora[0], lora[1], lora[4])
    act = silu(gu[:, :inter]) * gu[:, inter:]
    y = act @ w2.T
    if lora is not None:
        y = y + lora_delta(act, lora[2], lora[3], lora[4])
    return y, gu


def routed_rows(x_bits, idx, w13_bits, w2_bits, tokens=None, lora=None):
    """Per-route expert outputs Y (route-major) and their gate/up values.

    Contract "Experts" bullet: each (token, route) row gets its own expert
    output, with no gate multiply and no sum inside the expert step.
    `tokens` restricts the work to a subset of tokens (rows are returned in
    the order of that subset, K per token).  `lora` (dict: a13 [E,r,H],
    b13 [E,2I,r], a2 [E,r,I], b2 [E,H,r] bf16 bits, scale) gives every
    routed expert its own adapter."""
    T, K = idx.shape
    tok = np.arange(T) if tokens is None else np.asarray(tokens)
    x64 = bf16_to_f64(x_bits)
    H = x64.shape[1]
    sub = idx[tok]                             # [n, K]
    flat = sub.reshape(-1)
    n2I = w13_bits.shape[1]
    y = np.zeros((flat.size, H), F64)
    gu = np.zeros((flat.size, n2I), F64)
    for e in np.unique(flat):
        rows = np.nonzero(flat == e)[0]
        ad = None if lora is None else (lora["a13"][e], lora["b13"][e], lora["a2"][e],
                                        lora["b2"][e], float(lora["scale"]))
        ye, gue = swiglu_expert(x64[tok[rows // K]], w13_bits[e], w2_bits[e], ad)
        y[rows] = ye
        gu[rows] = gue
    return y, gu


def shared_expert(x_bits, ws13_bits, ws2_bits, w_sgate_bits, tokens=None):
    """Shared expert S[t] = SwiGLU_s(x[t]) and its gate sg[t] = sigmoid(w_sg . x[t])."""
    x64 = bf16_to_f64(x_bits)
    if tokens is not None:
        x64 = x64[np.asarray(tokens)]
    s, sgu = swiglu_expert(x64, ws13_bits, ws2_bits)
    sg = sigmoid(x64 @ bf16_to_f64(w_sgate_bits))
    return s, sg, sgu


def combine(y, gates, s=None, sg=None) -> np.ndarray:
    """out[t] = sum_k g[t,k] Y[t,k] (+ sg[t] S[t]).

    Contract "Combine" bullet: the ten route terms summed in route order,
    with one cast to bf16 at the end (exact arithmetic here, so the order is
    immaterial)."""
    T, K = gates.shape
    out = np.einsum("tk,tkh->th", gates, y.reshape(T, K, -1))
    if s is not None:
        out = out + sg[:, None] * s
    return out


def forward(layer: dict, x_bits, top_k: int = 10, tokens=None, forced_idx=None,
            lora=None) -> dict:
    """Whole forward pass in float64.

    layer: w_router [E,H] f32, router_bias [E] f32|None, w13 [E,2I,H] bf16,
    w2 [E,H,I] bf16, ws13/ws2/w_sgate bf16 or None.  `tokens` restricts the
    token-wise outputs to a subset; the permutation is returned only for the
    full batch.  `forced_idx` (full [T,K]) replaces the selection, as when
    routes are replayed.  `lora` adds per-expert LoRA adapters to the routed
    experts (see routed_rows); the router and the shared expert have none."""
    T = x_bits.shape[0]
    E = layer["w_router"].shape[0]
    tok = np.arange(T) if tokens is None else np.asarray(tokens)
    logits = router_logits(x_bits[tok], layer["w_router"], layer.get("router_bias"))
    if forced_idx is not None:
        idx_sub = np.asarray(forced_idx, np.int32)[tok]
    else:
        idx_sub = select_routes(logits, top_k)
    g = route_gates(logits, idx_sub)
    y, gu = routed_rows(x_bits[tok], idx_sub, layer["w13"], layer["w2"], lora=lora)
    res = {"tokens": tok, "logits": logits, "idx": idx_sub, "gates": g, "y": y, "gu": gu}
    if layer.get("ws13") is not None:
        s, sg, sgu = shared_expert(x_bits[tok], layer["ws13"], layer["ws2"], layer["w_sgate"])
        res.update(s=s, sg=sg, sgu=sgu)
        res["out"] = combine(y, g, s, sg)
    else:
        res["out"] = combine(y, g)
    if tokens is None:
        off, srt, pos = permute_routes(idx_sub, E)
        res.update(expert_offsets=off, sorted_route=srt, route_pos=pos)
    return res


# --------------------------------------------------------------------------
# backward
# --------------------------------------------------------------------------
def _swiglu_backward(dy, gu, x_rows, w13_bits, w2_bits):
    """Backward of one SwiGLU expert for a block of rows.

    dact = dy W2; dgate = dact*up*s*(1+gate*(1-s)) with s = sigmoid(gate);
    dup = dact*silu(gate); dx = [dgate, dup] W13; dW2 = dy^T act;
    dW13 = [dgate, dup]^T x."""
    w13 = bf16_to_f64(w13_bits)
    w2 = bf16_to_f64(w2_bits)
    inter = w13.shape[0] // 2
    gate, up = gu[:, :inter], gu[:, inter:]
    s = sigmoid(gate)
    act = gate * s * up
    dact = dy @ w2
    dgate = dact * up * s * (1.0 + gate * (1.0 - s))
    dup = dact * gate * s
    dgu = np.concatenate([dgate, dup], axis=1)
    return dgu @ w13, dy.T @ act, dgu.T @ x_rows, dgu


def _swiglu_backward_lora(dy, gu, x_rows, w13_bits, w2_bits, ad):
    """Backward of one SwiGLU expert whose projections carry the LoRA
    update of swiglu_expert (ad = (a13, b13, a2, b2, scale)).

    With z13 = x A13^T and z2 = act A2^T the forward is gu = x W13^T + s
    z13 B13^T and y = act W2^T + s z2 B2^T, so by the chain rule (every
    product a plain matrix product):
      v    = dy B2                      (route x rank)
      dact = dy W2 + s v A2
      dgu  = SwiGLU backward of dact, as in _swiglu_backward
      u    = dgu B13                    (route x rank)
      dx   = dgu W13 + s u A13
      dW2  = dy^T act,  dW13 = dgu^T x
      dA13 = s u^T x,   dB13 = s dgu^T z13
      dA2  = s v^T act, dB2  = s dy^T z2.
    Returns (dx, dW2, dW13, dA13, dB13, dA2, dB2)."""
    w13 = bf16_to_f64(w13_bits)
    w2 = bf16_to_f64(w2_bits)
    a13, b13, a2, b2 = (bf16_to_f64(m) for m in ad[:4])
    scale = float(ad[4])
    inter = w13.shape[0] // 2
    gate, up = gu[:, :inter], gu[:, inter:]
    s = sigmoid(gate)
    act = gate * s * up
    z13 = x_rows @ a13.T
    z2 = act @ a2.T
    v = dy @ b2
    dact = dy @ w2 + scale * (v @ a2)
    dgate = dact * up * s * (1.0 + gate * (1.0 - s))
    dup = dact * gate * s
    dgu = np.concatenate([dgate, dup], axis=1)
    u = dgu @ b13
    dx = dgu @ w13 + scale * (u @ a13)
    return (dx, dy.T @ act, dgu.T @ x_rows, scale * (u.T @ x_rows), scale * (dgu.T @ z13),
            scale * (v.T @ act), scale * (dy.T @ z2))


def backward(layer: dict, x_bits, fwd: dict, d_out_bits, lora=None) -> dict:
    """Gradients of every input of the layer for upstream gradient dOut.

    Contract "Backward" bullet: per-expert weight gradients into one dense
    buffer, per-route input gradients summed per token (the sum order is
    immaterial in exact arithmetic; the GPU's order is its own contract).
    The route-weight gradient dg = <dOut, Y> and its softmax backward
    through the renormalised gates follow from the combine definition.
    Needs the full batch (fwd from forward(..., tokens=None)).  `lora`
    (the dict of forward(); fwd must come from the same adapters) adds the
    routed experts' adapter terms and returns their gradients d_a13, d_b13,
    d_a2, d_b2 too."""
    x64 = bf16_to_f64(x_bits)
    dO = bf16_to_f64(d_out_bits)
    idx, g = fwd["idx"], fwd["gates"]
    T, K = idx.shape
    E, H = layer["w_router"].shape
    y = fwd["y"].reshape(T, K, H)
    # route-weight gradient and softmax backward over the selected logits
    dg = np.einsum("th,tkh->tk", dO, y)
    dl_sel = g * (dg - (g * dg).sum(axis=1, keepdims=True))
    dl = np.zeros((T, E), F64)
    np.put_along_axis(dl, idx.astype(np.int64), dl_sel, axis=1)
    wr = np.asarray(layer["w_router"]).astype(F64)
    d_w_router = dl.T @ x64
    dx = dl @ wr
    # routed experts
    d_w13 = np.zeros(layer["w13"].shape, F64)
    d_w2 = np.zeros(layer["w2"].shape, F64)
    if lora is not None:
        lg = {k: np.zeros(np.shape(lora[k[2:]]), F64) for k in ("d_a13", "d_b13", "d_a2", "d_b2")}
    flat = idx.reshape(-1)
    gflat = g.reshape(-1)
    for e in np.unique(flat):
        rows = np.nonzero(flat == e)[0]
        t = rows // K
        dy = gflat[rows, None] * dO[t]
        if lora is None:
            dxr, dw2, dw13, _ = _swiglu_backward(dy, fwd["gu"][rows], x64[t], layer["w13"][e], layer["w2"][e])
        else:
            ad = (lora["a13"][e], lora["b13"][e], lora["a2"][e], lora["b2"][e], float(lora["scale"]))
            dxr, dw2, dw13, *dad = _swiglu_backward_lora(dy, fwd["gu"][rows], x64[t], layer["w13"][e],
                                                          layer["w2"][e], ad)
            for key, val in zip(("d_a13", "d_b13", "d_a2", "d_b2"), dad):
                lg[key][e] = val
        np.add.at(dx, t, dxr)
        d_w2[e] = dw2
        d_w13[e] = dw13
    res = {"dg": dg, "dl": dl_sel, "d_w_router": d_w_router, "d_w13": d_w13, "d_w2": d_w2}
    if lora is not None:
        res.update(lg)
    if layer.get("ws13") is not None:
        s, sg = fwd["s"], fwd["sg"]
        dz = (dO * s).sum(axis=1) * sg * (1.0 - sg)
        wsg = bf16_to_f64(layer["w_sgate"])
        ds = sg[:, None] * dO
        dxs, dws2, dws13, _ = _swiglu_backward(ds, fwd["sgu"], x64, layer["ws13"], layer["ws2"])
        dx = dx + dxs + dz[:, None] * wsg[None, :]
        res.update(dz=dz, d_w_sgate=dz @ x64, d_ws13=dws13, d_ws2=dws2)
    res["dx"] = dx
    return res


def shared_expert_grads(layer: dict, x_bits, d_out_bits) -> dict:
    """Gradients of the shared expert and its gate alone (they sum over all
    tokens): dz = <dOut, S> sg (1 - sg), d_w_sgate = sum_t dz x, and the
    SwiGLU backward with dy = sg * dOut.  Same formulas as backward()."""
    x64 = bf16_to_f64(x_bits)
    dO = bf16_to_f64(d_out_bits)
    s, sg, sgu = shared_expert(x_bits, layer["ws13"], layer["ws2"], layer["w_sgate"])
    dz = (dO * s).sum(axis=1) * sg * (1.0 - sg)
    dxs, dws2, dws13, _ = _swiglu_backward(sg[:, None] * dO, sgu, x64, layer["ws13"], layer["ws2"])
    return {"dz": dz, "d_w_sgate": dz @ x64, "d_ws13": dws13, "d_ws2": dws2, "dx_shared": dxs}


def expert_weight_grads(layer: dict, x_bits, d_out_bits, idx, gates, gu_rows, expert: int):
    """dW13_e and dW2_e of one expert from its own routes only (for spot
    checks at sizes where the full backward is too large).  gu_rows are the
    gate/up values of that expert's routes in ascending route id."""
    T, K = idx.shape
    flat = idx.reshape(-1)
    rows = np.nonzero(flat == expert)[0]
    t = rows // K
    dy = gates.reshape(-1)[rows, None] * bf16_to_f64(d_out_bits)[t]
    _, dw2, dw13, _ = _swiglu_backward(dy, gu_rows, bf16_to_f64(x_bits)[t],
                                       layer["w13"][expert], layer["w2"][expert])
    return dw13, dw2


# --------------------------------------------------------------------------
# brute force (per token, explicit loops) -- the oracle's own cross-check
# --------------------------------------------------------------------------
def brute_force_forward(layer: dict, x_bits, top_k: int = 10):
    """Token-by-token forward with a full sort and explicit per-route FFNs.

    Shares nothing with the vectorised functions above except the exact
    bf16 decode; used to pin them on small inputs."""
    T, H = x_bits.shape
    wr = np.asarray(layer["w_router"]).astype(F64)
    E = wr.shape[0]
    bias = layer.get("router_bias")
    out = np.zeros((T, H), F64)
    routes = np.zeros((T, top_k), np.int32)
    for t in range(T):
        xt = bf16_to_f64(x_bits[t])
        lt = [float(np.dot(wr[e], xt)) + (float(bias[e]) if bias is not None else 0.0)
              for e in range(E)]
        ranked = sorted(range(E), key=lambda e: (-np.float32(lt[e]), e))[:top_k]
        routes[t] = ranked
        m = max(lt[e] for e in ranked)
        w = [np.exp(lt[e] - m) for e in ranked]
        den = sum(w)
        acc = np.zeros(H, F64)
        for k, e in enumerate(ranked):
            w13 = bf16_to_f64(layer["w13"][e])
            w2 = bf16_to_f64(layer["w2"][e])
            inter = w13.shape[0] // 2
            act = np.array([silu(np.dot(w13[i], xt)) * np.dot(w13[inter + i], xt) for i in range(inter)])
            acc += (w[k] / den) * (w2 @ act)
        if layer.get("ws13") is not None:
            ws13 = bf16_to_f64(layer["ws13"])
            ws2 = bf16_to_f64(layer["ws2"])
            inter = ws13.shape[0] // 2
            act = np.array([silu(np.dot(ws13[i], xt)) * np.dot(ws13[inter + i], xt) for i in range(inter)])
            gate = 1.0 / (1.0 + np.exp(-np.dot(bf16_to_f64(layer["w_sgate"]), xt)))
            acc += gate * (ws2 @ act)
        out[t] = acc
    return routes, out
