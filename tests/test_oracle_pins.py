"""Pins of the FP64 oracle against facts that do not come from the oracle.

Each test ties one part of the oracle to something independent of it:
brute-force per-token loops, special cases that reduce to a dense MLP or a
closed form, the tie rule of the pages' routing step, invariants of a
permutation, central finite differences and an independent torch float64
autograd of the same layer definition.  A plausible slip anywhere in the
oracle (a dropped shared term, a transposed weight, a wrong slot order, a
sign in the softmax backward) fails at least one of them.
"""
import dataclasses

import numpy as np
import pytest

import oracle as O
import workloads as W

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def small_cfg(**kw):
    base = dict(name="small", tokens=24, hidden=64, experts=32, top_k=4, inter=32, shared_inter=32)
    base.update(kw)
    return W.MoEConfig(**base)


def layer_and_x(cfg):
    layer = W.make_layer(cfg)
    return layer, W.tokens(cfg)


# ---------------------------------------------------------------- P1 brute force
@pytest.mark.parametrize("cfgname", ["small", "tiny"])
def test_brute_force_matches_vectorised(cfgname):
    cfg = small_cfg() if cfgname == "small" else W.CONFIGS["tiny"]
    layer, x = layer_and_x(cfg)
    x = x[:48]
    fwd = O.forward(layer, x, cfg.top_k)
    routes, out = O.brute_force_forward(layer, x, cfg.top_k)
    assert np.array_equal(routes, fwd["idx"])
    assert np.max(np.abs(out - fwd["out"])) <= 1e-12


def test_brute_force_at_production_shape():
    """Eight tokens of the 2048-hidden, 512-intermediate layer; only the
    experts those tokens touch are generated (the rest stay zero and are
    never read)."""
    cfg = W.CONFIGS["moe1k"]
    layer = W.make_layer(cfg, with_experts=False)
    x = W.tokens(cfg)[:8]
    idx = O.select_routes(O.router_logits(x, layer["w_router"]), cfg.top_k)
    E, H, I = cfg.experts, cfg.hidden, cfg.inter
    w13 = np.zeros((E, 2 * I, H), np.uint16)
    w2 = np.zeros((E, H, I), np.uint16)
    for e in np.unique(idx):
        a, b = W.expert_weights(cfg, int(e), 1)
        w13[e], w2[e] = a[0], b[0]
    layer["w13"], layer["w2"] = w13, w2
    fwd = O.forward(layer, x, cfg.top_k)
    routes, out = O.brute_force_forward(layer, x, cfg.top_k)
    assert np.array_equal(routes, fwd["idx"])
    assert np.max(np.abs(out - fwd["out"])) <= 1e-12


# ---------------------------------------------------------------- P2 identical experts
def test_identical_experts_reduce_to_dense_mlp():
    """All experts equal and no shared expert: the gates sum to one, so the
    layer is one dense SwiGLU MLP whatever the routing."""
    cfg = small_cfg(shared_inter=0)
    layer, x = layer_and_x(cfg)
    layer["w13"] = np.broadcast_to(layer["w13"][3], layer["w13"].shape)
    layer["w2"] = np.broadcast_to(layer["w2"][3], layer["w2"].shape)
    fwd = O.forward(layer, x, cfg.top_k)
    xf = O.bf16_to_f64(x)
    w13 = O.bf16_to_f64(layer["w13"][0])
    w2 = O.bf16_to_f64(layer["w2"][0])
    h = xf @ w13.T
    g, u = h[:, : cfg.inter], h[:, cfg.inter:]
    dense = (g / (1 + np.exp(-g)) * u) @ w2.T
    assert np.max(np.abs(fwd["out"] - dense)) <= 1e-12


# ---------------------------------------------------------------- P3 zero router
def test_zero_router_picks_lowest_ids_with_equal_gates():
    """All logits equal: the tie rule keeps experts 0..K-1 in order, and the
    renormalised gates are exactly 1/K."""
    cfg = small_cfg()
    layer, x = layer_and_x(cfg)
    layer["w_router"] = np.zeros_like(layer["w_router"])
    fwd = O.forward(layer, x, cfg.top_k)
    assert np.array_equal(fwd["idx"], np.tile(np.arange(cfg.top_k, dtype=np.int32), (cfg.tokens, 1)))
    assert np.all(fwd["gates"] == 1.0 / cfg.top_k)


# ---------------------------------------------------------------- P4 forced bias
def test_forced_bias_orders_slots_descending():
    """A bias of -100*e dominates the O(1) logits: slot k holds expert k,
    and the gates equal scipy's softmax of those ten logits."""
    from scipy.special import softmax
    cfg = small_cfg()
    layer, x = layer_and_x(cfg)
    layer["router_bias"] = (-100.0 * np.arange(cfg.experts)).astype(np.float32)
    fwd = O.forward(layer, x, cfg.top_k)
    assert np.array_equal(fwd["idx"], np.tile(np.arange(cfg.top_k, dtype=np.int32), (cfg.tokens, 1)))
    ref = softmax(fwd["logits"][:, : cfg.top_k], axis=1)
    assert np.max(np.abs(fwd["gates"] - ref)) <= 1e-15
    assert np.all(np.diff(fwd["logits"][:, : cfg.top_k], axis=1) < 0)


def test_tie_goes_to_lower_id_inside_the_top_k():
    """Two experts with bit-equal logits: the lower id takes the earlier slot."""
    cfg = small_cfg()
    layer, x = layer_and_x(cfg)
    wr = layer["w_router"].copy()
    wr[7] = wr[19]
    bias = np.zeros(cfg.experts, np.float32)
    bias[[7, 19]] = 50.0
    layer["w_router"], layer["router_bias"] = wr, bias
    fwd = O.forward(layer, x, cfg.top_k)
    assert np.all(fwd["idx"][:, 0] == 7) and np.all(fwd["idx"][:, 1] == 19)
    assert np.allclose(fwd["gates"][:, 0], fwd["gates"][:, 1], rtol=0, atol=0)


# ---------------------------------------------------------------- P5 expert-id probe
def test_expert_id_probe_maps_routes_to_their_experts():
    """Experts built so that expert e outputs the constant c_e on every
    hidden unit: x[:,0] = 1, every gate row = (a,0,...), every up row =
    (b_e,0,...), W2[:,0] = 1.  Then out[t] = sum_k g[t,k] silu(a) b_{e_k}
    exactly, which checks that each route reaches its own expert and its own
    slot's gate."""
    cfg = small_cfg(shared_inter=0)
    layer, x = layer_and_x(cfg)
    x = x.copy()
    x[:, 0] = W.f32_to_bf16_bits(np.ones(1, np.float32))[0]
    E, H, I = cfg.experts, cfg.hidden, cfg.inter
    a = 1.5
    b = np.array([2.0 ** (e // 8 - 2) * (1 + (e % 8) / 8) for e in range(E)])
    w13 = np.zeros((E, 2 * I, H))
    w13[:, :I, 0] = a
    w13[:, I:, 0] = b[:, None]
    w2 = np.zeros((E, H, I))
    w2[:, :, 0] = 1.0
    layer["w13"] = W.f32_to_bf16_bits(w13.astype(np.float32))
    layer["w2"] = W.f32_to_bf16_bits(w2.astype(np.float32))
    assert np.array_equal(O.bf16_to_f64(layer["w13"]), w13)
    fwd = O.forward(layer, x, cfg.top_k)
    c = a / (1 + np.exp(-a)) * b
    expect = (fwd["gates"] * c[fwd["idx"]]).sum(axis=1)
    assert np.max(np.abs(fwd["out"] - expect[:, None])) <= 1e-12


# ---------------------------------------------------------------- P6 invariants
def test_routing_and_permutation_invariants():
    cfg = W.CONFIGS["tiny"]
    layer, x = layer_and_x(cfg)
    fwd = O.forward(layer, x, cfg.top_k)
    idx, g = fwd["idx"], fwd["gates"]
    T, K, E = cfg.tokens, cfg.top_k, cfg.experts
    assert all(len(set(row)) == K for row in idx.tolist())
    assert np.max(np.abs(g.sum(axis=1) - 1.0)) <= 1e-12
    assert np.all(np.diff(g, axis=1) <= 0)       # slot 0 is the largest
    off, srt, pos = fwd["expert_offsets"], fwd["sorted_route"], fwd["route_pos"]
    assert off[0] == 0 and off[-1] == T * K and np.all(np.diff(off) >= 0)
    assert np.array_equal(np.sort(srt), np.arange(T * K))
    assert np.array_equal(pos[srt], np.arange(T * K))
    flat = idx.reshape(-1)
    for e in range(E):
        seg = srt[off[e]: off[e + 1]]
        assert np.all(flat[seg] == e)
        assert np.all(np.diff(seg) > 0)          # ascending route id inside a segment


def test_selection_matches_brute_force_ranking_on_random_logits():
    rng = np.random.default_rng(5)
    logits = rng.standard_normal((64, 512))
    logits[3, 10] = logits[3, 400]               # exact tie
    idx = O.select_routes(logits, 10)
    for t in range(64):
        ranked = sorted(range(512), key=lambda e: (-np.float32(logits[t, e]), e))[:10]
        assert list(idx[t]) == ranked


# ---------------------------------------------------------------- P7 backward
def _loss(layer, x, d_out, idx, top_k):
    fwd = O.forward(layer, x, top_k, forced_idx=idx)
    return float(np.sum(O.bf16_to_f64(d_out) * fwd["out"]))


def _tiny_float_layer():
    cfg = small_cfg(tokens=6, hidden=16, experts=8, top_k=3, inter=8, shared_inter=8)
    layer, x = layer_and_x(cfg)
    f = {k: (O.bf16_to_f64(v) if v is not None and v.dtype == np.uint16 else v) for k, v in layer.items()}
    f["w_router"] = layer["w_router"].astype(np.float64) * 20.0   # spread the gates
    return cfg, f, O.bf16_to_f64(x), W.grad_out(cfg)


@pytest.mark.parametrize("name", ["w_router", "w13", "w2", "ws13", "ws2", "w_sgate", "x"])
def test_backward_matches_central_differences(name):
    cfg, layer, x, d_out = _tiny_float_layer()
    fwd = O.forward(layer, x, cfg.top_k)
    idx = fwd["idx"]
    grads = O.backward(layer, x, fwd, d_out)
    key = {"x": "dx", "w_router": "d_w_router"}.get(name, "d_" + name)
    g = grads[key]
    base = x if name == "x" else layer[name]
    rng = np.random.default_rng(1)
    flat_ids = rng.choice(base.size, size=min(24, base.size), replace=False)
    h = 1e-6
    for fi in flat_ids:
        pert = base.copy().reshape(-1)
        orig = pert[fi]
        vals = []
        for s in (+1, -1):
            pert[fi] = orig + s * h
            arr = pert.reshape(base.shape)
            if name == "x":
                vals.append(_loss(layer, arr, d_out, idx, cfg.top_k))
            else:
                lay = dict(layer)
                lay[name] = arr
                vals.append(_loss(lay, x, d_out, idx, cfg.top_k))
        fd = (vals[0] - vals[1]) / (2 * h)
        an = g.reshape(-1)[fi]
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (name, fi, fd, an)


def test_backward_matches_torch_float64_autograd():
    torch = pytest.importorskip("torch")
    cfg, layer, x, d_out = _tiny_float_layer()
    fwd = O.forward(layer, x, cfg.top_k)
    idx = fwd["idx"]
    grads = O.backward(layer, x, fwd, d_out)
    T = lambda a: torch.tensor(np.asarray(a, np.float64), requires_grad=True)
    tx, twr, tw13, tw2 = T(x), T(layer["w_router"]), T(layer["w13"]), T(layer["w2"])
    tws13, tws2, twsg = T(layer["ws13"]), T(layer["ws2"]), T(layer["w_sgate"])
    I = cfg.inter
    logits = tx @ twr.T
    sel = torch.gather(logits, 1, torch.tensor(idx, dtype=torch.int64))
    gates = torch.softmax(sel, dim=1)
    out = torch.zeros(cfg.tokens, cfg.hidden, dtype=torch.float64)
    for t in range(cfg.tokens):
        for k in range(cfg.top_k):
            e = int(idx[t, k])
            h = tw13[e] @ tx[t]
            act = torch.nn.functional.silu(h[:I]) * h[I:]
            out[t] = out[t] + gates[t, k] * (tw2[e] @ act)
    hs = tx @ tws13.T
    s = (torch.nn.functional.silu(hs[:, :I]) * hs[:, I:]) @ tws2.T
    out = out + torch.sigmoid(tx @ twsg)[:, None] * s
    (out * torch.tensor(O.bf16_to_f64(d_out))).sum().backward()
    pairs = [("dx", tx), ("d_w_router", twr), ("d_w13", tw13), ("d_w2", tw2),
             ("d_ws13", tws13), ("d_ws2", tws2), ("d_w_sgate", twsg)]
    assert np.max(np.abs(fwd["out"] - out.detach().numpy())) <= 1e-12
    for key, tt in pairs:
        assert np.max(np.abs(grads[key] - tt.grad.numpy())) <= 1e-12, key


def test_expert_weight_grads_match_full_backward():
    cfg, layer, x, d_out = _tiny_float_layer()
    fwd = O.forward(layer, x, cfg.top_k)
    grads = O.backward(layer, x, fwd, d_out)
    flat = fwd["idx"].reshape(-1)
    for e in np.unique(flat):
        rows = np.nonzero(flat == e)[0]
        dw13, dw2 = O.expert_weight_grads(layer, x, d_out, fwd["idx"], fwd["gates"], fwd["gu"][rows], int(e))
        assert np.max(np.abs(dw13 - grads["d_w13"][e])) <= 1e-13
        assert np.max(np.abs(dw2 - grads["d_w2"][e])) <= 1e-13


def test_shared_expert_grads_match_full_backward():
    cfg, layer, x, d_out = _tiny_float_layer()
    fwd = O.forward(layer, x, cfg.top_k)
    full = O.backward(layer, x, fwd, d_out)
    sh = O.shared_expert_grads(layer, x, d_out)
    for k in ("dz", "d_w_sgate", "d_ws13", "d_ws2"):
        assert np.max(np.abs(sh[k] - full[k])) <= 1e-13, k


def test_token_subset_backward_gives_the_same_input_gradient_rows():
    """dX of a token depends only on that token: the backward of a token
    subset reproduces the full batch's dX rows (used for sampled GPU checks)."""
    cfg, layer, x, d_out = _tiny_float_layer()
    fwd = O.forward(layer, x, cfg.top_k)
    full = O.backward(layer, x, fwd, d_out)
    sub = np.array([1, 4, 5])
    fs = O.forward(layer, x[sub], cfg.top_k)
    part = O.backward(layer, x[sub], fs, d_out[sub])
    assert np.max(np.abs(part["dx"] - full["dx"][sub])) <= 1e-13
    assert np.max(np.abs(part["dl"] - full["dl"][sub])) <= 1e-13


# ---------------------------------------------------------------- subsets and bf16 report
def test_token_subset_equals_full_rows():
    cfg = small_cfg()
    layer, x = layer_and_x(cfg)
    full = O.forward(layer, x, cfg.top_k)
    sub = [0, 5, 23, 11]
    part = O.forward(layer, x, cfg.top_k, tokens=sub)
    assert np.array_equal(part["idx"], full["idx"][sub])
    # BLAS may block a float64 product differently for a different row count
    assert np.max(np.abs(part["out"] - full["out"][sub])) <= 1e-15
    K = cfg.top_k
    rows = np.concatenate([np.arange(t * K, t * K + K) for t in sub])
    assert np.max(np.abs(part["y"] - full["y"][rows])) <= 1e-15


def test_bf16_round_trip_and_rounding():
    vals = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -9, -2.5, 3.0e-3])
    bits = O.f64_to_bf16_bits(vals)
    back = O.bf16_to_f64(bits)
    assert back[0] == 1.0
    assert back[1] == 1.0                # tie -> even
    assert back[2] == 1.0 + 2.0 ** -7    # above the half-way point -> up
    assert back[3] == -2.5
    # half an ulp of the binade [2^-9, 2^-8): 2^-9 * 2^-8
    assert abs(back[4] - 3.0e-3) <= 2.0 ** -17


# ------------------------------------------------- block-scaled FP8 weights
def test_e4m3_decode_matches_the_format_definition():
    """OCP MX v1.0, E4M3 element type: bias 7, 3 mantissa bits, exponent
    field 0 subnormal (m x 2^-9), S.1111.111 NaN, largest normal 448."""
    d = O.e4m3_to_f64
    assert d(0x00) == 0.0 and np.signbit(d(0x80))
    assert d(0x01) == 2.0 ** -9                      # smallest subnormal
    assert d(0x07) == 0.875 * 2.0 ** -6              # largest subnormal
    assert d(0x08) == 2.0 ** -6                      # smallest normal
    assert d(0x38) == 1.0 and d(0xB8) == -1.0
    assert d(0x39) == 1.125 and d(0x3F) == 1.875
    assert d(0x7E) == 448.0 and d(0xFE) == -448.0    # largest normal
    assert np.isnan(d(0x7F)) and np.isnan(d(0xFF))
    # every finite code: exponent/mantissa composition, brute force
    for c in range(256):
        if c & 0x7F == 0x7F:
            continue
        e, m, s = (c >> 3) & 15, c & 7, -1.0 if c & 0x80 else 1.0
        want = s * (m / 8.0 * 2.0 ** -6 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7))
        assert d(c) == want


def test_e8m0_and_block_scaling():
    assert O.e8m0_to_f64(127) == 1.0
    assert O.e8m0_to_f64(0) == 2.0 ** -127 and O.e8m0_to_f64(254) == 2.0 ** 127
    assert np.isnan(O.e8m0_to_f64(255))
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 0x7F, size=(3, 96)).astype(np.uint8)
    scales = rng.integers(100, 140, size=(3, 3)).astype(np.uint8)
    got = O.mx_to_f64(codes, scales)
    for r in range(3):
        for i in range(96):
            assert got[r, i] == O.e4m3_to_f64(codes[r, i]) * 2.0 ** (int(scales[r, i // 32]) - 127)


def test_mx_encoder_picks_the_nearest_representable_weight():
    """The input encoder (workloads.mx) against brute force over the oracle's
    decoding of all finite codes: each element is the nearest E4M3 value of
    the scaled weight (ties to the even code), clamped at 448, and the block
    scale is 2^(floor(log2 amax) - 8)."""
    import workloads.mx as MX
    finite = np.array([c for c in range(256) if c & 0x7F != 0x7F], np.uint8)
    fvals = O.e4m3_to_f64(finite)
    rng = np.random.default_rng(11)
    w = rng.standard_normal((4, 64)).astype(np.float32) * np.float32(0.02)
    w[0, :32] = 0.0                                    # an all-zero block
    w[1, 3] = np.float32(5.0)                          # a block dominated by one value
    bits = W.f32_to_bf16_bits(w)
    codes, sc = MX.encode_mx(bits)
    v = O.bf16_to_f64(bits)
    for r in range(4):
        for b in range(2):
            blk = v[r, 32 * b:32 * b + 32]
            amax = np.abs(blk).max()
            want_s = 127 if amax == 0 else int(np.floor(np.log2(amax))) - 8 + 127
            assert sc[r, b] == want_s
            X = 2.0 ** (int(sc[r, b]) - 127)
            for i in range(32):
                y = min(max(blk[i] / X, -448.0), 448.0)
                dist = np.abs(fvals - y)
                best = finite[dist == dist.min()]
                if len(best) > 1:                       # a tie: the even mantissa
                    best = best[(best & 1) == 0]
                    best = best[np.signbit(O.e4m3_to_f64(best)) == np.signbit(y)] if len(best) > 1 else best
                assert O.e4m3_to_f64(codes[r, 32 * b + i]) == O.e4m3_to_f64(best[0])


# ---------------------------------------------------------------- LoRA adapters
BF16_ONE = 0x3F80


def lora_for(cfg, rank, scale=0.75):
    import workloads.lora as WL
    return WL.lora_adapters(cfg, rank, scale)


def test_expert_lora_rank_matches_the_pages():
    """ROLL pull request 502 page, "What this changes": an adapter of rank
    64 over a top-10 router gives rank-6 expert adapters."""
    assert O.expert_lora_rank(64, 10) == 6


def test_lora_with_zero_expand_is_the_base_layer():
    cfg = small_cfg()
    layer, x = layer_and_x(cfg)
    ad = lora_for(cfg, 3)
    ad["b13"][:] = 0
    ad["b2"][:] = 0
    base = O.forward(layer, x, cfg.top_k)
    lo = O.forward(layer, x, cfg.top_k, lora=ad)
    for key in ("y", "gu", "out"):
        assert np.array_equal(base[key], lo[key])


def test_lora_equals_the_merged_weight_layer():
    """LoRA's defining identity W x + s B (A x) = (W + s B A) x, route by
    route: the merged weights (float64, no longer bf16) go through a plain
    per-route SwiGLU written here."""
    cfg = small_cfg()
    layer, x = layer_and_x(cfg)
    ad = lora_for(cfg, 3)
    s = ad["scale"]
    fwd = O.forward(layer, x, cfg.top_k, lora=ad)
    bf = O.bf16_to_f64
    x64 = bf(x)
    I, K = cfg.inter, cfg.top_k
    merged = {}
    for t in range(cfg.tokens):
        for k in range(K):
            e = int(fwd["idx"][t, k])
            if e not in merged:
                merged[e] = (bf(layer["w13"][e]) + s * bf(ad["b13"][e]) @ bf(ad["a13"][e]),
                             bf(layer["w2"][e]) + s * bf(ad["b2"][e]) @ bf(ad["a2"][e]))
            w13, w2 = merged[e]
            gu = w13 @ x64[t]
            act = gu[:I] / (1.0 + np.exp(-gu[:I])) * gu[I:]
            y = w2 @ act
            r = t * K + k
            assert np.max(np.abs(gu - fwd["gu"][r])) <= 1e-12
            assert np.max(np.abs(y - fwd["y"][r])) <= 1e-12
    # the update is not negligible at these magnitudes
    base = O.forward(layer, x, cfg.top_k)
    assert np.max(np.abs(base["y"] - fwd["y"])) > 1e-4


def test_lora_one_hot_up_adapter_moves_one_gate_up_column():
    """Rank 1, A13 one-hot at input feature h0, B13 one-hot at gate/up
    column c0: only gu[:, c0] changes, by scale * x[token, h0].  A
    transposed factor, a wrong axis or a misplaced scale fails this."""
    cfg = small_cfg()
    layer, x = layer_and_x(cfg)
    E, H, I, K = cfg.experts, cfg.hidden, cfg.inter, cfg.top_k
    h0, c0, s = 5, I + 7, 0.75
    ad = {"a13": np.zeros((E, 1, H), np.uint16), "b13": np.zeros((E, 2 * I, 1), np.uint16),
          "a2": np.zeros((E, 1, I), np.uint16), "b2": np.zeros((E, H, 1), np.uint16), "scale": s}
    ad["a13"][:, 0, h0] = BF16_ONE
    ad["b13"][:, c0, 0] = BF16_ONE
    base = O.forward(layer, x, K)
    lo = O.forward(layer, x, K, lora=ad)
    d = lo["gu"] - base["gu"]
    want = s * O.bf16_to_f64(x)[np.repeat(np.arange(cfg.tokens), K), h0]
    assert np.max(np.abs(d[:, c0] - want)) <= 1e-15
    assert not np.any(np.delete(d, c0, axis=1))


def test_lora_one_hot_down_adapter_moves_one_hidden_column():
    """Rank 1, A2 one-hot at activation column i0, B2 one-hot at hidden
    column h1: only y[:, h1] changes, by scale * act[:, i0] (act from the
    unchanged gate/up values)."""
    cfg = small_cfg()
    layer, x = layer_and_x(cfg)
    E, H, I, K = cfg.experts, cfg.hidden, cfg.inter, cfg.top_k
    i0, h1, s = 3, 11, 0.75
    ad = {"a13": np.zeros((E, 1, H), np.uint16), "b13": np.zeros((E, 2 * I, 1), np.uint16),
          "a2": np.zeros((E, 1, I), np.uint16), "b2": np.zeros((E, H, 1), np.uint16), "scale": s}
    ad["a2"][:, 0, i0] = BF16_ONE
    ad["b2"][:, h1, 0] = BF16_ONE
    base = O.forward(layer, x, K)
    lo = O.forward(layer, x, K, lora=ad)
    assert np.array_equal(lo["gu"], base["gu"])
    gu = base["gu"]
    act = gu[:, :I] / (1.0 + np.exp(-gu[:, :I])) * gu[:, I:]
    d = lo["y"] - base["y"]
    assert np.max(np.abs(d[:, h1] - s * act[:, i0])) <= 1e-15
    assert not np.any(np.delete(d, h1, axis=1))


def test_lora_merged_weights_at_production_shape():
    """The merged-weight identity on four tokens of the 2048-hidden,
    512-intermediate layer with rank-6 adapters (only the touched experts'
    weights are generated)."""
    import workloads.lora as WL
    cfg = W.CONFIGS["moe1k"]
    layer = W.make_layer(cfg, with_experts=False)
    x = W.tokens(cfg)[:4]
    idx = O.select_routes(O.router_logits(x, layer["w_router"]), cfg.top_k)
    E, H, I, K = cfg.experts, cfg.hidden, cfg.inter, cfg.top_k
    w13 = np.zeros((E, 2 * I, H), np.uint16)
    w2 = np.zeros((E, H, I), np.uint16)
    for e in np.unique(idx):
        a, b = W.expert_weights(cfg, int(e), 1)
        w13[e], w2[e] = a[0], b[0]
    layer["w13"], layer["w2"] = w13, w2
    ad = WL.lora_adapters(cfg)
    s = ad["scale"]
    fwd = O.forward(layer, x, K, lora=ad)
    bf = O.bf16_to_f64
    x64 = bf(x)
    for t in range(4):
        for k in range(K):
            e = int(fwd["idx"][t, k])
            gu = (bf(w13[e]) + s * bf(ad["b13"][e]) @ bf(ad["a13"][e])) @ x64[t]
            act = gu[:I] / (1.0 + np.exp(-gu[:I])) * gu[I:]
            y = (bf(w2[e]) + s * bf(ad["b2"][e]) @ bf(ad["a2"][e])) @ act
            assert np.max(np.abs(y - fwd["y"][t * K + k])) <= 1e-12


def test_lora_adapter_inputs_are_seeded_and_shaped():
    """The adapter generator (input side only) is a pure function of the
    seed: same bits on every call, one stream per matrix and expert."""
    import workloads.lora as WL
    cfg = small_cfg()
    a, b = WL.lora_adapters(cfg, 3), WL.lora_adapters(cfg, 3)
    E, H, I = cfg.experts, cfg.hidden, cfg.inter
    shapes = {"a13": (E, 3, H), "b13": (E, 2 * I, 3), "a2": (E, 3, I), "b2": (E, H, 3)}
    for k, shp in shapes.items():
        assert a[k].shape == shp and a[k].dtype == np.uint16
        assert np.array_equal(a[k], b[k])
    assert not np.array_equal(a["a13"][0], a["a13"][1])
    assert a["rank"] == 3 and a["scale"] == WL.DEFAULT_SCALE


@pytest.mark.parametrize("name,gaps", [("tiny", (1e-3, 1e-2, 3e-2)), ("moe8k", (1e-4, 1e-3, 1e-2))])
def test_selection_boundary_spacing_matches_the_closed_form(name, gaps):
    """Tie-rate pin: at the selection threshold the gap between the K-th and
    (K+1)-th largest exact logits is about exponential with rate
    rho = E phi(z) / sigma_l, z = Phi^-1(1 - (K + 1/2) / E), sigma_l =
    0.02 sqrt(H) for unit-variance tokens (order statistics of E normal
    logits).  Counted on the oracle's own logits at gaps where the counts
    are large, the observed rate agrees with T (1 - exp(-rho d)) within
    Poisson noise plus 15%, which pins the expected number of fp32 router
    ties (gap < 1e-6) at T rho 1e-6: 0.014 for the 256-token layer, 0.23 at
    8192 tokens of hidden 2048."""
    from scipy.stats import norm
    cfg = W.CONFIGS[name]
    layer = W.make_layer(cfg, with_experts=False)
    logits = O.router_logits(W.tokens(cfg), layer["w_router"])
    top = -np.sort(-logits, axis=1)[:, :cfg.top_k + 1]
    gap = top[:, cfg.top_k - 1] - top[:, cfg.top_k]
    z = norm.ppf(1.0 - (cfg.top_k + 0.5) / cfg.experts)
    rho = cfg.experts * norm.pdf(z) / (cfg.w_sigma * np.sqrt(cfg.hidden))
    for d in gaps:
        expected = cfg.tokens * (1.0 - np.exp(-rho * d))
        observed = int((gap < d).sum())
        assert abs(observed - expected) <= 5.0 * np.sqrt(expected) + 0.15 * expected, (d, observed, expected)
    assert {"tiny": 0.014, "moe8k": 0.23}[name] == pytest.approx(cfg.tokens * rho * 1e-6, rel=0.03)


# ---------------------------------------------------------------- LoRA backward
def _tiny_lora_float(cfg, rank=3, scale=0.75):
    rng = np.random.default_rng(5)
    E, H, I = cfg.experts, cfg.hidden, cfg.inter
    return {"a13": rng.normal(0, 0.3, (E, rank, H)), "b13": rng.normal(0, 0.3, (E, 2 * I, rank)),
            "a2": rng.normal(0, 0.3, (E, rank, I)), "b2": rng.normal(0, 0.3, (E, H, rank)), "rank": rank,
            "scale": scale}


def _lora_loss(layer, x, d_out, idx, top_k, lora):
    fwd = O.forward(layer, x, top_k, forced_idx=idx, lora=lora)
    return float(np.sum(O.bf16_to_f64(d_out) * fwd["out"]))


@pytest.mark.parametrize("name", ["a13", "b13", "a2", "b2", "w13", "w2", "w_router", "x"])
def test_lora_backward_matches_central_differences(name):
    """Every adapter matrix, the base expert weights, the router and the
    input: the oracle's LoRA backward against central differences of the
    LoRA forward (routing frozen)."""
    cfg, layer, x, d_out = _tiny_float_layer()
    ad = _tiny_lora_float(cfg)
    fwd = O.forward(layer, x, cfg.top_k, lora=ad)
    idx = fwd["idx"]
    grads = O.backward(layer, x, fwd, d_out, lora=ad)
    key = {"x": "dx", "w_router": "d_w_router"}.get(name, "d_" + name)
    g = grads[key]
    if name in ("a13", "b13", "a2", "b2"):
        base = ad[name]
    else:
        base = x if name == "x" else layer[name]
    rng = np.random.default_rng(2)
    h = 1e-6
    for fi in rng.choice(base.size, size=min(24, base.size), replace=False):
        pert = base.copy().reshape(-1)
        orig = pert[fi]
        vals = []
        for s in (+1, -1):
            pert[fi] = orig + s * h
            arr = pert.reshape(base.shape)
            lay, xx, aa = layer, x, ad
            if name in ("a13", "b13", "a2", "b2"):
                aa = dict(ad)
                aa[name] = arr
            elif name == "x":
                xx = arr
            else:
                lay = dict(layer)
                lay[name] = arr
            vals.append(_lora_loss(lay, xx, d_out, idx, cfg.top_k, aa))
        fd = (vals[0] - vals[1]) / (2 * h)
        an = g.reshape(-1)[fi]
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (name, fi, fd, an)


def test_lora_backward_matches_torch_float64_autograd():
    """An independently written LoRA forward in torch float64 (per token,
    per route, the update scale * B (A v) on both projections), its autograd
    gradients against the oracle's."""
    torch = pytest.importorskip("torch")
    cfg, layer, x, d_out = _tiny_float_layer()
    ad = _tiny_lora_float(cfg)
    fwd = O.forward(layer, x, cfg.top_k, lora=ad)
    idx = fwd["idx"]
    grads = O.backward(layer, x, fwd, d_out, lora=ad)
    T = lambda a: torch.tensor(np.asarray(a, np.float64), requires_grad=True)
    tx, twr, tw13, tw2 = T(x), T(layer["w_router"]), T(layer["w13"]), T(layer["w2"])
    tws13, tws2, twsg = T(layer["ws13"]), T(layer["ws2"]), T(layer["w_sgate"])
    ta13, tb13, ta2, tb2 = T(ad["a13"]), T(ad["b13"]), T(ad["a2"]), T(ad["b2"])
    sc = ad["scale"]
    I = cfg.inter
    logits = tx @ twr.T
    gates = torch.softmax(torch.gather(logits, 1, torch.tensor(idx, dtype=torch.int64)), dim=1)
    out = torch.zeros(cfg.tokens, cfg.hidden, dtype=torch.float64)
    for t in range(cfg.tokens):
        for k in range(cfg.top_k):
            e = int(idx[t, k])
            h = tw13[e] @ tx[t] + sc * (tb13[e] @ (ta13[e] @ tx[t]))
            act = torch.nn.functional.silu(h[:I]) * h[I:]
            y = tw2[e] @ act + sc * (tb2[e] @ (ta2[e] @ act))
            out[t] = out[t] + gates[t, k] * y
    hs = tx @ tws13.T
    s = (torch.nn.functional.silu(hs[:, :I]) * hs[:, I:]) @ tws2.T
    out = out + torch.sigmoid(tx @ twsg)[:, None] * s
    (out * torch.tensor(O.bf16_to_f64(d_out))).sum().backward()
    assert np.max(np.abs(fwd["out"] - out.detach().numpy())) <= 1e-12
    pairs = [("dx", tx), ("d_w_router", twr), ("d_w13", tw13), ("d_w2", tw2), ("d_ws13", tws13),
             ("d_ws2", tws2), ("d_w_sgate", twsg), ("d_a13", ta13), ("d_b13", tb13), ("d_a2", ta2),
             ("d_b2", tb2)]
    for key, tt in pairs:
        assert np.max(np.abs(grads[key] - tt.grad.numpy())) <= 1e-12, key


def test_lora_backward_with_zero_expand():
    """B13 = B2 = 0: the adapters change nothing, so every base gradient is
    the plain backward's, the shrink matrices get no gradient, and the
    expand matrices' gradients are s * dgu^T (x A13^T) and s * dy^T (act
    A2^T) route by route."""
    cfg, layer, x, d_out = _tiny_float_layer()
    ad = _tiny_lora_float(cfg)
    ad["b13"][:] = 0.0
    ad["b2"][:] = 0.0
    fwd = O.forward(layer, x, cfg.top_k, lora=ad)
    plain = O.backward(layer, x, O.forward(layer, x, cfg.top_k), d_out)
    lo = O.backward(layer, x, fwd, d_out, lora=ad)
    for key in ("dx", "d_w_router", "d_w13", "d_w2", "d_ws13", "d_ws2", "d_w_sgate"):
        assert np.max(np.abs(lo[key] - plain[key])) <= 1e-13, key
    assert not lo["d_a13"].any() and not lo["d_a2"].any()
    K, I = cfg.top_k, cfg.inter
    dO = O.bf16_to_f64(d_out)
    flat = fwd["idx"].reshape(-1)
    for e in np.unique(flat):
        rows = np.nonzero(flat == e)[0]
        t = rows // K
        dy = fwd["gates"].reshape(-1)[rows, None] * dO[t]
        gu = fwd["gu"][rows]
        act = O.silu(gu[:, :I]) * gu[:, I:]
        dgu = O.swiglu_backward(dy, gu, x[t], layer["w13"][e], layer["w2"][e])[3]
        assert np.max(np.abs(lo["d_b13"][e] - ad["scale"] * dgu.T @ (x[t] @ ad["a13"][e].T))) <= 1e-13
        assert np.max(np.abs(lo["d_b2"][e] - ad["scale"] * dy.T @ (act @ ad["a2"][e].T))) <= 1e-13
