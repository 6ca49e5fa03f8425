"""Pins of the oracle's decode layer (CPU): library routines, closed forms,
invariants and a pure-Python brute force on tiny shapes."""
import dataclasses
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import layer as ol
from oracle.numerics import round_bf16


def rnd(rng, *shape, s=1.0):
    return rng.standard_normal(shape) * s


# ----------------------------------------------------------------------------- rmsnorm
def test_rmsnorm_matches_torch():
    rng = np.random.default_rng(0)
    x = rnd(rng, 5, 48)
    g = rnd(rng, 48)
    ref = F.rms_norm(torch.tensor(x), (48,), weight=torch.tensor(g), eps=1e-5).numpy()
    np.testing.assert_allclose(ol.rmsnorm(x, g, 1e-5), ref, rtol=1e-13, atol=1e-14)


def test_rmsnorm_constant_and_scale_invariance():
    g = np.linspace(0.5, 2.0, 16)
    for c in (-3.0, 0.7):
        np.testing.assert_allclose(ol.rmsnorm(np.full((1, 16), c), g, 0.0)[0], np.sign(c) * g, rtol=1e-14)
    x = np.random.default_rng(1).standard_normal((3, 16))
    np.testing.assert_allclose(ol.rmsnorm(7.5 * x, g, 0.0), ol.rmsnorm(x, g, 0.0), rtol=1e-13)


# ----------------------------------------------------------------------------- attention
def sdpa_with_sink(q, K, V, sinks, scale):
    """torch SDPA (float64, CPU) with the sink as an extra key of score sink_h
    and a zero value vector; grouped-query through enable_gqa."""
    Hq, D = q.shape
    Hkv, n, _ = K.shape
    qt = torch.tensor(q)[None, :, None, :]
    Kt = torch.cat([torch.zeros(Hkv, 1, D, dtype=torch.float64), torch.tensor(K)], dim=1)[None]
    Vt = torch.cat([torch.zeros(Hkv, 1, D, dtype=torch.float64), torch.tensor(V)], dim=1)[None]
    mask = torch.zeros(1, Hq, 1, n + 1, dtype=torch.float64)
    mask[0, :, 0, 0] = torch.tensor(sinks)
    return F.scaled_dot_product_attention(qt, Kt, Vt, attn_mask=mask, scale=scale, enable_gqa=True)[0, :, 0, :].numpy()


@pytest.mark.parametrize("Hq,Hkv,n,D", [(8, 1, 37, 16), (8, 2, 5, 8), (4, 4, 64, 64), (64, 8, 300, 64)])
def test_attention_matches_sdpa_with_sink_token(Hq, Hkv, n, D):
    rng = np.random.default_rng(Hq * 100 + n)
    q, K, V = rnd(rng, Hq, D), rnd(rng, Hkv, n, D), rnd(rng, Hkv, n, D)
    sinks = rnd(rng, Hq)
    o, p, ps = ol.decode_attention(q, K, V, sinks, 1 / math.sqrt(D))
    np.testing.assert_allclose(o, sdpa_with_sink(q, K, V, sinks, 1 / math.sqrt(D)), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(p.sum(axis=1) + ps, 1.0, rtol=0, atol=1e-14)


def test_attention_single_key_closed_form():
    rng = np.random.default_rng(3)
    q, K, V, sinks = rnd(rng, 4, 8), rnd(rng, 2, 1, 8), rnd(rng, 2, 1, 8), rnd(rng, 4)
    o, _, _ = ol.decode_attention(q, K, V, sinks, 0.25)
    for h in range(4):
        g = h // 2
        s0 = 0.25 * float(q[h] @ K[g, 0])
        np.testing.assert_allclose(o[h], V[g, 0] / (1 + math.exp(sinks[h] - s0)), rtol=1e-13)


def test_attention_identical_keys_gives_scaled_mean():
    rng = np.random.default_rng(4)
    q, V, sinks = rnd(rng, 2, 8), rnd(rng, 1, 9, 8), rnd(rng, 2)
    K = np.repeat(rnd(rng, 1, 1, 8), 9, axis=1)
    o, _, ps = ol.decode_attention(q, K, V, sinks, 0.3)
    for h in range(2):
        np.testing.assert_allclose(o[h], (1 - ps[h]) * V[0].mean(axis=0), rtol=1e-13)


def test_attention_without_sink_is_textbook_softmax():
    rng = np.random.default_rng(5)
    q, K, V = rnd(rng, 6, 16), rnd(rng, 3, 20, 16), rnd(rng, 3, 20, 16)
    o, _, ps = ol.decode_attention(q, K, V, np.full(6, -1e300), 0.25)
    ref = F.scaled_dot_product_attention(torch.tensor(q)[None, :, None], torch.tensor(K)[None],
                                         torch.tensor(V)[None], scale=0.25, enable_gqa=True)[0, :, 0].numpy()
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-13)
    assert np.all(ps == 0.0)


def test_attention_window_bounds():
    assert ol.attention_window("full", 300, 128) == (0, 300)
    assert ol.attention_window("sliding", 300, 128) == (172, 300)
    assert ol.attention_window("sliding", 100, 128) == (0, 100)
    assert ol.attention_window("sliding", 128, 128) == (0, 128)
    assert ol.attention_window("sliding", 129, 128) == (1, 129)


# ----------------------------------------------------------------------------- router
def test_router_topk_matches_torch_and_sorted_order():
    rng = np.random.default_rng(6)
    for _ in range(50):
        l = rng.standard_normal(128).astype(np.float32)
        idx, margin = ol.router_topk(l, 4)
        tv, ti = torch.topk(torch.tensor(l), 5)
        np.testing.assert_array_equal(idx, ti[:4].numpy())
        assert margin == pytest.approx(float(tv[3] - tv[4]), abs=0)


def test_router_ties_go_to_lower_index():
    l = np.array([0.5, 2.0, 1.0, 2.0, 1.0, -1.0], np.float32)
    idx, margin = ol.router_topk(l, 3)
    np.testing.assert_array_equal(idx, [1, 3, 2])
    assert margin == 0.0


def test_route_weights_is_renormalised_full_softmax():
    rng = np.random.default_rng(7)
    l = rng.standard_normal(32) * 3
    idx, _ = ol.router_topk(l.astype(np.float32), 4)
    w = ol.route_weights(l, idx)
    full = torch.softmax(torch.tensor(l), 0).numpy()
    np.testing.assert_allclose(w, full[idx] / full[idx].sum(), rtol=1e-13)
    assert w.sum() == pytest.approx(1.0, abs=1e-15)
    # E == k: the weights are the full softmax in pick order
    idx8, m8 = ol.router_topk(l[:8].astype(np.float32), 8)
    np.testing.assert_allclose(ol.route_weights(l[:8], idx8), torch.softmax(torch.tensor(l[:8]), 0).numpy()[idx8],
                               rtol=1e-13)
    assert m8 == float("inf")


def test_router_column_permutation_permutes_indices():
    rng = np.random.default_rng(8)
    l = rng.standard_normal(64).astype(np.float32)
    perm = rng.permutation(64)
    idx, _ = ol.router_topk(l, 4)
    idx2, _ = ol.router_topk(l[perm], 4)
    np.testing.assert_array_equal(perm[idx2], idx)


# ----------------------------------------------------------------------------- permutation
@pytest.mark.parametrize("B,k,E", [(4, 2, 8), (64, 4, 4), (64, 4, 128), (7, 3, 5), (1, 1, 1)])
def test_permutation_invariants_and_brute_force(B, k, E):
    rng = np.random.default_rng(B * 1000 + E)
    g = rng.integers(0, E, (B, k))
    counts, offsets, row_tok, row_slot, inv = ol.permutation(g, E)
    assert counts.sum() == B * k and offsets[0] == 0 and offsets[-1] == B * k
    np.testing.assert_array_equal(np.diff(offsets), counts)
    # brute force: walk experts, then tokens, then picks
    rows = [(b, s) for e in range(E) for b in range(B) for s in range(k) if g[b, s] == e]
    np.testing.assert_array_equal(row_tok, [r[0] for r in rows])
    np.testing.assert_array_equal(row_slot, [r[1] for r in rows])
    for b in range(B):
        for s in range(k):
            r = inv[b, s]
            assert row_tok[r] == b and row_slot[r] == s and offsets[g[b, s]] <= r < offsets[g[b, s] + 1]


# ----------------------------------------------------------------------------- experts
def test_silu_matches_torch():
    v = np.linspace(-30, 30, 1001)
    np.testing.assert_allclose(ol.silu(v), F.silu(torch.tensor(v)).numpy(), rtol=1e-14, atol=1e-300)


def _tiny(E=8, E_res=8, k=2, H=32, I=24, Hq=4, Hkv=2, D=8, W=6):
    return ol.Dims(H, Hq, Hkv, D, E, E_res, k, I, W)


def _params(dims, rng, gate_zero=False, wd_mult=1.0):
    H, D = dims.hidden, dims.head_dim
    dense = {
        "wqkv": rnd(rng, (dims.n_q_heads + 2 * dims.n_kv_heads) * D, H, s=0.2),
        "wo": rnd(rng, H, dims.n_q_heads * D, s=0.2),
        "wr": rnd(rng, dims.n_experts, H, s=1 / math.sqrt(H)),
        "sinks": rnd(rng, dims.n_q_heads),
        "gamma1": 1 + 0.1 * rnd(rng, H),
        "gamma2": 1 + 0.1 * rnd(rng, H),
    }
    experts = {}
    for e in range(dims.n_resident):
        wgu = rnd(rng, 2 * dims.inter, H, s=0.2)
        if gate_zero:
            wgu[: dims.inter] = 0.0
        experts[e] = {"wgu": wgu, "wd": wd_mult * rnd(rng, H, dims.inter, s=0.2)}
    return dense, experts


def _history(dims, rng, B, Lmax):
    Kh = rnd(rng, B, dims.n_kv_heads, Lmax, dims.head_dim)
    Vh = rnd(rng, B, dims.n_kv_heads, Lmax, dims.head_dim)
    return Kh, Vh, (lambda b, lo, hi: (Kh[b][:, lo:hi], Vh[b][:, lo:hi]))


def test_single_expert_top1_equals_dense_swiglu_mlp():
    dims = _tiny(E=1, E_res=1, k=1)
    rng = np.random.default_rng(9)
    dense, experts = _params(dims, rng)
    B, L = 3, [5, 2, 9]
    _, _, hist = _history(dims, rng, B, 10)
    x = rnd(rng, B, dims.hidden)
    rec = ol.layer_forward(dims, ol.Numerics(), "full", x, dense, experts.__getitem__, L, hist)
    hn = torch.tensor(rec.hn)
    gu = F.linear(hn, torch.tensor(experts[0]["wgu"]))
    mlp = F.linear(F.silu(gu[:, :dims.inter]) * gu[:, dims.inter:], torch.tensor(experts[0]["wd"])).numpy()
    np.testing.assert_allclose(rec.x_next, rec.h + mlp, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(rec.weights, 1.0)


def test_zero_gate_gives_identity_moe_and_doubling_down_doubles_term():
    dims = _tiny()
    B, L = 4, [3, 7, 1, 6]
    x = rnd(np.random.default_rng(10), B, dims.hidden)
    outs = []
    for gz, mult in ((True, 1.0), (False, 1.0), (False, 2.0)):
        rng = np.random.default_rng(11)
        dense, experts = _params(dims, rng, gate_zero=gz, wd_mult=mult)
        _, _, hist = _history(dims, rng, B, 8)
        outs.append(ol.layer_forward(dims, ol.Numerics(), "full", x, dense, experts.__getitem__, L, hist))
    np.testing.assert_array_equal(outs[0].x_next, outs[0].h)
    np.testing.assert_allclose(outs[2].x_next - outs[2].h, 2 * (outs[1].x_next - outs[1].h), rtol=1e-13, atol=1e-14)


# ----------------------------------------------------------------------------- whole layer
# Pure-Python roundings of the stored formats, written from the format
# definitions (not from oracle.numerics): a value's significand is taken from
# math.frexp and rounded with Python's round(), which breaks ties to even.
def py_bf16(v):
    """bfloat16: 8 significant bits, fp32's exponent range (normal inputs)."""
    if v == 0.0:
        return 0.0
    m, e = math.frexp(v)                 # v = m * 2^e, 0.5 <= |m| < 1
    return round(m * 256.0) * 2.0 ** (e - 8)


def py_e4m3(v):
    """OCP E4M3 (|v| <= 448): 4 significant bits for normals (leading-bit
    exponent >= -6), a fixed quantum of 2^-9 below that."""
    if v == 0.0:
        return 0.0
    _, e = math.frexp(abs(v))
    lead = max(e - 1, -6)                # exponent of the leading bit, clamped at the subnormal range
    q = 2.0 ** (lead - 3)
    return math.copysign(round(abs(v) / q) * q, v)


def py_pow2_scale(amax):
    """Smallest power of two s with amax <= 448 s (1 for an all-zero row)."""
    if amax == 0.0:
        return 1.0
    s = 1.0
    while amax > 448.0 * s:
        s *= 2.0
    while amax <= 448.0 * s / 2.0:
        s /= 2.0
    return s


def py_e4m3_row(row):
    """A row stored as E4M3 codes times one power-of-two scale."""
    s = py_pow2_scale(max(abs(v) for v in row))
    return [py_e4m3(v / s) * s for v in row]


def py_e4m3_decode(code):
    """Value of an OCP E4M3 byte: sign, 4 exponent bits (bias 7), 3 mantissa bits."""
    sign = -1.0 if code & 0x80 else 1.0
    ex, man = (code >> 3) & 15, code & 7
    if ex == 0:
        return sign * man * 2.0 ** -9
    return sign * (1.0 + man / 8.0) * 2.0 ** (ex - 7)


IDENT = lambda row: list(row)
QUANT = {
    "pure": {"act": IDENT, "kv": IDENT, "ex": IDENT},
    "bf16": {"act": lambda r: [py_bf16(v) for v in r], "kv": lambda r: [py_bf16(v) for v in r],
             "ex": lambda r: [py_bf16(v) for v in r]},
    "e4m3": {"act": lambda r: [py_bf16(v) for v in r], "kv": lambda r: [py_bf16(v) for v in r],
             "ex": py_e4m3_row},
}
NUMERICS = {"pure": ol.Numerics(), "bf16": ol.Numerics("bf16", "bf16", "bf16"),
            "e4m3": ol.Numerics("bf16", "bf16", "e4m3")}


def brute_expert(ew, I, H):
    """An expert's (wgu, wd) as nested lists: given values, or E4M3 codes times
    the scale of their output channel (the matrix row)."""
    if "wgu_codes" in ew:
        return ([[py_e4m3_decode(int(ew["wgu_codes"][j][i])) * float(ew["wgu_scale"][j]) for i in range(H)]
                 for j in range(2 * I)],
                [[py_e4m3_decode(int(ew["wd_codes"][i][j])) * float(ew["wd_scale"][i]) for j in range(I)]
                 for i in range(H)])
    return [list(map(float, r)) for r in ew["wgu"]], [list(map(float, r)) for r in ew["wd"]]


def brute_layer(dims, kind, x, dense, experts, L, Kh, Vh, quant="pure"):
    """Pure-Python loops over every index of the layer (float64). With
    dims.rope_theta > 0 the q heads and the new k heads are turned pair by
    pair at position L - 1 (RoFormer's rotary embedding). `quant` names the
    stored formats: "pure" (none), "bf16" (xn, q, the new K/V, o, the expert
    input hn and z rounded to bf16) or "e4m3" (as bf16, but hn and z stored as
    per-row power-of-two-scaled E4M3; experts given as E4M3 codes and
    per-output-channel scales)."""
    qa, qk, qe = QUANT[quant]["act"], QUANT[quant]["kv"], QUANT[quant]["ex"]
    H, Hq, Hkv, D, I = dims.hidden, dims.n_q_heads, dims.n_kv_heads, dims.head_dim, dims.inter
    G = Hq // Hkv
    ex_w = {e: brute_expert(experts[e], I, H) for e in experts}
    out = []
    for b in range(len(x)):
        xb = [float(v) for v in x[b]]
        ms = sum(v * v for v in xb) / H
        xn = qa([xb[i] * dense["gamma1"][i] / math.sqrt(ms + dims.eps) for i in range(H)])
        qkv = [sum(xn[i] * dense["wqkv"][r][i] for i in range(H)) for r in range((Hq + 2 * Hkv) * D)]
        if dims.rope_theta > 0:
            for head in range(Hq + Hkv):          # q heads, then k heads
                for i in range(D // 2):
                    ang = (L[b] - 1) / dims.rope_theta ** (2 * i / D)
                    u, v = qkv[head * D + 2 * i], qkv[head * D + 2 * i + 1]
                    qkv[head * D + 2 * i] = u * math.cos(ang) - v * math.sin(ang)
                    qkv[head * D + 2 * i + 1] = u * math.sin(ang) + v * math.cos(ang)
        qkv = qa(qkv[:Hq * D]) + qk(qkv[Hq * D:])   # q as the attention input, new K/V as stored
        lo = 0 if kind == "full" else max(0, L[b] - dims.window)
        att = []
        for hq in range(Hq):
            g = hq // G
            qv = qkv[hq * D:(hq + 1) * D]
            keys, vals = [], []
            for pos in range(lo, L[b]):
                if pos == L[b] - 1:
                    keys.append(qkv[(Hq + g) * D:(Hq + g + 1) * D])
                    vals.append(qkv[(Hq + Hkv + g) * D:(Hq + Hkv + g + 1) * D])
                else:
                    keys.append(list(Kh[b][g][pos]))
                    vals.append(list(Vh[b][g][pos]))
            sc = [sum(qv[d] * kk[d] for d in range(D)) / math.sqrt(D) for kk in keys]
            M = max([dense["sinks"][hq]] + sc)
            ex = [math.exp(s - M) for s in sc]
            Z = math.exp(dense["sinks"][hq] - M) + sum(ex)
            att += [sum(ex[j] * vals[j][d] for j in range(len(vals))) / Z for d in range(D)]
        att = qa(att)
        hb = [xb[i] + sum(att[j] * dense["wo"][i][j] for j in range(Hq * D)) for i in range(H)]
        ms2 = sum(v * v for v in hb) / H
        hn = [hb[i] * dense["gamma2"][i] / math.sqrt(ms2 + dims.eps) for i in range(H)]
        logits = [sum(hn[i] * dense["wr"][e][i] for i in range(H)) for e in range(dims.n_experts)]
        ranked = sorted(range(dims.n_experts), key=lambda e: (-np.float32(logits[e]), e))[:dims.top_k]
        mx = max(logits[t] for t in ranked)
        wsum = sum(math.exp(logits[t] - mx) for t in ranked)
        hx = qe(hn)                               # the experts' input row
        res = list(hb)
        for t in ranked:
            wgu, wd = ex_w[t % dims.n_resident]
            z = []
            for j in range(I):
                gte = sum(hx[i] * wgu[j][i] for i in range(H))
                up = sum(hx[i] * wgu[I + j][i] for i in range(H))
                z.append(gte / (1 + math.exp(-gte)) * up)
            z = qe(z)
            wt = math.exp(logits[t] - mx) / wsum
            for i in range(H):
                res[i] += wt * sum(z[j] * wd[i][j] for j in range(I))
        out.append(res)
    return np.array(out)


@pytest.mark.parametrize("kind,E_res,theta", [("full", 8, 0.0), ("sliding", 8, 0.0), ("sliding", 3, 0.0),
                                                ("full", 8, 10000.0), ("sliding", 3, 500.0)])
def test_layer_matches_brute_force(kind, E_res, theta):
    dims = dataclasses.replace(_tiny(E_res=E_res), rope_theta=theta)
    rng = np.random.default_rng(12)
    dense, experts = _params(dims, rng)
    B, L = 3, [9, 4, 6]
    Kh, Vh, hist = _history(dims, rng, B, 10)
    x = rnd(rng, B, dims.hidden)
    rec = ol.layer_forward(dims, ol.Numerics(), kind, x, dense, experts.__getitem__, L, hist)
    np.testing.assert_allclose(rec.x_next, brute_layer(dims, kind, x, dense, experts, L, Kh, Vh),
                               rtol=1e-11, atol=1e-11)


def _e4m3_table():
    """E4M3-exact value -> code, for every non-NaN code (pure-Python decode)."""
    return {py_e4m3_decode(c): c for c in range(256) if (c & 0x7F) != 0x7F}


def _to_e4m3_expert(ew, rng):
    """Quantise an expert's float matrices per output channel (row): scale =
    a random positive value near amax / 448, codes of the nearest E4M3 value
    of w / scale (saturated). Distinct scales per row, so a scale applied
    along the wrong axis changes the result."""
    table = _e4m3_table()
    out = {}
    for name in ("wgu", "wd"):
        w = np.asarray(ew[name], np.float64)
        sc = np.max(np.abs(w), axis=1) / 448.0 * rng.uniform(0.6, 1.0, w.shape[0])
        codes = np.empty(w.shape, np.uint8)
        for r in range(w.shape[0]):
            for c in range(w.shape[1]):
                v = max(-448.0, min(448.0, w[r, c] / sc[r]))
                codes[r, c] = table[py_e4m3(v)]
        out[name + "_codes"] = codes
        out[name + "_scale"] = sc.astype(np.float32)
    return out


@pytest.mark.parametrize("quant,kind,E_res,theta", [("bf16", "full", 8, 0.0), ("bf16", "sliding", 3, 500.0),
                                                     ("e4m3", "full", 8, 0.0), ("e4m3", "sliding", 3, 10000.0)])
def test_quantised_layer_matches_brute_force(quant, kind, E_res, theta):
    """The mirrored rounding points (bf16 xn, q, new K/V, o, hn, z; or E4M3
    hn and z with power-of-two row scales and E4M3 expert weights with
    per-channel scales) against the pure-Python loops with their own
    roundings."""
    dims = dataclasses.replace(_tiny(E_res=E_res), rope_theta=theta)
    rng = np.random.default_rng(21)
    dense, experts = _params(dims, rng)
    if quant == "e4m3":
        experts = {e: _to_e4m3_expert(ew, rng) for e, ew in experts.items()}
    B, L = 3, [9, 4, 6]
    Kh, Vh, hist = _history(dims, rng, B, 10)
    x = rnd(rng, B, dims.hidden)
    rec = ol.layer_forward(dims, NUMERICS[quant], kind, x, dense, experts.__getitem__, L, hist)
    ref = brute_layer(dims, kind, x, dense, experts, L, Kh, Vh, quant)
    np.testing.assert_allclose(rec.x_next, ref, rtol=1e-11, atol=1e-11)
    # the rounding points matter at this size: without them the layer is measurably different
    pure = brute_layer(dims, kind, x, dense, experts, L, Kh, Vh, "pure")
    assert np.max(np.abs(pure - ref)) > 1e-6 * np.max(np.abs(ref))


def test_e4m3_expert_dequantisation_uses_the_output_channel_scale():
    """wgu [2I][H] and wd [H][I] (non-square): element (n, k) is the code's
    value times the scale of output channel n."""
    rng = np.random.default_rng(22)
    I, H = 5, 7
    ew = {"wgu_codes": rng.integers(0, 0x7F, (2 * I, H)).astype(np.uint8),
          "wgu_scale": rng.uniform(0.5, 4.0, 2 * I).astype(np.float32),
          "wd_codes": rng.integers(0x80, 0xFF, (H, I)).astype(np.uint8),
          "wd_scale": rng.uniform(0.5, 4.0, H).astype(np.float32)}
    wgu, wd = ol.expert_matrices(ew)
    bgu, bd = brute_expert(ew, I, H)
    np.testing.assert_array_equal(wgu, np.array(bgu))
    np.testing.assert_array_equal(wd, np.array(bd))


def test_e4m3_scale_one_equals_plain_weights_and_pow2_down_scale_is_exact():
    """Codes with scale 1 are the code values themselves: the layer equals the
    same layer given those values as plain weights, bit for bit. Doubling every
    down-projection scale doubles the MoE term exactly (z does not depend on it)."""
    dims = _tiny()
    rng = np.random.default_rng(23)
    dense, experts = _params(dims, rng)
    q = {e: _to_e4m3_expert({k: v / 448.0 for k, v in ew.items()}, rng) for e, ew in experts.items()}
    one = {e: dict(ew, wgu_scale=np.ones_like(ew["wgu_scale"]), wd_scale=np.ones_like(ew["wd_scale"]))
           for e, ew in q.items()}
    plain = {e: {"wgu": np.array([[py_e4m3_decode(int(c)) for c in r] for r in ew["wgu_codes"]]),
                 "wd": np.array([[py_e4m3_decode(int(c)) for c in r] for r in ew["wd_codes"]])}
             for e, ew in q.items()}
    dbl = {e: dict(ew, wd_scale=2 * ew["wd_scale"]) for e, ew in q.items()}
    _, _, hist = _history(dims, rng, 3, 10)
    x = rnd(rng, 3, dims.hidden)
    run = lambda ex: ol.layer_forward(dims, NUMERICS["e4m3"], "full", x, dense, ex.__getitem__, [9, 4, 6], hist)
    a, b = run(one), run(plain)
    np.testing.assert_array_equal(a.x_next, b.x_next)
    c, d = run(q), run(dbl)
    np.testing.assert_array_equal(d.y, 2 * c.y)
    np.testing.assert_array_equal(d.weights, c.weights)


def test_oracle_roundings_match_pure_python():
    """oracle.numerics against the pure-Python roundings above, ties included."""
    from oracle.numerics import quant_rows_pow2_e4m3, round_e4m3
    rng = np.random.default_rng(24)
    v = np.concatenate([rng.standard_normal(3000) * 10.0 ** rng.uniform(-6, 2, 3000),
                        (np.arange(1, 600) + 0.5) * 2.0 ** -16,          # halfway points (bf16 ties)
                        [1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8)]])
    np.testing.assert_array_equal(round_bf16(v), [py_bf16(float(t)) for t in v])
    w = np.concatenate([rng.uniform(-448, 448, 2000), rng.standard_normal(2000) * 2.0 ** -8,
                        (np.arange(1, 64) + 0.5) * 2.0 ** -9, [1.0625, 1.1875, 3.0 * 2 ** -10, 416.0 + 16.0]])
    np.testing.assert_array_equal(round_e4m3(w), [py_e4m3(float(t)) for t in w])
    rows = rng.standard_normal((40, 33)) * 10.0 ** rng.uniform(-5, 5, (40, 1))
    rows[3] = 0.0
    rows[4, 0] = 448.0 * 2.0 ** -7        # amax exactly at a power-of-two boundary
    got, sc = quant_rows_pow2_e4m3(rows)
    np.testing.assert_array_equal(got, [py_e4m3_row(list(r)) for r in rows])
    np.testing.assert_array_equal(sc, [py_pow2_scale(float(np.max(np.abs(r)))) for r in rows])


def test_sliding_with_wide_window_equals_full():
    dims = _tiny(W=64)
    rng = np.random.default_rng(13)
    dense, experts = _params(dims, rng)
    _, _, hist = _history(dims, rng, 2, 10)
    x = rnd(rng, 2, dims.hidden)
    a = ol.layer_forward(dims, ol.Numerics(), "sliding", x, dense, experts.__getitem__, [9, 3], hist)
    b = ol.layer_forward(dims, ol.Numerics(), "full", x, dense, experts.__getitem__, [9, 3], hist)
    np.testing.assert_array_equal(a.x_next, b.x_next)


def test_token_permutation_equivariance_and_subset_independence():
    dims = _tiny()
    rng = np.random.default_rng(14)
    dense, experts = _params(dims, rng)
    B = 5
    L = [3, 8, 6, 1, 5]
    Kh, Vh, _ = _history(dims, rng, B, 9)
    x = rnd(rng, B, dims.hidden)

    def run(order):
        hist = lambda b, lo, hi: (Kh[order[b]][:, lo:hi], Vh[order[b]][:, lo:hi])
        return ol.layer_forward(dims, ol.Numerics("bf16", "bf16", "bf16"), "sliding", x[order], dense,
                                experts.__getitem__, [L[i] for i in order], hist)

    full = run(list(range(B)))
    perm = [3, 0, 4, 1, 2]
    pr = run(perm)
    # BLAS may block a product differently for another row count: equal up to rounding
    np.testing.assert_allclose(pr.x_next, full.x_next[perm], rtol=1e-12, atol=1e-13)
    np.testing.assert_array_equal(pr.topk, full.topk[perm])
    sub = run([4, 1])
    np.testing.assert_allclose(sub.x_next, full.x_next[[4, 1]], rtol=1e-12, atol=1e-13)
    np.testing.assert_array_equal(sub.topk, full.topk[[4, 1]])


def test_bf16_mirror_points_round_the_stored_tensors():
    dims = _tiny()
    rng = np.random.default_rng(15)
    dense, experts = _params(dims, rng)
    _, _, hist = _history(dims, rng, 2, 10)
    x = rnd(rng, 2, dims.hidden)
    rec = ol.layer_forward(dims, ol.Numerics("bf16", "bf16", "bf16"), "full", x, dense, experts.__getitem__,
                           [9, 3], hist)
    for t in (rec.q, rec.k_new, rec.v_new):
        np.testing.assert_array_equal(round_bf16(t), t)
    pure = ol.layer_forward(dims, ol.Numerics(), "full", x, dense, experts.__getitem__, [9, 3], hist)
    rms = np.sqrt(np.mean(pure.x_next ** 2))
    err = np.max(np.abs(rec.x_next - pure.x_next))
    assert 0 < err < 2e-2 * rms
