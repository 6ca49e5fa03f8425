"""The decode layer, one operator at a time, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Follows the operator list of one MoE transformer layer in Figure 3 of the
SubGPU Pipelining paper (RMSNorm, Q/KV projections, attention, output
projection, Add+Norm, router gating, top-k dispatch, expert up, SwiGLU,
expert down, combine) and its section 5.1 statement that GPT-OSS layers
alternate between sliding-window and full attention. The pages give the
operator names but not their formulas; the readings taken here are:

  * pre-norm residual block: xn = RMSNorm(x); h = x + Attn(xn) Wo^T;
    hn = RMSNorm(h); x' = h + MoE(hn); RMSNorm(v) = v * gamma / sqrt(mean(v^2) + eps);
  * RoPE (listed in Figure 3) is optional (Dims.rope_theta > 0): the
    rotary embedding of the original RoFormer formulation, adjacent pairs
    (2i, 2i+1) of a head turned by pos * theta^(-2i/D), applied to q and to
    the new k at the decoded position L-1 before they are stored; the cache
    holds keys already rotated at their own positions, which for the
    synthetic history means the generated values are taken as rotated keys.
    rope_theta = 0 leaves it out;
  * grouped-query attention with contiguous groups: query head h reads KV
    head h // (Hq / Hkv); scores scaled by 1/sqrt(D);
  * one learned sink logit per query head joins the softmax denominator and
    has no value vector;
  * the sliding window holds the last W positions including the new token
    (all of them when L <= W);
  * router: fp32 logits of an unbiased linear map; top-k ordered by logit,
    ties to the lower expert index; weights = softmax over the k picks;
  * expert pick t runs on resident expert t mod E_res (the identity when all
    experts are resident);
  * SwiGLU: z = silu(gate) * up, gate rows 0..I-1 and up rows I..2I-1 of the
    expert's first matrix, no biases; silu(v) = v / (1 + exp(-v));
  * combine: x' = h + sum over the k picks, in pick order, of w * y.

Quantisation points: the stored formats round a value where the method hands
a tensor to a matrix product or to the KV cache. With `Numerics.act == "bf16"`
xn, q, the new K/V, o, hn (expert input) and z are rounded to bf16; with
`expert_act == "e4m3"` the expert inputs hn and z are instead per-row
power-of-two-scaled E4M3. Everything else is float64.
"""
from __future__ import annotations

import dataclasses
from typing import Callable, Dict, List, Optional, Sequence, Tuple

import numpy as np

from .numerics import e4m3_decode, quant_rows_pow2_e4m3, round_bf16


@dataclasses.dataclass(frozen=True)
class Dims:
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    n_experts: int
    n_resident: int
    top_k: int
    inter: int
    window: int
    eps: float = 1e-5
    rope_theta: float = 0.0    # 0: no rotary embedding


@dataclasses.dataclass(frozen=True)
class Numerics:
    act: str = "none"          # "none" | "bf16": dense-product inputs, q, o
    kv: str = "none"           # "none" | "bf16": stored K/V of the new token
    expert_act: str = "none"   # "none" | "bf16" | "e4m3": expert inputs hn and z


def _q(a, mode: str):
    if mode == "none":
        return np.asarray(a, np.float64)
    if mode == "bf16":
        return round_bf16(a)
    if mode == "e4m3":
        return quant_rows_pow2_e4m3(a)[0]
    raise ValueError(mode)


# --------------------------------------------------------------------------
# operators
# --------------------------------------------------------------------------
def rmsnorm(x, gamma, eps: float) -> np.ndarray:
    """Figure 3 "RMSNorm" / "Add+Norm": v * gamma / sqrt(mean(v^2) + eps), per row."""
    x = np.asarray(x, np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x * np.asarray(gamma, np.float64) / np.sqrt(ms + eps)


def linear(x, w) -> np.ndarray:
    """y = x W^T with W stored [out][in] (Figure 3 "Q proj", "KV proj", "Output proj")."""
    return np.asarray(x, np.float64) @ np.asarray(w, np.float64).T


def rope(x, pos: int, theta: float) -> np.ndarray:
    """Figure 3 "RoPE" on the last axis of x (length D, even): the pair
    (x[2i], x[2i+1]) is turned by the angle pos * theta^(-2i/D):
      out[2i]   = x[2i] cos(a) - x[2i+1] sin(a)
      out[2i+1] = x[2i] sin(a) + x[2i+1] cos(a)."""
    x = np.asarray(x, np.float64)
    D = x.shape[-1]
    i = np.arange(D // 2, dtype=np.float64)
    a = float(pos) * np.power(float(theta), -2.0 * i / D)
    c, s = np.cos(a), np.sin(a)
    out = np.empty_like(x)
    out[..., 0::2] = x[..., 0::2] * c - x[..., 1::2] * s
    out[..., 1::2] = x[..., 0::2] * s + x[..., 1::2] * c
    return out


def attention_window(kind: str, L: int, window: int) -> Tuple[int, int]:
    """Positions [lo, L) the decoded token attends to (section 5.1: sliding or full)."""
    if kind == "sliding":
        return max(0, L - window), L
    if kind == "full":
        return 0, L
    raise ValueError(kind)


def decode_attention(q, K, V, sinks, scale: float):
    """Figure 3 "FMHA" for one decoded token, grouped-query, with sinks.

    q [Hq][D]; K, V [Hkv][n][D] (the attended positions); sinks [Hq].
    For head h of group g = h // (Hq/Hkv):
      s_j = scale * q_h . K[g, j];  M = max(sink_h, max_j s_j);
      Z = exp(sink_h - M) + sum_j exp(s_j - M);  p_j = exp(s_j - M) / Z;
      o_h = sum_j p_j V[g, j];  p_sink_h = exp(sink_h - M) / Z.
    Returns (o [Hq][D], p [Hq][n], p_sink [Hq]) in float64 (two passes).
    """
    q = np.asarray(q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    Hq, D = q.shape
    Hkv, n, _ = K.shape
    G = Hq // Hkv
    o = np.empty((Hq, D))
    p_all = np.empty((Hq, n))
    p_sink = np.empty(Hq)
    for h in range(Hq):
        g = h // G
        s = scale * (K[g] @ q[h])
        sink = float(sinks[h])
        M = max(sink, float(s.max())) if n else sink
        e = np.exp(s - M)
        es = np.exp(sink - M)
        Z = es + e.sum()
        p_all[h] = e / Z
        p_sink[h] = es / Z
        o[h] = p_all[h] @ V[g]
    return o, p_all, p_sink


def router_topk(logits32, k: int):
    """Figure 3 "Router gating" + "TopK dispatch" for one token.

    Selection is decided on the fp32 logits: the k largest, ordered by value
    descending, ties to the lower index. Returns (indices, margin) where margin
    is the gap between the k-th and (k+1)-th largest logit (inf when k == E).
    """
    l = np.asarray(logits32, np.float32)
    order = sorted(range(l.shape[0]), key=lambda i: (-float(l[i]), i))
    idx = np.array(order[:k], np.int64)
    margin = float(l[order[k - 1]]) - float(l[order[k]]) if k < l.shape[0] else float("inf")
    return idx, margin


def route_weights(logits64, idx) -> np.ndarray:
    """Softmax over the selected logits: w_t = exp(l_t - l_max) / sum_u exp(l_u - l_max)."""
    sel = np.asarray(logits64, np.float64)[np.asarray(idx)]
    e = np.exp(sel - sel.max())
    return e / e.sum()


def permutation(groups, n_groups: int):
    """Token->expert dispatch order (Figure 3 "TopK dispatch").

    groups [B][k]: the resident expert of each (token, pick). Rows are grouped
    by expert, and inside an expert ordered by (token, pick) ascending.
    Returns counts [n_groups], offsets [n_groups+1], row_tok [R], row_slot [R]
    and inv [B][k] (the row holding each (token, pick)).
    """
    g = np.asarray(groups, np.int64)
    B, k = g.shape
    flat = g.reshape(-1)
    counts = np.bincount(flat, minlength=n_groups).astype(np.int64)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    order = np.argsort(flat, kind="stable")       # stable: keeps (token, pick) order
    row_tok = order // k
    row_slot = order % k
    inv = np.empty(B * k, np.int64)
    inv[order] = np.arange(B * k)
    return counts, offsets, row_tok, row_slot, inv.reshape(B, k)


def silu(v) -> np.ndarray:
    v = np.asarray(v, np.float64)
    return v / (1.0 + np.exp(-v))


def expert_swiglu(xq, wgu, wd, inter: int, z_mode: str):
    """Figure 3 "Expert up (BMM)", "SwiGLU", "Expert down" for rows of one expert.

    xq [R][H] (already at the expert-input format); wgu [2I][H]; wd [H][I].
    g = xq Wg^T, u = xq Wu^T, z = silu(g) * u, y = Q(z) Wd^T. Returns (y, z).
    """
    gu = linear(xq, wgu)
    z = silu(gu[:, :inter]) * gu[:, inter:]
    y = linear(_q(z, z_mode), wd)
    return y, z


def expert_matrices(ew: Dict[str, np.ndarray]):
    """Dequantised (wgu, wd) of one expert: bf16/fp32 values as given, or
    E4M3 code value times its output channel's fp32 scale."""
    if "wgu_codes" in ew:
        wgu = e4m3_decode(ew["wgu_codes"]) * np.asarray(ew["wgu_scale"], np.float64)[:, None]
        wd = e4m3_decode(ew["wd_codes"]) * np.asarray(ew["wd_scale"], np.float64)[:, None]
        return wgu, wd
    return np.asarray(ew["wgu"], np.float64), np.asarray(ew["wd"], np.float64)


# --------------------------------------------------------------------------
# the layer
# --------------------------------------------------------------------------
@dataclasses.dataclass
class LayerRecord:
    xn: np.ndarray
    q: np.ndarray
    k_new: np.ndarray
    v_new: np.ndarray
    o: np.ndarray
    p_sink: np.ndarray
    h: np.ndarray
    hn: np.ndarray
    logits: np.ndarray        # float64
    logits32: np.ndarray
    topk: np.ndarray          # [B][k] router picks (0..E-1)
    weights: np.ndarray       # [B][k]
    margin: np.ndarray        # [B]
    groups: np.ndarray        # [B][k] resident expert per pick
    y: np.ndarray             # [B][k][H]
    x_next: np.ndarray


def layer_forward(dims: Dims, num: Numerics, kind: str, x, dense: Dict[str, np.ndarray],
                  expert: Callable[[int], Dict[str, np.ndarray]], L: Sequence[int],
                  history: Callable[[int, int, int], Tuple[np.ndarray, np.ndarray]]) -> LayerRecord:
    """One decode step of one layer for a batch of tokens.

    x [B][H]: residual rows. dense: wqkv, wo, wr, sinks, gamma1, gamma2.
    expert(e): weights of resident expert e. L[b]: sequence length including
    the decoded token (its new K/V lands at position L[b]-1). history(b, lo, hi)
    returns the cached K, V [Hkv][hi-lo][D] of positions [lo, hi).
    """
    H, Hq, Hkv, D = dims.hidden, dims.n_q_heads, dims.n_kv_heads, dims.head_dim
    x = np.asarray(x, np.float64)
    B = x.shape[0]

    # Norm + QKV (RMSNorm, Q proj, KV proj) [+ RoPE of q and the new k at L-1]
    xn = rmsnorm(x, dense["gamma1"], dims.eps)
    qkv = linear(_q(xn, num.act), dense["wqkv"])
    q = qkv[:, : Hq * D].reshape(B, Hq, D)
    k_new = qkv[:, Hq * D: (Hq + Hkv) * D].reshape(B, Hkv, D)
    if dims.rope_theta > 0:
        q = np.stack([rope(q[b], int(L[b]) - 1, dims.rope_theta) for b in range(B)])
        k_new = np.stack([rope(k_new[b], int(L[b]) - 1, dims.rope_theta) for b in range(B)])
    q = _q(q, num.act)
    k_new = _q(k_new, num.kv)
    v_new = _q(qkv[:, (Hq + Hkv) * D:], num.kv).reshape(B, Hkv, D)

    # Attention (FMHA over the window, the new token appended at L-1)
    o = np.empty((B, Hq, D))
    p_sink = np.empty((B, Hq))
    for b in range(B):
        lo, hi = attention_window(kind, int(L[b]), dims.window)
        Kh, Vh = history(b, lo, hi - 1)
        Kb = np.concatenate([np.asarray(Kh, np.float64), k_new[b][:, None, :]], axis=1)
        Vb = np.concatenate([np.asarray(Vh, np.float64), v_new[b][:, None, :]], axis=1)
        o[b], _, p_sink[b] = decode_attention(q[b], Kb, Vb, dense["sinks"], 1.0 / np.sqrt(D))

    # Output proj + Add + Norm
    h = x + linear(_q(o.reshape(B, Hq * D), num.act), dense["wo"])
    hn = rmsnorm(h, dense["gamma2"], dims.eps)

    # Router gating + TopK
    logits = linear(hn, dense["wr"])
    logits32 = logits.astype(np.float32)
    k = dims.top_k
    topk = np.empty((B, k), np.int64)
    weights = np.empty((B, k))
    margin = np.empty(B)
    for b in range(B):
        topk[b], margin[b] = router_topk(logits32[b], k)
        weights[b] = route_weights(logits[b], topk[b])
    groups = topk % dims.n_resident

    # Experts (grouped by resident expert) + combine
    hq = _q(hn, num.expert_act)
    y = np.zeros((B, k, H))
    for e in np.unique(groups):
        sel = np.argwhere(groups == e)                 # (token, pick) pairs in order
        wgu, wd = expert_matrices(expert(int(e)))
        ye, _ = expert_swiglu(hq[sel[:, 0]], wgu, wd, dims.inter, num.expert_act)
        y[sel[:, 0], sel[:, 1]] = ye
    x_next = h.copy()
    for s in range(k):
        x_next += weights[:, s: s + 1] * y[:, s]
    return LayerRecord(xn, q, k_new, v_new, o, p_sink, h, hn, logits, logits32, topk, weights,
                       margin, groups, y, x_next)


def iteration_forward(dims: Dims, num: Numerics, kinds: Sequence[str], x,
                      layer_params: Callable[[int], Tuple[Dict, Callable]], L: Sequence[int],
                      history: Callable[[int, int, int, int], Tuple[np.ndarray, np.ndarray]],
                      keep_records: bool = False):
    """A decode iteration: the layers in order, each on the previous one's output.

    layer_params(l) -> (dense, expert) for layer l; history(l, b, lo, hi).
    Returns (x after the last layer, per-layer top-k picks [n_layers][B][k],
    per-layer margins [n_layers][B], records if keep_records).
    """
    x = np.asarray(x, np.float64)
    picks, margins, recs = [], [], []
    for l, kind in enumerate(kinds):
        dense, expert = layer_params(l)
        rec = layer_forward(dims, num, kind, x, dense, expert, L,
                            lambda b, lo, hi, _l=l: history(_l, b, lo, hi))
        picks.append(rec.topk)
        margins.append(rec.margin)
        if keep_records:
            recs.append(rec)
        x = rec.x_next
    return x, np.array(picks), np.array(margins), recs
