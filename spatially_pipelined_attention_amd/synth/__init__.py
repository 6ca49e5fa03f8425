"""Seeded synthetic inputs for the spatially pipelined MoE decode layer.

This module is shared by the tests, the benchmark and the CPU reference: it
holds the workload shapes and the counter-based generator, and none of the
layer's arithmetic. Every element of every input tensor is a pure function of
(seed, tensor tag, layer, sub-stream, element index), so any slice can be
regenerated on its own, on the host (gen_host.c) or in HBM (gen_dev.hip),
with identical bits.

Value recipe (shapes follow the GPT-OSS-style decode layer used in the
SubGPU Pipelining paper's evaluation, section 5.1, one MoE transformer layer
as drawn in its Figure 3):
  * residual stream x: N(0, 1);
  * dense and expert matrices: N(0, 0.02^2), rounded to bf16 unless fp32;
  * router matrix (fp32): N(0, 1/H), so router logits are roughly N(0, 1)
    for a unit-RMS normalised input (N(0, 0.02^2) for the tiny fp32 case);
  * attention sink logits: N(0, 1), one per query head, fp32;
  * KV history: N(0, 1), rounded to the cache dtype;
  * KV lengths: fixed, or uniform integers in [lo, hi];
  * RMSNorm gains: ones.
"N(0, s^2)" is an Irwin-Hall(4) draw scaled to variance s^2.
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
import os
from typing import Dict, List, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
HOST_LIB_PATH = os.path.join(_HERE, "libspa_synth_host.so")
DEV_LIB_PATH = os.path.join(_HERE, "libspa_synth_dev.so")

# tensor tags of the counter-based streams
TAG_X = 1
TAG_WQKV = 2
TAG_WO = 3
TAG_WR = 4
TAG_WGU = 5
TAG_WD = 6
TAG_SINK = 7
TAG_KHIST = 8
TAG_VHIST = 9
TAG_KVLEN = 10

# KV history element (b, g, pos, d) has draw index ((b*Hkv + g) << KV_POS_BITS | pos) * D + d
KV_POS_BITS = 24


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shapes, dtypes and value recipe of one synthetic decode workload."""
    name: str
    seed: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    n_experts: int          # router width E
    n_resident: int         # experts resident on this GPU (pick t -> t % n_resident)
    top_k: int
    inter: int
    window: int
    n_layers: int
    batch: int
    kv_len_lo: int          # KV length (including the token being decoded)
    kv_len_hi: int
    layer_kinds: tuple      # per layer: "sliding" or "full"
    w_dtype: str            # "f32" or "bf16" (dense + experts)
    expert_dtype: str       # "f32", "bf16" or "e4m3"
    kv_dtype: str           # "f32" or "bf16"
    w_std: float = 0.02
    router_std: Optional[float] = None   # None: 1/sqrt(hidden)
    eps: float = 1e-5
    rope_theta: float = 0.0              # rotary embedding base (0: none)

    @property
    def qkv_rows(self) -> int:
        return (self.n_q_heads + 2 * self.n_kv_heads) * self.head_dim

    @property
    def router_sigma(self) -> float:
        return self.router_std if self.router_std is not None else 1.0 / math.sqrt(self.hidden)

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


def _alternating(n_layers: int) -> tuple:
    # even layers sliding-window, odd layers full attention
    return tuple("sliding" if l % 2 == 0 else "full" for l in range(n_layers))


WORKLOADS: Dict[str, Workload] = {
    # tiny fp32 layer: correctness only
    "tiny_fp32": Workload("tiny_fp32", 1001, 256, 4, 1, 64, 8, 8, 2, 256, 128, 1, 4,
                          128, 128, ("full",), "f32", "f32", "f32", router_std=0.02),
    # one GPT-OSS-120B-shaped full-attention layer, KV 4096, 128 experts top-4
    "gptoss_layer_full": Workload("gptoss_layer_full", 1002, 2880, 64, 8, 64, 128, 128, 4, 2880,
                                  128, 1, 64, 4096, 4096, ("full",), "bf16", "bf16", "bf16"),
    # same layer, sliding window 128, batch 256 (4 microbatches of 64)
    "gptoss_layer_sliding_b256": Workload("gptoss_layer_sliding_b256", 1003, 2880, 64, 8, 64, 128,
                                          128, 4, 2880, 128, 1, 256, 4096, 4096, ("sliding",),
                                          "bf16", "bf16", "bf16"),
    # 36-layer iteration, one GPU's share: 64 sequences, KV U[1024, 8192], 4 resident experts
    "gptoss_36l_b64": Workload("gptoss_36l_b64", 1004, 2880, 64, 8, 64, 128, 4, 4, 2880, 128, 36,
                               64, 1024, 8192, _alternating(36), "bf16", "bf16", "bf16"),
    # the same with fp8 e4m3 experts (per-output-channel fp32 scale)
    "gptoss_36l_fp8": Workload("gptoss_36l_fp8", 1005, 2880, 64, 8, 64, 128, 4, 4, 2880, 128, 36,
                               64, 1024, 8192, _alternating(36), "bf16", "e4m3", "bf16"),
    # the SubGPU Pipelining paper's own shape (section 5.1: KV history 32,768):
    # every sequence at 32,768 positions, otherwise the 36-layer share above
    "gptoss_36l_kv32k": Workload("gptoss_36l_kv32k", 1006, 2880, 64, 8, 64, 128, 4, 4, 2880, 128, 36,
                                 64, 32768, 32768, _alternating(36), "bf16", "bf16", "bf16"),
    # the 36-layer one-GPU share with the rotary embedding of Figure 3 (base 10000)
    "gptoss_36l_b64_rope": Workload("gptoss_36l_b64_rope", 1007, 2880, 64, 8, 64, 128, 4, 4, 2880, 128, 36,
                                    64, 1024, 8192, _alternating(36), "bf16", "bf16", "bf16", rope_theta=10000.0),
}


# ----------------------------------------------------------------------------
# host generator (ctypes over gen_host.c)
# ----------------------------------------------------------------------------
_host = None


def host_lib():
    global _host
    if _host is None:
        if not os.path.exists(HOST_LIB_PATH):
            raise RuntimeError(f"{HOST_LIB_PATH} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(HOST_LIB_PATH)
        lib.spa_gen_stream_key.restype = ctypes.c_uint64
        lib.spa_gen_stream_key.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32]
        lib.spa_gen_normal_scale.restype = ctypes.c_float
        lib.spa_gen_normal_scale.argtypes = [ctypes.c_double]
        vp, i64, u64, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64, ctypes.c_float
        lib.spa_gen_normal_f32.argtypes = [vp, i64, u64, i64, f32]
        lib.spa_gen_normal_bf16.argtypes = [vp, i64, u64, i64, f32]
        lib.spa_gen_uniform_int.argtypes = [vp, i64, u64, i64, ctypes.c_int32, ctypes.c_int32]
        lib.spa_quant_rows_e4m3.argtypes = [vp, i64, i64, vp, vp]
        lib.spa_e4m3_decode.argtypes = [vp, i64, vp]
        _host = lib
    return _host


def stream_key(seed: int, tag: int, layer: int = 0, sub: int = 0) -> int:
    return int(host_lib().spa_gen_stream_key(seed, tag, layer, sub))


def normal_scale(std: float) -> float:
    return float(host_lib().spa_gen_normal_scale(std))


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def normal_f32(n: int, key: int, i0: int, std: float) -> np.ndarray:
    out = np.empty(n, np.float32)
    host_lib().spa_gen_normal_f32(_ptr(out), n, key, i0, normal_scale(std))
    return out


def normal_bf16_bits(n: int, key: int, i0: int, std: float) -> np.ndarray:
    out = np.empty(n, np.uint16)
    host_lib().spa_gen_normal_bf16(_ptr(out), n, key, i0, normal_scale(std))
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32 values."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


def uniform_int(n: int, key: int, i0: int, lo: int, hi: int) -> np.ndarray:
    out = np.empty(n, np.int32)
    host_lib().spa_gen_uniform_int(_ptr(out), n, key, i0, lo, hi)
    return out


def quant_rows_e4m3(w: np.ndarray):
    """Offline per-output-channel fp8 weights: (codes uint8, scales fp32)."""
    w = np.ascontiguousarray(w, np.float32)
    rows, cols = w.reshape(-1, w.shape[-1]).shape
    codes = np.empty((rows, cols), np.uint8)
    scales = np.empty(rows, np.float32)
    host_lib().spa_quant_rows_e4m3(_ptr(w), rows, cols, _ptr(codes), _ptr(scales))
    return codes.reshape(w.shape), scales.reshape(w.shape[:-1])


# ----------------------------------------------------------------------------
# workload tensors (host, logical layouts)
# ----------------------------------------------------------------------------
def _matrix(wl: Workload, tag: int, layer: int, sub: int, rows: int, cols: int, std: float,
            dtype: str) -> np.ndarray:
    """Values of a [rows][cols] weight matrix as float32 (bf16-exact when dtype is bf16)."""
    key = stream_key(wl.seed, tag, layer, sub)
    if dtype == "f32":
        return normal_f32(rows * cols, key, 0, std).reshape(rows, cols)
    return bf16_bits_to_f32(normal_bf16_bits(rows * cols, key, 0, std)).reshape(rows, cols)


def kv_lengths(wl: Workload) -> np.ndarray:
    """L_b per sequence (the count of cached positions including the decoded token)."""
    if wl.kv_len_lo == wl.kv_len_hi:
        return np.full(wl.batch, wl.kv_len_lo, np.int32)
    return uniform_int(wl.batch, stream_key(wl.seed, TAG_KVLEN), 0, wl.kv_len_lo, wl.kv_len_hi)


def x_rows(wl: Workload, tokens: Sequence[int], resample: Optional[Dict[int, int]] = None) -> np.ndarray:
    """Initial residual rows x[b] (fp32). `resample[b]` selects a re-drawn variant of token b."""
    resample = resample or {}
    out = np.empty((len(tokens), wl.hidden), np.float32)
    for i, b in enumerate(tokens):
        key = stream_key(wl.seed, TAG_X, 0, int(resample.get(int(b), 0)))
        out[i] = normal_f32(wl.hidden, key, int(b) * wl.hidden, 1.0)
    return out


def dense_weights(wl: Workload, layer: int) -> Dict[str, np.ndarray]:
    """Per-layer dense parameters: wqkv [(Hq+2Hkv)D][H], wo [H][Hq D], wr [E][H],
    sinks [Hq], gamma1/gamma2 [H] (all float32 values)."""
    H, qd = wl.hidden, wl.n_q_heads * wl.head_dim
    return {
        "wqkv": _matrix(wl, TAG_WQKV, layer, 0, wl.qkv_rows, H, wl.w_std, wl.w_dtype),
        "wo": _matrix(wl, TAG_WO, layer, 0, H, qd, wl.w_std, wl.w_dtype),
        "wr": _matrix(wl, TAG_WR, layer, 0, wl.n_experts, H, wl.router_sigma, "f32"),
        "sinks": normal_f32(wl.n_q_heads, stream_key(wl.seed, TAG_SINK, layer), 0, 1.0),
        "gamma1": np.ones(H, np.float32),
        "gamma2": np.ones(H, np.float32),
    }


def expert_weights(wl: Workload, layer: int, e: int) -> Dict[str, np.ndarray]:
    """Resident expert e of a layer: wgu [2I][H] (rows 0..I-1 gate, I..2I-1 up), wd [H][I].
    For e4m3 experts also the codes and per-output-channel scales."""
    I, H = wl.inter, wl.hidden
    if wl.expert_dtype == "e4m3":
        gu = _matrix(wl, TAG_WGU, layer, e, 2 * I, H, wl.w_std, "f32")
        d = _matrix(wl, TAG_WD, layer, e, H, I, wl.w_std, "f32")
        gu_c, gu_s = quant_rows_e4m3(gu)
        d_c, d_s = quant_rows_e4m3(d)
        return {"wgu_codes": gu_c, "wgu_scale": gu_s, "wd_codes": d_c, "wd_scale": d_s}
    return {
        "wgu": _matrix(wl, TAG_WGU, layer, e, 2 * I, H, wl.w_std, wl.expert_dtype),
        "wd": _matrix(wl, TAG_WD, layer, e, H, I, wl.w_std, wl.expert_dtype),
    }


def kv_base_index(wl: Workload, b: int, g: int, pos0: int) -> int:
    return (((b * wl.n_kv_heads + g) << KV_POS_BITS) + pos0) * wl.head_dim


def kv_history(wl: Workload, layer: int, b: int, pos0: int, pos1: int):
    """Cached K and V of sequence b for positions [pos0, pos1): float32 arrays [Hkv][n][D]."""
    n = max(0, pos1 - pos0)
    D, G = wl.head_dim, wl.n_kv_heads
    K = np.empty((G, n, D), np.float32)
    V = np.empty((G, n, D), np.float32)
    if n == 0:
        return K, V
    for tag, out in ((TAG_KHIST, K), (TAG_VHIST, V)):
        key = stream_key(wl.seed, tag, layer)
        for g in range(G):
            i0 = kv_base_index(wl, b, g, pos0)
            if wl.kv_dtype == "f32":
                out[g] = normal_f32(n * D, key, i0, 1.0).reshape(n, D)
            else:
                out[g] = bf16_bits_to_f32(normal_bf16_bits(n * D, key, i0, 1.0)).reshape(n, D)
    return K, V


def history_range(wl: Workload, layer: int, L: int):
    """Positions of the cached history a decode step at length L can attend to
    (the newest position L-1 is produced by the step itself)."""
    if wl.layer_kinds[layer] == "sliding":
        return max(0, L - wl.window), L - 1
    return 0, L - 1


# ----------------------------------------------------------------------------
# device generator (ctypes over gen_dev.hip); needs a GPU
# ----------------------------------------------------------------------------
_dev = None


def dev_lib():
    global _dev
    if _dev is None:
        if not os.path.exists(DEV_LIB_PATH):
            raise RuntimeError(f"{DEV_LIB_PATH} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(DEV_LIB_PATH)
        vp, i64, u64, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64, ctypes.c_float
        for name in ("spa_gen_dev_normal_f32", "spa_gen_dev_normal_bf16"):
            getattr(lib, name).argtypes = [vp, i64, u64, i64, f32, vp]
            getattr(lib, name).restype = ctypes.c_int
        for name in ("spa_gen_dev_rows_bf16", "spa_gen_dev_rows_f32"):
            getattr(lib, name).argtypes = [vp, i64, i64, vp, u64, f32, vp]
            getattr(lib, name).restype = ctypes.c_int
        _dev = lib
    return _dev


def _check(rc: int, what: str):
    if rc != 0:
        raise RuntimeError(f"{what}: hip error {rc}")


def dev_fill_normal(t, key: int, i0: int, std: float, stream: int = 0):
    """Fill a contiguous torch CUDA tensor (float32 or bfloat16) with draws i0.."""
    import torch
    n = t.numel()
    if t.dtype == torch.float32:
        _check(dev_lib().spa_gen_dev_normal_f32(t.data_ptr(), n, key, i0, normal_scale(std), stream), "gen f32")
    elif t.dtype == torch.bfloat16:
        _check(dev_lib().spa_gen_dev_normal_bf16(t.data_ptr(), n, key, i0, normal_scale(std), stream), "gen bf16")
    else:
        raise TypeError(t.dtype)


def dev_fill_rows(t, bases, key: int, std: float, stream: int = 0):
    """Fill a [rows][row_len] torch CUDA tensor: row r holds draws bases[r] + c."""
    import torch
    assert t.is_contiguous() and t.dim() == 2
    b = torch.as_tensor(np.asarray(bases, np.int64)).to(t.device)
    if t.dtype == torch.float32:
        fn = dev_lib().spa_gen_dev_rows_f32
    elif t.dtype == torch.bfloat16:
        fn = dev_lib().spa_gen_dev_rows_bf16
    else:
        raise TypeError(t.dtype)
    _check(fn(t.data_ptr(), t.shape[0], t.shape[1], b.data_ptr(), key, normal_scale(std), stream), "gen rows")
    return b  # keep alive until the stream has consumed it
