"""Rounding and decoding of the narrow formats the layer stores (float64 in/out).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages fix no precision for the layer; the synthetic workloads store
weights and KV in bf16 (or fp32, or OCP E4M3 expert weights) with fp32
accumulation. These helpers give the exact value such a store holds.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def round_bf16(a) -> np.ndarray:
    """Nearest bfloat16 value of each float64 element, ties to even.

    bfloat16 keeps 8 significant bits and fp32's exponent range; inputs here
    are normal numbers in that range, so rounding the float64 significand to
    8 bits is exact RNE. Result is float64 holding the bf16 value.
    """
    a = np.ascontiguousarray(a, dtype=np.float64)
    u = a.view(np.uint64)
    drop = np.uint64(45)                      # 52 - 7 fraction bits dropped
    lsb = (u >> drop) & np.uint64(1)
    half = np.uint64((1 << 44) - 1)
    r = (u + half + lsb) & ~np.uint64((1 << 45) - 1)
    return r.view(np.float64)


def round_e4m3(a) -> np.ndarray:
    """Nearest OCP E4M3 value (bias 7, 3 mantissa bits, smallest normal 2^-6,
    subnormal quantum 2^-9), ties to even. Inputs must satisfy |a| <= 448."""
    a = np.asarray(a, dtype=np.float64)
    mag = np.abs(a)
    if np.any(mag > E4M3_MAX):
        raise ValueError("e4m3 rounding input beyond 448")
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(mag > 0, mag, 1.0)))
    e = np.maximum(e, -6.0)
    quantum = np.exp2(e - 3.0)
    return np.round(a / quantum) * quantum   # numpy rounds half to even


def e4m3_decode(codes) -> np.ndarray:
    """Value of each OCP E4M3 byte (S.EEEE.MMM); 0x7F/0xFF (NaN) map to nan."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (8 + m) * np.exp2(e - 10.0))
    v = s * mag
    return np.where((c & 0x7F) == 0x7F, np.nan, v)


def pow2_scale(amax) -> np.ndarray:
    """Smallest power of two s with amax <= 448 * s (1 where amax is 0)."""
    amax = np.asarray(amax, dtype=np.float64)
    safe = np.where(amax > 0, amax, E4M3_MAX)
    k = np.ceil(np.log2(safe / E4M3_MAX))
    # settle the boundary exactly (448 * 2^k is exact in binary floating point)
    k = np.where(safe > E4M3_MAX * np.exp2(k), k + 1, k)
    k = np.where(safe <= E4M3_MAX * np.exp2(k - 1), k - 1, k)
    return np.where(amax > 0, np.exp2(k), 1.0)


def quant_rows_pow2_e4m3(a):
    """Per-row fp8 activation: s = pow2_scale(max |row|), value = s * E4M3(row / s).
    Dividing by a power of two is exact, so only the E4M3 rounding is lossy.
    Returns (dequantised values, per-row scales)."""
    a = np.asarray(a, dtype=np.float64)
    s = pow2_scale(np.max(np.abs(a), axis=-1))
    return round_e4m3(a / s[..., None]) * s[..., None], s
