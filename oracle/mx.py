"""MX (microscaling) codecs in plain fp64 — part of the CPU oracle (test infrastructure).

The block's weights and activations are MX tensors: element codes plus one shared E8M0 scale per
32 consecutive elements along the reduction dimension. The MiniMax-M3-on-MI355X page ("Lần theo
điểm nghẽn: Tối ưu MiniMax M3 trên AMD Instinct MI355X", results passage and the quantisation /
"three data planes" passage) serves MXFP8 and MXFP4 weights but does not define the encodings;
they follow the OCP Microscaling Formats (MX) v1.0 specification:

  * E8M0 scale byte b:  2^(b - 127); b = 255 is NaN.
  * E4M3 ("fn", OCP; not the FNUZ variant the same page warns about for MI300X in its
    correctness-contracts passage): 1 sign, 4 exponent (bias 7), 3 mantissa bits. No infinities;
    S.1111.111 is NaN; largest finite 448; subnormals m * 2^-9.
  * E2M1: 1 sign, 2 exponent (bias 1), 1 mantissa bit: magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}.

Conversion of a block of 32 values to MX (the specification's rule, applied by the oracle to
weights at load and to activations on the fly):
    shared_exp = floor(log2(max |x|)) - emax_elem        (emax_elem = 8 for E4M3, 2 for E2M1)
    scale byte = clamp(shared_exp, -127, 127) + 127       (all-zero block: byte 0)
    code       = nearest element value to x / 2^shared_exp, ties to the even code, saturated to
                 the largest finite magnitude; the sign is kept (so -tiny gives a negative zero).

E2M1 codes are returned one per uint8 (0..15); packing two per byte is a layout matter that the
tests do on their side.

This module is test infrastructure: only tests/, the package smoke check and the bench's CPU
baseline use it. It shares no code with the GPU path.
"""
from __future__ import annotations

import numpy as np

BLOCK = 32

FORMATS = ("e4m3", "e2m1")
EMAX = {"e4m3": 8, "e2m1": 2}
CODE_BITS = {"e4m3": 8, "e2m1": 4}


# ---------------------------------------------------------------- element decoding (formulas)
def e8m0_value(b: int) -> float:
    if not 0 <= b <= 255:
        raise ValueError(b)
    return float("nan") if b == 255 else 2.0 ** (b - 127)


def e4m3_value(code: int) -> float:
    if not 0 <= code <= 255:
        raise ValueError(code)
    sign = -1.0 if code & 0x80 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return float("nan")
    if exp == 0:
        return sign * man * 2.0 ** -9                 # subnormal: 0.mmm * 2^(1-7)
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


def e2m1_value(code: int) -> float:
    if not 0 <= code <= 15:
        raise ValueError(code)
    sign = -1.0 if code & 0x8 else 1.0
    exp = (code >> 1) & 0x3
    man = code & 0x1
    if exp == 0:
        return sign * man * 0.5                       # subnormal: 0.m * 2^(1-1)
    return sign * (1.0 + man / 2.0) * 2.0 ** (exp - 1)


E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
E2M1_TABLE = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)
E8M0_TABLE = np.array([e8m0_value(b) for b in range(256)], dtype=np.float64)

# Non-negative finite magnitudes indexed by code (codes 0..max are increasing in value).
_MAGS = {"e4m3": E4M3_TABLE[:0x7F], "e2m1": E2M1_TABLE[:8]}
_SIGN = {"e4m3": 0x80, "e2m1": 0x8}


def decode(codes: np.ndarray, fmt: str) -> np.ndarray:
    table = E4M3_TABLE if fmt == "e4m3" else E2M1_TABLE
    return table[np.asarray(codes, dtype=np.int64)]


# ---------------------------------------------------------------- element encoding
def encode_nearest(v: np.ndarray, fmt: str) -> np.ndarray:
    """Round each value to the nearest representable element (ties to the even code), saturating
    to the largest finite magnitude; keeps the sign bit of v."""
    v = np.asarray(v, dtype=np.float64)
    if not np.all(np.isfinite(v)):
        raise ValueError("non-finite input to the MX encoder")
    mags = _MAGS[fmt]
    a = np.minimum(np.abs(v), mags[-1])
    hi = np.searchsorted(mags, a, side="left")             # first magnitude >= a
    hi = np.minimum(hi, len(mags) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - mags[lo]
    d_hi = mags[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.int64)
    code = np.where(np.signbit(v), code | _SIGN[fmt], code)
    return code.astype(np.uint8)


def shared_exponent(amax: np.ndarray, fmt: str) -> np.ndarray:
    """floor(log2(amax)) - emax_elem, clamped to the E8M0 range [-127, 127]; amax == 0 -> -127."""
    amax = np.asarray(amax, dtype=np.float64)
    m, e = np.frexp(amax)                  # amax = m * 2^e with 0.5 <= m < 1  ->  floor(log2) = e-1
    fl = e.astype(np.int64) - 1
    se = np.where(amax > 0, fl - EMAX[fmt], -127)
    return np.clip(se, -127, 127)


def quantize(x: np.ndarray, fmt: str):
    """MX-quantise along the last axis (its length a multiple of 32).

    Returns (codes uint8 [..., K], scale bytes uint8 [..., K/32])."""
    x = np.asarray(x, dtype=np.float64)
    K = x.shape[-1]
    if K % BLOCK:
        raise ValueError("last axis must be a multiple of 32")
    xb = x.reshape(x.shape[:-1] + (K // BLOCK, BLOCK))
    se = shared_exponent(np.max(np.abs(xb), axis=-1), fmt)
    v = xb / np.ldexp(1.0, se)[..., None]                  # exact: power-of-two scaling
    codes = encode_nearest(v, fmt).reshape(x.shape)
    return codes, (se + 127).astype(np.uint8)


def dequantize(codes: np.ndarray, scales: np.ndarray, fmt: str) -> np.ndarray:
    """codes [..., K], scale bytes [..., K/32] -> fp64 values code_value * 2^(byte - 127)."""
    vals = decode(codes, fmt)
    K = vals.shape[-1]
    s = E8M0_TABLE[np.asarray(scales, dtype=np.int64)]
    return (vals.reshape(vals.shape[:-1] + (K // BLOCK, BLOCK)) * s[..., None]).reshape(vals.shape)


def quantize_dequantize(x: np.ndarray, fmt: str) -> np.ndarray:
    c, s = quantize(x, fmt)
    return dequantize(c, s, fmt)


# ---------------------------------------------------------------- bf16 rounding
def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Nearest bf16 value (ties to even) of each fp64 input, returned as fp64, rounded once and
    directly from the exact value. bf16 keeps 8 significant bits: for |x| in [2^(e-1), 2^e) the
    grid step is 2^(e-8), and below the smallest normal (2^-126) the step stays 2^-133. Finite
    inputs within the bf16 range."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)                               # x = m * 2^e, 0.5 <= |m| < 1
    q = np.maximum(e.astype(np.int64), -125) - 8     # exponent of the grid step
    return np.ldexp(np.rint(np.ldexp(x, -q)), q)     # np.rint: nearest, ties to even
