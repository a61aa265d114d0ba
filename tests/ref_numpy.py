"""Independent NumPy float64 re-derivation of the tail, used only to pin the
CPU oracle on tiny shapes.  It shares nothing with the oracle: formats are
decoded from their closed forms, quantization codes come from a brute-force
nearest-value search, and every sum is a float64 matrix product.

Decisions that turn floating point into codes (the 1x128 FP8 quantizer, the
top-k argmax, bf16 rounding) are taken in FP32, the method's precision.
"""
from __future__ import annotations

import numpy as np


def e4m3_values() -> np.ndarray:
    """Value of each of the 256 e4m3 codes from the OCP 8-bit FP closed form."""
    v = np.empty(256, np.float64)
    for c in range(256):
        s, e, m = c >> 7, (c >> 3) & 15, c & 7
        if e == 15 and m == 7:
            v[c] = np.nan
            continue
        mag = m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
        v[c] = -mag if s else mag
    return v


E4M3 = e4m3_values()
_POS = E4M3[:127]          # finite non-negative magnitudes, ascending


def e4m3_encode_bruteforce(x32: np.ndarray) -> np.ndarray:
    """Nearest finite e4m3 value, ties to the even code, saturating at 448,
    sign kept; by exhaustive distance comparison against all 127 magnitudes."""
    x = np.asarray(x32, np.float32).astype(np.float64)
    a = np.minimum(np.abs(x), 448.0)
    d = np.abs(a[..., None] - _POS)                       # [..., 127]
    best = d.min(axis=-1, keepdims=True)
    cand = d == best
    # among equidistant codes pick the even one (at most two candidates)
    idx = np.arange(127)
    even = cand & (idx % 2 == 0)
    code = np.where(even.any(axis=-1), np.argmax(even, axis=-1), np.argmax(cand, axis=-1))
    return (code | (np.signbit(x).astype(np.int64) << 7)).astype(np.uint8)


def quant_1x128(x32: np.ndarray):
    x32 = np.asarray(x32, np.float32)
    rows, cols = x32.shape
    xb = x32.reshape(rows, cols // 128, 128)
    amax = np.abs(xb).max(axis=2)
    s = np.where(amax == 0, np.float32(1), amax / np.float32(448)).astype(np.float32)
    q = e4m3_encode_bruteforce((xb / s[:, :, None]).astype(np.float32)).reshape(rows, cols)
    return q, s


def bf16_round(x: np.ndarray) -> np.ndarray:
    """fp64 -> fp32 -> bf16 (RNE) -> value as fp64."""
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    keep = u >> 16
    rest = u & 0xFFFF
    up = (rest > 0x8000) | ((rest == 0x8000) & ((keep & 1) == 1))
    b = (keep + up).astype(np.uint32) << 16
    return b.astype(np.uint32).view(np.float32).astype(np.float64)


def bf16_val(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, np.uint32) << 16).view(np.float32).astype(np.float64)


def e2m1_values() -> np.ndarray:
    mags = [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    return np.array([(-1) ** (c >> 3) * mags[c & 7] for c in range(16)], np.float64)


def dequant_fp8(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """[E, N, K] codes with [E, N/128, K/128] scales -> fp64 weights."""
    v = E4M3[codes]
    s = np.repeat(np.repeat(scales.astype(np.float64), 128, axis=1), 128, axis=2)
    return v * s


def dequant_mxfp4(packed: np.ndarray, e8m0: np.ndarray) -> np.ndarray:
    lo = packed & 0xF
    hi = packed >> 4
    nib = np.stack([lo, hi], axis=-1).reshape(*packed.shape[:-1], packed.shape[-1] * 2)
    v = e2m1_values()[nib]
    s = np.repeat(2.0 ** (e8m0.astype(np.float64) - 127), 32, axis=-1)
    return v * s


def dequant_nvfp4(packed: np.ndarray, s16: np.ndarray, g: np.ndarray) -> np.ndarray:
    """[E, N, K/2] e2m1 pairs, [E, N, K/16] e4m3 scales, [E] fp32 matrix
    scales -> fp64 weights e2m1 * e4m3 * g (exact in fp64)."""
    lo = packed & 0xF
    hi = packed >> 4
    nib = np.stack([lo, hi], axis=-1).reshape(*packed.shape[:-1], packed.shape[-1] * 2)
    v = e2m1_values()[nib]
    s = np.repeat(E4M3[s16], 16, axis=-1)
    return v * s * np.asarray(g, np.float64)[:, None, None]


def silu_mul(g, u):
    return g / (1 + np.exp(-g)) * u
