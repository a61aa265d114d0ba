"""Parity metrics shared by the GPU tests and the benchmark.

Relative error of element i against the oracle's FP32 output o:
    rel_i = |g_i - o_i| / max(|o_i|, rms(o))
(an elementwise |g - o| / |o| is ill-posed where the routed and shared parts
cancel).  The bar: max_i rel_i <= 2e-2 and mean_i rel_i <= 3e-3.
"""
from __future__ import annotations

import numpy as np

MAX_REL = 2e-2
MEAN_REL = 3e-3


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits).astype(np.uint32) << 16).view(np.float32)


def rel_errors(got: np.ndarray, want: np.ndarray) -> tuple[float, float]:
    g = np.asarray(got, np.float64)
    o = np.asarray(want, np.float64)
    if o.size == 0:
        return 0.0, 0.0
    rms = np.sqrt(np.mean(o * o))
    rel = np.abs(g - o) / np.maximum(np.abs(o), max(rms, 1e-30))
    return float(rel.max()), float(rel.mean())


def e4m3_value(code: np.ndarray) -> np.ndarray:
    c = np.asarray(code, np.int64)
    s, e, m = c >> 7, (c >> 3) & 15, c & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (1 + m / 8.0) * 2.0 ** (e.astype(np.float64) - 7))
    return np.where(s == 1, -mag, mag)


def check_h_codes(gpu_hq, gpu_sh, orc_hq, orc_sh, orc_h, tol=1e-5):
    """The rule for re-quantized activations computed by two different FP32
    summation orders: scales agree to `tol` relative; codes agree except where
    the oracle's h lies within tol * block amax of a rounding midpoint, and
    then by exactly one code step.  Returns (n_mismatch, n_total)."""
    gpu_hq = np.asarray(gpu_hq)
    orc_hq = np.asarray(orc_hq)
    rs = np.abs(np.asarray(gpu_sh, np.float64) - orc_sh) / np.abs(orc_sh)
    assert np.all(rs <= tol), f"h scale mismatch {rs.max():.3e}"
    mism = gpu_hq != orc_hq
    n = int(mism.sum())
    if n:
        rows, cols = np.nonzero(mism.reshape(-1, gpu_hq.shape[-1]))
        g = gpu_hq.reshape(-1, gpu_hq.shape[-1])[rows, cols]
        o = orc_hq.reshape(-1, orc_hq.shape[-1])[rows, cols]
        h = np.asarray(orc_h, np.float64).reshape(-1, orc_hq.shape[-1])[rows, cols]
        s = np.asarray(orc_sh, np.float64).reshape(-1, orc_sh.shape[-1])[rows, cols // 128]
        gv, ov = e4m3_value(g), e4m3_value(o)
        # adjacent codes of the same sign (or +-0 around zero)
        step = np.abs(g.astype(np.int64) & 0x7F) - np.abs(o.astype(np.int64) & 0x7F)
        same_sign = ((g ^ o) & 0x80) == 0
        assert np.all((np.abs(step) == 1) & (same_sign | (np.minimum(g & 0x7F, o & 0x7F) == 0))), \
            "h code differs by more than one step"
        mid = (gv + ov) / 2 * s
        amax = 448.0 * s
        assert np.all(np.abs(h - mid) <= tol * amax), "h code flip away from a rounding midpoint"
    return n, gpu_hq.size
