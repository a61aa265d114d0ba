"""Parity metrics shared by the GPU tests.

Two statistics of an output g against the oracle's FP32 output o, with the
bar max <= 2e-2 and mean <= 3e-3:

* elementwise: rel_i = |g_i - o_i| / max(|o_i|, rms(o)) over every compared
  element (the floor rms(o) keeps the ratio defined where the routed and the
  shared parts cancel);
* per token, normwise: rel_t = ||g_t - o_t||_2 / ||o_t||_2.

The GPU and the oracle sum the routed L1 in different orders, so h differs
by a few 1e-5 of its block amax and its FP8 codes differ where h lies that
close to a rounding midpoint (check_h_codes states and checks the rule).  Each
such flip moves whole output rows: a single element of out by up to about 1 %,
so the largest elementwise error over a workload grows with the number of
elements compared, while the per-token error and the mean stay put.  The
outputs are therefore compared twice:

* directly with the oracle's own pipeline: per token (max and mean) and
  elementwise mean against the bar; the elementwise max is reported;
* with the oracle continuing from the GPU's own h codes (oracle.forward's
  h_codes): every step after the h quantization, checked elementwise and per
  token against the full bar, with the h-code flips taken out.

Intermediates downstream of h (the routed L2 output y of one (token, slot)
row, the normalized latent rn) are compared per row with the same bar.
"""
from __future__ import annotations

import numpy as np

MAX_REL = 2e-2
MEAN_REL = 3e-3
MAX_REL_INTERMEDIATE = MAX_REL


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits).astype(np.uint32) << 16).view(np.float32)


def row_rel_errors(got: np.ndarray, want: np.ndarray) -> tuple[float, float]:
    """(max, mean) over rows of ||g_row - o_row|| / ||o_row||."""
    g = np.asarray(got, np.float64).reshape(-1, np.shape(want)[-1])
    o = np.asarray(want, np.float64).reshape(-1, np.shape(want)[-1])
    if o.size == 0:
        return 0.0, 0.0
    rel = np.linalg.norm(g - o, axis=1) / np.maximum(np.linalg.norm(o, axis=1), 1e-30)
    return float(rel.max()), float(rel.mean())


def rel_errors(got: np.ndarray, want: np.ndarray) -> tuple[float, float]:
    """Elementwise (max, mean) of |g - o| / max(|o|, rms(o))."""
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


# h is computed twice by different summation procedures: the oracle's
# sequential FP32 loop and the matrix cores, which sum the 128 FP8 products of
# one block instruction with an internal precision coarser than FP32 (see
# tests/test_gpu_mfma_precision.py, which measures it and checks that on the
# workloads' own operands it moves h by at most H_TOL / 5 of the block amax).
H_TOL = 5e-4


def assert_output_gate(got: np.ndarray, want: np.ndarray, what: str, elementwise_max: bool = True) -> dict:
    """Both output statistics against the bar (the elementwise max only when
    `elementwise_max`); returns them."""
    emax, emean = rel_errors(got, want)
    tmax, tmean = row_rel_errors(got, want)
    st = {f"{what}_elementwise": (emax, emean), f"{what}_per_token": (tmax, tmean)}
    assert emean <= MEAN_REL and (emax <= MAX_REL or not elementwise_max), st
    assert tmax <= MAX_REL and tmean <= MEAN_REL, st
    return st


def e4m3_ordinal(code: np.ndarray) -> np.ndarray:
    """Position of an e4m3 code on the number line (+0 and -0 both 0)."""
    c = np.asarray(code, np.int64)
    mag = c & 0x7F
    return np.where(c >> 7 == 1, -mag, mag)


def e4m3_encode_np(x: np.ndarray) -> np.ndarray:
    """Nearest e4m3 code (ties to even), saturating at 448, sign kept."""
    vals = e4m3_value(np.arange(127))
    x = np.asarray(x, np.float64)
    a = np.minimum(np.abs(x), 448.0)
    hi = np.searchsorted(vals, a, side="left").clip(0, 126)
    lo = np.maximum(hi - 1, 0)
    dlo, dhi = a - vals[lo], vals[hi] - a
    code = np.where(dhi < dlo, hi, np.where(dlo < dhi, lo, np.where(lo % 2 == 0, lo, hi)))
    code = np.where(vals[hi] == a, hi, code)
    return (code | (np.signbit(x).astype(np.int64) << 7)).astype(np.uint8)


def e4m3_spacing(code: np.ndarray) -> np.ndarray:
    """Distance from an e4m3 code's magnitude to the next larger one (in
    units of the scale)."""
    mag = np.asarray(code, np.int64) & 0x7F
    return e4m3_value(np.minimum(mag + 1, 126)) - e4m3_value(np.minimum(mag, 125))


def check_h_codes(gpu_hq, gpu_sh, orc_hq, orc_sh, orc_h, tol=H_TOL):
    """The rule for re-quantized activations computed by two different
    summation procedures: scales agree to `tol` relative, and every GPU code
    is the rounding (with the GPU's scale) of some value within tol * block
    amax of the oracle's h -- so codes differ only where h sits that close to
    a rounding midpoint.  Where that band is narrower than the code spacing
    (every normal code of the larger values) a differing code is exactly one
    step from the oracle's; near zero, where the subnormal codes are spaced
    2^-9 of the scale apart, the band spans several codes and the band rule
    alone applies.  Returns (n_mismatch, n_total, max scale deviation,
    n_mismatch more than one step apart)."""
    gpu_hq = np.asarray(gpu_hq)
    orc_hq = np.asarray(orc_hq)
    rs = np.abs(np.asarray(gpu_sh, np.float64) - orc_sh) / np.abs(orc_sh)
    assert np.all(rs <= tol), f"h scale mismatch {rs.max():.3e}"
    mism = (gpu_hq != orc_hq) & (e4m3_ordinal(gpu_hq) != e4m3_ordinal(orc_hq))  # (+0 and -0 are equal)
    n = int(mism.sum())
    multi = 0
    if n:
        ncol = gpu_hq.shape[-1]
        rows, cols = np.nonzero(mism.reshape(-1, ncol))
        g = gpu_hq.reshape(-1, ncol)[rows, cols]
        o = orc_hq.reshape(-1, ncol)[rows, cols]
        h = np.asarray(orc_h, np.float64).reshape(-1, ncol)[rows, cols]
        s_orc = np.asarray(orc_sh, np.float64).reshape(-1, ncol // 128)[rows, cols // 128]
        s_gpu = np.asarray(gpu_sh, np.float64).reshape(-1, ncol // 128)[rows, cols // 128]
        band = tol * 448.0 * s_orc
        lo = e4m3_value(e4m3_encode_np((h - band) / s_gpu))
        hi = e4m3_value(e4m3_encode_np((h + band) / s_gpu))
        gv = e4m3_value(g)
        assert np.all((gv >= lo) & (gv <= hi)), "h code flip away from a rounding midpoint"
        step = np.abs(e4m3_ordinal(g) - e4m3_ordinal(o))
        narrow = 2.0 * band < e4m3_spacing(np.minimum(g & 0x7F, o & 0x7F)) * s_orc
        assert np.all(step[narrow] == 1), f"h codes more than one step apart: {np.bincount(step[narrow])}"
        multi = int(np.count_nonzero(step > 1))
    return n, gpu_hq.size, float(rs.max(initial=0.0)), multi
