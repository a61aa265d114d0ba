"""Seeded synthetic inputs for the latent-MoE layer tail.

This module only *draws* inputs: activations, router weights, quantized routed
expert weights and the BF16 dense weights.  It holds no step of the tail
itself (no routing, activation quantization, GEMM, SwiGLU or norm), so that the
CPU oracle and the HIP path can both consume exactly the same bytes while
sharing no arithmetic.

Workloads follow the widths of the Kimi-K3 latent-MoE tail described in
"[Kimi K3][Kernel] Fuse BF16 shared experts into latent MegaMoE tail"
(Summary: a 3584-wide routed latent, a 7168-wide shared hidden vector).  The
five named workloads fix token counts, expert counts, top-k, intermediate sizes
and weight formats.

Recipe (all draws are independent counter-style streams so the expert weights
can be drawn in parallel and reproduced one expert at a time):

* every tensor has its own ``numpy.random.Generator(PCG64(SeedSequence([seed,
  tag, index])))``; ``tag`` names the tensor, ``index`` the expert (0 for
  non-expert tensors);
* x_lat, x_hid ~ N(0, 1) rounded to bf16 (RNE); W_g ~ N(0, 0.02) fp32;
* routed W1 [E, 2I, L] ~ N(0, 1/sqrt(L)), W2 [E, L, I] ~ N(0, 1/sqrt(I));
  FP8 e4m3 with one fp32 scale per 128x128 block (scale = block amax / 448,
  1.0 for an all-zero block), or MXFP4 (e2m1 elements, one e8m0 scale per 32
  along K, OCP MX v1.0 scale rule floor(log2(amax)) - 2);
* W_up [H, L] ~ N(0, 1/sqrt(L)), Ws1 [2 I_s, H] ~ N(0, 1/sqrt(H)),
  Ws2 [H, I_s] ~ N(0, 1/sqrt(I_s)), all rounded to bf16;
* gamma ~ U(0.5, 1.5) rounded to bf16;
* router bias: zero, or for the skewed-load workload b[e] = -s * ln(e + 1)
  (log of an unnormalised Zipf(s) pmf, expert 0 most popular).

Rows 0..I-1 of W1 (and of Ws1) are the gate projection, rows I..2I-1 the up
projection.  FP4 bytes hold two elements, the even K index in the low nibble.

bf16 values are carried as uint16 bit patterns.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np
import torch

HIDDEN = 7168
LATENT = 3584

WFMT_FP8 = 0
WFMT_MXFP4 = 1
WFMT_NVFP4 = 3

# tensor tags for the per-tensor seed streams
_T_XLAT, _T_WG, _T_W1, _T_W2, _T_GAMMA, _T_WUP, _T_XHID, _T_WS1, _T_WS2 = range(1, 10)
_T_RESID = 10  # the add3 residual stream


@dataclass(frozen=True)
class Workload:
    name: str
    Mr: int
    Ms: int
    E: int
    k: int
    I: int
    Is: int
    wfmt: int
    seed: int
    zipf_s: float = 0.0
    H: int = HIDDEN
    L: int = LATENT
    rms_eps: float = 1e-6
    zero_router: bool = False       # W_g = 0 (all-equal logits)
    zero_shared: bool = False       # Ws1 = Ws2 = 0
    identical_experts: bool = False  # every expert gets expert 0's weights


# The five workloads of the tail (token counts, experts, top-k, widths, formats).
WORKLOADS = {
    "tiny": Workload("tiny", Mr=16, Ms=16, E=8, k=2, I=512, Is=512, wfmt=WFMT_FP8, seed=0),
    "decode": Workload("decode", Mr=128, Ms=128, E=64, k=8, I=2048, Is=2048, wfmt=WFMT_FP8, seed=1),
    "prefill": Workload("prefill", Mr=4096, Ms=4096, E=64, k=8, I=2048, Is=2048, wfmt=WFMT_FP8, seed=2),
    "mxfp4": Workload("mxfp4", Mr=1024, Ms=1024, E=128, k=8, I=2048, Is=2048, wfmt=WFMT_MXFP4, seed=3,
                      zipf_s=1.2),
    "indep": Workload("indep", Mr=2048, Ms=8192, E=384, k=8, I=2048, Is=2048, wfmt=WFMT_FP8, seed=4),
    # the decode shape with NVFP4 routed weights (e2m1, an e4m3 scale per 16
    # along K and an fp32 scale per expert matrix)
    "nvfp4": Workload("nvfp4", Mr=128, Ms=128, E=64, k=8, I=2048, Is=2048, wfmt=WFMT_NVFP4, seed=5),
}


def _rng(seed: int, tag: int, index: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tag, index])))


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (RNE) with torch's CPU cast; returns uint16 bit patterns."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


def _quant_fp8_block128(w: np.ndarray):
    """w [N, K] fp32 -> (codes [N, K] u8 e4m3, scales [N/128, K/128] fp32)."""
    n, kk = w.shape
    blocks = w.reshape(n // 128, 128, kk // 128, 128)
    amax = np.abs(blocks).max(axis=(1, 3))
    scale = np.where(amax == 0, np.float32(1.0), amax / np.float32(448.0)).astype(np.float32)
    scaled = blocks / scale[:, None, :, None]
    t = torch.from_numpy(np.ascontiguousarray(scaled.reshape(n, kk), dtype=np.float32))
    codes = t.clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, scale


def _e2m1_codes(v: np.ndarray) -> np.ndarray:
    """Nearest e2m1 code of each value (ties to the even code), saturating at
    6, sign in bit 3: the grid has spacing 0.5 below 2, 1 in [2, 4) and 2 from
    4 on, so the nearest code is an integer rounding (numpy's rint: ties to
    even) per range."""
    mag = np.abs(v)
    code = np.where(mag < 2, np.rint(mag * 2),
                    np.where(mag < 4, np.rint(mag) + 2, np.minimum(np.rint(mag * 0.5), 3) + 4)).astype(np.uint8)
    return code | (np.signbit(v).astype(np.uint8) << 3)


def _quant_nvfp4(w: np.ndarray):
    """w [N, K] fp32 -> (packed [N, K/2] u8 e2m1, scales [N, K/16] u8 e4m3,
    tensor scale fp32).

    NVFP4 as served with --quantization nvfp4: one fp32 scale g for the whole
    matrix, g = amax / (448 * 6), so that each 16-element block's scale
    amax16 / (6 g) fits the e4m3 range; that block scale is rounded to e4m3
    (nearest, torch's cast), and each element w / (s16 g) to the nearest e2m1
    (saturating at 6; 0 where the block scale rounded to 0)."""
    n, kk = w.shape
    amax = np.float32(np.abs(w).max())
    g = np.float32(1.0) if amax == 0 else np.float32(amax / np.float32(448.0 * 6.0))
    blocks = w.reshape(n, kk // 16, 16)
    bmax = np.abs(blocks).max(axis=2)
    sv = np.minimum(bmax / (np.float32(6.0) * g), np.float32(448.0)).astype(np.float32)
    scodes = torch.from_numpy(np.ascontiguousarray(sv)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    sdec = torch.from_numpy(scodes.copy()).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    den = (sdec * g).astype(np.float32)
    v = np.where(den[:, :, None] > 0, blocks / np.where(den > 0, den, 1)[:, :, None], 0).astype(np.float32)
    code = _e2m1_codes(v).reshape(n, kk)
    packed = (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8)
    return packed, scodes, g


def _quant_mxfp4(w: np.ndarray):
    """w [N, K] fp32 -> (packed [N, K/2] u8, e8m0 scales [N, K/32] u8).

    OCP MX v1.0: shared exponent X = floor(log2(amax)) - emax(e2m1)=2, element =
    w / 2^X rounded to nearest e2m1 (ties to even code), saturating at 6.
    The e2m1 grid has spacing 0.5 below 2, 1 in [2, 4) and 2 from 4 on, so the
    nearest code is an integer rounding (numpy's rint: ties to even) per range.
    """
    n, kk = w.shape
    blocks = w.reshape(n, kk // 32, 32)
    amax = np.abs(blocks).max(axis=2)
    _, ex = np.frexp(amax)                      # amax = m * 2^ex, m in [0.5, 1)
    X = np.where(amax == 0, 0, ex.astype(np.int32) - 1 - 2)
    X = np.clip(X, -127, 127)
    e8m0 = (X + 127).astype(np.uint8)
    v = blocks * np.ldexp(np.float32(1.0), -X)[:, :, None].astype(np.float32)
    code = _e2m1_codes(v).reshape(n, kk)
    packed = (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8)
    return packed, e8m0


@dataclass
class Inputs:
    wl: Workload
    x_lat: np.ndarray            # [Mr, L] bf16 bits
    x_hid: np.ndarray            # [Ms, H] bf16 bits
    gate: np.ndarray             # [E, L] fp32
    gate_bias: np.ndarray        # [E] fp32
    w1: np.ndarray               # FP8 [E, 2I, L] u8 | MXFP4, NVFP4 [E, 2I, L/2] u8
    w1_scale: np.ndarray         # FP8 [E, 2I/128, L/128] f32 | MXFP4 [E, 2I, L/32] u8 e8m0 | NVFP4 [E, 2I, L/16] u8 e4m3
    w2: np.ndarray               # FP8 [E, L, I] u8 | MXFP4, NVFP4 [E, L, I/2] u8
    w2_scale: np.ndarray         # FP8 [E, L/128, I/128] f32 | MXFP4 [E, L, I/32] u8 e8m0 | NVFP4 [E, L, I/16] u8 e4m3
    gamma: np.ndarray            # [L] bf16 bits
    w_up: np.ndarray             # [H, L] bf16 bits
    ws1: np.ndarray              # [2 Is, H] bf16 bits
    ws2: np.ndarray              # [H, Is] bf16 bits
    extra: dict = field(default_factory=dict)
    w1_tscale: np.ndarray = field(default_factory=lambda: np.zeros(0, np.float32))  # NVFP4: [E] fp32
    w2_tscale: np.ndarray = field(default_factory=lambda: np.zeros(0, np.float32))  # NVFP4: [E] fp32


def _normal(seed, tag, idx, shape, std):
    r = _rng(seed, tag, idx)
    a = r.standard_normal(int(np.prod(shape)), dtype=np.float32).reshape(shape)
    if std != 1.0:
        a *= np.float32(std)
    return a


def _expert_weights(wl: Workload, tag: int, e: int, n: int, kk: int, out_codes, out_scales, out_tscale):
    src = 0 if wl.identical_experts else e
    w = _normal(wl.seed, tag, src, (n, kk), 1.0 / np.sqrt(kk))
    if wl.wfmt == WFMT_FP8:
        c, s = _quant_fp8_block128(w)
    elif wl.wfmt == WFMT_NVFP4:
        c, s, g = _quant_nvfp4(w)
        out_tscale[e] = g
    else:
        c, s = _quant_mxfp4(w)
    out_codes[e] = c
    out_scales[e] = s


def make_inputs(wl: Workload | str, Mr: int | None = None, Ms: int | None = None,
                routing_only: bool = False) -> Inputs:
    """Draw every input of one workload.  ``Mr``/``Ms`` override token counts
    (the streams of x_lat / x_hid are then a prefix-compatible redraw).
    ``routing_only`` draws x_lat and the router only (other tensors empty)."""
    if isinstance(wl, str):
        wl = WORKLOADS[wl]
    if Mr is not None or Ms is not None:
        from dataclasses import replace
        wl = replace(wl, Mr=wl.Mr if Mr is None else Mr, Ms=wl.Ms if Ms is None else Ms)
    E, L, H, I, Is = wl.E, wl.L, wl.H, wl.I, wl.Is
    x_lat = f32_to_bf16_bits(_normal(wl.seed, _T_XLAT, 0, (wl.Mr, L), 1.0))
    if wl.zero_router:
        gate = np.zeros((E, L), np.float32)
    else:
        gate = _normal(wl.seed, _T_WG, 0, (E, L), 0.02)
    if wl.zipf_s:
        gate_bias = (-wl.zipf_s * np.log(np.arange(1, E + 1, dtype=np.float64))).astype(np.float32)
    else:
        gate_bias = np.zeros(E, np.float32)
    if routing_only:
        e8, e16 = np.zeros(0, np.uint8), np.zeros(0, np.uint16)
        return Inputs(wl, x_lat, e16, gate, gate_bias, e8, np.zeros(0, np.float32), e8, np.zeros(0, np.float32),
                      e16, e16, e16, e16)
    w1t = np.zeros(E if wl.wfmt == WFMT_NVFP4 else 0, np.float32)
    w2t = np.zeros(E if wl.wfmt == WFMT_NVFP4 else 0, np.float32)
    if wl.wfmt == WFMT_FP8:
        w1 = np.empty((E, 2 * I, L), np.uint8)
        w1s = np.empty((E, 2 * I // 128, L // 128), np.float32)
        w2 = np.empty((E, L, I), np.uint8)
        w2s = np.empty((E, L // 128, I // 128), np.float32)
    elif wl.wfmt == WFMT_NVFP4:
        w1 = np.empty((E, 2 * I, L // 2), np.uint8)
        w1s = np.empty((E, 2 * I, L // 16), np.uint8)
        w2 = np.empty((E, L, I // 2), np.uint8)
        w2s = np.empty((E, L, I // 16), np.uint8)
    else:
        w1 = np.empty((E, 2 * I, L // 2), np.uint8)
        w1s = np.empty((E, 2 * I, L // 32), np.uint8)
        w2 = np.empty((E, L, I // 2), np.uint8)
        w2s = np.empty((E, L, I // 32), np.uint8)
    jobs = [(_T_W1, e, 2 * I, L, w1, w1s, w1t) for e in range(E)] + \
           [(_T_W2, e, L, I, w2, w2s, w2t) for e in range(E)]
    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(lambda j: _expert_weights(wl, *j), jobs))
    r = _rng(wl.seed, _T_GAMMA, 0)
    gamma = f32_to_bf16_bits(r.uniform(0.5, 1.5, L).astype(np.float32))
    w_up = f32_to_bf16_bits(_normal(wl.seed, _T_WUP, 0, (H, L), 1.0 / np.sqrt(L)))
    x_hid = f32_to_bf16_bits(_normal(wl.seed, _T_XHID, 0, (wl.Ms, H), 1.0))
    if wl.zero_shared:
        ws1 = np.zeros((2 * Is, H), np.uint16)
        ws2 = np.zeros((H, Is), np.uint16)
    else:
        ws1 = f32_to_bf16_bits(_normal(wl.seed, _T_WS1, 0, (2 * Is, H), 1.0 / np.sqrt(H)))
        ws2 = f32_to_bf16_bits(_normal(wl.seed, _T_WS2, 0, (H, Is), 1.0 / np.sqrt(Is)))
    return Inputs(wl, x_lat, x_hid, gate, gate_bias, w1, w1s, w2, w2s, gamma, w_up, ws1, ws2,
                  w1_tscale=w1t, w2_tscale=w2t)


def make_residual(wl: Workload | str, Mr: int | None = None) -> np.ndarray:
    """The residual stream joined by the add3 epilogue: [Mr, H] bf16 bits,
    N(0, 1), its own stream of the workload's seed."""
    if isinstance(wl, str):
        wl = WORKLOADS[wl]
    Mr = wl.Mr if Mr is None else Mr
    return f32_to_bf16_bits(_normal(wl.seed, _T_RESID, 0, (Mr, wl.H), 1.0))


def algorithmic_bytes(wl: Workload, touched_experts: int | None = None) -> dict:
    """Bytes the tail must move at least once: touched routed experts' weights
    and scales, W_up, shared weights, W_g, gamma, inputs, outputs."""
    E = wl.E if touched_experts is None else touched_experts
    L, H, I, Is = wl.L, wl.H, wl.I, wl.Is
    if wl.wfmt == WFMT_FP8:
        routed = E * (2 * I * L + L * I) + E * 4 * ((2 * I // 128) * (L // 128) + (L // 128) * (I // 128))
    elif wl.wfmt == WFMT_NVFP4:
        routed = E * (2 * I * L // 2 + L * I // 2) + E * (2 * I * L // 16 + L * I // 16) + E * 8
    else:
        routed = E * (2 * I * L // 2 + L * I // 2) + E * (2 * I * L // 32 + L * I // 32)
    dense = 2 * (H * L + 2 * Is * H + H * Is) + 4 * wl.E * L + 2 * L
    io = 2 * (wl.Mr * L + wl.Ms * H) + 2 * wl.Ms * H
    return {"routed": routed, "dense": dense, "io": io, "total": routed + dense + io}


def algorithmic_flops(wl: Workload) -> dict:
    R = wl.Mr * wl.k
    L, H, I, Is = wl.L, wl.H, wl.I, wl.Is
    lowp = 2 * R * (2 * I) * L + 2 * R * L * I
    bf16 = 2 * wl.Ms * (2 * Is) * H + 2 * wl.Ms * H * Is + 2 * wl.Mr * H * L
    return {"lowp": lowp, "bf16": bf16, "router": 2 * wl.Mr * wl.E * L}
