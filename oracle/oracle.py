"""ctypes front end of the CPU oracle (``libmoe_tail_oracle.so``).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product package.  It marshals numpy
arrays; all arithmetic happens in ``moe_tail_oracle.cpp``.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_tail_oracle.cpp")
LIB_PATH = os.path.join(_HERE, "libmoe_tail_oracle.so")

BUILD_CMD = ["g++", "-O2", "-std=c++17", "-fopenmp", "-fno-fast-math", "-ffp-contract=off",
             "-fPIC", "-shared", "-Wall", _SRC, "-o", LIB_PATH]


def build() -> str:
    subprocess.run(BUILD_CMD, check=True)
    return LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < os.path.getmtime(_SRC):
            build()
        _lib = C.CDLL(LIB_PATH)
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


def bf16_from_f32(x):
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().oracle_bf16_from_f32(_p(x), C.c_int64(x.size), _p(out))
    return out


def e4m3_decode(codes):
    codes = _c(codes, np.uint8)
    out = np.empty(codes.shape, np.float32)
    lib().oracle_e4m3_decode(_p(codes), C.c_int64(codes.size), _p(out))
    return out


def e4m3_encode(x):
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint8)
    lib().oracle_e4m3_encode(_p(x), C.c_int64(x.size), _p(out))
    return out


def e2m1_decode(nibbles):
    nibbles = _c(nibbles, np.uint8)
    out = np.empty(nibbles.shape, np.float32)
    lib().oracle_e2m1_decode(_p(nibbles), C.c_int64(nibbles.size), _p(out))
    return out


def e8m0_decode(e):
    e = _c(e, np.uint8)
    out = np.empty(e.shape, np.float32)
    lib().oracle_e8m0_decode(_p(e), C.c_int64(e.size), _p(out))
    return out


def quant_1x128(x):
    x = _c(x, np.float32)
    rows, cols = x.shape
    q = np.empty((rows, cols), np.uint8)
    s = np.empty((rows, cols // 128), np.float32)
    lib().oracle_quant_1x128(_p(x), C.c_int(rows), C.c_int(cols), _p(q), _p(s))
    return q, s


def rmsnorm(z, gamma_bits, eps):
    z = _c(z, np.float32)
    rows, n = z.shape
    out = np.empty((rows, n), np.uint16)
    lib().oracle_rmsnorm(_p(z), C.c_int(rows), C.c_int(n), _p(_c(gamma_bits, np.uint16)), C.c_float(eps), _p(out))
    return out


def router_logits(x_lat, gate, bias):
    x_lat = _c(x_lat, np.uint16)
    gate = _c(gate, np.float32)
    Mr, L = x_lat.shape
    E = gate.shape[0]
    out = np.empty((Mr, E), np.float32)
    lib().oracle_router_logits(C.c_int(L), C.c_int(E), C.c_int(Mr), _p(x_lat), _p(gate),
                               _p(None if bias is None else _c(bias, np.float32)), _p(out))
    return out


def topk_softmax(logits, k):
    logits = _c(logits, np.float32)
    Mr, E = logits.shape
    ids = np.empty((Mr, k), np.int32)
    w = np.empty((Mr, k), np.float32)
    lib().oracle_topk_softmax(C.c_int(E), C.c_int(k), C.c_int(Mr), _p(logits), _p(ids), _p(w))
    return ids, w


def route(x_lat, gate, bias, k):
    x_lat = _c(x_lat, np.uint16)
    gate = _c(gate, np.float32)
    Mr, L = x_lat.shape
    E = gate.shape[0]
    ids = np.empty((Mr, k), np.int32)
    w = np.empty((Mr, k), np.float32)
    lib().oracle_route(C.c_int(L), C.c_int(E), C.c_int(k), C.c_int(Mr), _p(x_lat), _p(gate),
                       _p(None if bias is None else _c(bias, np.float32)), _p(ids), _p(w), None)
    return ids, w


def permute(ids, E):
    ids = _c(ids, np.int32)
    Mr, k = ids.shape
    off = np.empty(E + 1, np.int32)
    sp = np.empty(Mr * k, np.int32)
    p2r = np.empty(Mr * k, np.int32)
    lib().oracle_permute(C.c_int(E), C.c_int(k), C.c_int(Mr), _p(ids), _p(off), _p(sp), _p(p2r))
    return off, sp, p2r


@dataclass
class ForwardResult:
    sel: np.ndarray
    out_f32: np.ndarray     # [n, H]
    out_bf16: np.ndarray    # [n, H] bf16 bits
    xq: np.ndarray          # [n, L]
    sx: np.ndarray          # [n, L/128]
    hq: np.ndarray          # [n, k, I]
    sh: np.ndarray          # [n, k, I/128]
    h: np.ndarray           # [n, k, I]
    y: np.ndarray           # [n, k, L]
    rn: np.ndarray          # [n, L] bf16 bits
    hs: np.ndarray          # [n, Is] bf16 bits
    sbf: np.ndarray         # [n, H] bf16 bits


def forward(inp, topk_ids, topk_w, sel=None, Mr=None, Ms=None, residual=None, h_codes=None) -> ForwardResult:
    """Run the oracle on ``synth.Inputs`` for the tokens in ``sel`` (default all).
    ``residual`` ([Mr, H] bf16 bits, row t for token t) is added to the routed
    rows after the shared add, before the one rounding ("add3").
    ``h_codes`` (optional ``(hq [n, k, I] u8, sh [n, k, I/128] f32)``, rows in
    ``sel`` order): the h codes and scales to continue from instead of the
    oracle's own (the routed L1 is skipped; ``h`` then reads 0)."""
    wl = inp.wl
    Mr = inp.x_lat.shape[0] if Mr is None else Mr
    Ms = inp.x_hid.shape[0] if Ms is None else Ms
    if sel is None:
        sel = np.arange(Ms, dtype=np.int32)
    sel = _c(sel, np.int32)
    n = sel.size
    H, L, I, Is, k = wl.H, wl.L, wl.I, wl.Is, wl.k
    r = ForwardResult(
        sel=sel,
        out_f32=np.zeros((n, H), np.float32), out_bf16=np.zeros((n, H), np.uint16),
        xq=np.zeros((n, L), np.uint8), sx=np.zeros((n, L // 128), np.float32),
        hq=np.zeros((n, k, I), np.uint8), sh=np.zeros((n, k, I // 128), np.float32),
        h=np.zeros((n, k, I), np.float32), y=np.zeros((n, k, L), np.float32),
        rn=np.zeros((n, L), np.uint16), hs=np.zeros((n, Is), np.uint16), sbf=np.zeros((n, H), np.uint16))
    arrs = [_c(inp.w1, np.uint8), _c(inp.w1_scale, inp.w1_scale.dtype), _c(inp.w2, np.uint8),
            _c(inp.w2_scale, inp.w2_scale.dtype), _c(inp.gamma, np.uint16), _c(inp.w_up, np.uint16),
            _c(inp.ws1, np.uint16), _c(inp.ws2, np.uint16), _c(inp.x_lat, np.uint16), _c(inp.x_hid, np.uint16),
            _c(topk_ids, np.int32), _c(topk_w, np.float32)]
    res = None if residual is None else _c(residual, np.uint16)
    hq_in = sh_in = None
    if h_codes is not None:
        hq_in, sh_in = _c(h_codes[0], np.uint8), _c(h_codes[1], np.float32)
        if hq_in.shape != (n, k, I) or sh_in.shape != (n, k, I // 128):
            raise ValueError("h_codes must be [n, k, I] codes and [n, k, I/128] scales")
    if res is not None and res.shape != (Mr, H):
        raise ValueError("residual must be [Mr, H]")
    rc = lib().oracle_forward(
        C.c_int(H), C.c_int(L), C.c_int(wl.E), C.c_int(k), C.c_int(I), C.c_int(Is), C.c_int(wl.wfmt),
        C.c_float(wl.rms_eps),
        _p(arrs[0]), _p(arrs[1]), _p(arrs[2]), _p(arrs[3]), _p(arrs[4]), _p(arrs[5]), _p(arrs[6]), _p(arrs[7]),
        _p(arrs[8]), C.c_int(Mr), _p(arrs[9]), C.c_int(Ms), _p(arrs[10]), _p(arrs[11]), _p(res),
        C.c_int(n), _p(sel),
        _p(r.out_f32), _p(r.out_bf16), _p(r.xq), _p(r.sx), _p(r.hq), _p(r.sh), _p(r.h), _p(r.y), _p(r.rn),
        _p(r.hs), _p(r.sbf), _p(hq_in), _p(sh_in),
        _p(_c(inp.w1_tscale, np.float32) if wl.wfmt == 3 else None),
        _p(_c(inp.w2_tscale, np.float32) if wl.wfmt == 3 else None))
    if rc != 0:
        raise ValueError("oracle_forward rejected its arguments")
    return r
