"""Pins of the oracle's pipeline: an independent NumPy float64 re-derivation on
tiny shapes, stage by stage, plus invariants that hold at any size.  CPU only."""
from dataclasses import replace

import numpy as np
import pytest

from latent_moe_layer_amd import synth
from oracle import oracle as orc
from tests import ref_numpy as ref

PIN = synth.Workload("pin", Mr=5, Ms=7, E=4, k=2, I=128, Is=128, wfmt=synth.WFMT_FP8, seed=11, H=384, L=256)


def _rel_close(got, want, tol):
    scale = max(np.sqrt(np.mean(np.asarray(want, np.float64) ** 2)), 1e-30)
    return np.max(np.abs(np.asarray(got, np.float64) - want)) <= tol * scale


def _dequant(inp, which):
    if inp.wl.wfmt == synth.WFMT_FP8:
        return ref.dequant_fp8(getattr(inp, which), getattr(inp, which + "_scale"))
    if inp.wl.wfmt == synth.WFMT_NVFP4:
        return ref.dequant_nvfp4(getattr(inp, which), getattr(inp, which + "_scale"), getattr(inp, which + "_tscale"))
    return ref.dequant_mxfp4(getattr(inp, which), getattr(inp, which + "_scale"))


@pytest.mark.parametrize("wfmt", [synth.WFMT_FP8, synth.WFMT_MXFP4, synth.WFMT_NVFP4])
def test_pipeline_against_float64_stagewise(wfmt):
    wl = replace(PIN, wfmt=wfmt, zipf_s=1.2 if wfmt else 0.0)
    inp = synth.make_inputs(wl)
    Mr, Ms, k, E, L, H, I, Is = wl.Mr, wl.Ms, wl.k, wl.E, wl.L, wl.H, wl.I, wl.Is

    # router: fixed-order FP32 logits vs float64 dot products
    logits = orc.router_logits(inp.x_lat, inp.gate, inp.gate_bias)
    x64 = ref.bf16_val(inp.x_lat)
    l64 = x64 @ inp.gate.astype(np.float64).T + inp.gate_bias
    bound = 1e-5 * (np.abs(x64) @ np.abs(inp.gate.astype(np.float64)).T + np.abs(inp.gate_bias))
    assert np.all(np.abs(logits - l64) <= bound)
    ids, w = orc.route(inp.x_lat, inp.gate, inp.gate_bias, k)
    ids64 = np.argsort(-l64, axis=1, kind="stable")[:, :k]
    assert np.array_equal(ids, ids64)
    sel64 = np.take_along_axis(l64, ids64, 1)
    w64 = np.exp(sel64 - sel64[:, :1])
    w64 /= w64.sum(axis=1, keepdims=True)
    assert np.max(np.abs(w - w64)) <= 1e-6

    res = orc.forward(inp, ids, w)
    r = slice(0, Mr)

    # x codes/scales: the FP32 quantizer decision, by brute force
    xq, sx = ref.quant_1x128(x64.astype(np.float32))
    assert np.array_equal(res.xq[r], xq) and np.array_equal(res.sx[r], sx)

    # L1 + SwiGLU from the oracle's codes, in float64
    W1 = _dequant(inp, "w1")
    W2 = _dequant(inp, "w2")
    xhat = ref.E4M3[xq] * np.repeat(sx.astype(np.float64), 128, axis=1)
    h64 = np.zeros((Mr, k, I))
    for t in range(Mr):
        for j in range(k):
            g = W1[ids[t, j]] @ xhat[t]
            h64[t, j] = ref.silu_mul(g[:I], g[I:])
    amax = np.abs(h64).reshape(Mr, k, I // 128, 128).max(axis=3)
    err = np.abs(res.h[r] - h64).reshape(Mr, k, I // 128, 128).max(axis=3)
    assert np.all(err <= 1e-5 * amax + 1e-30)

    # h codes: exactly the FP32 quantizer applied to the oracle's FP32 h
    hq_b, sh_b = ref.quant_1x128(res.h[r].reshape(Mr * k, I))
    assert np.array_equal(res.hq[r].reshape(Mr * k, I), hq_b)
    assert np.array_equal(res.sh[r].reshape(Mr * k, I // 128), sh_b)

    # L2 from the oracle's h codes
    hhat = ref.E4M3[res.hq[r]] * np.repeat(res.sh[r].astype(np.float64), 128, axis=2)
    y64 = np.stack([np.stack([W2[ids[t, j]] @ hhat[t, j] for j in range(k)]) for t in range(Mr)])
    assert _rel_close(res.y[r], y64, 1e-5)

    # combine + RMSNorm from the oracle's y: rn within one bf16 rounding
    z = np.einsum("tj,tjn->tn", w.astype(np.float64), res.y[r].astype(np.float64))
    rn64 = z / np.sqrt((z ** 2).mean(axis=1, keepdims=True) + wl.rms_eps) * ref.bf16_val(inp.gamma)
    rn = ref.bf16_val(res.rn[r])
    assert np.all(np.abs(rn - rn64) <= np.abs(rn64) * (2.0 ** -8 + 1e-5) + 1e-30)
    assert np.mean(rn == ref.bf16_round(rn64)) > 0.99

    # shared expert, each stage from the oracle's previous bf16 tensor
    xh = ref.bf16_val(inp.x_hid)
    gs = xh @ ref.bf16_val(inp.ws1).T
    hs64 = ref.silu_mul(gs[:, :Is], gs[:, Is:])
    hs = ref.bf16_val(res.hs)
    assert np.all(np.abs(hs - hs64) <= np.abs(hs64) * (2.0 ** -8 + 1e-5) + 1e-30)
    s64 = hs @ ref.bf16_val(inp.ws2).T
    sb = ref.bf16_val(res.sbf)
    assert np.all(np.abs(sb - s64) <= np.abs(s64) * (2.0 ** -8 + 1e-5) + 1e-30)

    # up-projection + FP32 shared add
    out64 = rn @ ref.bf16_val(inp.w_up).T + sb[r]
    assert _rel_close(res.out_f32[r], out64, 1e-5)
    assert np.array_equal(ref.bf16_val(res.out_bf16[r]), ref.bf16_round(res.out_f32[r]))
    # shared-only rows carry s_bf unchanged
    assert np.array_equal(res.out_bf16[Mr:], res.sbf[Mr:])


def test_zero_router_gives_first_k_experts_equal_weights():
    wl = replace(PIN, zero_router=True, k=3)
    inp = synth.make_inputs(wl)
    ids, w = orc.route(inp.x_lat, inp.gate, None, 3)
    assert np.array_equal(ids, np.tile(np.arange(3, dtype=np.int32), (wl.Mr, 1)))
    assert np.all(w == np.float32(1.0) / np.float32(3.0))


def test_topk_bruteforce_and_weight_sum():
    rng = np.random.default_rng(7)
    for E, k in [(8, 2), (64, 8), (384, 8), (1024, 16), (5, 5)]:
        logits = rng.standard_normal((33, E)).astype(np.float32)
        logits[0, :] = 0.5                      # all-equal row: lowest indices win
        logits[1, 3 % E] = logits[1, 1 % E]     # a tie
        ids, w = orc.topk_softmax(logits, k)
        for t in range(33):
            order = sorted(range(E), key=lambda e: (-logits[t, e], e))[:k]
            assert list(ids[t]) == order
        assert np.all(np.abs(w.sum(axis=1) - 1) <= k * 2.0 ** -23)
        assert np.all(np.diff(w, axis=1) <= 0)


def test_permutation_properties():
    rng = np.random.default_rng(8)
    for E, k, Mr in [(8, 2, 16), (64, 8, 128), (384, 8, 300), (4, 4, 1), (16, 2, 0)]:
        ids = np.array([rng.permutation(E)[:k] for _ in range(Mr)], np.int32).reshape(Mr, k)
        off, sp, p2r = orc.permute(ids, E)
        R = Mr * k
        cnt = np.bincount(ids.ravel(), minlength=E)
        assert off[0] == 0 and off[E] == R and np.array_equal(np.diff(off), cnt)
        assert np.array_equal(np.sort(sp), np.arange(R))
        assert np.array_equal(p2r[sp], np.arange(R))
        for e in range(E):
            seg = sp[off[e]:off[e + 1]]
            assert np.all(ids.ravel()[seg] == e)
            assert np.all(np.diff(seg // k) > 0)


def test_zero_shared_weights_gives_routed_only():
    wl = replace(PIN, zero_shared=True)
    inp = synth.make_inputs(wl)
    ids, w = orc.route(inp.x_lat, inp.gate, inp.gate_bias, wl.k)
    res = orc.forward(inp, ids, w)
    assert np.all(res.sbf == 0) and np.all(res.hs == 0)
    rn = ref.bf16_val(res.rn[:wl.Mr])
    up64 = rn @ ref.bf16_val(inp.w_up).T
    assert _rel_close(res.out_f32[:wl.Mr], up64, 1e-5)
    assert np.all(res.out_bf16[wl.Mr:] == 0)


@pytest.mark.parametrize("k", [1, 2])
def test_identical_experts_equal_dense_mlp(k):
    """Identical experts with all-equal logits: the routed latent equals a single
    dense FP8 MLP (the same pipeline with one expert, top-1), bit for bit."""
    wl = replace(PIN, identical_experts=True, zero_router=True, k=k)
    inp = synth.make_inputs(wl)
    ids, w = orc.route(inp.x_lat, inp.gate, None, k)
    res = orc.forward(inp, ids, w)
    dense = replace(wl, E=1, k=1)
    dinp = synth.make_inputs(dense)
    dids, dw = orc.route(dinp.x_lat, dinp.gate, None, 1)
    dres = orc.forward(dinp, dids, dw)
    assert np.array_equal(res.rn, dres.rn)
    assert np.array_equal(res.out_bf16, dres.out_bf16)


def test_identical_experts_k8_within_ulps():
    wl = replace(PIN, identical_experts=True, zero_router=True, k=4, E=8)
    inp = synth.make_inputs(wl)
    ids, w = orc.route(inp.x_lat, inp.gate, None, 4)
    res = orc.forward(inp, ids, w)
    dres = orc.forward(synth.make_inputs(replace(wl, E=1, k=1)), np.zeros((wl.Mr, 1), np.int32),
                       np.ones((wl.Mr, 1), np.float32))
    a, b = ref.bf16_val(res.rn), ref.bf16_val(dres.rn)
    assert np.all(np.abs(a - b) <= np.abs(b) * 2.0 ** -7 + 1e-30)


def test_token_permutation_invariance():
    inp = synth.make_inputs(PIN)
    Mr, Ms = PIN.Mr, PIN.Ms
    ids, w = orc.route(inp.x_lat, inp.gate, inp.gate_bias, PIN.k)
    res = orc.forward(inp, ids, w)
    rng = np.random.default_rng(9)
    pr = rng.permutation(Mr)
    ps = np.concatenate([pr, Mr + rng.permutation(Ms - Mr)])
    inp2 = synth.make_inputs(PIN)
    inp2.x_lat = inp.x_lat[pr].copy()
    inp2.x_hid = inp.x_hid[ps].copy()
    ids2, w2 = orc.route(inp2.x_lat, inp2.gate, inp2.gate_bias, PIN.k)
    assert np.array_equal(ids2, ids[pr]) and np.array_equal(w2, w[pr])
    res2 = orc.forward(inp2, ids2, w2)
    assert np.array_equal(res2.out_bf16, res.out_bf16[ps])
    assert np.array_equal(res2.out_f32, res.out_f32[ps])


def test_shared_rows_independent_of_routed_count():
    inp = synth.make_inputs(PIN)
    ids, w = orc.route(inp.x_lat, inp.gate, inp.gate_bias, PIN.k)
    full = orc.forward(inp, ids, w)
    none = orc.forward(inp, ids[:0], w[:0], Mr=0)
    assert np.array_equal(full.out_bf16[PIN.Mr:], none.out_bf16[PIN.Mr:])
    assert np.array_equal(full.sbf, none.sbf)


def test_subset_selection_matches_full_run():
    inp = synth.make_inputs(PIN)
    ids, w = orc.route(inp.x_lat, inp.gate, inp.gate_bias, PIN.k)
    full = orc.forward(inp, ids, w)
    sel = np.array([6, 2, 0], np.int32)
    part = orc.forward(inp, ids, w, sel=sel)
    assert np.array_equal(part.out_bf16, full.out_bf16[sel])
    assert np.array_equal(part.hq, full.hq[sel])


def test_given_h_codes_continue_the_same_pipeline():
    # Given the oracle's own h codes back, every later step is bit for bit the
    # plain run's; given one code moved by a step, only that (token, slot)'s y
    # row changes, by the moved value times the W2 column (float64 check).
    inp = synth.make_inputs(PIN)
    ids, w = orc.route(inp.x_lat, inp.gate, inp.gate_bias, PIN.k)
    sel = np.array([4, 0, 2, 6], np.int32)
    plain = orc.forward(inp, ids, w, sel=sel)
    same = orc.forward(inp, ids, w, sel=sel, h_codes=(plain.hq, plain.sh))
    for name in ("y", "rn", "out_f32", "out_bf16", "hq", "sh", "sbf"):
        assert np.array_equal(getattr(same, name), getattr(plain, name)), name
    assert np.all(same.h == 0)  # the L1 is skipped
    hq = plain.hq.copy()
    s_, j_, i_ = 2, 1, 37          # token 2 (row 2 of sel), slot 1, h column 37
    old = hq[s_, j_, i_]
    hq[s_, j_, i_] = (old & 0x80) | ((old & 0x7F) + 1)
    moved = orc.forward(inp, ids, w, sel=sel, h_codes=(hq, plain.sh))
    dy = moved.y.astype(np.float64) - plain.y
    mask = np.zeros(dy.shape, bool)
    mask[s_, j_] = True
    assert np.all(dy[~mask] == 0)
    W2 = _dequant(inp, "w2")
    dh = (ref.E4M3[hq[s_, j_, i_]] - ref.E4M3[old]) * np.float64(plain.sh[s_, j_, i_ // 128])
    want = dh * W2[ids[sel[s_], j_]][:, i_]
    # (dy is the difference of two FP32 sums: compare at the scale of the y row)
    yscale = np.sqrt(np.mean(plain.y[s_, j_].astype(np.float64) ** 2))
    assert np.max(np.abs(dy[s_, j_] - want)) <= 1e-5 * yscale
    assert np.max(np.abs(dy[s_, j_] - want)) <= 1e-2 * np.max(np.abs(want))


def test_nvfp4_with_power_of_two_scales_is_mxfp4():
    # NVFP4 whose e4m3 block scales are powers of two, equal over each
    # 32-wide group, and whose matrix scale is a power of two, encodes the same
    # weights as MXFP4 with e8m0 = log2(block scale * matrix scale) + 127: every
    # output of the pipeline is then bit for bit the MXFP4 one
    wl4 = replace(PIN, wfmt=synth.WFMT_MXFP4, zipf_s=0.7)
    inp4 = synth.make_inputs(wl4)
    ids, w = orc.route(inp4.x_lat, inp4.gate, inp4.gate_bias, wl4.k)
    base = orc.forward(inp4, ids, w)
    nv = synth.make_inputs(replace(wl4, wfmt=synth.WFMT_NVFP4))
    nv.w1, nv.w2 = inp4.w1, inp4.w2
    for which, src in (("w1", inp4.w1_scale), ("w2", inp4.w2_scale)):
        X = src.astype(np.int64) - 127 + 3          # block exponent against a matrix scale of 2^-3
        assert np.all((X >= -9) & (X <= 8))         # a power of two e4m3 can hold
        s16 = np.repeat(P_E4M3_POW2[X + 9], 2, axis=-1)
        setattr(nv, which + "_scale", s16.astype(np.uint8))
        setattr(nv, which + "_tscale", np.full(wl4.E, 2.0 ** -3, np.float32))
    got = orc.forward(nv, ids, w)
    for name in ("hq", "sh", "y", "rn", "out_f32", "out_bf16"):
        assert np.array_equal(getattr(got, name), getattr(base, name)), name


# e4m3 codes of 2^-9 .. 2^8 (index X + 9): subnormal 2^-9 .. 2^-7 (mantissa
# 1, 2, 4), normal 2^-6 .. 2^8 (exponent field X + 7, mantissa 0)
P_E4M3_POW2 = np.array([1, 2, 4] + [(x + 7) << 3 for x in range(-6, 9)], np.int64)


def test_nvfp4_dequantization_against_float64():
    wl = replace(PIN, wfmt=synth.WFMT_NVFP4)
    inp = synth.make_inputs(wl)
    assert inp.w1.shape == (wl.E, 2 * wl.I, wl.L // 2) and inp.w1_scale.shape == (wl.E, 2 * wl.I, wl.L // 16)
    assert inp.w1_scale.dtype == np.uint8 and inp.w1_tscale.shape == (wl.E,)
    # the oracle's L1 output of one token and expert against float64 from the codes
    ids, w = orc.route(inp.x_lat, inp.gate, inp.gate_bias, wl.k)
    res = orc.forward(inp, ids, w, sel=np.array([0], np.int32))
    W1 = _dequant(inp, "w1")
    xq, sx = ref.quant_1x128(ref.bf16_val(inp.x_lat[:1]).astype(np.float32))
    xhat = ref.E4M3[xq[0]] * np.repeat(sx[0].astype(np.float64), 128)
    for j in range(wl.k):
        g = W1[ids[0, j]] @ xhat
        h64 = ref.silu_mul(g[:wl.I], g[wl.I:])
        amax = np.abs(h64).reshape(-1, 128).max(axis=1)
        err = np.abs(res.h[0, j] - h64).reshape(-1, 128).max(axis=1)
        assert np.all(err <= 1e-5 * amax)
    # the generator's scales: every block scale times the matrix scale covers the block
    w64 = _dequant(inp, "w1")
    assert np.all(np.isfinite(w64)) and np.abs(w64).max() > 0
