"""Pins of the oracle's add3 epilogue (routed up-projection + shared output +
residual, added in FP32 in that order and rounded to bf16 once; tokenspeed PR
"MNNVL CuTe-DSL finalize tail + K3 comm layer extraction", commit log).  CPU only."""
from dataclasses import replace

import numpy as np

from latent_moe_layer_amd import synth
from oracle import oracle as orc
from tests import ref_numpy as ref

PIN = synth.Workload("pin", Mr=5, Ms=7, E=4, k=2, I=128, Is=128, wfmt=synth.WFMT_FP8, seed=11, H=384, L=256)


def _run(wl, inp=None, residual=None, sel=None):
    inp = synth.make_inputs(wl) if inp is None else inp
    ids, w = orc.route(inp.x_lat, inp.gate, inp.gate_bias, wl.k)
    return inp, orc.forward(inp, ids, w, sel=sel, residual=residual)


def test_add3_is_one_fp32_add_after_the_shared_add():
    """out_f32(add3) = fp32(out_f32(plain) + residual) bit for bit: the residual
    comes after the shared add, in FP32, and the result is rounded once."""
    inp, plain = _run(PIN)
    r = synth.make_residual(PIN)
    _, add3 = _run(PIN, inp, r)
    Mr = PIN.Mr
    want = plain.out_f32[:Mr] + ref.bf16_val(r).astype(np.float32)  # one FP32 add
    assert want.dtype == np.float32
    assert np.array_equal(add3.out_f32[:Mr].view(np.uint32), want.view(np.uint32))
    assert np.array_equal(add3.out_bf16[:Mr], synth.f32_to_bf16_bits(want))
    # shared rows (t >= Mr) take no residual
    assert np.array_equal(add3.out_bf16[Mr:], plain.out_bf16[Mr:])
    assert np.array_equal(add3.out_f32[Mr:], plain.out_f32[Mr:])


def test_add3_with_zero_weights_returns_the_residual():
    """No up-projection and no shared expert: each routed row is its residual
    row exactly (a bf16 value survives the FP32 add of zeros and the rounding)."""
    wl = replace(PIN, zero_shared=True)
    inp = synth.make_inputs(wl)
    inp.w_up = np.zeros_like(inp.w_up)
    r = synth.make_residual(wl)
    _, res = _run(wl, inp, r)
    assert np.array_equal(res.out_bf16[:wl.Mr], r)
    assert np.all(res.out_bf16[wl.Mr:] == 0)


def test_add3_zero_residual_equals_plain_forward():
    inp, plain = _run(PIN)
    _, add3 = _run(PIN, inp, np.zeros((PIN.Mr, PIN.H), np.uint16))
    assert np.array_equal(add3.out_bf16, plain.out_bf16)
    assert np.array_equal(add3.out_f32, plain.out_f32)


def test_add3_residual_row_follows_the_token():
    """Row s of a selection takes the residual of token sel[s], not of row s."""
    inp = synth.make_inputs(PIN)
    r = synth.make_residual(PIN)
    _, full = _run(PIN, inp, r)
    sel = np.array([4, 6, 1, 3], np.int32)
    _, part = _run(PIN, inp, r, sel=sel)
    assert np.array_equal(part.out_bf16, full.out_bf16[sel])
    assert np.array_equal(part.out_f32, full.out_f32[sel])


def test_add3_against_float64():
    """The final join recomputed in float64 from the oracle's own rn and shared
    output: within a few FP32 roundings of the float64 sum."""
    inp = synth.make_inputs(PIN)
    r = synth.make_residual(PIN)
    _, res = _run(PIN, inp, r)
    Mr = PIN.Mr
    up64 = ref.bf16_val(res.rn[:Mr]).astype(np.float64) @ ref.bf16_val(inp.w_up).astype(np.float64).T
    want = up64 + ref.bf16_val(res.sbf[:Mr]) + ref.bf16_val(r)
    scale = np.sqrt(np.mean(want ** 2))
    assert np.max(np.abs(res.out_f32[:Mr] - want)) <= 1e-5 * scale
