"""The seeded input generator: weight quantization rules checked by brute
force, reproducibility, shapes.  CPU only."""
from dataclasses import replace

import numpy as np

from latent_moe_layer_amd import synth
from tests import ref_numpy as ref


def test_fp8_block_quantization_rule():
    rng = np.random.default_rng(0)
    w = rng.standard_normal((256, 384)).astype(np.float32) * 0.05
    w[128:, 256:] = 0.0
    codes, scales = synth._quant_fp8_block128(w)
    assert codes.shape == w.shape and scales.shape == (2, 3)
    for bi in range(2):
        for bj in range(3):
            blk = w[128 * bi:128 * bi + 128, 128 * bj:128 * bj + 128]
            amax = np.abs(blk).max()
            s = np.float32(1.0) if amax == 0 else np.float32(amax) / np.float32(448)
            assert scales[bi, bj] == s
            want = ref.e4m3_encode_bruteforce((blk / s).astype(np.float32))
            assert np.array_equal(codes[128 * bi:128 * bi + 128, 128 * bj:128 * bj + 128], want)


def test_mxfp4_quantization_rule_bruteforce():
    rng = np.random.default_rng(1)
    w = (rng.standard_normal((64, 256)) * rng.choice([1e-3, 1, 40], (64, 1))).astype(np.float32)
    w[3, :32] = 0.0
    # exact ties on the e2m1 grid of a block whose amax is 6 * 2^0 (X = 0)
    w[5, :32] = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0] * 4, np.float32)
    packed, e8m0 = synth._quant_mxfp4(w)
    vals = ref.e2m1_values()
    nib = np.stack([packed & 0xF, packed >> 4], axis=-1).reshape(64, 256)
    for r in range(64):
        for b in range(8):
            blk = w[r, 32 * b:32 * b + 32].astype(np.float64)
            amax = np.abs(blk).max()
            X = 0 if amax == 0 else int(np.floor(np.log2(amax))) - 2
            assert e8m0[r, b] == X + 127
            v = blk / 2.0 ** X
            for i in range(32):
                d = np.abs(vals[:8] - min(abs(v[i]), 6.0))
                cands = np.flatnonzero(d == d.min())
                c = cands[0] if len(cands) == 1 else [x for x in cands if x % 2 == 0][0]
                assert nib[r, 32 * b + i] & 7 == c, (r, b, i, v[i])
                if v[i] != 0:
                    assert (nib[r, 32 * b + i] >> 3) == (v[i] < 0)
    assert list(nib[5, :8] & 7) == [0, 2, 2, 4, 4, 6, 6, 7]


def test_reproducible_and_prefix_stable():
    wl = synth.Workload("t", Mr=5, Ms=7, E=3, k=2, I=128, Is=128, wfmt=0, seed=3, H=256, L=256)
    a, b = synth.make_inputs(wl), synth.make_inputs(wl)
    for name in ("x_lat", "x_hid", "gate", "w1", "w1_scale", "w2", "w2_scale", "gamma", "w_up", "ws1", "ws2"):
        assert np.array_equal(getattr(a, name), getattr(b, name)), name
    c = synth.make_inputs(wl, Mr=3, Ms=9)
    assert np.array_equal(c.x_lat, a.x_lat[:3]) and np.array_equal(c.x_hid[:7], a.x_hid)
    assert np.array_equal(c.w1, a.w1)


def test_shapes_and_distributions():
    wl = replace(synth.WORKLOADS["tiny"], E=2)
    inp = synth.make_inputs(wl)
    assert inp.w1.shape == (2, 1024, 3584) and inp.w1_scale.shape == (2, 8, 28)
    assert inp.w2.shape == (2, 3584, 512) and inp.w2_scale.shape == (2, 28, 4)
    assert inp.w_up.shape == (7168, 3584) and inp.ws1.shape == (1024, 7168) and inp.ws2.shape == (7168, 512)
    x = ref.bf16_val(inp.x_lat)
    assert abs(x.std() - 1) < 0.02 and abs(inp.gate.std() - 0.02) < 0.001
    g = ref.bf16_val(inp.gamma)
    assert g.min() >= 0.5 and g.max() <= 1.5
    wup = ref.bf16_val(inp.w_up)
    assert abs(wup.std() * np.sqrt(3584) - 1) < 0.01
    z = replace(synth.WORKLOADS["mxfp4"], E=4, Mr=4, Ms=4, I=128, Is=128)
    zi = synth.make_inputs(z)
    assert np.allclose(zi.gate_bias, -1.2 * np.log(np.arange(1, 5)), rtol=1e-6)
    assert zi.w1.shape == (4, 256, 1792) and zi.w1_scale.shape == (4, 256, 112)
