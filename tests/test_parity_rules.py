"""The parity rules themselves, on CPU: the h-code rule accepts codes that
round a value near a midpoint and rejects anything else."""
import numpy as np
import pytest

from oracle import oracle as orc
from tests import parity as P


def test_encode_np_matches_oracle():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100000) * rng.choice([1e-3, 1, 100], 100000)).astype(np.float32)
    x = np.concatenate([x, P.e4m3_value(np.arange(127)).astype(np.float32), [0.0, -0.0, 500.0]]).astype(np.float32)
    assert np.array_equal(P.e4m3_encode_np(x), orc.e4m3_encode(x))


def _block(seed):
    rng = np.random.default_rng(seed)
    h = rng.standard_normal((4, 256)).astype(np.float32)
    q, s = orc.quant_1x128(h)
    return h, q, s


def test_h_rule_accepts_identical_and_midpoint_flips():
    h, q, s = _block(1)
    assert P.check_h_codes(q, s, q, s, h)[:2] == (0, q.size)
    # move one value exactly onto a midpoint and flip it to the other side
    vals = P.e4m3_value(np.arange(127))
    h2 = h.copy()
    r, c = 1, 5
    mid = (vals[60] + vals[61]) / 2 * s[r, c // 128]
    h2[r, c] = mid
    q2, _ = orc.quant_1x128(h2)
    g = q2.copy()
    g[r, c] = q2[r, c] ^ 1 if (q2[r, c] & 0x7F) in (60, 61) else q2[r, c]
    assert P.check_h_codes(g, s, q2, s, h2)[0] <= 1
    # across zero: a tiny h may land on +0 / -0 / the smallest codes
    h3 = h.copy()
    h3[2, 7] = 1e-9
    q3, _ = orc.quant_1x128(h3)
    g3 = q3.copy()
    g3[2, 7] = 0x80  # -0 against +0: the same value, not a flip
    assert P.check_h_codes(g3, s, q3, s, h3)[0] == 0
    g3[2, 7] = 0x01  # the smallest subnormal: one step from zero
    assert P.check_h_codes(g3, s, q3, s, h3)[0] == 1


def test_h_rule_rejects_far_flips_and_scale_drift():
    h, q, s = _block(2)
    g = q.copy()
    i = np.argmax(np.abs(h[0, :128]))
    g[0, i] = (g[0, i] & 0x80) | ((g[0, i] & 0x7F) - 2)
    with pytest.raises(AssertionError):
        P.check_h_codes(g, s, q, s, h)
    with pytest.raises(AssertionError):
        P.check_h_codes(q, s * 1.01, q, s, h)


def test_rel_errors_definition():
    o = np.array([1.0, -1.0, 0.0, 1e-6])
    g = o + np.array([0.01, 0.0, 0.001, 0.0])
    mx, mean = P.rel_errors(g, o)
    rms = np.sqrt(np.mean(o ** 2))
    assert np.isclose(mx, 0.01) and np.isclose(mean, (0.01 + 0.001 / rms) / 4)


def test_row_rel_errors_definition():
    o = np.array([[3.0, 4.0], [1.0, 0.0]])
    g = o + np.array([[0.05, 0.0], [0.0, 0.01]])
    mx, mean = P.row_rel_errors(g, o)
    assert np.isclose(mx, 0.01) and np.isclose(mean, 0.01)


def test_h_rule_one_step_where_the_band_is_narrower_than_the_spacing():
    # the largest value of a block sits at a normal code whose spacing is far
    # wider than the band: moving it onto a midpoint, only the neighbouring
    # code is admitted, never one two steps away
    h, q, s = _block(3)
    i = int(np.argmax(np.abs(h[1, :128])))
    vals = P.e4m3_value(np.arange(127))
    c = int(q[1, i] & 0x7F)
    h2 = h.copy()
    h2[1, i] = np.copysign((vals[c - 1] + vals[c - 2]) / 2 * s[1, 0], h[1, i])  # midpoint of codes c-2, c-1
    q2, _ = orc.quant_1x128(h2)
    g = q2.copy()
    g[1, i] = (q2[1, i] & 0x80) | ((q2[1, i] & 0x7F) ^ 1)  # the other code of the midpoint pair
    assert P.check_h_codes(g, s, q2, s, h2)[0] == 1
    g[1, i] = (q2[1, i] & 0x80) | ((q2[1, i] & 0x7F) - 2)
    with pytest.raises(AssertionError):
        P.check_h_codes(g, s, q2, s, h2)


def test_h_rule_admits_several_subnormal_steps_inside_the_band():
    # near zero the codes are 2^-9 of the scale apart, far below the band:
    # a value of a few subnormal steps may come out a few codes away
    h, q, s = _block(5)
    h2 = h.copy()
    h2[0, 3] = 5 * 2.0 ** -9 * s[0, 0]   # code 5 (subnormal)
    q2, _ = orc.quant_1x128(h2)
    g = q2.copy()
    g[0, 3] = (q2[0, 3] & 0x80) | 7      # two subnormal steps away: inside 5e-4 of the amax
    n, _, _, multi = P.check_h_codes(g, s, q2, s, h2)
    assert n == 1 and multi == 1


def test_output_gate_checks_both_statistics():
    rng = np.random.default_rng(4)
    o = rng.standard_normal((8, 64))
    P.assert_output_gate(o * (1 + 1e-3), o, "out")
    # one element off by 5 % of the rms: the elementwise max fails, the per-token norm passes
    g = o.copy()
    g[3, 5] += 0.05 * np.sqrt(np.mean(o * o))
    assert P.row_rel_errors(g, o)[0] <= 2e-2
    with pytest.raises(AssertionError):
        P.assert_output_gate(g, o, "out")
