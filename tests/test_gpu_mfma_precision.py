"""How the matrix cores round the FP8 block product of the routed GEMMs, and
what that does to h.  This is the measurement the h-code tolerance H_TOL
rests on.  MI355X only (marker ``gpu``).

The routed L1 sums K = 3584 products as 28 block products of 128 (one
matrix-core instruction each, unit scales), each promoted by its two block
scales and added in FP32.  The oracle sums the same dequantized products one
by one in FP32.  The two sums differ, so h = silu(gate) * up differs, and the
h codes can differ where h lies close to a rounding midpoint.

The probe (moe_tail_probe_mfma_fp8) runs the same instruction on given codes:
* sums whose every partial sum is exact in a short significand come out
  exact;
* a small product beside a large one in the same instruction may lose low
  bits (the instruction's internal precision is coarser than FP32);
* on the decode workload's own x codes and W1 weights, h formed from the
  instruction's block sums moves by at most H_TOL / 5 of its 1x128 block
  amax, and so does the oracle's FP32 h.  Both are measured against the exact
  (float64) h of the same quantized operands, so the two sides can differ by
  at most 2 H_TOL / 5 < H_TOL.
"""
import numpy as np
import pytest
import torch

from latent_moe_layer_amd import binding as B
from latent_moe_layer_amd import synth
from oracle import oracle as orc
from tests import parity as P

pytestmark = pytest.mark.gpu

E4M3_ONE = 0x38
E4M3_448 = 0x7E


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.probes()


def mfma(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """[n, 16, 128] codes x [n, 16, 128] codes -> [n, 16, 16] f32 on the GPU."""
    a = np.ascontiguousarray(a, np.uint8)
    b = np.ascontiguousarray(b, np.uint8)
    n = a.shape[0]
    da, db = torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda()
    dc = torch.empty((n, 16, 16), dtype=torch.float32, device="cuda")
    B.moe_tail_probe_mfma_fp8(da, db, dc, n)
    torch.cuda.synchronize()
    return dc.cpu().numpy()


def exact(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """The same block products in float64 (exact for e4m3 operands)."""
    return np.einsum("nik,njk->nij", P.e4m3_value(a), P.e4m3_value(b))


def e4m3_code(v: float) -> int:
    return int(P.e4m3_encode_np(np.array([v]))[0])


def test_exact_when_every_partial_sum_is_short():
    # values in {+-0.5, +-1, +-1.5, +-2}: products are multiples of 1/4 below 4 in
    # magnitude, so every partial sum has a few significant bits
    rng = np.random.default_rng(0)
    pool = np.array([e4m3_code(v) for v in (0.5, 1.0, 1.5, 2.0, -0.5, -1.0, -1.5, -2.0)], np.uint8)
    a = rng.choice(pool, (64, 16, 128))
    b = rng.choice(pool, (64, 16, 128))
    assert np.array_equal(mfma(a, b).astype(np.float64), exact(a, b))


def test_small_products_beside_a_large_one():
    """448 * 1 at K index 0 and small addends 2^-j * 1 elsewhere: what the
    instruction keeps of them (printed), and the bounds asserted below."""
    rows = []
    cases = []
    for j in range(0, 19):
        for kk in (1, 7, 8, 31, 64, 127):
            a = np.zeros((16, 128), np.uint8)
            b = np.zeros((16, 128), np.uint8)
            a[0, 0], b[0, 0] = E4M3_448, E4M3_ONE
            # 2^-j as (2^-ja) * (2^-jb), each factor an e4m3 value
            ja, jb = min(j, 9), j - min(j, 9)
            a[0, kk], b[0, kk] = e4m3_code(2.0 ** -ja), e4m3_code(2.0 ** -jb)
            cases.append((j, kk))
            rows.append((a, b))
    a = np.stack([r[0] for r in rows])
    b = np.stack([r[1] for r in rows])
    got = mfma(a, b)[:, 0, 0].astype(np.float64)
    kept = got - 448.0
    table = {}
    for (j, kk), kv in zip(cases, kept):
        addend = 2.0 ** -j
        table.setdefault(j, []).append(kv / addend)
        # never more than the addend is lost, nothing is invented
        assert -1e-12 <= kv <= addend * (1 + 1e-12), (j, kk, kv)
        # addends down to 2^-5 (2^-13.8 of the large product) are kept exactly
        if j <= 5:
            assert kv == addend, (j, kk, kv)
    print("fraction of a 2^-j addend kept beside 448 (K index 1, 7, 8, 31, 64, 127):")
    for j, fr in table.items():
        print(f"  j={j:2d}: " + " ".join(f"{f:.3f}" for f in fr))

    # many small addends beside the large one: the worst case of the loss
    a = np.zeros((1, 16, 128), np.uint8)
    b = np.zeros((1, 16, 128), np.uint8)
    a[0, 0, 0], b[0, 0, 0] = E4M3_448, E4M3_ONE
    a[0, 0, 1:] = e4m3_code(2.0 ** -9)
    b[0, 0, 1:] = E4M3_ONE
    lost = float(exact(a, b)[0, 0, 0] - mfma(a, b)[0, 0, 0])
    print(f"127 addends of 2^-9 beside 448: lost {lost:.6g} ({lost / 448.0:.3e} of the large product)")
    assert 0.0 <= lost <= 127 * 2.0 ** -9


def test_random_operands_error_bound():
    """Full-range random codes: |instruction - exact| against the sum of the
    magnitudes of the products (printed: the measured ratio)."""
    rng = np.random.default_rng(1)
    codes = rng.integers(0, 256, (2048, 16, 128)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0  # no NaN codes
    a, b = codes[:1024], codes[1024:]
    got = mfma(a, b).astype(np.float64)
    ex = exact(a, b)
    mag = np.einsum("nik,njk->nij", np.abs(P.e4m3_value(a)), np.abs(P.e4m3_value(b)))
    ratio = np.abs(got - ex) / np.maximum(mag, 1e-300)
    print(f"random codes: max |err| / sum|p| = {ratio.max():.3e} (2^{np.log2(max(ratio.max(), 1e-300)):.1f})")
    assert ratio.max() <= 2.0 ** -12


def _h_from_g(g: np.ndarray, I: int) -> np.ndarray:
    gate, up = g[..., :I], g[..., I:]
    return gate / (1.0 + np.exp(-gate)) * up


def test_h_deviation_on_workload_operands():
    """The decode workload's own x codes and W1 weights: h formed from the
    instruction's block sums (promoted by the block scales, as the routed L1
    does) and the oracle's FP32 h, each against the exact h of the same
    quantized operands, in units of the 1x128 block amax of the exact h."""
    wl = synth.WORKLOADS["decode"]
    inp = synth.make_inputs(wl)
    L, I = wl.L, wl.I
    nkb = L // 128
    toks = np.arange(16)
    xq, sx = orc.quant_1x128(P.bf16_to_f32(inp.x_lat[toks]))           # [16, L], [16, L/128]
    probes = ((0, 0), (7, 5), (33, 15), (63, 9))  # (expert, 128-column block of h)
    # the oracle's FP32 h of these tokens for these experts: routing given to
    # it directly, one probed expert per slot
    ids = np.tile(np.array([e for e, _ in probes] + [1, 2, 3, 4], np.int32), (wl.Mr, 1))
    ref = orc.forward(inp, ids, np.full(ids.shape, 1.0 / wl.k, np.float32), sel=toks.astype(np.int32))
    worst_mfma = worst_orc = 0.0
    for slot, (e, hb) in enumerate(probes):
        rows = np.concatenate([np.arange(128 * hb, 128 * hb + 128), I + np.arange(128 * hb, 128 * hb + 128)])
        wq = inp.w1[e][rows]                                           # [256, L] codes
        ws = inp.w1_scale[e][rows // 128]                              # [256, L/128]
        # block products on the GPU: [kb][row block of 16 weight rows] -> 16 x 16
        a = np.stack([xq[:, 128 * kb:128 * kb + 128] for kb in range(nkb) for _ in range(16)])
        b = np.stack([wq[16 * rb:16 * rb + 16, 128 * kb:128 * kb + 128] for kb in range(nkb) for rb in range(16)])
        c = mfma(a, b).astype(np.float64).reshape(nkb, 16, 16, 16)     # [kb, rb, tok, row in rb]
        c = c.transpose(0, 2, 1, 3).reshape(nkb, 16, 256)              # [kb, tok, row]
        ce = exact(a, b).reshape(nkb, 16, 16, 16).transpose(0, 2, 1, 3).reshape(nkb, 16, 256)
        sig = sx.T[:, :, None] * ws.T[:, None, :]                      # [kb, tok, row]
        g_mfma = np.sum(c * sig, axis=0)
        g_exact = np.sum(ce * sig, axis=0)
        h_mfma, h_exact = _h_from_g(g_mfma, 128), _h_from_g(g_exact, 128)
        amax = np.max(np.abs(h_exact), axis=1, keepdims=True)
        worst_mfma = max(worst_mfma, float(np.max(np.abs(h_mfma - h_exact) / amax)))
        h_orc = ref.h[:, slot, 128 * hb:128 * hb + 128].astype(np.float64)
        worst_orc = max(worst_orc, float(np.max(np.abs(h_orc - h_exact) / amax)))
    print(f"h deviation / block amax: matrix cores {worst_mfma:.3e}, oracle FP32 {worst_orc:.3e}; "
          f"H_TOL / 5 = {P.H_TOL / 5:.1e}")
    assert worst_mfma <= P.H_TOL / 5
    assert worst_orc <= P.H_TOL / 5
