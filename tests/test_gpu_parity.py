"""Parity of the HIP path against the CPU oracle on small and ragged tails,
edge cases and invariants.  Runs on an MI355X only (marker ``gpu``)."""
from dataclasses import replace

import numpy as np
import pytest
import torch

from latent_moe_layer_amd import binding as B
from latent_moe_layer_amd import synth
from latent_moe_layer_amd.device import DeviceTail, to_np
from oracle import oracle as orc
from tests import parity as P

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()  # a missing library fails loudly here


def run(inp, Mr=None, Ms=None, residual=None):
    dev = DeviceTail(inp, "cuda:0", Mr=Mr, Ms=Ms)
    dev.set_residual(residual)
    dev.route()
    dev.forward()
    torch.cuda.synchronize()
    return dev


def check_routing(dev, inp):
    Mr, wl = dev.Mr, inp.wl
    ids, w = to_np(dev.topk_ids), to_np(dev.topk_w)
    oids, ow = orc.route(inp.x_lat[:Mr], inp.gate, inp.gate_bias, wl.k)
    assert np.array_equal(ids, oids), "expert ids differ"
    assert np.max(np.abs(w - ow), initial=0.0) <= 1e-6, "routing weights differ"
    off, sp, p2r = orc.permute(oids, wl.E)
    assert np.array_equal(to_np(dev.offsets), off)
    assert np.array_equal(to_np(dev.sorted_pair), sp)
    assert np.array_equal(to_np(dev.pair_to_row), p2r)
    return oids, ow, p2r


def check_forward(dev, inp, sel=None, report=None, residual=None):
    """Compare outputs and intermediates on the tokens in `sel` (default all);
    `residual` ([Mr, H] bf16 bits): the add3 output is expected.

    Two comparisons with the oracle (the rule in tests/parity.py):
    * direct: the oracle's own pipeline.  x codes bit for bit, h codes by the
      midpoint rule, y and rn per row, out per token and by the elementwise
      mean (the elementwise max is reported: legitimate h-code flips set it);
      shared_out (no h on its path) elementwise and per token;
    * given the GPU's h codes: the oracle continues from exactly the codes the
      GPU produced, so every later step (routed L2, combine, RMSNorm, shared
      expert, up-projection, the joins) is checked elementwise and per token
      with the full bar."""
    wl, Mr, Ms = inp.wl, dev.Mr, dev.Ms
    oids, ow, p2r = check_routing(dev, inp)
    if sel is None:
        sel = np.arange(Ms, dtype=np.int32)
    sel = np.asarray(sel, np.int32)
    ref = orc.forward(inp, oids, ow, sel=sel, Mr=Mr, Ms=Ms, residual=residual)
    inter = {k: to_np(v) for k, v in dev.intermediates().items()}
    rsel = np.flatnonzero(sel < Mr)
    ssel = np.flatnonzero(sel >= Mr)
    stats = {}
    if rsel.size:
        toks = sel[rsel]
        # x codes and scales: bit-exact
        assert np.array_equal(inter["xq"][toks], ref.xq[rsel]), "x codes differ"
        assert np.array_equal(inter["sx"][toks], ref.sx[rsel]), "x scales differ"
        # h codes: the midpoint rule, one code step at most
        rows = p2r.reshape(Mr, wl.k)[toks]                      # [n, k]
        n_mis, n_tot, sdev, multi = P.check_h_codes(inter["hq"][rows], inter["sh"][rows], ref.hq[rsel],
                                                    ref.sh[rsel], ref.h[rsel])
        stats["h_flips"] = (n_mis, n_tot)
        stats["h_flips_multi_step_near_zero"] = multi
        stats["h_scale_dev"] = sdev
        # routed L2 output and the normalized latent, per row
        ymax, ymean = P.row_rel_errors(inter["y"][rows], ref.y[rsel])
        rmax, rmean = P.row_rel_errors(P.bf16_to_f32(inter["rn"][toks]), P.bf16_to_f32(ref.rn[rsel]))
        stats["y"] = (ymax, ymean)
        stats["rn"] = (rmax, rmean)
        assert ymax <= P.MAX_REL_INTERMEDIATE and ymean <= P.MEAN_REL, stats
        assert rmax <= P.MAX_REL_INTERMEDIATE and rmean <= P.MEAN_REL, stats
        # final output against the oracle's FP32 value: elementwise and per token
        got = P.bf16_to_f32(to_np(dev.out)[toks])
        stats["out_bitwise_frac"] = float(np.mean(to_np(dev.out)[toks] == ref.out_bf16[rsel]))
        stats.update(P.assert_output_gate(got, ref.out_f32[rsel], "out", elementwise_max=False))
        # the oracle continued from the GPU's own h codes
        hq_g = np.zeros((sel.size, wl.k, wl.I), np.uint8)
        sh_g = np.ones((sel.size, wl.k, wl.I // 128), np.float32)
        hq_g[rsel] = inter["hq"][rows]
        sh_g[rsel] = inter["sh"][rows]
        cref = orc.forward(inp, oids, ow, sel=sel, Mr=Mr, Ms=Ms, residual=residual, h_codes=(hq_g, sh_g))
        cy = P.row_rel_errors(inter["y"][rows], cref.y[rsel])
        stats["given_h_y_elementwise"] = P.rel_errors(inter["y"][rows], cref.y[rsel])
        stats["given_h_y"] = cy
        assert cy[0] <= P.MAX_REL and cy[1] <= P.MEAN_REL, stats
        stats.update(P.assert_output_gate(got, cref.out_f32[rsel], "given_h_out"))
    if ssel.size:
        got = P.bf16_to_f32(to_np(dev.shared_out)[sel[ssel] - Mr])
        stats.update(P.assert_output_gate(got, ref.out_f32[ssel], "shared_out"))
    if report is not None:
        report.update(stats)
    print(stats)
    return stats


# ------------------------------------------------------------------ tests --

def test_quantizer_bit_exact():
    rng = np.random.default_rng(0)
    rows, cols = 97, 1024
    x = (rng.standard_normal((rows, cols)) * rng.choice([1e-4, 1e-2, 1, 50, 3e4], (rows, 1))).astype(np.float32)
    x[1, :128] = 0.0
    x[2, 128:256] = -0.0
    x[3, :] = np.float32(448.0)
    vals = P.e4m3_value(np.arange(127))
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    # block amax 448 -> scale exactly 1: every midpoint between codes, and one ulp below it
    x[4:6, :] = 0.0
    x[4, :126] = mids[:126]
    x[4, 127] = 448.0
    x[5, :126] = np.nextafter(mids[:126], np.float32(0))
    x[5, 127] = 448.0
    xd = torch.from_numpy(x).cuda()
    q = torch.empty((rows, cols), dtype=torch.uint8, device="cuda")
    s = torch.empty((rows, cols // 128), dtype=torch.float32, device="cuda")
    B.moe_tail_quant_fp8_1x128(xd, False, rows, cols, q, s)
    oq, os_ = orc.quant_1x128(x)
    torch.cuda.synchronize()
    assert np.array_equal(to_np(q), oq)
    assert np.array_equal(to_np(s), os_)
    # bf16 input path
    xb = synth.f32_to_bf16_bits(x)
    B.moe_tail_quant_fp8_1x128(torch.from_numpy(xb.view(np.int16)).cuda(), True, rows, cols, q, s)
    oq, os_ = orc.quant_1x128(P.bf16_to_f32(xb))
    torch.cuda.synchronize()
    assert np.array_equal(to_np(q), oq)
    assert np.array_equal(to_np(s), os_)


# Shapes of every routing path: top-k and permutation in one workgroup (Mr <= 16: 1, 2, 6 and 16
# experts per lane), top-k then the one-workgroup permutation (from 17 tokens), and the grid-wide
# permutation (more than 24 groups of 64 tokens).  Each is routed twice in a row, the outputs
# poisoned before each call.
@pytest.mark.parametrize("E,k,Mr,zipf", [(8, 2, 16, 0.0), (64, 8, 128, 0.0), (64, 8, 4096, 0.0), (128, 8, 1024, 1.2),
                                         (384, 8, 2048, 0.0), (1024, 16, 200, 0.0), (5, 5, 70, 0.0), (9, 3, 1, 0.0),
                                         (16, 4, 130, 0.0), (64, 8, 530, 0.0), (32, 4, 1600, 0.0),
                                         (128, 8, 16, 1.2), (384, 8, 13, 0.0), (1024, 16, 16, 0.0), (64, 8, 17, 0.0),
                                         (256, 8, 100, 1.2), (64, 8, 511, 0.0)])
def test_route_bit_exact(E, k, Mr, zipf):
    wl = synth.Workload("r", Mr=Mr, Ms=Mr, E=E, k=k, I=128, Is=128, wfmt=0, seed=100 + E, zipf_s=zipf)
    inp = synth.make_inputs(wl, routing_only=True)
    dev = DeviceTail(inp, "cuda:0", Mr=Mr, Ms=Mr)
    for _ in range(2):
        for t in (dev.topk_ids, dev.offsets, dev.sorted_pair, dev.pair_to_row):
            t.fill_(-1)
        dev.topk_w.fill_(float("nan"))
        dev.route()
        torch.cuda.synchronize()
        check_routing(dev, inp)


@pytest.mark.parametrize("L,Mr,E,k", [(256, 7, 12, 3), (768, 33, 20, 4), (256, 64, 16, 2)])
def test_route_bit_exact_narrow_latent(L, Mr, E, k):
    # the few-token logits tiling (2 tokens x 1 expert per wave) at narrow
    # latents: L = 256 makes its x tile exactly one 1 KB block; odd token and
    # expert counts leave partial tiles (rows past Mr and experts past E)
    wl = synth.Workload("rn", Mr=Mr, Ms=Mr, E=E, k=k, I=128, Is=128, wfmt=0, seed=200 + L + E, H=256, L=L)
    inp = synth.make_inputs(wl, routing_only=True)
    dev = DeviceTail(inp, "cuda:0", Mr=Mr, Ms=Mr)
    for t in (dev.topk_ids, dev.offsets, dev.sorted_pair, dev.pair_to_row):
        t.fill_(-1)
    dev.topk_w.fill_(float("nan"))
    dev.route()
    torch.cuda.synchronize()
    check_routing(dev, inp)


def test_route_all_equal_logits():
    wl = synth.Workload("r", Mr=70, Ms=70, E=16, k=4, I=128, Is=128, wfmt=0, seed=5, zero_router=True)
    inp = synth.make_inputs(wl, routing_only=True)
    dev = DeviceTail(inp, "cuda:0", Mr=70, Ms=70)
    dev.route()
    torch.cuda.synchronize()
    ids = to_np(dev.topk_ids)
    assert np.array_equal(ids, np.tile(np.arange(4, dtype=np.int32), (70, 1)))
    assert np.all(to_np(dev.topk_w) == np.float32(0.25))
    check_routing(dev, inp)


def test_forward_tiny_full():
    inp = synth.make_inputs("tiny")
    dev = run(inp)
    check_forward(dev, inp)


@pytest.mark.parametrize("wfmt", [synth.WFMT_FP8, synth.WFMT_MXFP4, synth.WFMT_NVFP4])
def test_forward_ragged(wfmt):
    # several tiles and a ragged tail in every dimension the grid splits.  I is
    # the smallest workload's 512: one legitimate h-code flip moves the output
    # by about 1/sqrt(I) of its rms, so much narrower experts would need a
    # looser bar than the workloads' 2e-2.
    wl = synth.Workload("ragged", Mr=37, Ms=53, E=8, k=3, I=512, Is=384, wfmt=wfmt, seed=21,
                        zipf_s=1.2 if wfmt == synth.WFMT_MXFP4 else 0.0)
    inp = synth.make_inputs(wl)
    dev = run(inp)
    check_forward(dev, inp)


def test_forward_mxfp4_width_not_a_multiple_of_256():
    # MXFP4 experts 640 wide: the tiled kernel's small MXFP4 tiles step 256 K
    # at a time, so every routed GEMM runs on the row-streaming kernel here
    wl = synth.Workload("fp4w640", Mr=37, Ms=53, E=8, k=3, I=640, Is=384, wfmt=synth.WFMT_MXFP4, seed=26,
                        zipf_s=1.2, H=1024, L=512)
    inp = synth.make_inputs(wl)
    dev = run(inp)
    check_forward(dev, inp)


@pytest.mark.parametrize("wfmt", [synth.WFMT_FP8, synth.WFMT_MXFP4, synth.WFMT_NVFP4])
def test_forward_tiled_path(wfmt):
    # Past 256 tokens FP8 experts with >= 128 rows take 128-row tiles (here
    # most experts, ~150 rows each: full and partial 128-row tiles), the
    # others 32- or 64-row tiles; MXFP4 experts take 32- and 64-row tiles,
    # NVFP4 experts several 32-row tiles; M > 128 takes the tiled dense
    # kernel for the shared expert and the up-projection.
    wl = synth.Workload("tiled", Mr=300, Ms=333, E=16 if wfmt == synth.WFMT_MXFP4 else 18, k=8, I=512, Is=512, wfmt=wfmt, seed=30,
                        zipf_s=0.3 if wfmt == synth.WFMT_MXFP4 else 0.0)
    inp = synth.make_inputs(wl)
    dev = run(inp)
    loads = np.diff(to_np(dev.offsets))
    assert loads.max() >= 128 and loads.min() < 128, loads
    rng = np.random.default_rng(3)
    sel = np.concatenate([np.sort(rng.choice(300, 24, replace=False)), [0, 299, 300, 332]]).astype(np.int32)
    check_forward(dev, inp, sel=np.unique(sel))


@pytest.mark.parametrize("wfmt", [synth.WFMT_FP8, synth.WFMT_MXFP4])
def test_forward_tiled_several_tiles_per_workgroup(wfmt):
    # ~36 row tiles x 16 n tiles (L1) and x 8 (L2): more tiles than workgroups,
    # so each persistent workgroup runs two or three tiles back to back and
    # loads the next tile's rows, pair ids and weight scales while the
    # current one finishes.  Outputs are checked on a sample of tokens.
    wl = synth.Workload("multi", Mr=1024, Ms=1184, E=8, k=4, I=2048, Is=256, wfmt=wfmt, seed=31, H=2048, L=2048,
                        zipf_s=0.4 if wfmt else 0.0)
    inp = synth.make_inputs(wl)
    dev = run(inp)
    loads = np.diff(to_np(dev.offsets))
    assert loads.min() >= 128, loads
    rng = np.random.default_rng(5)
    sel = np.concatenate([np.sort(rng.choice(1024, 40, replace=False)), [0, 1023, 1024, 1183]]).astype(np.int32)
    check_forward(dev, inp, sel=np.unique(sel))


# ------------------------------------------------------------------- add3 --
# The up-projection epilogue joining the residual stream: out = bf16((up +
# shared) + residual), one rounding (tokenspeed PR "MNNVL CuTe-DSL finalize
# tail + K3 comm layer extraction", commit log).

@pytest.mark.parametrize("Mr,Ms", [(40, 56), (300, 320)])  # small-M dense path, tiled dense path
def test_forward_add3(Mr, Ms):
    wl = synth.Workload("add3", Mr=Mr, Ms=Ms, E=8, k=2, I=256, Is=256, wfmt=0, seed=41 + Mr, H=1024, L=512)
    inp = synth.make_inputs(wl)
    r = synth.make_residual(wl)
    dev = run(inp, residual=r)
    check_forward(dev, inp, residual=r)
    # the same call without the residual: shared_out rows are untouched by it
    plain = run(inp)
    assert np.array_equal(to_np(dev.shared_out), to_np(plain.shared_out))


def test_forward_add3_decode_sampled():
    wl = synth.WORKLOADS["decode"]
    inp = synth.make_inputs(wl)
    r = synth.make_residual(wl)
    dev = run(inp, residual=r)
    sel = np.array([0, 1, 37, 64, 100, 127], np.int32)
    check_forward(dev, inp, sel=sel, residual=r)


def test_forward_add3_without_routed_tokens():
    # Mr = 0: no up-projection, the residual may be NULL, the shared rows are the plain ones
    wl = synth.Workload("a3mr0", Mr=0, Ms=20, E=4, k=2, I=128, Is=256, wfmt=0, seed=24)
    inp = synth.make_inputs(wl)
    dev = DeviceTail(inp, "cuda:0")
    B.moe_tail_forward_add3(dev.dims, dev.weights, dev.t["x_lat"], 0, dev.t["x_hid"], dev.Ms, dev.routing, None,
                            dev.out, dev.shared_out, dev.ws, dev.ws_bytes)
    torch.cuda.synchronize()
    got = to_np(dev.shared_out)
    plain = run(inp)
    assert np.array_equal(got, to_np(plain.shared_out))


@pytest.mark.parametrize("wfmt", [0, 1])
def test_forward_256_row_tiles(wfmt):
    # about 490 rows per expert: a full 256-row tile and a ragged second one
    # (experts between 385 and 512 rows take 256-row tiles)
    wl = synth.Workload("huge", Mr=960, Ms=1100, E=4, k=2, I=512, Is=256, wfmt=wfmt, seed=51, H=1024, L=512)
    inp = synth.make_inputs(wl)
    dev = run(inp)
    loads = np.diff(to_np(dev.offsets))
    assert loads.min() > 384 and loads.max() <= 512 and np.all(loads % 256 != 0), loads
    check_forward(dev, inp)


@pytest.mark.parametrize("wfmt", [0, 1])
def test_forward_256_row_tiles_short_tail(wfmt):
    # about 300 rows per expert: one full 256-row tile and a tail of at most
    # 128 rows, which goes to a 128-row tile past the expert's 256-row tiles
    wl = synth.Workload("tail", Mr=600, Ms=640, E=4, k=2, I=512, Is=256, wfmt=wfmt, seed=52, H=1024, L=512)
    inp = synth.make_inputs(wl)
    dev = run(inp)
    loads = np.diff(to_np(dev.offsets))
    assert loads.min() > 256 and loads.max() <= 384, loads
    check_forward(dev, inp)


@pytest.mark.parametrize("wfmt", [0, 1])
@pytest.mark.parametrize("Mr,E", [(200, 8), (600, 16)])
def test_forward_64_row_tiles(Mr, E, wfmt):
    # experts averaging more than 32 rows: those with 33 .. 127 rows take
    # 64-row tiles (ragged), the others 32-row tiles, and from 257 tokens on
    # experts with 128 rows or more take the 128- and 256-row tiles
    wl = synth.Workload("mid", Mr=Mr, Ms=Mr + 20, E=E, k=2, I=512, Is=256, wfmt=wfmt, seed=53 + E, H=1024, L=512,
                        zipf_s=0.6)
    inp = synth.make_inputs(wl)
    dev = run(inp)
    loads = np.diff(to_np(dev.offsets))
    assert np.any((loads > 32) & (loads < 128)) and np.any(loads % 64 != 0), loads
    check_forward(dev, inp)


@pytest.mark.parametrize("Mr", [40, 300])
def test_forward_mxfp4_skewed_loads(Mr):
    # strongly skewed MXFP4 loads (at 300 tokens: 0 .. 15, 20, 49, 100, 152,
    # 251, 296, 300 rows): every tile size at once, experts with a handful of
    # rows on the 32-row tiles, with MXFP4's two K blocks per step; more
    # shared than routed tokens keeps the forward on one launch per stage
    wl = synth.Workload("tiny16", Mr=Mr, Ms=320, E=16, k=4, I=512, Is=256, wfmt=synth.WFMT_MXFP4, seed=87,
                        H=1024, L=512, zipf_s=1.2)
    inp = synth.make_inputs(wl)
    dev = run(inp)
    loads = np.diff(to_np(dev.offsets))
    assert np.any((loads > 0) & (loads <= 16)) and np.any(loads > 16), loads
    check_forward(dev, inp)


def test_forward_heavy_expert_many_row_tiles():
    # all-equal logits: every token goes to experts 0..k-1, 100 rows each (4 row tiles per expert)
    wl = synth.Workload("heavy", Mr=100, Ms=100, E=6, k=2, I=512, Is=128, wfmt=0, seed=22, zero_router=True)
    inp = synth.make_inputs(wl)
    dev = run(inp)
    check_forward(dev, inp)


@pytest.mark.parametrize("wfmt", [synth.WFMT_FP8, synth.WFMT_MXFP4, synth.WFMT_NVFP4])
def test_forward_top16(wfmt):
    # the widest routing the kernels take (k = 16): every lane of a 1x128
    # block's 16 writes its slot's copy of the x scale (the by-row copy the
    # tiled routed L1 reads), and every token reaches 16 of 24 experts; the
    # decode-sized schedule, one expert past 32 rows on several tiles
    wl = synth.Workload("top16", Mr=45, Ms=60, E=24, k=16, I=512, Is=256, wfmt=wfmt, seed=95, H=1024, L=768,
                        zipf_s=0.8)
    inp = synth.make_inputs(wl)
    dev = run(inp)
    loads = np.diff(to_np(dev.offsets))
    assert loads.sum() == 45 * 16 and loads.max() > 32, loads
    check_forward(dev, inp)


@pytest.mark.parametrize("wfmt,E,k,I,L", [(synth.WFMT_FP8, 512, 8, 512, 512), (synth.WFMT_MXFP4, 512, 8, 512, 512),
                                          (synth.WFMT_FP8, 1024, 16, 512, 256)])
def test_forward_expert_count_limits(wfmt, E, k, I, L):
    # 512 experts: the most the tiled kernels hold in their LDS expert tables
    # (32-row tiles for most experts, 64- and 128-row ones for the heavy ones
    # of the skewed loads); 1024 experts at top-16: past that limit, every
    # routed GEMM on the row-streaming kernels (L = 256 keeps them there).
    # More shared than routed tokens, every token compared.  (Experts at
    # least 512 wide: at 128, one legitimate h-code flip of a large code
    # moves its routed row's y by about 2 %, the per-row bar itself.)
    Mr = 700 if E <= 512 else 300
    wl = synth.Workload("maxe", Mr=Mr, Ms=Mr + 20, E=E, k=k, I=I, Is=128, wfmt=wfmt, seed=97 + E + wfmt, H=512, L=L,
                        zipf_s=0.15)
    inp = synth.make_inputs(wl)
    dev = run(inp)
    loads = np.diff(to_np(dev.offsets))
    assert loads.sum() == Mr * k and np.count_nonzero(loads) > E // 2, loads
    if E <= 512:
        assert loads.max() >= 128, loads.max()  # heavy experts on the larger tiles
    check_forward(dev, inp)


@pytest.mark.parametrize("wfmt,I,L", [(synth.WFMT_FP8, 512, 8192), (synth.WFMT_FP8, 8192, 512),
                                      (synth.WFMT_MXFP4, 512, 8192), (synth.WFMT_MXFP4, 8192, 512),
                                      (synth.WFMT_NVFP4, 384, 8192), (synth.WFMT_NVFP4, 8064, 512)])
def test_forward_width_limits(wfmt, I, L):
    # the widest reductions the kernels take: L = 8192 (the routed L1's and
    # the up-projection's K, and RMSNorm's width) and I = 8192 (the routed
    # L2's K), 64 scale blocks along K, which fill the kernels' LDS scale
    # tables; FP8 and MXFP4 on the tiled kernels, NVFP4 with the other
    # width not a multiple of 256, so on the row-streaming kernels
    wl = synth.Workload("maxw", Mr=24, Ms=30, E=3, k=2, I=I, Is=256, wfmt=wfmt, seed=131 + wfmt, H=1024, L=L)
    inp = synth.make_inputs(wl)
    dev = run(inp)
    check_forward(dev, inp)


def test_forward_nvfp4_skewed_and_narrow():
    # NVFP4 weights on skewed loads (a few heavy experts, many empty ones),
    # with more shared than routed tokens; experts 384 wide (not a multiple
    # of 256) keep the routed GEMMs on the row-streaming kernels
    wl = synth.Workload("nv", Mr=96, Ms=120, E=32, k=4, I=384, Is=256, wfmt=synth.WFMT_NVFP4, seed=91, zipf_s=1.2)
    inp = synth.make_inputs(wl)
    dev = run(inp)
    loads = np.diff(to_np(dev.offsets))
    assert np.any(loads == 0) and loads.max() > 32, loads
    check_forward(dev, inp)


def test_forward_no_routed_tokens():
    wl = synth.Workload("mr0", Mr=0, Ms=20, E=4, k=2, I=128, Is=256, wfmt=0, seed=23)
    inp = synth.make_inputs(wl)
    dev = run(inp)
    check_forward(dev, inp)


def test_forward_single_token_all_experts():
    wl = synth.Workload("e_eq_k", Mr=1, Ms=1, E=4, k=4, I=128, Is=128, wfmt=0, seed=24)
    inp = synth.make_inputs(wl)
    dev = run(inp)
    check_forward(dev, inp)


def test_zero_shared_weights():
    wl = replace(synth.WORKLOADS["tiny"], zero_shared=True, seed=25)
    inp = synth.make_inputs(wl)
    dev = run(inp)
    assert np.all(to_np(dev.intermediates()["s"]) == 0)
    check_forward(dev, inp)


def test_identical_experts_match_dense():
    wl = replace(synth.WORKLOADS["tiny"], identical_experts=True, zero_router=True, k=2, seed=26)
    inp = synth.make_inputs(wl)
    dev = run(inp)
    check_forward(dev, inp)
    dense = synth.make_inputs(replace(wl, E=1, k=1))
    ddev = run(dense)
    a = P.bf16_to_f32(to_np(dev.intermediates()["rn"]))
    b = P.bf16_to_f32(to_np(ddev.intermediates()["rn"]))
    mx, mean = P.row_rel_errors(a, b)
    assert mx <= 2e-2 and mean <= 3e-3


def test_deterministic_bitwise():
    inp = synth.make_inputs(synth.Workload("det", Mr=45, Ms=60, E=16, k=4, I=256, Is=256, wfmt=0, seed=27))
    a = run(inp)
    out1, so1, hq1 = to_np(a.out).copy(), to_np(a.shared_out).copy(), to_np(a.intermediates()["hq"]).copy()
    a.route()
    a.forward()
    torch.cuda.synchronize()
    assert np.array_equal(to_np(a.out), out1)
    assert np.array_equal(to_np(a.shared_out), so1)
    assert np.array_equal(to_np(a.intermediates()["hq"]), hq1)


def test_shared_rows_independent_of_routed_count():
    wl = synth.Workload("t5", Mr=24, Ms=40, E=8, k=2, I=128, Is=256, wfmt=0, seed=28)
    inp = synth.make_inputs(wl)
    a = run(inp)
    b = run(inp, Mr=0, Ms=40)
    assert np.array_equal(to_np(a.shared_out), to_np(b.shared_out)[24:])
    # and rows < Mr of the shared output equal the Mr=0 run's rows
    assert np.array_equal(to_np(a.intermediates()["s"]), to_np(b.shared_out)[:24])


def test_token_permutation():
    wl = synth.Workload("perm", Mr=33, Ms=33, E=8, k=2, I=256, Is=128, wfmt=0, seed=29)
    inp = synth.make_inputs(wl)
    a = run(inp)
    perm = np.random.default_rng(1).permutation(33)
    inp2 = synth.make_inputs(wl)
    inp2.x_lat = inp.x_lat[perm].copy()
    inp2.x_hid = inp.x_hid[perm].copy()
    b = run(inp2)
    ga, gb = P.bf16_to_f32(to_np(a.out)[perm]), P.bf16_to_f32(to_np(b.out))
    mx, mean = P.row_rel_errors(gb, ga)
    assert mx <= 2e-2 and mean <= 3e-3
    print("bitwise-equal fraction under permutation:", float(np.mean(to_np(a.out)[perm] == to_np(b.out))))
