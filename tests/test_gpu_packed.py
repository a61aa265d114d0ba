"""MXFP4 and NVFP4 scales in the tiled kernels' order
(moe_tail_pack_mxfp4_scales, moe_tail_pack_nvfp4_scales): the pack kernels
against the orders written out here from their definitions, and the forward
on packed scales bit for bit the forward on natural ones, on every path that
reads them (one launch per stage with every tile size, the six-launch decode
forward, the single-launch tail, add3).  The pages' routed FP8/FP4 experts
(DeepGEMM PR 416 mirror, Summary) and the NVFP4 recipe (tokenspeed recipe
"Kimi-K3 DEP16 with sharded shared experts", Allocation and launch) fix the
scale formats, not their order in memory.  MI355X only (marker ``gpu``)."""
from dataclasses import replace

import numpy as np
import pytest
import torch

from latent_moe_layer_amd import binding as B
from latent_moe_layer_amd import synth
from latent_moe_layer_amd.device import DeviceTail, to_np
from tests.test_gpu_fused import _snapshot, _poison

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()


def packed_order(S: np.ndarray, paired_half: int) -> np.ndarray:
    """P[e][t][s][h][j][g] = S[e][n(t, j)][8 s + 4 h + g] for natural scales
    S [E, N, K/32]; tile row j of tile t is weight row 256 t + j, or (paired)
    gate row 128 t + j / up row half + 128 t + j - 128."""
    E, N, KB = S.shape
    T, NS = N // 256, KB // 8
    t = np.arange(T)[:, None]
    j = np.arange(256)[None, :]
    if paired_half:
        rows = np.where(j < 128, 128 * t + j, paired_half + 128 * t + (j - 128))
    else:
        rows = 256 * t + j
    out = np.empty((E, T, NS, 2, 256, 4), np.uint8)
    for s in range(NS):
        for h in range(2):
            cols = 8 * s + 4 * h + np.arange(4)
            out[:, :, s, h, :, :] = S[:, rows, :][:, :, :, cols]
    return out.reshape(E, N, KB)


@pytest.mark.parametrize("E,I,L", [(3, 512, 768), (2, 256, 512)])
def test_pack_kernel_matches_the_order(E, I, L):
    rng = np.random.default_rng(E * 1000 + I)
    s1 = rng.integers(0, 256, (E, 2 * I, L // 32), dtype=np.uint8)
    s2 = rng.integers(0, 256, (E, L, I // 32), dtype=np.uint8)
    d = B.make_dims(1024, L, E, 2, I, 256, B.MOE_TAIL_W_MXFP4, 1e-6)
    t1, t2 = torch.from_numpy(s1).cuda(), torch.from_numpy(s2).cuda()
    p1, p2 = torch.empty_like(t1), torch.empty_like(t2)
    B.moe_tail_pack_mxfp4_scales(d, t1, t2, p1, p2)
    torch.cuda.synchronize()
    assert np.array_equal(to_np(p1), packed_order(s1, I))
    assert np.array_equal(to_np(p2), packed_order(s2, 0))


def packed_order_nv(S: np.ndarray, paired_half: int) -> np.ndarray:
    """P[e][t][s][j][q] = S[e][n(t, j)][16 s + q] for natural e4m3 scales
    S [E, N, K/16]; tile rows as in packed_order."""
    E, N, KB = S.shape
    T, NS = N // 256, KB // 16
    t = np.arange(T)[:, None]
    j = np.arange(256)[None, :]
    if paired_half:
        rows = np.where(j < 128, 128 * t + j, paired_half + 128 * t + (j - 128))
    else:
        rows = 256 * t + j
    out = np.empty((E, T, NS, 256, 16), np.uint8)
    for s in range(NS):
        out[:, :, s, :, :] = S[:, rows, 16 * s:16 * s + 16]
    return out.reshape(E, N, KB)


@pytest.mark.parametrize("E,I,L", [(3, 512, 768), (2, 256, 512)])
def test_pack_nvfp4_kernel_matches_the_order(E, I, L):
    rng = np.random.default_rng(E * 1000 + I + 7)
    s1 = rng.integers(0, 256, (E, 2 * I, L // 16), dtype=np.uint8)
    s2 = rng.integers(0, 256, (E, L, I // 16), dtype=np.uint8)
    d = B.make_dims(1024, L, E, 2, I, 256, B.MOE_TAIL_W_NVFP4, 1e-6)
    t1, t2 = torch.from_numpy(s1).cuda(), torch.from_numpy(s2).cuda()
    p1, p2 = torch.empty_like(t1), torch.empty_like(t2)
    B.moe_tail_pack_nvfp4_scales(d, t1, t2, p1, p2)
    torch.cuda.synchronize()
    assert np.array_equal(to_np(p1), packed_order_nv(s1, I))
    assert np.array_equal(to_np(p2), packed_order_nv(s2, 0))


def _forward(inp, pack, residual=None, fused=False, events=None):
    dev = DeviceTail(inp, "cuda:0", pack_scales=pack)
    dev.set_residual(residual)
    dev.route()
    _poison(dev)
    dev.forward(fused=fused, events=events)
    torch.cuda.synchronize()
    return _snapshot(dev)


def _same(a, b):
    for k in a:
        assert np.array_equal(a[k], b[k]), f"{k} differs between packed and natural scales"


CASES = {
    # decode sizes: the six-launch forward (and below the single launch)
    "ragged": synth.Workload("ragged4", Mr=37, Ms=53, E=8, k=3, I=512, Is=384, wfmt=1, seed=21, H=1024, L=512,
                             zipf_s=1.2),
    # one launch per stage, every tile size (32, 64, 128, 256 rows, short tails)
    "skewed": synth.Workload("skew", Mr=300, Ms=320, E=16, k=4, I=512, Is=256, wfmt=1, seed=87, H=1024, L=512,
                             zipf_s=1.2),
    # several tiles per persistent workgroup on the 128- and 256-row tiles
    "multi": synth.Workload("multi", Mr=1024, Ms=1184, E=8, k=4, I=2048, Is=256, wfmt=1, seed=31, H=2048,
                            L=2048, zipf_s=0.4),
    # NVFP4: the six-launch decode forward, and the 32-row tiles of the
    # one-launch-per-stage path with several tiles per expert
    "ragged_nv4": synth.Workload("raggednv", Mr=37, Ms=53, E=8, k=3, I=512, Is=384, wfmt=synth.WFMT_NVFP4, seed=27,
                                 H=1024, L=512, zipf_s=1.2),
    "skewed_nv4": synth.Workload("skewnv", Mr=300, Ms=320, E=16, k=4, I=512, Is=256, wfmt=synth.WFMT_NVFP4, seed=88,
                                 H=1024, L=768, zipf_s=1.2),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_packed_forward_equals_natural(case):
    inp = synth.make_inputs(CASES[case])
    _same(_forward(inp, False), _forward(inp, True))


@pytest.mark.parametrize("case", ["ragged", "ragged_nv4"])
def test_packed_single_launch_and_add3(case):
    wl = CASES[case]
    inp = synth.make_inputs(wl)
    _same(_forward(inp, False, fused=True), _forward(inp, True, fused=True))
    r = synth.make_residual(wl)
    _same(_forward(inp, False, residual=r), _forward(inp, True, residual=r))


def test_packed_mxfp4_workload():
    # the 1024-token MXFP4 workload itself: bit for bit the natural order
    inp = synth.make_inputs(synth.WORKLOADS["mxfp4"])
    a, b = _forward(inp, False), _forward(inp, True)
    _same(a, b)


def test_packed_nvfp4_workload():
    # the decode-shape NVFP4 workload: bit for bit the natural order
    inp = synth.make_inputs(synth.WORKLOADS["nvfp4"])
    _same(_forward(inp, False), _forward(inp, True))


def test_packed_declines_other_widths():
    wl = replace(CASES["ragged"], I=640)
    dev = DeviceTail(synth.make_inputs(wl), "cuda:0")
    with pytest.raises(B.MoeTailError) as e:
        B.moe_tail_pack_mxfp4_scales(dev.dims, dev.t["w1_scale"], dev.t["w2_scale"],
                                     torch.empty_like(dev.t["w1_scale"]), torch.empty_like(dev.t["w2_scale"]))
    assert e.value.status == B.MOE_TAIL_ERR_UNSUPPORTED
