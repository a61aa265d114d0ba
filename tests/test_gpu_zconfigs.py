"""Parity at the five full workload sizes, in the launch configuration the
benchmark times.  Routing, permutation and x codes are compared bit for bit on
every token; outputs, h codes, y and the normalized latent on every token up
to 128 tokens, and beyond that on a sample the oracle computes one by one: the
tokens of every touched expert's first and last row (so each expert's first
and last row tile is checked), and random tokens up to at least 128.  MI355X
only (marker ``gpu``)."""
import numpy as np
import pytest
import torch

from latent_moe_layer_amd import synth
from latent_moe_layer_amd.device import DeviceTail, to_np
from oracle import oracle as orc
from tests.test_gpu_parity import check_forward

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _sample(n, m, seed):
    rng = np.random.default_rng(seed)
    s = np.unique(np.concatenate([[0, n - 1], rng.choice(n, size=min(n, m), replace=False)]))
    return s.astype(np.int32)


def boundary_tokens(offsets, sorted_pair, k, n_min, seed):
    """The tokens of each touched expert's first and last row, topped up with
    random tokens to at least n_min."""
    Mr = sorted_pair.size // k
    first = offsets[:-1][np.diff(offsets) > 0]
    last = offsets[1:][np.diff(offsets) > 0] - 1
    toks = np.unique(sorted_pair[np.concatenate([first, last])] // k)
    if toks.size < n_min:
        rng = np.random.default_rng(seed)
        rest = np.setdiff1d(np.arange(Mr), toks)
        toks = np.union1d(toks, rng.choice(rest, size=min(rest.size, n_min - toks.size), replace=False))
    return np.union1d(toks, [0, Mr - 1]).astype(np.int32)


@pytest.mark.parametrize("name,n_shared", [("tiny", 0), ("decode", 0), ("prefill", 0), ("mxfp4", 0), ("indep", 32),
                                           ("nvfp4", 0)])
def test_workload(name, n_shared):
    wl = synth.WORKLOADS[name]
    print(f"[{name}] generating inputs", flush=True)
    inp = synth.make_inputs(wl)
    # (MXFP4 and NVFP4 on packed scales, as the benchmark runs them; the
    # natural order is bit for bit the same, test_gpu_packed)
    dev = DeviceTail(inp, "cuda:0", pack_scales=wl.wfmt in (synth.WFMT_MXFP4, synth.WFMT_NVFP4))
    stream = torch.cuda.Stream()
    print(f"[{name}] route + forward on the GPU", flush=True)
    dev.route(stream)
    dev.forward(stream)
    torch.cuda.synchronize()
    # every token: x codes and scales bit-exact
    xq, sx = orc.quant_1x128((inp.x_lat.astype(np.uint32) << 16).view(np.float32))
    inter = dev.intermediates()
    assert np.array_equal(to_np(inter["xq"]), xq)
    assert np.array_equal(to_np(inter["sx"]), sx)
    offsets, sorted_pair = to_np(dev.offsets), to_np(dev.sorted_pair)
    if wl.Mr <= 128:
        sel = np.arange(wl.Ms, dtype=np.int32) if n_shared == 0 else None
    else:
        sel = boundary_tokens(offsets, sorted_pair, wl.k, 128, wl.seed)
    if n_shared:
        base = np.arange(wl.Mr, dtype=np.int32) if sel is None else sel
        sel = np.concatenate([base, wl.Mr + _sample(wl.Ms - wl.Mr, n_shared, wl.seed + 1)]).astype(np.int32)
    loads = np.diff(offsets)
    print(f"[{name}] oracle on {len(sel)} tokens ({np.count_nonzero(sel < wl.Mr)} routed)", flush=True)
    stats = check_forward(dev, inp, sel=sel)
    print(f"[{name}] expert loads min/max {loads.min()}/{loads.max()}, touched {np.count_nonzero(loads)}; {stats}",
          flush=True)
