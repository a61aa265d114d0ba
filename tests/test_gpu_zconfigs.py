"""Parity at the five full workload sizes, in the launch configuration the
benchmark times.  Routing, permutation and x codes are compared bit for bit on
every token; outputs, h codes, y and the normalized latent on a sample of
tokens that the oracle computes one by one.  MI355X only (marker ``gpu``)."""
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


@pytest.mark.parametrize("name,n_routed,n_shared", [("tiny", None, 0), ("decode", None, 0), ("prefill", 12, 0),
                                                   ("mxfp4", 12, 0), ("indep", 10, 10)])
def test_workload(name, n_routed, n_shared):
    wl = synth.WORKLOADS[name]
    print(f"[{name}] generating inputs", flush=True)
    inp = synth.make_inputs(wl)
    # (MXFP4 on packed scales, as the benchmark runs it; the natural order is
    # bit for bit the same, test_gpu_packed)
    dev = DeviceTail(inp, "cuda:0", pack_scales=wl.wfmt == synth.WFMT_MXFP4)
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
    if n_routed is None:
        sel = None
    else:
        sel = _sample(wl.Mr, n_routed, wl.seed)
        if n_shared:
            sel = np.concatenate([sel, wl.Mr + _sample(wl.Ms - wl.Mr, n_shared, wl.seed + 1)]).astype(np.int32)
    print(f"[{name}] oracle on {'all' if sel is None else len(sel)} tokens", flush=True)
    stats = check_forward(dev, inp, sel=sel)
    loads = np.diff(to_np(dev.offsets))
    print(f"[{name}] expert loads min/max {loads.min()}/{loads.max()}, touched {np.count_nonzero(loads)}; {stats}",
          flush=True)
