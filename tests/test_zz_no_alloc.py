"""The allocation-free forward (moe_tail_forward_noalloc): the library's own
static device workspace instead of a caller's.  Two calls in a row on one GPU,
the second on a smaller input, each bit for bit moe_tail_forward's result on
its own workspace (which the parity tests hold to the oracle).  MI355X only
(marker ``gpu``)."""
import numpy as np
import pytest
import torch

from latent_moe_layer_amd import binding as B
from latent_moe_layer_amd import synth
from latent_moe_layer_amd.device import DeviceTail, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()


def _noalloc_equals_forward(wl):
    inp = synth.make_inputs(wl)
    dev = DeviceTail(inp, "cuda:0")
    dev.route()
    dev.forward()
    torch.cuda.synchronize()
    want_out = to_np(dev.out).copy()
    want_so = None if dev.shared_out is None else to_np(dev.shared_out).copy()
    dev.out.fill_(-1)
    if dev.shared_out is not None:
        dev.shared_out.fill_(-1)
    print(f"[{wl.name}] moe_tail_forward_noalloc Mr={dev.Mr} Ms={dev.Ms}", flush=True)
    B.moe_tail_forward_noalloc(dev.dims, dev.weights, dev.t["x_lat"], dev.Mr, dev.t["x_hid"], dev.Ms, dev.routing,
                               dev.out, dev.shared_out)
    torch.cuda.synchronize()
    assert np.array_equal(to_np(dev.out), want_out)
    if want_so is not None:
        assert np.array_equal(to_np(dev.shared_out), want_so)


def test_noalloc_two_calls_second_smaller():
    # the decode workload (the six-launch schedule, whose ticket counter lives
    # in the scratch), then a smaller tail with shared-only rows (one launch per
    # stage), then the decode workload again on what the smaller call left
    big = synth.WORKLOADS["decode"]
    small = synth.Workload("small", Mr=24, Ms=40, E=8, k=2, I=512, Is=256, wfmt=0, seed=71)
    assert B.moe_tail_workspace_bytes(B.make_dims(big.H, big.L, big.E, big.k, big.I, big.Is, 0, 1e-6), 128, 128) \
        <= B.MOE_TAIL_NOALLOC_MAX_BYTES
    _noalloc_equals_forward(big)
    _noalloc_equals_forward(small)
    _noalloc_equals_forward(big)


def test_noalloc_rejects_sizes_beyond_its_scratch():
    wl = synth.Workload("wide", Mr=512, Ms=512, E=8, k=8, I=512, Is=256, wfmt=0, seed=72)
    dims = B.make_dims(wl.H, wl.L, wl.E, wl.k, wl.I, wl.Is, 0, 1e-6)
    assert B.moe_tail_workspace_bytes(dims, 512, 512) > B.MOE_TAIL_NOALLOC_MAX_BYTES
    inp = synth.make_inputs(wl)
    dev = DeviceTail(inp, "cuda:0")
    with pytest.raises(B.MoeTailError) as e:
        B.moe_tail_forward_noalloc(dev.dims, dev.weights, dev.t["x_lat"], dev.Mr, dev.t["x_hid"], dev.Ms,
                                   dev.routing, dev.out, dev.shared_out)
    assert e.value.status == B.MOE_TAIL_ERR_WORKSPACE
