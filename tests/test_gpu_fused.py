"""The single-launch tail (moe_tail_forward_fused): bit for bit the
multi-launch forward on the same inputs (every output and materialized
intermediate), parity with the oracle, repeated calls, graph replay, and the
sizes it declines.  The pages' producer schedules routed and shared work in
one kernel (DeepGEMM PR 416 mirror, Summary).  MI355X only (marker ``gpu``)."""
import ctypes as C
from dataclasses import replace

import numpy as np
import pytest
import torch

from latent_moe_layer_amd import binding as B
from latent_moe_layer_amd import synth
from latent_moe_layer_amd.device import DeviceTail, to_np
from tests.test_gpu_parity import check_forward

pytestmark = pytest.mark.gpu

# The launch's counters: 16 words of the workspace ending with the status word
# (moe_tail_workspace_layout, MOE_TAIL_WS_STATUS): one word per stage (the
# workgroups that finished it, the last one the count of finished workgroups)
# and the error word.
SEGMENTS = 8
SYNC_ERR = 15
BF16_NAN = 0x7FC0


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()


def _sync_base(dev):
    return dev.layout[B.MOE_TAIL_WS_STATUS] - 4 * SYNC_ERR


def _poison(dev):
    """Fill outputs and intermediates with a pattern no result has (0xFFFF
    bf16 is a NaN, 0xFF codes and all-ones floats too)."""
    dev.out.fill_(-1)
    if dev.shared_out is not None:
        dev.shared_out.fill_(-1)
    end = _sync_base(dev) if dev.layout[B.MOE_TAIL_WS_STATUS] != B.SIZE_MAX else dev.ws_bytes
    dev.ws[:end].fill_(255)


def _snapshot(dev):
    snap = {"out": to_np(dev.out).copy()}
    if dev.shared_out is not None:
        snap["shared_out"] = to_np(dev.shared_out).copy()
    for k, v in dev.intermediates().items():
        snap[k] = to_np(v).copy()
    return snap


def _sync_words(dev):
    base = _sync_base(dev)
    return to_np(dev.ws[base: base + 64].view(torch.int32))


def _grid():
    n = torch.cuda.get_device_properties(0).multi_processor_count
    return n // 8 * 8


def staged_and_fused(inp, residual=None, Mr=None, Ms=None):
    dev = DeviceTail(inp, "cuda:0", Mr=Mr, Ms=Ms)
    dev.set_residual(residual)
    dev.route()
    _poison(dev)
    dev.forward()
    torch.cuda.synchronize()
    staged = _snapshot(dev)
    _poison(dev)
    dev.forward(fused=True)
    torch.cuda.synchronize()
    return dev, staged, _snapshot(dev)


def assert_same(staged, fused, keys=None):
    for k in keys or staged:
        assert np.array_equal(staged[k], fused[k]), f"{k} differs between the staged and the single-launch forward"


def assert_counters(dev):
    words = _sync_words(dev)
    assert words[SYNC_ERR] == 0, "a segment wait timed out"
    assert np.all(words[:SEGMENTS] == _grid()), words[:SEGMENTS]


CASES = {
    # the smallest workload: 8 experts, 16 tokens
    "tiny": synth.WORKLOADS["tiny"],
    # ragged everywhere, more shared than routed tokens (shared_out rows)
    "ragged": synth.Workload("ragged", Mr=37, Ms=53, E=8, k=3, I=512, Is=384, wfmt=0, seed=21, H=1024, L=512),
    "ragged_fp4": synth.Workload("ragged4", Mr=37, Ms=53, E=8, k=3, I=512, Is=384, wfmt=1, seed=21, H=1024, L=512,
                                 zipf_s=1.2),
    # NVFP4 weights on skewed loads (experts past 32 rows take several tiles)
    "ragged_nv4": synth.Workload("raggednv", Mr=37, Ms=53, E=8, k=3, I=512, Is=384, wfmt=synth.WFMT_NVFP4, seed=27,
                                 H=1024, L=512, zipf_s=1.2),
    # all-equal logits: two experts with 100 rows each, four 32-row tiles apiece
    "heavy": synth.Workload("heavy", Mr=100, Ms=100, E=6, k=2, I=512, Is=128, wfmt=0, seed=22, zero_router=True,
                            H=1024, L=512),
    # one token on every expert
    "one_token": synth.Workload("one", Mr=1, Ms=1, E=4, k=4, I=384, Is=128, wfmt=0, seed=24, H=1024, L=512),
    # the largest shared count it takes, with few routed tokens
    "ms128": synth.Workload("ms128", Mr=9, Ms=128, E=16, k=4, I=512, Is=256, wfmt=0, seed=61, H=1024, L=512),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_fused_equals_staged_bitwise(case):
    inp = synth.make_inputs(CASES[case])
    dev, staged, fused = staged_and_fused(inp)
    assert_same(staged, fused)
    assert_counters(dev)


@pytest.mark.parametrize("case", ["tiny", "ragged", "ragged_fp4", "ragged_nv4"])
def test_fused_against_oracle(case):
    inp = synth.make_inputs(CASES[case])
    dev = DeviceTail(inp, "cuda:0")
    dev.route()
    _poison(dev)
    dev.forward(fused=True)
    torch.cuda.synchronize()
    check_forward(dev, inp)


def test_fused_add3_equals_staged():
    wl = CASES["ragged"]
    inp = synth.make_inputs(wl)
    r = synth.make_residual(wl)
    dev, staged, fused = staged_and_fused(inp, residual=r)
    assert_same(staged, fused)
    check_forward(dev, inp, residual=r)


def test_fused_decode_full_size():
    # the decode workload itself (128 tokens, 64 experts, top-8, the served
    # widths): every output bit equal to the staged forward's, a sample of
    # tokens against the oracle
    wl = synth.WORKLOADS["decode"]
    inp = synth.make_inputs(wl)
    r = synth.make_residual(wl)
    dev, staged, fused = staged_and_fused(inp)
    assert_same(staged, fused)
    assert_counters(dev)
    check_forward(dev, inp, sel=np.array([0, 5, 63, 64, 127], np.int32))
    dev.set_residual(r)
    _poison(dev)
    dev.forward()
    torch.cuda.synchronize()
    staged3 = _snapshot(dev)
    _poison(dev)
    dev.forward(fused=True)
    torch.cuda.synchronize()
    assert_same(staged3, _snapshot(dev))


def test_fused_repeated_calls_and_graph_replay():
    # the counters are cleared by every call's first launch: back-to-back
    # calls, and replays of a captured graph with eager work in between, all
    # give the first call's bits
    inp = synth.make_inputs(CASES["ragged"])
    dev = DeviceTail(inp, "cuda:0")
    dev.route()
    dev.forward(fused=True)
    torch.cuda.synchronize()
    ref = _snapshot(dev)
    for _ in range(3):
        _poison(dev)
        dev.forward(fused=True)
    torch.cuda.synchronize()
    assert_same(ref, _snapshot(dev))
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        dev.forward(stream=s, fused=True)  # warm-up on the capture stream
        s.synchronize()
        with torch.cuda.graph(g, stream=s):
            dev.route(stream=s)
            dev.forward(stream=s, fused=True)
    for _ in range(3):
        _poison(dev)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert_same(ref, _snapshot(dev))
        assert_counters(dev)


def test_fused_without_routed_tokens():
    wl = synth.Workload("mr0", Mr=0, Ms=20, E=4, k=2, I=384, Is=256, wfmt=0, seed=23, H=1024, L=512)
    inp = synth.make_inputs(wl)
    dev, staged, fused = staged_and_fused(inp)
    assert_same(staged, fused, keys=["shared_out", "hs"])


def _hip_events(n):
    rt = C.CDLL("libamdhip64.so")
    rt.hipEventCreate.argtypes = [C.POINTER(C.c_void_p)]
    out = []
    for _ in range(n):
        h = C.c_void_p()
        assert rt.hipEventCreate(C.byref(h)) == 0
        out.append(h.value)
    return out


@pytest.mark.parametrize("case", ["tiny", "ragged", "ragged_fp4", "ragged_nv4", "ms128", "decode"])
def test_coscheduled_forward_equals_one_launch_per_stage(case):
    # At decode sizes moe_tail_forward runs the tail as six launches with
    # independent stages sharing a launch (routed L2 with the shared L1's
    # items, combine with the shared L1's reduction, shared L2 with the
    # up-projection); the profiled entry point keeps one launch per stage.
    # Same tiles, same summation orders: the same bits.
    wl = synth.WORKLOADS["decode"] if case == "decode" else CASES[case]
    inp = synth.make_inputs(wl)
    dev = DeviceTail(inp, "cuda:0")
    dev.route()
    _poison(dev)
    dev.forward()
    torch.cuda.synchronize()
    co = _snapshot(dev)
    _poison(dev)
    dev.forward(events=_hip_events(B.MOE_TAIL_NUM_STAGES + 1))
    torch.cuda.synchronize()
    assert_same(co, _snapshot(dev))


# FP8 weights, experts averaging 50 rows (32/64-row tiles) and more than twice
# as many shared as routed tokens: moe_tail_forward runs the shared L1 and L2
# on a second stream beside the routed work (each on its share of the CUs).
COSCHED = synth.Workload("cosched", Mr=300, Ms=700, E=48, k=8, I=512, Is=256, wfmt=0, seed=61, H=1024, L=512)


def test_shared_on_second_stream_equals_one_stream():
    # The forward with the shared expert on a second stream against one
    # launch per stage on the caller's stream: the same tiles with the same
    # summation orders, so the same bits; parity with the oracle; the
    # caller's stream alone orders the outputs (a wait on that stream, not on
    # the device, finds them complete); graph replays, with eager work in
    # between, give the same bits each time.
    inp = synth.make_inputs(COSCHED)
    dev = DeviceTail(inp, "cuda:0")
    dev.route()
    _poison(dev)
    dev.forward(events=_hip_events(B.MOE_TAIL_NUM_STAGES + 1))
    torch.cuda.synchronize()
    ref = _snapshot(dev)
    check_forward(dev, inp)
    s = torch.cuda.Stream()
    for _ in range(2):
        _poison(dev)
        torch.cuda.synchronize()
        dev.forward(stream=s)
        s.synchronize()
        assert_same(ref, _snapshot(dev))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            dev.route(stream=s)
            dev.forward(stream=s)
    for _ in range(3):
        _poison(dev)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert_same(ref, _snapshot(dev))
        dev.forward()  # eager work between replays
        torch.cuda.synchronize()


def test_shared_on_second_stream_add3_and_one_stream_entry_points():
    # The same sizes through the other entry points: add3 (the shared expert
    # on the second stream) against the timed entry point with the same
    # residual (one stream), and the plain forward against the
    # allocation-free one (one stream, its own scratch): the same bits.
    inp = synth.make_inputs(COSCHED)
    dev = DeviceTail(inp, "cuda:0")
    dev.route()
    dev.set_residual(synth.make_residual(COSCHED))
    _poison(dev)
    dev.forward()
    torch.cuda.synchronize()
    two = _snapshot(dev)
    _poison(dev)
    dev.forward_timed(None, _hip_events(B.MOE_TAIL_NUM_STAGES + 1))
    torch.cuda.synchronize()
    assert_same(two, _snapshot(dev))
    dev.set_residual(None)
    _poison(dev)
    dev.forward()
    torch.cuda.synchronize()
    ref = _snapshot(dev)
    out = torch.full_like(dev.out, -1)
    shared_out = torch.full_like(dev.shared_out, -1)
    B.moe_tail_forward_noalloc(dev.dims, dev.weights, dev.t["x_lat"], dev.Mr, dev.t["x_hid"], dev.Ms, dev.routing,
                               out, shared_out, None)
    torch.cuda.synchronize()
    assert np.array_equal(to_np(out), ref["out"])
    assert np.array_equal(to_np(shared_out), ref["shared_out"])


@pytest.mark.parametrize("case", ["ragged", "decode"])
def test_fused_wait_given_up_fails_closed(case):
    # Every stage wait forced to give up from the host (max_polls = 0): the
    # launch still finishes, out and shared_out hold NaN in every element and
    # the status word reads 1.  The next complete call on the same workspace
    # clears the word and gives the staged forward's bits again.
    wl = synth.WORKLOADS["decode"] if case == "decode" else CASES[case]
    inp = synth.make_inputs(wl)
    dev = DeviceTail(inp, "cuda:0")
    dev.route()
    dev.forward()
    torch.cuda.synchronize()
    ref = _snapshot(dev)
    print(f"[{case}] fused launch with every wait given up", flush=True)
    B.moe_tail_forward_fused_bounded(dev.dims, dev.weights, dev.t["x_lat"], dev.Mr, dev.t["x_hid"], dev.Ms,
                                     dev.routing, None, dev.out, dev.shared_out, dev.ws, dev.ws_bytes, None, 0)
    torch.cuda.synchronize()
    words = _sync_words(dev)
    assert words[SYNC_ERR] == 1
    assert words[SEGMENTS - 1] == _grid()  # every workgroup finished
    assert np.all(to_np(dev.out) == BF16_NAN)
    if dev.shared_out is not None:
        assert np.all(to_np(dev.shared_out) == BF16_NAN)
    dev.forward(fused=True)
    torch.cuda.synchronize()
    assert _sync_words(dev)[SYNC_ERR] == 0
    assert_same(ref, _snapshot(dev), keys=["out"] + (["shared_out"] if dev.shared_out is not None else []))
    assert_counters(dev)


def test_fused_declines_large_token_counts():
    wl = synth.Workload("big", Mr=16, Ms=129, E=4, k=2, I=384, Is=128, wfmt=0, seed=62, H=1024, L=512)
    inp = synth.make_inputs(wl)
    dev = DeviceTail(inp, "cuda:0")
    dev.route()
    with pytest.raises(B.MoeTailError) as e:
        dev.forward(fused=True)
    assert e.value.status == B.MOE_TAIL_ERR_UNSUPPORTED
    # narrow experts (I < 384) are declined too, and MXFP4 experts whose width
    # is not a multiple of 256
    for wl2 in (replace(wl, Ms=16, I=128), replace(wl, Ms=16, I=640, wfmt=synth.WFMT_MXFP4)):
        dev2 = DeviceTail(synth.make_inputs(wl2), "cuda:0")
        dev2.route()
        with pytest.raises(B.MoeTailError) as e:
            dev2.forward(fused=True)
        assert e.value.status == B.MOE_TAIL_ERR_UNSUPPORTED
