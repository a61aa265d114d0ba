"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every function include/moe_tail.h declares, sizes its workspace, and rejects
bad arguments before touching the device ("fail closed")."""
import ctypes as C
import os
import re

import pytest

from latent_moe_layer_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions(header):
    text = open(os.path.join(ROOT, "include", header)).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return set(re.findall(r"\b(moe_tail_\w+)\s*\(", text))


# every header under include/ and the library that implements it
HEADERS = {"moe_tail.h": (B.lib, B.EXPORTED), "moe_tail_probes.h": (B.probes, B.PROBES_EXPORTED)}


def test_every_header_has_a_library():
    assert sorted(f for f in os.listdir(os.path.join(ROOT, "include")) if f.endswith(".h")) == sorted(HEADERS)


@pytest.mark.parametrize("header", sorted(HEADERS))
def test_library_exports_every_declared_function(header):
    load, exported = HEADERS[header]
    lib = load()
    declared = _declared_functions(header)
    assert declared == set(exported)
    for name in declared:
        assert hasattr(lib, name), name


DIMS = dict(hidden=7168, latent=3584, num_experts=64, top_k=8, inter=2048, shared_inter=2048, wfmt=0, rms_eps=1e-6)


def dims(**kw):
    d = dict(DIMS)
    d.update(kw)
    return B.make_dims(**d)


def test_workspace_bytes_and_layout():
    d = dims()
    n = B.moe_tail_workspace_bytes(d, 128, 128)
    offs = B.moe_tail_workspace_layout(d, 128, 128)
    regions, status = offs[:B.MOE_TAIL_WS_STATUS], offs[B.MOE_TAIL_WS_STATUS]
    assert n > 0 and all(o % 256 == 0 for o in regions) and max(regions) < n
    assert sorted(regions) == regions
    # decode sizes have the single-launch path: its status word is the last word of the workspace's counters
    assert status % 4 == 0 and max(regions) < status <= n - 4
    # sizes without that path have no status word
    assert B.moe_tail_workspace_layout(d, 2048, 2048)[B.MOE_TAIL_WS_STATUS] == B.SIZE_MAX
    # y holds Mr*k rows of fp32 latent
    assert offs[B.MOE_TAIL_WS_RN] - offs[B.MOE_TAIL_WS_Y] >= 128 * 8 * 3584 * 4
    # the independent-count case (more shared than routed tokens)
    assert B.moe_tail_workspace_bytes(dims(num_experts=384), 2048, 8192) > 0
    assert B.moe_tail_workspace_bytes(d, 0, 0) >= 0


@pytest.mark.parametrize("kw,Mr,Ms", [
    (dict(top_k=0), 16, 16),
    (dict(top_k=9, num_experts=8), 16, 16),
    (dict(rms_eps=0.0), 16, 16),
    (dict(rms_eps=float("nan")), 16, 16),
    (dict(hidden=-7168), 16, 16),
    ({}, 17, 16),          # Mr > Ms
    ({}, -1, 16),
    ({}, 16, (1 << 20) + 1),
])
def test_invalid_args_size_zero(kw, Mr, Ms):
    assert B.moe_tail_workspace_bytes(dims(**kw), Mr, Ms) == 0


@pytest.mark.parametrize("kw", [dict(hidden=7000), dict(latent=3600), dict(inter=2000), dict(shared_inter=100),
                                dict(num_experts=1025), dict(top_k=17, num_experts=64), dict(wfmt=5),
                                dict(latent=16384)])
def test_unsupported_dims(kw):
    offs = (C.c_size_t * B.MOE_TAIL_WS_NUM)()
    rc = B.lib().moe_tail_workspace_layout(C.byref(dims(**kw)), 16, 16, offs)
    assert rc == B.MOE_TAIL_ERR_UNSUPPORTED


def _fake_weights(align=256):
    # host addresses that are never dereferenced: every call below fails its checks first
    base = 1 << 40
    names = ("gate", "gate_bias", "w1", "w1_scale", "w2", "w2_scale", "rms_gamma", "w_up", "ws1", "ws2")
    return B.Weights(**{n: base + i * (1 << 30) + (0 if align else 8) for i, n in enumerate(names)})


def _fake_routing(null=None, misalign=None):
    base = 1 << 41
    names = ("topk_ids", "topk_weights", "expert_offsets", "sorted_pair", "pair_to_row")
    vals = {n: base + i * (1 << 30) for i, n in enumerate(names)}
    if null:
        vals[null] = None
    if misalign:
        vals[misalign] += 4
    return B.Routing(**vals)


def _route(d, w, x, Mr, r, ws, nbytes):
    return B.lib().moe_tail_route(C.byref(d), C.byref(w), x, Mr, C.byref(r), ws, nbytes, None)


def _fwd(d, w, x_lat, Mr, x_hid, Ms, r, out, shared_out, ws, nbytes):
    return B.lib().moe_tail_forward(C.byref(d), C.byref(w), x_lat, Mr, x_hid, Ms, C.byref(r), out, shared_out, ws,
                                    nbytes, None)


X = 1 << 42
OUT = 1 << 43
SOUT = 1 << 44
WS = 1 << 45


def test_route_rejections():
    d, w = dims(), _fake_weights()
    need = B.moe_tail_workspace_bytes(d, 16, 16)
    assert _route(d, w, X, 16, _fake_routing(null="sorted_pair"), WS, need) == B.MOE_TAIL_ERR_INVALID
    assert _route(d, w, X, 16, _fake_routing(misalign="topk_ids"), WS, need) == B.MOE_TAIL_ERR_INVALID
    assert _route(d, w, None, 16, _fake_routing(), WS, need) == B.MOE_TAIL_ERR_INVALID
    assert _route(d, w, X + 2, 16, _fake_routing(), WS, need) == B.MOE_TAIL_ERR_INVALID
    assert _route(d, w, X, -3, _fake_routing(), WS, need) == B.MOE_TAIL_ERR_INVALID
    assert _route(d, w, X, 16, _fake_routing(), WS, 0) == B.MOE_TAIL_ERR_WORKSPACE
    assert _route(dims(wfmt=5), w, X, 16, _fake_routing(), WS, need) == B.MOE_TAIL_ERR_UNSUPPORTED
    wn = _fake_weights()
    wn.gate = None
    assert _route(d, wn, X, 16, _fake_routing(), WS, need) == B.MOE_TAIL_ERR_INVALID


def test_forward_rejections():
    d, w, r = dims(), _fake_weights(), _fake_routing()
    need = B.moe_tail_workspace_bytes(d, 16, 32)
    # shared_out must be given exactly when Ms > Mr
    assert _fwd(d, w, X, 16, X, 32, r, OUT, None, WS, need) == B.MOE_TAIL_ERR_INVALID
    need16 = B.moe_tail_workspace_bytes(d, 16, 16)
    assert _fwd(d, w, X, 16, X, 16, r, OUT, SOUT, WS, need16) == B.MOE_TAIL_ERR_INVALID
    assert _fwd(d, w, X, 17, X, 16, r, OUT, None, WS, need16) == B.MOE_TAIL_ERR_INVALID
    assert _fwd(d, w, X, 16, X, 32, r, OUT, SOUT, WS, need - 1) == B.MOE_TAIL_ERR_WORKSPACE
    assert _fwd(d, w, X, 16, X, 32, r, None, SOUT, WS, need) == B.MOE_TAIL_ERR_INVALID
    assert _fwd(d, w, X, 16, X, 32, r, OUT + 8, SOUT, WS, need) == B.MOE_TAIL_ERR_INVALID
    assert _fwd(d, w, X, 16, X, 32, _fake_routing(null="pair_to_row"), OUT, SOUT, WS, need) == B.MOE_TAIL_ERR_INVALID
    assert _fwd(d, _fake_weights(align=0), X, 16, X, 32, r, OUT, SOUT, WS, need) == B.MOE_TAIL_ERR_INVALID
    assert _fwd(dims(hidden=7040), w, X, 16, X, 32, r, OUT, SOUT, WS, need) == B.MOE_TAIL_ERR_UNSUPPORTED
    wn = _fake_weights()
    wn.ws2 = None
    assert _fwd(d, wn, X, 16, X, 32, r, OUT, SOUT, WS, need) == B.MOE_TAIL_ERR_INVALID
    assert B.lib().moe_tail_forward_profiled(C.byref(d), C.byref(w), X, 16, X, 32, C.byref(r), OUT, SOUT, WS, need,
                                             None, None) == B.MOE_TAIL_ERR_INVALID


def test_forward_nvfp4_needs_its_matrix_scales():
    d, r = dims(wfmt=B.MOE_TAIL_W_NVFP4), _fake_routing()
    need = B.moe_tail_workspace_bytes(d, 16, 16)
    w = _fake_weights()
    assert _fwd(d, w, X, 16, X, 16, r, OUT, None, WS, need) == B.MOE_TAIL_ERR_INVALID  # no matrix scales
    w.w1_tensor_scale, w.w2_tensor_scale = 1 << 47, (1 << 47) + 4096
    assert _fwd(d, w, X, 16, X, 16, r, OUT, None, WS, need - 1) == B.MOE_TAIL_ERR_WORKSPACE
    w.w2_tensor_scale += 4  # misaligned
    assert _fwd(d, w, X, 16, X, 16, r, OUT, None, WS, need) == B.MOE_TAIL_ERR_INVALID
    # the single launch and the packed-scale entry points decline NVFP4
    w.w2_tensor_scale -= 4
    f = B.lib().moe_tail_forward_fused
    assert f(C.byref(d), C.byref(w), X, 16, X, 16, C.byref(r), None, OUT, None, WS, need, None) == \
        B.MOE_TAIL_ERR_UNSUPPORTED
    assert B.lib().moe_tail_pack_mxfp4_scales(C.byref(d), X, None, OUT, None, None) == B.MOE_TAIL_ERR_INVALID


def test_forward_add3_rejections():
    d, w, r = dims(), _fake_weights(), _fake_routing()
    need = B.moe_tail_workspace_bytes(d, 16, 16)
    f = B.lib().moe_tail_forward_add3
    RES = 1 << 46
    # the residual is required when there are routed tokens, and 16-byte aligned
    assert f(C.byref(d), C.byref(w), X, 16, X, 16, C.byref(r), None, OUT, None, WS, need, None) == \
        B.MOE_TAIL_ERR_INVALID
    assert f(C.byref(d), C.byref(w), X, 16, X, 16, C.byref(r), RES + 2, OUT, None, WS, need, None) == \
        B.MOE_TAIL_ERR_INVALID
    # every other check is the plain forward's
    assert f(C.byref(d), C.byref(w), X, 16, X, 16, C.byref(r), RES, OUT, None, WS, need - 1, None) == \
        B.MOE_TAIL_ERR_WORKSPACE
    assert f(C.byref(d), C.byref(w), X, 17, X, 16, C.byref(r), RES, OUT, None, WS, need, None) == \
        B.MOE_TAIL_ERR_INVALID


def test_forward_fused_rejections():
    d, w, r = dims(), _fake_weights(), _fake_routing()
    f = B.lib().moe_tail_forward_fused
    need = B.moe_tail_workspace_bytes(d, 16, 16)
    RES = 1 << 46
    # the plain forward's checks come first
    assert f(C.byref(d), C.byref(w), X, 17, X, 16, C.byref(r), None, OUT, None, WS, need, None) == \
        B.MOE_TAIL_ERR_INVALID
    assert f(C.byref(d), C.byref(w), X, 16, X, 16, C.byref(r), None, OUT, None, WS, need - 1, None) == \
        B.MOE_TAIL_ERR_WORKSPACE
    assert f(C.byref(d), C.byref(w), X, 16, X, 16, C.byref(r), RES + 2, OUT, None, WS, need, None) == \
        B.MOE_TAIL_ERR_INVALID
    assert f(C.byref(d), C.byref(w), X, 16, X, 16, C.byref(r), None, OUT, SOUT, WS, need, None) == \
        B.MOE_TAIL_ERR_INVALID
    # sizes outside the single launch's range are declined (nothing enqueued)
    need129 = B.moe_tail_workspace_bytes(d, 16, 129)
    assert f(C.byref(d), C.byref(w), X, 16, X, 129, C.byref(r), None, OUT, SOUT, WS, need129, None) == \
        B.MOE_TAIL_ERR_UNSUPPORTED
    dn = dims(inter=256)
    needn = B.moe_tail_workspace_bytes(dn, 16, 16)
    assert f(C.byref(dn), C.byref(w), X, 16, X, 16, C.byref(r), None, OUT, None, WS, needn, None) == \
        B.MOE_TAIL_ERR_UNSUPPORTED


def test_forward_fused_bounded_rejections():
    d, w, r = dims(), _fake_weights(), _fake_routing()
    f = B.lib().moe_tail_forward_fused_bounded
    need = B.moe_tail_workspace_bytes(d, 16, 16)
    assert f(C.byref(d), C.byref(w), X, 16, X, 16, C.byref(r), None, OUT, None, WS, need, None, -1) == \
        B.MOE_TAIL_ERR_INVALID
    assert f(C.byref(d), C.byref(w), X, 16, X, 16, C.byref(r), None, OUT, None, WS, need - 1, None, 0) == \
        B.MOE_TAIL_ERR_WORKSPACE
    need129 = B.moe_tail_workspace_bytes(d, 16, 129)
    assert f(C.byref(d), C.byref(w), X, 16, X, 129, C.byref(r), None, OUT, SOUT, WS, need129, None, 0) == \
        B.MOE_TAIL_ERR_UNSUPPORTED


def test_forward_noalloc_rejections():
    # every check runs before the runtime is asked for the scratch address
    f = B.lib().moe_tail_forward_noalloc
    w, r = _fake_weights(), _fake_routing()
    big = dims(num_experts=8, inter=512, shared_inter=256)
    assert B.moe_tail_workspace_bytes(big, 512, 512) > B.MOE_TAIL_NOALLOC_MAX_BYTES
    assert f(C.byref(big), C.byref(w), X, 512, X, 512, C.byref(r), OUT, None, None) == B.MOE_TAIL_ERR_WORKSPACE
    d = dims()
    assert f(C.byref(d), C.byref(w), X, 17, X, 16, C.byref(r), OUT, None, None) == B.MOE_TAIL_ERR_INVALID
    assert f(C.byref(d), C.byref(w), X, 16, X, 32, C.byref(r), OUT, None, None) == B.MOE_TAIL_ERR_INVALID
    assert f(C.byref(dims(hidden=7040)), C.byref(w), X, 16, X, 16, C.byref(r), OUT, None, None) == \
        B.MOE_TAIL_ERR_UNSUPPORTED


def test_probe_rejections():
    p = B.probes()
    assert p.moe_tail_probe_mfma_fp8(X, X, OUT, 0, None) == 1
    assert p.moe_tail_probe_mfma_fp8(X, X, OUT, 65537, None) == 1
    assert p.moe_tail_probe_mfma_fp8(X + 4, X, OUT, 1, None) == 1
    assert p.moe_tail_probe_copy(X, OUT, 100, None) == 1
    assert p.moe_tail_probe_copy(X, X + 16, 4096, None) == 1  # overlapping
    assert p.moe_tail_probe_copy(None, OUT, 4096, None) == 1
    assert p.moe_tail_probe_copy(X, OUT, 0, None) == 0
    assert p.moe_tail_probe_stream_read(X, 4000, OUT, 0, None) == 1
    assert p.moe_tail_probe_stream_read(X, 4096, None, 0, None) == 1
    assert p.moe_tail_probe_stream_read(X, 0, OUT, 0, None) == 0
    f = p.moe_tail_probe_stream_paths
    assert f(X, 1 << 20, 64, 0, 4, 128, OUT, 0, None) == 1          # no such mode
    assert f(X, 1 << 20, 0, 0, 0, 128, OUT, 0, None) == 1           # empty grid
    assert f(X, (1 << 20) + 1024, 64, 0, 0, 128, OUT, 0, None) == 1  # not whole 32 KB stages
    assert f(X, 1 << 31, 1, 0, 2, 128, OUT, 0, None) == 1            # past a buffer's 32-bit range
    assert f(X, 1 << 20, 64, 0, 1, 100, OUT, 0, None) == 1          # rows not whole 128-byte lines
    assert f(X, 32768 * 5, 64, 0, 1, 1792, OUT, 0, None) == 1       # not whole 256-row matrices
    assert f(X + 4, 1 << 20, 64, 0, 0, 128, OUT, 0, None) == 1
    assert f(X, 1 << 20, 64, 0, 0, 128, None, 0, None) == 1


def test_pack_mxfp4_scales_rejections():
    pk = B.lib().moe_tail_pack_mxfp4_scales
    d4 = dims(wfmt=B.MOE_TAIL_W_MXFP4)
    A, P = 1 << 44, 1 << 45  # placeholders: every call below fails before touching them
    # FP8 dims have no e8m0 scales
    assert pk(C.byref(dims()), A, A + (1 << 40), P, P + (1 << 40), None) == B.MOE_TAIL_ERR_INVALID
    # widths that are not multiples of 256
    assert pk(C.byref(dims(wfmt=1, inter=640)), A, None, P, None, None) == B.MOE_TAIL_ERR_UNSUPPORTED
    # an input without its output, misaligned or overlapping buffers
    assert pk(C.byref(d4), A, None, None, None, None) == B.MOE_TAIL_ERR_INVALID
    assert pk(C.byref(d4), A + 4, None, P, None, None) == B.MOE_TAIL_ERR_INVALID
    assert pk(C.byref(d4), A, None, A + 1024, None, None) == B.MOE_TAIL_ERR_INVALID
    # nothing to do
    assert pk(C.byref(d4), None, None, None, None, None) == B.MOE_TAIL_OK
    # a forward on packed scales needs the tiled kernels' shapes
    w, r = _fake_weights(), _fake_routing()
    dp = dims(wfmt=B.MOE_TAIL_W_MXFP4_PACKED, inter=640)
    need = B.moe_tail_workspace_bytes(dp, 16, 16)
    assert _fwd(dp, w, X, 16, X, 16, r, OUT, None, WS, need) == B.MOE_TAIL_ERR_UNSUPPORTED


def test_pack_nvfp4_scales_rejections():
    pk = B.lib().moe_tail_pack_nvfp4_scales
    dn = dims(wfmt=B.MOE_TAIL_W_NVFP4)
    A, P = 1 << 44, 1 << 45  # placeholders: every call below fails before touching them
    # FP8 and MXFP4 dims have no e4m3 block scales
    assert pk(C.byref(dims()), A, None, P, None, None) == B.MOE_TAIL_ERR_INVALID
    assert pk(C.byref(dims(wfmt=B.MOE_TAIL_W_MXFP4)), A, None, P, None, None) == B.MOE_TAIL_ERR_INVALID
    # widths that are not multiples of 256
    assert pk(C.byref(dims(wfmt=B.MOE_TAIL_W_NVFP4, inter=640)), A, None, P, None, None) == B.MOE_TAIL_ERR_UNSUPPORTED
    # an input without its output, misaligned or overlapping buffers
    assert pk(C.byref(dn), None, A, None, None, None) == B.MOE_TAIL_ERR_INVALID
    assert pk(C.byref(dn), A + 4, None, P, None, None) == B.MOE_TAIL_ERR_INVALID
    assert pk(C.byref(dn), A, None, A + 1024, None, None) == B.MOE_TAIL_ERR_INVALID
    assert pk(C.byref(dn), None, None, None, None, None) == B.MOE_TAIL_OK
    # a forward on packed scales needs the tiled kernels' shapes and the matrix scales
    w, r = _fake_weights(), _fake_routing()
    dp = dims(wfmt=B.MOE_TAIL_W_NVFP4_PACKED, inter=640)
    need = B.moe_tail_workspace_bytes(dp, 16, 16)
    w.w1_tensor_scale = w.w2_tensor_scale = 1 << 46
    assert _fwd(dp, w, X, 16, X, 16, r, OUT, None, WS, need) == B.MOE_TAIL_ERR_UNSUPPORTED
    dp = dims(wfmt=B.MOE_TAIL_W_NVFP4_PACKED)
    need = B.moe_tail_workspace_bytes(dp, 16, 16)
    w.w1_tensor_scale = None
    assert _fwd(dp, w, X, 16, X, 16, r, OUT, None, WS, need) == B.MOE_TAIL_ERR_INVALID


def test_quant_rejections():
    q = B.lib().moe_tail_quant_fp8_1x128
    assert q(X, 1, 4, 100, OUT, SOUT, None) == B.MOE_TAIL_ERR_INVALID
    assert q(X, 1, -1, 128, OUT, SOUT, None) == B.MOE_TAIL_ERR_INVALID
    assert q(None, 1, 4, 128, OUT, SOUT, None) == B.MOE_TAIL_ERR_INVALID
    assert q(X, 1, 4, 128, OUT + 1, SOUT, None) == B.MOE_TAIL_ERR_INVALID


def test_strerror():
    assert B.strerror(0) == "ok"
    assert "workspace" in B.strerror(B.MOE_TAIL_ERR_WORKSPACE)
    assert B.strerror(99) == "unknown status"


def test_status_error_type():
    with pytest.raises(B.MoeTailError) as e:
        B._check(B.MOE_TAIL_ERR_UNSUPPORTED, "x")
    assert e.value.status == B.MOE_TAIL_ERR_UNSUPPORTED


def test_bench_declines_several_gpus():
    # one GPU only: more is refused before any device work, with a message
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
