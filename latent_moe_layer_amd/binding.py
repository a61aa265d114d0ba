"""ctypes binding of ``libmoe_tail.so`` (the C ABI in include/moe_tail.h).

Argument marshalling only: every step of the tail runs in the HIP kernels
behind the C ABI.  Pointers may be given as torch tensors (their data_ptr is
used) or as plain integers; streams as torch.cuda.Stream, an integer handle, or
None for the null stream.  A non-zero status raises ``MoeTailError``.
"""
from __future__ import annotations

import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_tail.so")

MOE_TAIL_OK = 0
MOE_TAIL_ERR_INVALID = 1
MOE_TAIL_ERR_UNSUPPORTED = 2
MOE_TAIL_ERR_WORKSPACE = 3
MOE_TAIL_ERR_DEVICE = 4

MOE_TAIL_W_FP8_BLOCK128 = 0
MOE_TAIL_W_MXFP4 = 1
MOE_TAIL_W_MXFP4_PACKED = 2
MOE_TAIL_W_NVFP4 = 3
MOE_TAIL_W_NVFP4_PACKED = 4

MOE_TAIL_WS_XQ, MOE_TAIL_WS_SX, MOE_TAIL_WS_HQ, MOE_TAIL_WS_SH, MOE_TAIL_WS_Y, MOE_TAIL_WS_RN, \
    MOE_TAIL_WS_HS, MOE_TAIL_WS_S, MOE_TAIL_WS_STATUS = range(9)
MOE_TAIL_WS_NUM = 9
SIZE_MAX = 2 ** 64 - 1
MOE_TAIL_NUM_STAGES = 7

EXPORTED = ("moe_tail_workspace_bytes", "moe_tail_workspace_layout", "moe_tail_route", "moe_tail_forward",
            "moe_tail_forward_add3", "moe_tail_forward_noalloc", "moe_tail_forward_fused", "moe_tail_forward_fused_bounded",
            "moe_tail_forward_profiled", "moe_tail_forward_timed", "moe_tail_stage_name", "moe_tail_quant_fp8_1x128",
            "moe_tail_pack_mxfp4_scales", "moe_tail_pack_nvfp4_scales", "moe_tail_strerror")


class MoeTailError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {strerror(status)} (status {status})")


class Dims(C.Structure):
    _fields_ = [("hidden", C.c_int32), ("latent", C.c_int32), ("num_experts", C.c_int32), ("top_k", C.c_int32),
                ("inter", C.c_int32), ("shared_inter", C.c_int32), ("wfmt", C.c_int32), ("rms_eps", C.c_float)]


class Weights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("gate", "gate_bias", "w1", "w1_scale", "w2", "w2_scale", "rms_gamma",
                                          "w_up", "ws1", "ws2", "w1_tensor_scale", "w2_tensor_scale")]


class Routing(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("topk_ids", "topk_weights", "expert_offsets", "sorted_pair",
                                          "pair_to_row")]


_lib = None


def lib() -> C.CDLL:
    """Load the HIP library; fails loudly when it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = C.CDLL(LIB_PATH)
        L.moe_tail_workspace_bytes.restype = C.c_size_t
        L.moe_tail_workspace_bytes.argtypes = [C.POINTER(Dims), C.c_int32, C.c_int32]
        L.moe_tail_workspace_layout.restype = C.c_int
        L.moe_tail_workspace_layout.argtypes = [C.POINTER(Dims), C.c_int32, C.c_int32, C.POINTER(C.c_size_t)]
        L.moe_tail_route.restype = C.c_int
        L.moe_tail_route.argtypes = [C.POINTER(Dims), C.POINTER(Weights), C.c_void_p, C.c_int32,
                                     C.POINTER(Routing), C.c_void_p, C.c_size_t, C.c_void_p]
        fwd = [C.POINTER(Dims), C.POINTER(Weights), C.c_void_p, C.c_int32, C.c_void_p, C.c_int32,
               C.POINTER(Routing), C.c_void_p, C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]
        L.moe_tail_forward.restype = C.c_int
        L.moe_tail_forward.argtypes = fwd
        L.moe_tail_forward_noalloc.restype = C.c_int
        L.moe_tail_forward_noalloc.argtypes = fwd[:9] + [C.c_void_p]
        L.moe_tail_forward_add3.restype = C.c_int
        L.moe_tail_forward_add3.argtypes = fwd[:7] + [C.c_void_p] + fwd[7:]
        L.moe_tail_forward_fused.restype = C.c_int
        L.moe_tail_forward_fused.argtypes = fwd[:7] + [C.c_void_p] + fwd[7:]
        L.moe_tail_forward_fused_bounded.restype = C.c_int
        L.moe_tail_forward_fused_bounded.argtypes = fwd[:7] + [C.c_void_p] + fwd[7:] + [C.c_int32]
        L.moe_tail_forward_timed.restype = C.c_int
        L.moe_tail_forward_timed.argtypes = fwd[:7] + [C.c_void_p] + fwd[7:] + [C.POINTER(C.c_void_p)]
        L.moe_tail_stage_name.restype = C.c_char_p
        L.moe_tail_stage_name.argtypes = [C.POINTER(Dims), C.c_int32, C.c_int32, C.c_int32]
        L.moe_tail_forward_profiled.restype = C.c_int
        L.moe_tail_forward_profiled.argtypes = fwd + [C.POINTER(C.c_void_p)]
        L.moe_tail_quant_fp8_1x128.restype = C.c_int
        L.moe_tail_quant_fp8_1x128.argtypes = [C.c_void_p, C.c_int32, C.c_int32, C.c_int32, C.c_void_p,
                                               C.c_void_p, C.c_void_p]
        L.moe_tail_pack_mxfp4_scales.restype = C.c_int
        L.moe_tail_pack_mxfp4_scales.argtypes = [C.POINTER(Dims), C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                                 C.c_void_p]
        L.moe_tail_pack_nvfp4_scales.restype = C.c_int
        L.moe_tail_pack_nvfp4_scales.argtypes = [C.POINTER(Dims), C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                                 C.c_void_p]
        L.moe_tail_strerror.restype = C.c_char_p
        L.moe_tail_strerror.argtypes = [C.c_int]
        _lib = L
    return _lib


def ptr(x) -> int | None:
    """Device address of a torch tensor / integer / None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def stream_handle(stream) -> int | None:
    if stream is None:
        return None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def strerror(status: int) -> str:
    return lib().moe_tail_strerror(status).decode()


def _check(rc: int, where: str) -> None:
    if rc != MOE_TAIL_OK:
        raise MoeTailError(rc, where)


def make_dims(hidden, latent, num_experts, top_k, inter, shared_inter, wfmt, rms_eps) -> Dims:
    return Dims(hidden, latent, num_experts, top_k, inter, shared_inter, wfmt, rms_eps)


def make_weights(**kw) -> Weights:
    return Weights(**{k: ptr(v) for k, v in kw.items()})


def make_routing(**kw) -> Routing:
    return Routing(**{k: ptr(v) for k, v in kw.items()})


def moe_tail_workspace_bytes(dims: Dims, Mr: int, Ms: int) -> int:
    return lib().moe_tail_workspace_bytes(C.byref(dims), Mr, Ms)


def moe_tail_workspace_layout(dims: Dims, Mr: int, Ms: int) -> list[int]:
    offs = (C.c_size_t * MOE_TAIL_WS_NUM)()
    _check(lib().moe_tail_workspace_layout(C.byref(dims), Mr, Ms, offs), "moe_tail_workspace_layout")
    return list(offs)


def moe_tail_route(dims: Dims, weights: Weights, x_lat, Mr: int, routing: Routing, workspace, ws_bytes: int,
                   stream=None) -> None:
    _check(lib().moe_tail_route(C.byref(dims), C.byref(weights), ptr(x_lat), Mr, C.byref(routing), ptr(workspace),
                                ws_bytes, stream_handle(stream)), "moe_tail_route")


def moe_tail_forward(dims: Dims, weights: Weights, x_lat, Mr: int, x_hid, Ms: int, routing: Routing, out,
                     shared_out, workspace, ws_bytes: int, stream=None) -> None:
    _check(lib().moe_tail_forward(C.byref(dims), C.byref(weights), ptr(x_lat), Mr, ptr(x_hid), Ms,
                                  C.byref(routing), ptr(out), ptr(shared_out), ptr(workspace), ws_bytes,
                                  stream_handle(stream)), "moe_tail_forward")


MOE_TAIL_NOALLOC_MAX_BYTES = 48 << 20


def moe_tail_forward_noalloc(dims: Dims, weights: Weights, x_lat, Mr: int, x_hid, Ms: int, routing: Routing, out,
                             shared_out, stream=None) -> None:
    _check(lib().moe_tail_forward_noalloc(C.byref(dims), C.byref(weights), ptr(x_lat), Mr, ptr(x_hid), Ms,
                                          C.byref(routing), ptr(out), ptr(shared_out), stream_handle(stream)),
           "moe_tail_forward_noalloc")


def moe_tail_forward_add3(dims: Dims, weights: Weights, x_lat, Mr: int, x_hid, Ms: int, routing: Routing, residual,
                          out, shared_out, workspace, ws_bytes: int, stream=None) -> None:
    _check(lib().moe_tail_forward_add3(C.byref(dims), C.byref(weights), ptr(x_lat), Mr, ptr(x_hid), Ms,
                                       C.byref(routing), ptr(residual), ptr(out), ptr(shared_out), ptr(workspace),
                                       ws_bytes, stream_handle(stream)), "moe_tail_forward_add3")


def moe_tail_forward_fused(dims: Dims, weights: Weights, x_lat, Mr: int, x_hid, Ms: int, routing: Routing, residual,
                           out, shared_out, workspace, ws_bytes: int, stream=None) -> None:
    """``residual`` None: moe_tail_forward's result; else moe_tail_forward_add3's."""
    _check(lib().moe_tail_forward_fused(C.byref(dims), C.byref(weights), ptr(x_lat), Mr, ptr(x_hid), Ms,
                                        C.byref(routing), ptr(residual), ptr(out), ptr(shared_out), ptr(workspace),
                                        ws_bytes, stream_handle(stream)), "moe_tail_forward_fused")


def moe_tail_forward_fused_bounded(dims: Dims, weights: Weights, x_lat, Mr: int, x_hid, Ms: int, routing: Routing,
                                   residual, out, shared_out, workspace, ws_bytes: int, stream, max_polls: int) -> None:
    _check(lib().moe_tail_forward_fused_bounded(C.byref(dims), C.byref(weights), ptr(x_lat), Mr, ptr(x_hid), Ms,
                                                C.byref(routing), ptr(residual), ptr(out), ptr(shared_out),
                                                ptr(workspace), ws_bytes, stream_handle(stream), max_polls),
           "moe_tail_forward_fused_bounded")


def moe_tail_forward_profiled(dims: Dims, weights: Weights, x_lat, Mr: int, x_hid, Ms: int, routing: Routing, out,
                              shared_out, workspace, ws_bytes: int, stream, events) -> None:
    """``events``: MOE_TAIL_NUM_STAGES + 1 hipEvent_t handles (integers)."""
    arr = (C.c_void_p * len(events))(*events)
    _check(lib().moe_tail_forward_profiled(C.byref(dims), C.byref(weights), ptr(x_lat), Mr, ptr(x_hid), Ms,
                                           C.byref(routing), ptr(out), ptr(shared_out), ptr(workspace), ws_bytes,
                                           stream_handle(stream), arr), "moe_tail_forward_profiled")


def moe_tail_forward_timed(dims: Dims, weights: Weights, x_lat, Mr: int, x_hid, Ms: int, routing: Routing, residual,
                           out, shared_out, workspace, ws_bytes: int, stream, events) -> None:
    """``events``: MOE_TAIL_NUM_STAGES + 1 hipEvent_t handles (integers)."""
    arr = (C.c_void_p * len(events))(*events)
    _check(lib().moe_tail_forward_timed(C.byref(dims), C.byref(weights), ptr(x_lat), Mr, ptr(x_hid), Ms,
                                        C.byref(routing), ptr(residual), ptr(out), ptr(shared_out), ptr(workspace),
                                        ws_bytes, stream_handle(stream), arr), "moe_tail_forward_timed")


def moe_tail_stage_names(dims: Dims, Mr: int, Ms: int) -> list[str]:
    """Names of the launch groups of moe_tail_forward's schedule for these sizes."""
    names = []
    while True:
        n = lib().moe_tail_stage_name(C.byref(dims), Mr, Ms, len(names))
        if n is None:
            return names
        names.append(n.decode())


def moe_tail_pack_nvfp4_scales(dims: Dims, w1_scale, w2_scale, w1_scale_packed, w2_scale_packed, stream=None) -> None:
    _check(lib().moe_tail_pack_nvfp4_scales(C.byref(dims), ptr(w1_scale), ptr(w2_scale), ptr(w1_scale_packed),
                                            ptr(w2_scale_packed), stream_handle(stream)), "moe_tail_pack_nvfp4_scales")


def moe_tail_pack_mxfp4_scales(dims: Dims, w1_scale, w2_scale, w1_scale_packed, w2_scale_packed, stream=None) -> None:
    _check(lib().moe_tail_pack_mxfp4_scales(C.byref(dims), ptr(w1_scale), ptr(w2_scale), ptr(w1_scale_packed),
                                            ptr(w2_scale_packed), stream_handle(stream)), "moe_tail_pack_mxfp4_scales")


def moe_tail_quant_fp8_1x128(x, x_is_bf16: bool, rows: int, cols: int, codes, scales, stream=None) -> None:
    _check(lib().moe_tail_quant_fp8_1x128(ptr(x), int(bool(x_is_bf16)), rows, cols, ptr(codes), ptr(scales),
                                          stream_handle(stream)), "moe_tail_quant_fp8_1x128")


# ------------------------------------------------------------ probes --
# libmoe_tail_probes.so (include/moe_tail_probes.h): measurement kernels the
# tests and the benchmark use; not steps of the tail.

PROBES_PATH = os.path.join(_HERE, "libmoe_tail_probes.so")
PROBES_EXPORTED = ("moe_tail_probe_mfma_fp8", "moe_tail_probe_copy", "moe_tail_probe_stream_read",
                   "moe_tail_probe_stream_paths")

_probes = None


def probes() -> C.CDLL:
    """Load the probe library; fails loudly when it has not been built."""
    global _probes
    if _probes is None:
        if not os.path.exists(PROBES_PATH):
            raise ImportError(f"{PROBES_PATH} is missing: build it with __graft_entry__.build()")
        L = C.CDLL(PROBES_PATH)
        L.moe_tail_probe_mfma_fp8.restype = C.c_int
        L.moe_tail_probe_mfma_fp8.argtypes = [C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32, C.c_void_p]
        L.moe_tail_probe_copy.restype = C.c_int
        L.moe_tail_probe_copy.argtypes = [C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]
        L.moe_tail_probe_stream_read.restype = C.c_int
        L.moe_tail_probe_stream_read.argtypes = [C.c_void_p, C.c_size_t, C.c_void_p, C.c_uint32, C.c_void_p]
        L.moe_tail_probe_stream_paths.restype = C.c_int
        L.moe_tail_probe_stream_paths.argtypes = [C.c_void_p, C.c_size_t, C.c_int32, C.c_int32, C.c_int32, C.c_int32,
                                                  C.c_void_p, C.c_uint32, C.c_void_p]
        _probes = L
    return _probes


def _check_probe(rc: int, where: str) -> None:
    if rc != 0:
        raise MoeTailError(rc, where)


def moe_tail_probe_mfma_fp8(a, b, c, n: int, stream=None) -> None:
    _check_probe(probes().moe_tail_probe_mfma_fp8(ptr(a), ptr(b), ptr(c), n, stream_handle(stream)),
                 "moe_tail_probe_mfma_fp8")


def moe_tail_probe_copy(src, dst, nbytes: int, stream=None) -> None:
    _check_probe(probes().moe_tail_probe_copy(ptr(src), ptr(dst), nbytes, stream_handle(stream)),
                 "moe_tail_probe_copy")


def moe_tail_probe_stream_read(src, nbytes: int, sink, magic: int = 0x9E3779B9, stream=None) -> None:
    _check_probe(probes().moe_tail_probe_stream_read(ptr(src), nbytes, ptr(sink), magic, stream_handle(stream)),
                 "moe_tail_probe_stream_read")


def moe_tail_probe_stream_paths(src, per_wg: int, grid: int, shared: bool, mode: int, row_bytes: int, sink,
                                magic: int = 0x9E3779B9, stream=None) -> None:
    _check_probe(probes().moe_tail_probe_stream_paths(ptr(src), per_wg, grid, int(bool(shared)), mode, row_bytes,
                                                      ptr(sink), magic, stream_handle(stream)),
                 "moe_tail_probe_stream_paths")
