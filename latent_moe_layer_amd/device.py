"""Device-side buffers for one tail: uploads a seeded ``synth.Inputs`` with
torch (device memory and streams only) and calls the C ABI through
``binding``.  No arithmetic of the tail happens here."""
from __future__ import annotations

import numpy as np
import torch

from . import binding as B
from . import synth


def _dev(a: np.ndarray, device) -> torch.Tensor:
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


class DeviceTail:
    """Weights, inputs, routing, outputs and workspace of one tail on one GPU."""

    def __init__(self, inp: synth.Inputs, device="cuda:0", Mr: int | None = None, Ms: int | None = None,
                 pack_scales: bool = False):
        """``pack_scales`` (MXFP4 or NVFP4 weights): rearrange the block scales
        once with moe_tail_pack_mxfp4_scales / moe_tail_pack_nvfp4_scales and
        run the forward on the packed order."""
        wl = inp.wl
        self.inp = inp
        self.device = torch.device(device)
        self.Mr = inp.x_lat.shape[0] if Mr is None else Mr
        self.Ms = inp.x_hid.shape[0] if Ms is None else Ms
        self.dims = B.make_dims(wl.H, wl.L, wl.E, wl.k, wl.I, wl.Is, wl.wfmt, wl.rms_eps)
        d = self.device
        self.t = {name: _dev(getattr(inp, name), d) for name in
                  ("x_lat", "x_hid", "gate", "gate_bias", "w1", "w1_scale", "w2", "w2_scale", "gamma", "w_up",
                   "ws1", "ws2", "w1_tscale", "w2_tscale")}
        t = self.t
        if pack_scales:
            if wl.wfmt not in (synth.WFMT_MXFP4, synth.WFMT_NVFP4):
                raise ValueError("packed scales are an MXFP4 or NVFP4 layout")
            t["w1_scale"], natural1 = torch.empty_like(t["w1_scale"]), t["w1_scale"]
            t["w2_scale"], natural2 = torch.empty_like(t["w2_scale"]), t["w2_scale"]
            if wl.wfmt == synth.WFMT_MXFP4:
                B.moe_tail_pack_mxfp4_scales(self.dims, natural1, natural2, t["w1_scale"], t["w2_scale"])
                self.dims.wfmt = B.MOE_TAIL_W_MXFP4_PACKED
            else:
                B.moe_tail_pack_nvfp4_scales(self.dims, natural1, natural2, t["w1_scale"], t["w2_scale"])
                self.dims.wfmt = B.MOE_TAIL_W_NVFP4_PACKED
            torch.cuda.synchronize(d)
        self.weights = B.make_weights(gate=t["gate"], gate_bias=t["gate_bias"], w1=t["w1"], w1_scale=t["w1_scale"],
                                      w2=t["w2"], w2_scale=t["w2_scale"], rms_gamma=t["gamma"], w_up=t["w_up"],
                                      ws1=t["ws1"], ws2=t["ws2"],
                                      w1_tensor_scale=t["w1_tscale"] if wl.wfmt == synth.WFMT_NVFP4 else None,
                                      w2_tensor_scale=t["w2_tscale"] if wl.wfmt == synth.WFMT_NVFP4 else None)
        self.alloc(self.Mr, self.Ms)

    def alloc(self, Mr: int, Ms: int) -> None:
        """(Re)allocate routing, outputs and workspace for Mr routed / Ms shared tokens."""
        wl, d = self.inp.wl, self.device
        self.Mr, self.Ms = Mr, Ms
        R = Mr * wl.k
        self.topk_ids = torch.empty((Mr, wl.k), dtype=torch.int32, device=d)
        self.topk_w = torch.empty((Mr, wl.k), dtype=torch.float32, device=d)
        self.offsets = torch.empty(wl.E + 1, dtype=torch.int32, device=d)
        self.sorted_pair = torch.empty(R, dtype=torch.int32, device=d)
        self.pair_to_row = torch.empty(R, dtype=torch.int32, device=d)
        self.routing = B.make_routing(topk_ids=self.topk_ids, topk_weights=self.topk_w,
                                      expert_offsets=self.offsets, sorted_pair=self.sorted_pair,
                                      pair_to_row=self.pair_to_row)
        self.out = torch.empty((Mr, wl.H), dtype=torch.int16, device=d)
        self.shared_out = torch.empty((Ms - Mr, wl.H), dtype=torch.int16, device=d) if Ms > Mr else None
        self.ws_bytes = B.moe_tail_workspace_bytes(self.dims, Mr, Ms)
        if self.ws_bytes == 0 and (Mr or Ms):
            raise ValueError("dims or token counts rejected by moe_tail_workspace_bytes")
        self.ws = torch.empty(max(self.ws_bytes, 256), dtype=torch.uint8, device=d)
        self.layout = B.moe_tail_workspace_layout(self.dims, Mr, Ms)

    def route(self, stream=None) -> None:
        B.moe_tail_route(self.dims, self.weights, self.t["x_lat"], self.Mr, self.routing, self.ws, self.ws_bytes,
                         stream)

    def set_residual(self, residual: np.ndarray | None) -> None:
        """Upload the add3 residual ([Mr, H] bf16 bits); None goes back to the plain forward."""
        self.residual = None if residual is None else _dev(residual, self.device)

    def forward(self, stream=None, events=None, fused: bool = False) -> None:
        """The multi-launch forward (with stage events if given), or with
        ``fused`` the single-launch one (moe_tail_forward_fused)."""
        res = getattr(self, "residual", None)
        if fused:
            if events is not None:
                raise ValueError("the single-launch forward has no stage events")
            B.moe_tail_forward_fused(self.dims, self.weights, self.t["x_lat"], self.Mr, self.t["x_hid"], self.Ms,
                                     self.routing, res, self.out, self.shared_out, self.ws, self.ws_bytes, stream)
            return
        if res is not None:
            if events is not None:
                raise ValueError("the profiled forward has no add3 variant")
            B.moe_tail_forward_add3(self.dims, self.weights, self.t["x_lat"], self.Mr, self.t["x_hid"], self.Ms,
                                    self.routing, res, self.out, self.shared_out, self.ws, self.ws_bytes, stream)
            return
        args = (self.dims, self.weights, self.t["x_lat"], self.Mr, self.t["x_hid"], self.Ms, self.routing, self.out,
                self.shared_out, self.ws, self.ws_bytes, stream)
        if events is None:
            B.moe_tail_forward(*args)
        else:
            B.moe_tail_forward_profiled(*args, events)

    def forward_timed(self, stream, events) -> None:
        """moe_tail_forward's schedule (add3 if a residual is set) with an event
        before each launch group (moe_tail_forward_timed)."""
        B.moe_tail_forward_timed(self.dims, self.weights, self.t["x_lat"], self.Mr, self.t["x_hid"], self.Ms,
                                 self.routing, getattr(self, "residual", None), self.out, self.shared_out, self.ws,
                                 self.ws_bytes, stream, events)

    # -------- views of the materialized intermediates (tests) --------
    def _view(self, idx: int, dtype, shape):
        n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        off = self.layout[idx]
        return self.ws[off:off + n].view(dtype).view(*shape)

    def intermediates(self) -> dict:
        wl = self.inp.wl
        Mr, Ms, R = self.Mr, self.Ms, self.Mr * wl.k
        return {
            "xq": self._view(B.MOE_TAIL_WS_XQ, torch.uint8, (Mr, wl.L)),
            "sx": self._view(B.MOE_TAIL_WS_SX, torch.float32, (Mr, wl.L // 128)),
            "hq": self._view(B.MOE_TAIL_WS_HQ, torch.uint8, (R, wl.I)),
            # (stored K-block-major, [I/128, R]; viewed here as [R, I/128])
            "sh": self._view(B.MOE_TAIL_WS_SH, torch.float32, (wl.I // 128, R)).t(),
            "y": self._view(B.MOE_TAIL_WS_Y, torch.float32, (R, wl.L)),
            "rn": self._view(B.MOE_TAIL_WS_RN, torch.int16, (Mr, wl.L)),
            "hs": self._view(B.MOE_TAIL_WS_HS, torch.int16, (Ms, wl.Is)),
            "s": self._view(B.MOE_TAIL_WS_S, torch.int16, (Mr, wl.H)),
        }


def to_np(t: torch.Tensor) -> np.ndarray:
    a = t.detach().cpu().numpy()
    if a.dtype == np.int16:
        a = a.view(np.uint16)
    return a
