"""Benchmark of the latent-MoE layer tail on one MI355X.

One step = one pass of the whole tail (route + forward: router top-k and
permutation, x quantization, routed L1 + SwiGLU + h quantization, routed L2,
combine + RMSNorm, shared L1 + SwiGLU, shared L2, up-projection + FP32 shared
add) over one batch of seeded synthetic input already resident in HBM.  At
decode sizes moe_tail_forward runs independent stages in shared launches;
the per-stage breakdown (`stage_us`) comes from moe_tail_forward_profiled,
which keeps one launch per stage (the same kernels' bodies and bits).

Prints ONE JSON line.  `value` is the whole tail's achieved HBM throughput
(algorithmic bytes / time per layer); `us_per_layer` is the step time.  The
`roofline` object covers the dominant kernel (the routed L1 launch), timed with HIP events
recorded on the stream it runs on.  `cpu_baseline` times the CPU oracle on the
same inputs (rank 0, N = 1 only).
"""
from __future__ import annotations

import argparse
import ctypes as C
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "latent-MoE tail µs/layer + achieved HBM GB/s (M<=128) / MFMA TFLOP/s (M>=1024)"
HBM_PEAK_GBS = 8000.0
# HBM bytes per launch of the routed L1 kernel from FETCH_SIZE and WRITE_SIZE
# counter runs, scaled by the same counters' reading of a copy kernel of known
# size (profiles/decode_routed_traffic.md); taken on the current kernels.
MEASURED_L1_TRAFFIC = {"decode": 945.7e6}
# the same for the single-launch forward (quantizer + persistent tail)
MEASURED_FUSED_TRAFFIC: dict = {}
FP8_PEAK_TFLOPS = 5000.0
MXFP4_PEAK_TFLOPS = 10100.0
STAGES = ["quant_x", "routed_l1", "routed_l2", "combine_rmsnorm", "shared_l1", "shared_l2", "up_proj_add"]


class HipEvents:
    """hipEvent_t handles through the HIP runtime's C API (recorded by the
    library on the stream it launches on)."""

    def __init__(self, n: int):
        self.rt = C.CDLL("libamdhip64.so")
        self.rt.hipEventCreate.argtypes = [C.POINTER(C.c_void_p)]
        self.rt.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
        self.rt.hipEventSynchronize.argtypes = [C.c_void_p]
        self.rt.hipEventRecord.argtypes = [C.c_void_p, C.c_void_p]
        self.ev = []
        for _ in range(n):
            h = C.c_void_p()
            assert self.rt.hipEventCreate(C.byref(h)) == 0
            self.ev.append(h.value)

    def record(self, i: int, stream) -> None:
        assert self.rt.hipEventRecord(C.c_void_p(self.ev[i]), C.c_void_p(stream.cuda_stream)) == 0

    def elapsed_ms(self, a: int, b: int) -> float:
        ms = C.c_float()
        assert self.rt.hipEventSynchronize(C.c_void_p(self.ev[b])) == 0
        assert self.rt.hipEventElapsedTime(C.byref(ms), C.c_void_p(self.ev[a]), C.c_void_p(self.ev[b])) == 0
        return ms.value


def routed_l1_bytes(wl, touched: int) -> int:
    """Algorithmic bytes of the routed L1 launch: the touched experts' W1 and
    its scales, the x codes and scales it gathers, the h codes and scales it
    writes."""
    L, I, R = wl.L, wl.I, wl.Mr * wl.k
    if wl.wfmt == 0:
        w = touched * (2 * I * L + 4 * (2 * I // 128) * (L // 128))
    else:
        w = touched * (2 * I * L // 2 + 2 * I * L // 32)
    return w + wl.Mr * (L + 4 * L // 128) + R * (I + 4 * I // 128)


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="decode", choices=["tiny", "decode", "prefill", "mxfp4", "indep"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager", action="store_true", help="time eager launches instead of graph replays")
    ap.add_argument("--add3", action="store_true",
                    help="time moe_tail_forward_add3 (the residual joined in the up-projection epilogue)")
    ap.add_argument("--fused", action="store_true",
                    help="time moe_tail_forward_fused (the x quantizer, then one persistent launch for the rest)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs the tail on one GPU only; --gpus {args.gpus} is not supported "
              "(how the tail would shard over several GPUs is a design note, not code).", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from latent_moe_layer_amd import synth
    from latent_moe_layer_amd.device import DeviceTail, to_np

    wl = synth.WORKLOADS[args.workload]
    t0 = time.time()
    inp = synth.make_inputs(wl)
    gen_s = time.time() - t0
    # MXFP4 scales go in the tiled kernels' order once, as a server would at load
    dev = DeviceTail(inp, "cuda:0", pack_scales=wl.wfmt == synth.WFMT_MXFP4)
    if args.add3:
        dev.set_residual(synth.make_residual(wl))
    stream = torch.cuda.Stream()
    nst = len(STAGES)
    hev = HipEvents((args.steps + 1) * (nst + 1) + 2)

    def step(st, events=None):
        dev.route(st)
        dev.forward(st, events, fused=args.fused and events is None)

    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            step(stream)
    torch.cuda.synchronize()

    if args.eager:
        run_step = lambda: step(stream)  # noqa: E731
    else:
        # one step (route + forward, all kernels) captured as a HIP graph
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step(torch.cuda.current_stream())
        torch.cuda.synchronize()
        for _ in range(3):
            graph.replay()
        run_step = graph.replay

    # timed region: exactly K steps
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(torch.cuda.current_stream() if not args.eager else stream)
    for _ in range(args.steps):
        run_step()
    stop.record(torch.cuda.current_stream() if not args.eager else stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    ms_per_step = total_ms / args.steps

    # per-stage durations: K more eager steps, the library recording HIP events
    # on the stream its kernels run on (the profiled entry point has no add3
    # variant; the stages run the same kernels)
    residual, dev.residual = getattr(dev, "residual", None), None
    for i in range(args.steps):
        step(stream, hev.ev[i * (nst + 1):(i + 1) * (nst + 1)])
    torch.cuda.synchronize()
    dev.residual = residual
    stage_ms = np.zeros(nst)
    for i in range(args.steps):
        base = i * (nst + 1)
        for s in range(nst):
            stage_ms[s] += hev.elapsed_ms(base + s, base + s + 1)
    stage_ms /= args.steps

    fused_ms = None
    if args.fused:
        # the single-launch forward (x quantizer + persistent tail) bracketed
        # by HIP events on its stream, route outside the brackets
        base = args.steps * (nst + 1)
        tot = 0.0
        for i in range(args.steps):
            dev.route(stream)
            hev.record(base, stream)
            dev.forward(stream, fused=True)
            hev.record(base + 1, stream)
            tot += hev.elapsed_ms(base, base + 1)
        fused_ms = tot / args.steps

    offsets = to_np(dev.offsets)
    touched = int(np.count_nonzero(np.diff(offsets)))
    nbytes = synth.algorithmic_bytes(wl, touched)["total"] + (wl.Mr * wl.H * 2 if args.add3 else 0)
    flops = synth.algorithmic_flops(wl)
    us = ms_per_step * 1e3
    gbs = nbytes / (ms_per_step * 1e-3) / 1e9
    l1_bytes = routed_l1_bytes(wl, touched)
    l1_ms = float(stage_ms[1])
    if wl.Mr <= 128:
        roof = {"bound": "hbm", "achieved": l1_bytes / (l1_ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    else:
        l1_flops = 2 * wl.Mr * wl.k * 2 * wl.I * wl.L
        peak = FP8_PEAK_TFLOPS if wl.wfmt == 0 else MXFP4_PEAK_TFLOPS
        roof = {"bound": "mfma", "achieved": l1_flops / (l1_ms * 1e-3) / 1e12, "peak": peak, "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = MEASURED_L1_TRAFFIC.get(wl.name)
    # the routed L1 stage: the persistent tiled kernel's launches (32-row
    # tiles, or 32- and 64-row tiles in one launch; past 256 tokens, FP8 also
    # the 128-row and 256-row launches)
    fmt = "TF_FP8" if wl.wfmt == 0 else "TF_FP4"
    small = f"k_tile<TK_L1, {fmt}, 0, 32>" if wl.Mr * wl.k <= 32 * wl.E and wl.Mr <= 256 \
        else f"k_tile_small_mid<TK_L1, {fmt}>"
    roof["kernel"] = small + ("" if wl.Mr <= 256 or wl.wfmt != 0
                              else f" + k_tile<TK_L1, {fmt}, 0, 128> + k_tile<TK_L1, {fmt}, 0, 256>")
    roof["algorithmic_bytes_per_launch"] = l1_bytes
    roof["avg_launch_us"] = l1_ms * 1e3
    if fused_ms is not None:
        # the dominant launch is then the persistent tail itself: every byte of
        # the forward (all but the router's weights), timed with the quantizer
        # launch that precedes it
        fw_bytes = nbytes - 4 * wl.E * wl.L
        roof = {"bound": "hbm", "achieved": fw_bytes / (fused_ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s"}
        roof["frac"] = roof["achieved"] / roof["peak"]
        roof["traffic"] = MEASURED_FUSED_TRAFFIC.get(wl.name)
        roof["kernel"] = f"k_quant_clear + k_tail_small<{fmt}>"
        roof["algorithmic_bytes_per_launch"] = fw_bytes
        roof["avg_launch_us"] = fused_ms * 1e3

    cpu = None
    if not args.no_cpu_baseline:
        from oracle import oracle as orc
        sample = min(wl.Mr, 128)
        sel = np.linspace(0, wl.Mr - 1, sample).astype(np.int32) if sample < wl.Mr else None
        t1 = time.time()
        ids, w = orc.route(inp.x_lat, inp.gate, inp.gate_bias, wl.k)
        orc.permute(ids, wl.E)
        orc.forward(inp, ids, w, sel=sel)
        cpu_s = (time.time() - t1) * wl.Mr / sample
        cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
        cpu = {"value": nbytes / cpu_s / 1e9, "unit": "GB/s", "cores": cores, "kind": "oracle",
               "us_per_layer": cpu_s * 1e6,
               "sample": (f"route + permute + forward of all {wl.Mr} tokens" if sample == wl.Mr else
                          f"route of all tokens + forward of {sample} of {wl.Mr} tokens, scaled to {wl.Mr}")}

    out = {
        "metric": METRIC, "value": gbs, "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_per_step, "us_per_layer": us, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp8e4m3+bf16" if wl.wfmt == 0 else "mxfp4+fp8e4m3+bf16",
        "data": "synthetic (seeded; random-init weights of the tail's shapes)",
        "config": {"workload": f"{wl.name}: Mr={wl.Mr} Ms={wl.Ms} E={wl.E} top{wl.k} I={wl.I} I_s={wl.Is} "
                               f"H={wl.H} L={wl.L} {'FP8 128x128' if wl.wfmt == 0 else 'MXFP4 (e8m0 scales packed)'} routed weights",
                   "global_batch": wl.Mr, "parallelism": "single GPU",
                   "epilogue": "add3: up + shared + residual, one rounding" if args.add3 else "up + shared"},
        "algorithmic_bytes": nbytes, "touched_experts": touched,
        "tflops_lowp": flops["lowp"] / (ms_per_step * 1e-3) / 1e12,
        "tflops_bf16": flops["bf16"] / (ms_per_step * 1e-3) / 1e12,
        "hbm_frac": gbs / HBM_PEAK_GBS,
        "timing": ("eager launches" if args.eager else "HIP graph replay of route + forward") +
                  (" (single-launch forward)" if args.fused else ""),
        "stage_us": {n: float(v * 1e3) for n, v in zip(STAGES, stage_ms)},
        "stage_timing": "one launch per stage (moe_tail_forward_profiled), HIP events on its stream",
        "roofline": roof, "cpu_baseline": cpu, "input_gen_s": gen_s,
    }
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
