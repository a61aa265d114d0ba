"""Benchmark of the latent-MoE layer tail on one MI355X.

One step = one pass of the whole tail (route + forward: router top-k and
permutation, x quantization, routed L1 + SwiGLU + h quantization, routed L2,
combine + RMSNorm, shared L1 + SwiGLU, shared L2, up-projection + FP32 shared
add) over one batch of seeded synthetic input already resident in HBM,
captured as one HIP graph and replayed.

Prints ONE JSON line.  The headline is the decode workload (128 routed and
128 shared tokens, 64 experts, top-8, FP8 experts): `value` is the whole
tail's achieved HBM throughput (algorithmic bytes / mean time per layer over
the K timed replays, which run back to back between two events).  The same
line carries, under `legs`, the other workloads timed the same way (by
default all of them: prefill, the MFMA-bound half of the metric, tiny,
mxfp4, the independent-count workload and nvfp4), and for every workload:
  - median / p10 / p90 of the per-replay times (K replays before those, with
    an event between consecutive ones; `us_per_layer_evented` is their mean),
    and the same cache-cold (a 512 MiB streaming read between replays, outside
    the timed pair, evicts the 256 MB Infinity Cache);
  - `us_per_layer_5_per_graph`: context, the step captured five times in one
    graph (as a model's graph holds one per layer), per step;
  - `groups_us`: each launch group of the schedule the plain call runs, from
    moe_tail_forward_timed (events recorded on the library's stream; where
    the plain call runs the shared L1 and L2 on a second stream beside the
    routed GEMMs, the timed call keeps them on one stream, so its groups
    time each stage alone);
  - `roofline`: the routed L1 launch(es) against the bound of that workload
    (HBM for the weight-streaming workloads, FP8 MFMA for prefill), with the
    other unit alongside.
`stream_read_gbs` is a plain streaming read of 4 GiB (moe_tail_probe_stream
_read), the practical HBM read ceiling.  `cpu_baseline` times the CPU oracle
on the decode workload's tokens (rank 0, N = 1 only).

`--calibrate-copy` instead copies 512 MiB three times with the probe copy
kernel (for scaling the FETCH_SIZE / WRITE_SIZE counters under rocprofv3).
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
FP8_PEAK_TFLOPS = 5000.0     # dense FP8 (and FP8 x FP4: the scaled MFMA runs both at the FP8 rate)
BF16_PEAK_TFLOPS = 2500.0
# HBM bytes per launch of a routed L1 kernel from FETCH_SIZE and WRITE_SIZE
# counter runs, each scaled by the same counter's reading of the probe copy
# of 512 MiB (bench.py --calibrate-copy); see the traffic summaries under
# profiles/.  Only figures taken on the current kernels are listed.
MEASURED_L1_TRAFFIC = {
    "decode": 945.8e6,    # k_tile<0, 0, 0, 32>: 943.6 MB fetched + 2.2 MB written (profiles/decode_tail_traffic.md)
    "prefill": 1587.2e6,  # k_tile<0, 0, 0, 256> 1127.1 MB + k_tile<0, 0, 0, 128> 460.1 MB (profiles/prefill_tail_traffic.md)
    "mxfp4": 1084.5e6,    # k_tile_small_mid<0, 1> (profiles/mxfp4_tail_traffic.md)
    "nvfp4": 534.6e6,     # k_tile<0, 3, 0, 32> (profiles/nvfp4_tail_traffic.md)
    "indep": 5787.2e6,    # k_tile_small_mid<0, 0>: 5752.5 fetched + 34.8 written (profiles/indep_tail_traffic.md)
}
FORMATS = {0: "FP8 128x128", 1: "MXFP4 (e8m0 scales packed)", 3: "NVFP4 (e4m3 scale per 16 packed, fp32 per matrix)"}
DTYPES = {0: "fp8e4m3+bf16", 1: "mxfp4+fp8e4m3+bf16", 3: "nvfp4+fp8e4m3+fp16+bf16"}
# workloads whose routed GEMMs are bound by the matrix cores (the others stream weights)
MFMA_BOUND = {"prefill"}


class HipEvents:
    """hipEvent_t handles through the HIP runtime's C API (recorded by the
    library on the stream it launches on)."""

    def __init__(self, n: int):
        self.rt = C.CDLL("libamdhip64.so")
        self.rt.hipEventCreate.argtypes = [C.POINTER(C.c_void_p)]
        self.rt.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
        self.rt.hipEventSynchronize.argtypes = [C.c_void_p]
        self.ev = []
        for _ in range(n):
            h = C.c_void_p()
            assert self.rt.hipEventCreate(C.byref(h)) == 0
            self.ev.append(h.value)

    def record(self, i: int, stream) -> None:
        self.rt.hipEventRecord.argtypes = [C.c_void_p, C.c_void_p]
        assert self.rt.hipEventRecord(C.c_void_p(self.ev[i]), C.c_void_p(stream.cuda_stream)) == 0

    def elapsed_ms(self, a: int, b: int) -> float:
        ms = C.c_float()
        assert self.rt.hipEventSynchronize(C.c_void_p(self.ev[b])) == 0
        assert self.rt.hipEventElapsedTime(C.byref(ms), C.c_void_p(self.ev[a]), C.c_void_p(self.ev[b])) == 0
        return ms.value


def routed_l1_bytes(wl, touched: int) -> int:
    """Algorithmic bytes of the routed L1 launch(es): the touched experts' W1
    and its scales, the x codes and scales it gathers, the h codes and scales
    it writes."""
    L, I, R = wl.L, wl.I, wl.Mr * wl.k
    if wl.wfmt == 0:
        w = touched * (2 * I * L + 4 * (2 * I // 128) * (L // 128))
    elif wl.wfmt == 3:
        w = touched * (2 * I * L // 2 + 2 * I * L // 16 + 4)
    else:
        w = touched * (2 * I * L // 2 + 2 * I * L // 32)
    return w + wl.Mr * (L + 4 * L // 128) + R * (I + 4 * I // 128)


def routed_l2_bytes(wl, touched: int) -> int:
    """Algorithmic bytes of the routed L2 launch(es): W2 and scales of the
    touched experts, the h codes and scales, the FP32 y rows."""
    L, I, R = wl.L, wl.I, wl.Mr * wl.k
    if wl.wfmt == 0:
        w = touched * (L * I + 4 * (L // 128) * (I // 128))
    elif wl.wfmt == 3:
        w = touched * (L * I // 2 + L * I // 16 + 4)
    else:
        w = touched * (L * I // 2 + L * I // 32)
    return w + R * (I + 4 * I // 128) + R * L * 4


def pct(xs, q):
    import numpy as np
    return float(np.percentile(np.asarray(xs), q))


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def probe_paths(torch, B, reps: int = 3) -> dict:
    """Per-workgroup rates of the staging load paths (moe_tail_probe_stream_paths),
    best of `reps`: 64 workgroups on private runs (HBM, not saturated), 256 on
    private runs (HBM, the whole chip) and 256 on one shared run (L2)."""
    per = 7 << 20  # 16 matrices of 256 rows x 1792 B, 8 of 256 x 3584 B
    src = torch.empty(256 * per, dtype=torch.uint8, device="cuda").fill_(1)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    paths = [("lds_ring_contiguous", 0, 128), ("lds_ring_rows_1792B", 1, 1792), ("lds_ring_rows_3584B", 1, 3584),
             ("regs_whole_lines", 2, 128), ("regs_half_lines", 3, 128)]
    out = {"per_workgroup_bytes": per, "workgroup_threads": 512,
           "lds_ring": "4 stages of 32 KB, 3 in flight", "regs": "16 loads of 16 B in flight per lane", "results": []}
    for grid, shared in ((64, False), (256, False), (256, True)):
        for name, mode, rb in paths:
            best = 1e30
            for _ in range(reps + 1):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                B.moe_tail_probe_stream_paths(src, per, grid, shared, mode, rb, sink,
                                              stream=torch.cuda.current_stream())
                b.record()
                torch.cuda.synchronize()
                best = min(best, a.elapsed_time(b) * 1e-3)
            gbs = grid * per / best / 1e9
            out["results"].append({"path": name, "grid": grid, "source": "L2 (one shared run)" if shared else "HBM",
                                   "us": round(best * 1e6, 1), "total_GBps": round(gbs), "per_wg_GBps": round(gbs / grid, 1)})
    del src
    return out


def stream_read_gbs(torch, B, reps: int = 5) -> float:
    """Best-of-`reps` rate of one streaming read of 4 GiB."""
    nbytes = 4 << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    best = 0.0
    for _ in range(reps + 1):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        B.moe_tail_probe_stream_read(src, nbytes, sink, stream=torch.cuda.current_stream())
        b.record()
        torch.cuda.synchronize()
        best = max(best, nbytes / (a.elapsed_time(b) * 1e-3) / 1e9)
    del src
    return best


def measure(name: str, args, torch, np, B, synth, DeviceTail, to_np, flush) -> dict:
    wl = synth.WORKLOADS[name]
    t0 = time.time()
    inp = synth.make_inputs(wl)
    gen_s = time.time() - t0
    # FP4 block scales go in the tiled kernels' order once, as a server would at load
    dev = DeviceTail(inp, "cuda:0", pack_scales=wl.wfmt in (synth.WFMT_MXFP4, synth.WFMT_NVFP4))
    if args.add3:
        dev.set_residual(synth.make_residual(wl))
    stream = torch.cuda.Stream()
    K = args.steps

    def step(st):
        dev.route(st)
        dev.forward(st, fused=args.fused)

    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            step(stream)
    torch.cuda.synchronize()

    # one step (route + forward, all kernels) captured as a HIP graph
    if args.eager:
        class _Eager:
            @staticmethod
            def replay():
                step(torch.cuda.current_stream())
        graph = _Eager()
    else:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step(torch.cuda.current_stream())
    torch.cuda.synchronize()
    for _ in range(3):
        graph.replay()
    torch.cuda.synchronize()

    # the distribution over steps: K replays, an event between consecutive
    # ones (this pass also finishes the warm-up: the first pass after the
    # capture measured slower)
    cur = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    torch.cuda.synchronize()
    ev[0].record(cur)
    for i in range(K):
        graph.replay()
        ev[i + 1].record(cur)
    torch.cuda.synchronize()
    per = [ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(K)]
    evented_us = ev[0].elapsed_time(ev[K]) * 1e3 / K

    # timed region: exactly K replays between two events, nothing else
    # enqueued among them (an event recorded between replays costs about 5 us
    # a step at decode size)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(cur)
    for i in range(K):
        graph.replay()
    t1.record(cur)
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)

    # context: the step captured 5 times in one graph, as a model's graph
    # holds one per layer (no graph boundary between them)
    graph5_us = None
    if not args.eager:
        g5 = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g5):
            for _ in range(5):
                step(torch.cuda.current_stream())
        torch.cuda.synchronize()
        g5.replay()
        reps = max(1, K // 5)
        torch.cuda.synchronize()
        t0.record(cur)
        for _ in range(reps):
            g5.replay()
        t1.record(cur)
        torch.cuda.synchronize()
        graph5_us = t0.elapsed_time(t1) * 1e3 / (5 * reps)
        del g5

    # cache-cold: a 512 MiB streaming read before each replay, outside the pair
    cold = []
    if not args.no_cold:
        a = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
        b = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
        for i in range(K):
            B.moe_tail_probe_stream_read(flush["buf"], flush["bytes"], flush["sink"], stream=cur)
            a[i].record(cur)
            graph.replay()
            b[i].record(cur)
        torch.cuda.synchronize()
        cold = [a[i].elapsed_time(b[i]) * 1e3 for i in range(K)]

    # launch groups of the schedule the plain call runs (eager, events on its stream)
    # (the route, moe_tail_route's launches, from an event before it to the
    # forward's first event)
    names = B.moe_tail_stage_names(dev.dims, dev.Mr, dev.Ms)
    nev = B.MOE_TAIL_NUM_STAGES + 1
    per_step = nev + 1
    hev = HipEvents(K * per_step)
    groups = None
    if not args.fused:
        for i in range(K):
            hev.record(i * per_step, stream)
            dev.route(stream)
            dev.forward_timed(stream, hev.ev[i * per_step + 1:(i + 1) * per_step])
        torch.cuda.synchronize()
        gsum = np.zeros(len(names) + 1)
        for i in range(K):
            for g in range(len(names) + 1):
                gsum[g] += hev.elapsed_ms(i * per_step + g, i * per_step + g + 1)
        groups = {n: float(v * 1e3 / K) for n, v in zip(["route"] + names, gsum)}

    offsets = to_np(dev.offsets)
    loads = np.diff(offsets)
    touched = int(np.count_nonzero(loads))
    nbytes = synth.algorithmic_bytes(wl, touched)["total"] + (wl.Mr * wl.H * 2 if args.add3 else 0)
    flops = synth.algorithmic_flops(wl)
    us = total_ms * 1e3 / K
    leg = {
        "workload": f"{wl.name}: Mr={wl.Mr} Ms={wl.Ms} E={wl.E} top{wl.k} I={wl.I} I_s={wl.Is} H={wl.H} L={wl.L} "
                    f"{FORMATS[wl.wfmt]} routed weights",
        "us_per_layer": us, "us_median": pct(per, 50), "us_p10": pct(per, 10), "us_p90": pct(per, 90),
        "us_per_layer_evented": evented_us, "us_per_layer_5_per_graph": graph5_us,
        "cold_us_median": pct(cold, 50) if cold else None, "cold_us_p10": pct(cold, 10) if cold else None,
        "cold_us_p90": pct(cold, 90) if cold else None,
        "algorithmic_bytes": nbytes, "flops_lowp": flops["lowp"], "flops_bf16": flops["bf16"],
        "GBps": nbytes / (us * 1e-6) / 1e9, "hbm_frac": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS,
        "TFLOPs_lowp": flops["lowp"] / (us * 1e-6) / 1e12, "TFLOPs_bf16": flops["bf16"] / (us * 1e-6) / 1e12,
        "touched_experts": touched, "expert_rows_min_max": [int(loads.min()), int(loads.max())],
        "groups_us": groups, "input_gen_s": gen_s,
    }
    if groups is not None and "routed_l1" in groups:
        l1_us = groups["routed_l1"]
        l1_b = routed_l1_bytes(wl, touched)
        l1_f = 2 * wl.Mr * wl.k * 2 * wl.I * wl.L
        gbs = l1_b / (l1_us * 1e-6) / 1e9
        tfs = l1_f / (l1_us * 1e-6) / 1e12
        fmt = {0: "TF_FP8", 1: "TF_FP4", 3: "TF_NV4"}[wl.wfmt]
        if wl.wfmt == 3:
            kern = f"k_tile<TK_L1, {fmt}, 0, 32>"
        elif wl.Mr <= 256 and wl.Mr * wl.k <= 32 * wl.E:
            kern = f"k_tile<TK_L1, {fmt}, 0, 32>"
        else:
            kern = f"k_tile_small_mid<TK_L1, {fmt}>"
            if wl.Mr > 256 and wl.wfmt == 0:
                kern += f" + k_tile<TK_L1, {fmt}, 0, 128> + k_tile<TK_L1, {fmt}, 0, 256>"
        if name in MFMA_BOUND:
            roof = {"bound": "mfma", "achieved": tfs, "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "also": {"achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS}}
        else:
            roof = {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "also": {"achieved": tfs, "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                             "frac": tfs / FP8_PEAK_TFLOPS}}
        roof["frac"] = roof["achieved"] / roof["peak"]
        roof["traffic"] = MEASURED_L1_TRAFFIC.get(name)
        roof["kernel"] = kern
        roof["algorithmic_bytes_per_launch"] = l1_b
        roof["flops_per_launch"] = l1_f
        roof["avg_launch_us"] = l1_us
        roof["timing"] = "HIP events around the routed L1 launch group of moe_tail_forward_timed, on its stream"
        leg["roofline"] = roof
        if "routed_l2" in groups:
            l2_us = groups["routed_l2"]
            lf = 2 * wl.Mr * wl.k * wl.L * wl.I
            both = (l1_f + lf) / ((l1_us + l2_us) * 1e-6) / 1e12
            leg["routed_l1_l2"] = {"us": l1_us + l2_us, "TFLOPs": both, "mfma_frac": both / FP8_PEAK_TFLOPS,
                                   "GBps": (l1_b + routed_l2_bytes(wl, touched)) / ((l1_us + l2_us) * 1e-6) / 1e9}
    leg["_inp"] = inp
    leg["_dev"] = dev
    return leg


def oracle_timing(inp, leg, np) -> dict:
    """The CPU oracle on this workload's inputs: route and permutation of every
    routed token, the forward of at most 128 of the Ms tokens (evenly spread
    over routed and shared-only ones), the forward's time scaled to all Ms."""
    from oracle import oracle as orc
    wl = inp.wl
    sample = min(wl.Ms, 128)
    sel = np.linspace(0, wl.Ms - 1, sample).astype(np.int32) if sample < wl.Ms else None
    t1 = time.time()
    ids, w = orc.route(inp.x_lat, inp.gate, inp.gate_bias, wl.k)
    orc.permute(ids, wl.E)
    t2 = time.time()
    orc.forward(inp, ids, w, sel=sel)
    cpu_s = (t2 - t1) + (time.time() - t2) * wl.Ms / sample
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": leg["algorithmic_bytes"] / cpu_s / 1e9, "unit": "GB/s", "cores": cores, "kind": "oracle",
            "us_per_layer": cpu_s * 1e6, "cpu_model": cpu_model(),
            "sample": (f"route + permute + forward of all {wl.Ms} tokens" if sample == wl.Ms else
                       f"route + permute of all {wl.Mr} routed tokens, forward of {sample} of the {wl.Ms} tokens "
                       f"(evenly spread), scaled to {wl.Ms}")}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode", choices=["tiny", "decode", "prefill", "mxfp4", "indep", "nvfp4"],
                    help="the headline workload")
    ap.add_argument("--legs", default="prefill,tiny,mxfp4,indep,nvfp4",
                    help="other workloads timed on the same line (comma list, 'none', or 'all')")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-all", action="store_true", help="also time the CPU oracle on every leg's tokens")
    ap.add_argument("--no-cold", action="store_true", help="skip the cache-cold replays")
    ap.add_argument("--eager", action="store_true", help="time eager launches instead of graph replays")
    ap.add_argument("--add3", action="store_true",
                    help="time moe_tail_forward_add3 (the residual joined in the up-projection epilogue)")
    ap.add_argument("--fused", action="store_true",
                    help="time moe_tail_forward_fused (the x quantizer, then one persistent launch for the rest)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="copy 512 MiB three times with the probe copy kernel and exit")
    ap.add_argument("--probe-paths", action="store_true",
                    help="time the load-path probes (direct-to-LDS rings, register loads; HBM and L2) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs the tail on one GPU only; --gpus {args.gpus} is not supported "
              "(how the tail would shard over several GPUs is a design note, not code).", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from latent_moe_layer_amd import binding as B
    from latent_moe_layer_amd import synth
    from latent_moe_layer_amd.device import DeviceTail, to_np

    if args.calibrate_copy:
        nbytes = 512 << 20
        src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        torch.cuda.synchronize()
        for _ in range(3):
            B.moe_tail_probe_copy(src, dst, nbytes)
        torch.cuda.synchronize()
        assert torch.equal(src[::4096], dst[::4096])
        print(json.dumps({"calibration": "k_probe_copy", "bytes_read_per_launch": nbytes,
                          "bytes_written_per_launch": nbytes, "launches": 3}))
        return 0

    if args.probe_paths:
        print(json.dumps(probe_paths(torch, B)))
        return 0

    flush = None
    if not args.no_cold:
        fb = 512 << 20
        flush = {"buf": torch.empty(fb, dtype=torch.uint8, device="cuda").fill_(3), "bytes": fb,
                 "sink": torch.zeros(1, dtype=torch.int32, device="cuda")}
    def progress(what):  # one line per finished step of the run, on stderr (stdout carries only the JSON line)
        print(f"[bench] {what}", file=sys.stderr, flush=True)

    head = measure(args.workload, args, torch, np, B, synth, DeviceTail, to_np, flush)
    progress(f"{args.workload}: {head['us_per_layer']:.1f} us per layer")
    legs = {}
    names = [] if args.legs == "none" else \
        (["tiny", "decode", "prefill", "mxfp4", "indep", "nvfp4"] if args.legs == "all" else args.legs.split(","))
    inp, dev = head.pop("_inp"), head.pop("_dev")

    wl = synth.WORKLOADS[args.workload]
    cpu = None if args.no_cpu_baseline else oracle_timing(inp, head, np)
    if cpu is not None:
        progress(f"{args.workload}: oracle timed")
    del inp, dev
    torch.cuda.empty_cache()

    for n in names:
        if n and n != args.workload:
            leg = measure(n, args, torch, np, B, synth, DeviceTail, to_np, flush)
            progress(f"{n}: {leg['us_per_layer']:.1f} us per layer")
            linp = leg.pop("_inp")
            leg.pop("_dev")
            if args.cpu_all:
                leg["cpu_baseline"] = oracle_timing(linp, leg, np)
                progress(f"{n}: oracle timed")
            del linp
            legs[n] = leg
            torch.cuda.empty_cache()

    if flush is not None:
        del flush["buf"]
        torch.cuda.empty_cache()
    sread = stream_read_gbs(torch, B)

    us = head["us_per_layer"]
    out = {
        "metric": METRIC, "value": head["GBps"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": us * 1e-3, "us_per_layer": us, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": DTYPES[wl.wfmt],
        "data": "synthetic (seeded; random-init weights of the tail's shapes)",
        "config": {"workload": head["workload"], "global_batch": wl.Mr, "parallelism": "single GPU",
                   "epilogue": "add3: up + shared + residual, one rounding" if args.add3 else "up + shared"},
        "us_median": head["us_median"], "us_p10": head["us_p10"], "us_p90": head["us_p90"],
        "us_per_layer_evented": head["us_per_layer_evented"],
        "us_per_layer_5_per_graph": head["us_per_layer_5_per_graph"],
        "cold_us_median": head["cold_us_median"], "cold_us_p10": head["cold_us_p10"],
        "cold_us_p90": head["cold_us_p90"],
        "algorithmic_bytes": head["algorithmic_bytes"], "touched_experts": head["touched_experts"],
        "hbm_frac": head["hbm_frac"], "tflops_lowp": head["TFLOPs_lowp"], "tflops_bf16": head["TFLOPs_bf16"],
        "stream_read_gbs": sread, "frac_of_stream_read": head["GBps"] / sread,
        "timing": (("eager launches" if args.eager else "HIP graph replay") + " of route + forward" +
                   (" (single-launch forward)" if args.fused else "") +
                   "; value: K replays between two events; median / p10 / p90: K replays before those with an"
                   " event between consecutive ones (us_per_layer_evented their mean)"),
        "groups_us": head["groups_us"],
        "roofline": head.get("roofline"), "cpu_baseline": cpu, "input_gen_s": head["input_gen_s"],
        "legs": legs,
    }
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
