#!/usr/bin/env python3
"""Throughput of the routed MoE layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the whole hot path over one batch of synthetic tokens:
moe_route (router GEMV, top-6, gates) then moe_forward (histogram, prefix sum,
scatter, [token quantisation], grouped up GEMM + ReLU^2, [intermediate
quantisation], grouped down GEMM, combine); the stacked workload runs 23 such
layers with pre-norm and residual.  Inputs are resident in HBM before timing.
W untimed warm-up steps, then exactly K steps between two device
synchronisations, with no events.  Per-stage durations come from a second
pass of K steps with HIP events recorded at every stage boundary on the
stream the kernels run on, plus events stamped with the two GEMM kernels' own
start and end (hipExtLaunchKernel); before each of those steps a 512 MB buffer is
read outside the events, so no step finds the previous step's weights in the
256 MB Infinity Cache.  A third pass records one event before and one after
each step (the same read before each): `step_ms_events` gives the p10 / p50 /
p90 of those step times.

`--cache-slots N` instead times steps through moe_forward_cached, with the
expert bank in pinned host memory and N device slots (uploads included).
`--shared F_S` times the MoE block (a shared expert added to the routed
output), `--graph` also times captured replays, `--copy-calibration` and
`--gemm-ceiling` only run the reference copy and the platform BLAS.

Prints one JSON line.  `roofline` describes the dominant kernel (algorithmic
bytes or flops per launch / the mean of its kernel's own start-to-end
durations in the second pass): decode batches against HBM; 4096-token
batches against both the MFMA instruction the kernel runs and HBM, `bound`
naming the one that takes longer at its peak and the other nested inside;
`traffic` is the counted HBM bytes per launch while the GEMM sources match
the recorded counter passes.  `cpu_baseline` is the CPU
oracle timed on this host on a bounded sample of the same workload; `parity`
compares the timed run's output on those sampled tokens with the oracle's
(max |delta| / rms, near ties counted, id sets compared).  A single-layer
decode workload also carries a `prefill` record: the same measurement on the
4096-token prefill batch of the same format (the MFMA half of the metric),
unless --no-prefill.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s; HBM GB/s at T=64, MFMA TFLOP/s at T=4096 (1 GPU)"
HBM_PEAK_GBS = 8000.0
# nvfp4 runs on the fp16 MFMA after an exact expansion of its codes: same peak as bf16
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "nvfp4": 2500.0}
# the card's dense 4-bit MFMA peak, reported beside the fp16 one for nvfp4
FP4_PEAK_TFLOPS = 10100.0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=30)
    p.add_argument("--workload", default="decode_t64_bf16")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-prefill", action="store_true",
                   help="skip the 4096-token prefill record of a decode workload")
    p.add_argument("--shared", type=int, default=0, metavar="F_S",
                   help="time the MoE block: each layer adds a shared expert of this width "
                        "(moe_shared_forward accumulating into the routed y; 3712 is the "
                        "assumed width)")
    p.add_argument("--graph", action="store_true",
                   help="also capture one step into a HIP graph and time K replays "
                        "(reported beside the eager headline)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain 1 GiB device copy (reference for HBM byte counters)")
    p.add_argument("--gemm-ceiling", action="store_true",
                   help="only time the platform BLAS (torch.matmul / torch.bmm in bf16) on the "
                        "prefill GEMM shapes: one dense 24576 x 2688 x 1856 product each way, "
                        "and 128 equal 192-row expert products (no routing skew)")
    p.add_argument("--cache-slots", type=int, default=0,
                   help="single-layer workloads: keep the expert bank in pinned host memory and "
                        "run each step through moe_forward_cached with this many device slots, "
                        "cycling over 8 token batches (uploads over PCIe are in the timing)")
    return p.parse_args()


class Hip:
    """The few HIP runtime calls the timing needs (events)."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        e = ctypes.c_void_p()
        assert self.lib.hipEventCreate(ctypes.byref(e)) == 0
        return e.value

    def record(self, ev, stream):
        assert self.lib.hipEventRecord(ctypes.c_void_p(ev), ctypes.c_void_p(stream)) == 0

    def elapsed(self, a, b) -> float:
        ms = ctypes.c_float()
        assert self.lib.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b)) == 0
        return ms.value

    def destroy(self, ev):
        self.lib.hipEventDestroy(ctypes.c_void_p(ev))


def weight_bytes_per_expert(fmt, F, H):
    n = F * H
    if fmt == "bf16":
        return 2 * n
    if fmt == "fp8":
        return n + 4
    return n // 2 + n // 16 + 4


def cached_bench(args, wl):
    """Steps through moe_forward_cached: the expert bank lives in pinned host
    memory and `cache_slots` device slots hold the experts the batches select.
    The step cycles over 8 token batches of the workload's size, so the
    selected experts change from step to step; its time includes the upload of
    the missing experts over PCIe and the wait for the routing counts."""
    import torch

    import sparse_moe_routed_amd as moe
    from sparse_moe_routed_amd import synth

    T, fmt = wl["T"], wl["fmt"]
    ld = moe.LayerDims()
    dev = torch.device("cuda:0")
    w_r, b = synth.make_router(0)
    up, down = synth.make_experts(0)
    bank = moe.quantize_experts(up.to(dev), down.to(dev), fmt, ld)
    del up, down
    router = moe.pack_router(w_r.to(dev), b.to(dev), ld)
    cache = moe.ExpertCache(bank, args.cache_slots, ld)
    bank.up = bank.down = bank.up_bs = bank.down_bs = None  # the device keeps the slots and scales
    torch.cuda.empty_cache()
    xs = [synth.make_tokens_device(T, seed=9000 + i) for i in range(8)]
    ids = torch.empty((T, ld.top_k), dtype=torch.int32, device=dev)
    gates = torch.empty((T, ld.top_k), dtype=torch.float32, device=dev)
    y = torch.empty((T, ld.hidden), dtype=torch.float32, device=dev)
    ws = moe.workspace(ld, fmt, T, dev)
    rws = moe.route_workspace(ld, T, dev)
    totals = {"touched": 0, "hits": 0, "misses": 0, "bytes_uploaded": 0}

    def step(i, count):
        x = xs[i % len(xs)]
        moe.route(x, router, ld, ids=ids, gates=gates, ws=rws)
        _, st = moe.forward_cached(x, ids, gates, cache, ld, ws=ws, y=y)
        if count:
            for k in totals:
                totals[k] += st[k]

    for i in range(args.warmup):
        step(i, False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    out = {
        "metric": "MoE-layer tokens/s with the expert bank in host memory (1 GPU)",
        "value": round(T * args.steps / wall, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": fmt,
        "data": "synthetic (seeded; 8 token batches in turn)",
        "config": {"workload": args.workload, "T": T, "format": fmt,
                   "cache_slots": args.cache_slots, "batches": len(xs)},
        "cache": {"touched_per_step": round(totals["touched"] / args.steps, 2),
                  "hit_rate": round(totals["hits"] / max(1, totals["touched"]), 4),
                  "misses_per_step": round(totals["misses"] / args.steps, 2),
                  "uploaded_mb_per_step": round(totals["bytes_uploaded"] / args.steps / 1e6, 2),
                  "upload_gbs": round(totals["bytes_uploaded"] / wall / 1e9, 2)},
        "roofline": None,
    }
    print(json.dumps(out), flush=True)


def build_layers(fmt, n_layers, dev, ld, verbose=True):
    """Router and expert bank of each layer on the device (seeded synthetic)."""
    import torch

    import sparse_moe_routed_amd as moe
    from sparse_moe_routed_amd import synth

    t_setup = time.time()
    layers = []
    for l in range(n_layers):
        w_r, b = synth.make_router(l)
        up, down = synth.make_experts(l)
        up_d, down_d = up.to(dev), down.to(dev)
        del up, down
        bank = moe.quantize_experts(up_d, down_d, fmt, ld)
        if fmt != "bf16":
            del up_d, down_d
        layers.append(dict(router=moe.pack_router(w_r.to(dev), b.to(dev), ld), bank=bank))
        if verbose:
            print(f"# {fmt} layer {l} ready ({time.time() - t_setup:.1f}s)", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    return layers


def build_shared(fmt, n_layers, f_s, dev):
    """Shared expert of each layer on the device (seeded synthetic), or None."""
    import sparse_moe_routed_amd as moe
    from sparse_moe_routed_amd import synth

    if not f_s:
        return None
    sd = moe.shared_dims(synth.HIDDEN, f_s)
    out = []
    for l in range(n_layers):
        up, down = synth.make_shared_expert(l, ffn=f_s)
        out.append(moe.quantize_experts(up[None].to(dev), down[None].to(dev), fmt, sd))
    return sd, out


def measure(args, name, layers, hip, shared=None):
    """Time one workload (see the module docstring).  Returns (record, state):
    the record of the bench line without its headline keys, and the device
    tensors of the last step for the parity check."""
    import numpy as np
    import torch

    import sparse_moe_routed_amd as moe
    from sparse_moe_routed_amd import synth

    wl = synth.WORKLOADS[name]
    T, fmt, n_layers = wl["T"], wl["fmt"], wl["layers"]
    dims = synth.Dims()
    ld = moe.LayerDims()
    H, F, E, k = dims.hidden, dims.ffn, dims.n_experts, dims.top_k
    dev = torch.device("cuda:0")
    x0 = synth.make_tokens(T, outliers=wl["outliers"]).to(dev)
    ws = moe.workspace(ld, fmt, T, dev)
    rws = moe.route_workspace(ld, T, dev)
    y = torch.empty((T, H), dtype=torch.float32, device=dev)
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    gates = torch.empty((T, k), dtype=torch.float32, device=dev)
    xin = torch.empty_like(x0)
    xs = x0.clone()
    sws = None
    if shared:
        sws = moe.shared_workspace(shared[0], fmt, T, dev)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream().cuda_stream
    n_ev = moe.N_TIMED_EVENTS

    def run_layer(L, x_in, ev=None, li=0):
        """route + forward of one layer (+ the shared expert added into y);
        ev = (route events, stage events) or None"""
        if ev:
            hip.record(ev[0][0], stream)
        moe.route(x_in, L["router"], ld, ids=ids, gates=gates, ws=rws)
        if ev:
            hip.record(ev[0][1], stream)
            moe.forward_timed(x_in, ids, gates, L["bank"], ev[1], ld, ws=ws, y=y)
        else:
            moe.forward(x_in, ids, gates, L["bank"], ld, ws=ws, y=y)
        if shared:
            moe.shared_forward(x_in, shared[1][li], shared[0], y=y, accumulate=True, ws=sws)

    def step(evs=None):
        if n_layers == 1:
            run_layer(layers[0], x0, evs[0] if evs else None)
        else:
            # pre-norm, layer, then the residual fused with the next layer's
            # pre-norm; the last layer ends with the plain residual
            xs.copy_(x0)
            moe.prenorm(xs, xin)
            for li, L in enumerate(layers):
                run_layer(L, xin, evs[li] if evs else None, li)
                if li + 1 < n_layers:
                    moe.residual_prenorm(xs, y, xin)
                else:
                    moe.residual_add(xs, y)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # pass 1 (headline): exactly K steps between two synchronisations, no events
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    tokens_per_s = T * args.steps / wall
    # the last step's routing and output (single layer: the timed run's own
    # result for x0; every step computes the same)
    state = dict(ids=ids.clone(), gates=gates.clone(), y=y.clone(), x0=x0)

    # pass 2 (attribution): K more steps with HIP events at every stage
    # boundary, recorded on the stream the kernels run on (events add a few
    # microseconds per step, so pass 1 alone gives the headline), and on the
    # two GEMM launches themselves: hipExtLaunchKernel stamps those events
    # with the kernel's own start and end, the interval a kernel trace reports
    # (stacked workloads: events around every layer, averaged over the layers)
    stage_ms = {}
    # Before each step a 512 MB buffer is read (outside the events), more than
    # the 256 MB Infinity Cache, so no step finds the previous step's weights
    # in it.  Reading leaves clean lines; writing would leave dirty ones whose
    # write-back the next kernel would pay for.
    evs = [[([hip.event(), hip.event()], [hip.event() for _ in range(n_ev)])
            for _ in range(n_layers)] for _ in range(args.steps)]
    flush = torch.ones(128 << 20, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    for i in range(args.steps):
        flush.amax()
        step(evs[i])
    torch.cuda.synchronize()
    flat = [e for per_step in evs for e in per_step]
    stage_ms["route"] = float(np.mean([hip.elapsed(er[0], er[1]) for er, _ in flat]))
    for si, sname in enumerate(moe.STAGES):
        stage_ms[sname] = float(np.mean([hip.elapsed(es[si], es[si + 1]) for _, es in flat]))
    j0 = moe.N_STAGES + 1
    gemm_kernel_ms = {
        "up": float(np.mean([hip.elapsed(es[j0], es[j0 + 1]) for _, es in flat])),
        "down": float(np.mean([hip.elapsed(es[j0 + 2], es[j0 + 3]) for _, es in flat]))}
    for er, es in flat:
        for h in er + es:
            hip.destroy(h)

    # pass 3: the distribution of single-step times, with one event before and
    # one after each step (and the cache-clearing read before the first)
    ev2 = [(hip.event(), hip.event()) for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        flush.amax()
        hip.record(ev2[i][0], stream)
        step()
        hip.record(ev2[i][1], stream)
    torch.cuda.synchronize()
    del flush
    step_ev = sorted(hip.elapsed(a, b) for a, b in ev2)
    for a, b in ev2:
        hip.destroy(a)
        hip.destroy(b)
    q = lambda p_: step_ev[min(len(step_ev) - 1, int(round(p_ * (len(step_ev) - 1))))]
    step_pct = {"p10": round(q(0.1), 4), "p50": round(q(0.5), 4), "p90": round(q(0.9), 4)}

    # pass 4 (optional): the same step captured once into a HIP graph (the
    # library's calls hold no host sync, allocation or memset), K replays
    # between two synchronisations
    graph_rec = None
    if args.graph:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            graph.replay()
        torch.cuda.synchronize()
        gwall = time.perf_counter() - t0
        graph_rec = {"ms_per_step": round(gwall * 1e3 / args.steps, 4),
                     "value": round(T * args.steps / gwall, 1), "steps": args.steps}
        del graph

    # ---------------------------------------------------------------- roofline
    ids_h = ids.cpu().numpy()
    touched = int(np.unique(ids_h).size)
    R = T * k
    wbe = weight_bytes_per_expert(fmt, F, H)
    layer_bytes = touched * 2 * wbe + E * H * 4 + E * 4 + T * H * 2 + T * H * 4
    flops_up = 2.0 * R * F * H
    dom = "up" if gemm_kernel_ms["up"] >= gemm_kernel_ms["down"] else "down"
    dur_s = gemm_kernel_ms[dom] * 1e-3
    # algorithmic bytes of the dominant launch: the touched experts' weights
    # once, its activation input once, its output once (FP8 up projections
    # read the tokens as bf16 values of their codes, FP8 down projections read
    # E4M3 codes, NVFP4 reads fp16 values)
    a_in = {"bf16": 2, "fp8": 2 if dom == "up" else 1, "nvfp4": 2}[fmt]
    if dom == "up":
        alg = touched * wbe + T * H * a_in + R * F * 2
    else:
        alg = touched * wbe + R * F * a_in + R * H * 4
    hbm_gbs = alg / dur_s / 1e9
    if T <= 256:
        # weight-streaming launch
        roof = {"bound": "hbm", "achieved": round(hbm_gbs, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(hbm_gbs / HBM_PEAK_GBS, 4),
                "traffic": None, "kernel": f"grouped_gemm_{dom}", "alg_bytes": int(alg)}
    else:
        # both limits of the launch: the MFMA instruction it runs (the FP8 up
        # projection runs the bf16 one on exactly expanded codes, NVFP4 the
        # fp16 one) and HBM for its algorithmic bytes; the bound is the one
        # that takes longer at its peak
        inst = {"bf16": "bf16", "fp8": "bf16" if dom == "up" else "fp8", "nvfp4": "f16"}[fmt]
        peak = {"bf16": 2500.0, "fp8": 5000.0, "f16": 2500.0}[inst]
        tflops = flops_up / dur_s / 1e12
        mfma = {"achieved": round(tflops, 1), "peak": peak, "unit": "TFLOP/s",
                "frac": round(tflops / peak, 4), "alg_flops": flops_up,
                "instruction": f"{inst} MFMA"}
        if fmt == "fp8":
            mfma["frac_fp8_peak"] = round(tflops / MFMA_PEAK_TFLOPS["fp8"], 4)
        if fmt == "nvfp4":
            mfma["peak_fp4"] = FP4_PEAK_TFLOPS
            mfma["frac_fp4"] = round(tflops / FP4_PEAK_TFLOPS, 4)
        hbm = {"achieved": round(hbm_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
               "frac": round(hbm_gbs / HBM_PEAK_GBS, 4), "alg_bytes": int(alg)}
        t_mfma = flops_up / (peak * 1e12)
        t_hbm = alg / (HBM_PEAK_GBS * 1e9)
        if t_hbm >= t_mfma:
            roof = {"bound": "hbm", **{k2: hbm[k2] for k2 in ("achieved", "peak", "unit", "frac")},
                    "traffic": None, "kernel": f"grouped_gemm_{dom}", "alg_bytes": int(alg),
                    "mfma": mfma}
        else:
            roof = {"bound": "mfma", **{k2: mfma[k2] for k2 in ("achieved", "peak", "unit", "frac")},
                    "traffic": None, "kernel": f"grouped_gemm_{dom}", "alg_flops": flops_up,
                    "instruction": mfma["instruction"], "hbm": hbm}
            for k2 in ("frac_fp8_peak", "peak_fp4", "frac_fp4"):
                if k2 in mfma:
                    roof[k2] = mfma[k2]
    # HBM bytes per launch from the FETCH_SIZE / WRITE_SIZE counter passes,
    # used only while the GEMM sources are the ones the counters were taken on
    tf = os.path.join(ROOT, "profiles", f"traffic_{name}.json")
    if os.path.exists(tf):
        rec = json.load(open(tf))
        if rec.get("source_sha256") == gemm_source_sha256():
            roof["traffic"] = rec.get("bytes_per_launch", {}).get(roof["kernel"])

    layer_ms = ms_per_step / n_layers
    out = {
        "value": round(tokens_per_s, 1),
        "ms_per_step": round(ms_per_step, 4),
        "dtype": fmt,
        "config": {"workload": name, "T": T, "hidden": H, "ffn": F, "experts": E,
                   "top_k": k, "format": fmt, "layers": n_layers, "outlier_rows": wl["outliers"],
                   "shared_ffn": shared[0].ffn if shared else 0},
        "layer_hbm_gbs": round(layer_bytes / (layer_ms * 1e-3) / 1e9, 1),
        "layer_tflops": round(2 * flops_up / (layer_ms * 1e-3) / 1e12, 2),
        "experts_touched": touched,
        "stage_ms": {k2: round(v, 4) for k2, v in stage_ms.items()},
        "gemm_kernel_ms": {k2: round(v, 4) for k2, v in gemm_kernel_ms.items()},
        "step_ms_events": step_pct,
        "roofline": roof,
    }
    if graph_rec:
        out["graph"] = graph_rec
    return out, state


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus > 1 or world > 1:
        print(f"bench.py: measures one GPU only; --gpus {max(args.gpus, world)} "
              "is not supported (the layer would shard by expert parallelism; only the "
              "single-GPU kernels are built)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import sparse_moe_routed_amd as moe
    from sparse_moe_routed_amd import synth

    if args.copy_calibration:
        n = 1 << 30
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_each_way": n, "launches": args.steps}), flush=True)
        return

    if args.gemm_ceiling:
        print(json.dumps(gemm_ceiling(args)), flush=True)
        return

    if args.workload not in synth.WORKLOADS:
        sys.exit(f"unknown workload {args.workload}; choose from {sorted(synth.WORKLOADS)}")
    wl = synth.WORKLOADS[args.workload]
    fmt, n_layers = wl["fmt"], wl["layers"]
    if args.cache_slots:
        if n_layers != 1:
            sys.exit("--cache-slots applies to single-layer workloads")
        return cached_bench(args, wl)
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    hip = Hip()
    ld = moe.LayerDims()

    layers = build_layers(fmt, n_layers, dev, ld)
    shared = build_shared(fmt, n_layers, args.shared, dev)
    rec, state = measure(args, args.workload, layers, hip, shared)
    out = {
        "metric": METRIC,
        "value": rec.pop("value"),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": rec.pop("ms_per_step"),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": rec.pop("dtype"),
        "data": "synthetic (seeded; shapes and distributions of the Nemotron 3.5 Transcribe routed MoE layer)",
        "config": rec.pop("config"),
    }
    out.update(rec)
    if not args.no_cpu_baseline:
        out["cpu_baseline"], out["parity"] = cpu_baseline(args.workload, state)
        if n_layers > 1 or shared:
            # the timed step ends with the last layer's output; per-layer
            # parity of the stack is a GPU test (teacher-forced)
            out["parity"] = None

    # the MFMA half of the metric: the 4096-token prefill batch of the same
    # format, with the same layer weights
    pre = f"prefill_t4096_{fmt}"
    if (not args.no_prefill and not shared and n_layers == 1 and wl["T"] < 4096 and pre in synth.WORKLOADS
            and synth.WORKLOADS[pre]["layers"] == 1):
        del state
        torch.cuda.empty_cache()
        prec, pstate = measure(args, pre, layers, hip)
        if not args.no_cpu_baseline:
            prec["cpu_baseline"], prec["parity"] = cpu_baseline(pre, pstate)
        prec.pop("dtype")
        out["prefill"] = prec
    print(json.dumps(out), flush=True)


def gemm_ceiling(args):
    """TFLOP/s of the platform BLAS on the 4096-token prefill GEMMs (24576
    routed rows, 2688 x 1856 experts): a reference ceiling for the grouped
    kernels, which also carry the routing skew and ragged expert tiles."""
    import torch

    from sparse_moe_routed_amd import synth

    H, F, E, R = synth.HIDDEN, synth.FFN, synth.N_EXPERTS, 4096 * synth.TOP_K
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(0)

    def rand(*shape):
        return torch.randn(*shape, device=dev, dtype=torch.bfloat16, generator=g)

    def rate(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(args.steps):
            fn()
        e.record()
        torch.cuda.synchronize()
        sec = s.elapsed_time(e) * 1e-3 / args.steps
        return round(2.0 * R * H * F / sec / 1e12, 1), round(sec * 1e6, 1)

    a_up, w_up_t = rand(R, H), rand(H, F)      # contiguous operands only
    a_dn, w_dn_t = rand(R, F), rand(F, H)
    a_b, w_b = rand(E, R // E, H), rand(E, H, F)
    out = {"metric": "platform BLAS bf16 TFLOP/s on the prefill GEMM shapes", "peak": 2500.0,
           "steps": args.steps}
    for name, fn in (("dense_up", lambda: torch.matmul(a_up, w_up_t)),
                     ("dense_down", lambda: torch.matmul(a_dn, w_dn_t)),
                     ("batched_up_128x192", lambda: torch.bmm(a_b, w_b))):
        tf, us = rate(fn)
        out[name] = {"tflops": tf, "us": us, "frac": round(tf / 2500.0, 4)}
    return out


def gemm_source_sha256():
    """Hash of the sources the grouped GEMM kernels are built from."""
    h = hashlib.sha256()
    for f in ("gemm.hip", "moe_common.h", "moe_internal.h"):
        h.update(open(os.path.join(ROOT, "sparse_moe_routed_amd", "csrc", f), "rb").read())
    return h.hexdigest()


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(name, state):
    """The oracle as it stands, on a bounded token sample of the same workload,
    and the parity of the timed run's output on that sample: the oracle routes
    the sampled tokens itself (float64); tokens whose 6th/7th logit gap is
    under 1e-5 are near ties (counted; left out if their id sets differ), the
    other id sets must equal the GPU's, and the outputs are compared on the
    tokens with equal id sets (the oracle's own routing and gates)."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import moe as om
    from sparse_moe_routed_amd import synth

    wl = synth.WORKLOADS[name]
    T, fmt = wl["T"], wl["fmt"]
    x = synth.make_tokens(T, outliers=wl["outliers"]).float().numpy()
    w_r, b = synth.make_router(0)
    # bf16: the oracle needs no dequantisation, so a larger sample (the whole
    # decode batch; 192 tokens of a prefill batch, every 8th outlier row among
    # them).  fp8/nvfp4: the per-tensor scales of x and of the intermediate
    # cover the whole batch, so only the whole batch reproduces them; decode
    # batches run whole (the oracle re-quantises every touched expert on each
    # call: about 10 s at 4 tokens, 40-50 s at 64 on 16 cores), prefill
    # batches are timed on 4 tokens and their parity is not compared here
    whole_batch_only = fmt != "bf16"
    if fmt == "bf16":
        n = min(T, 192)
    elif T <= 64:
        n = T
    else:
        n = 4
    rng = np.random.default_rng(77)
    sample = np.arange(T) if n == T else np.sort(rng.choice(T, n, replace=False))
    xs = x[sample]
    # only the experts the sample can touch are generated (each from its own stream)
    ids_o, _, _, _ = om.route(xs, w_r.numpy(), b.numpy(), synth.TOP_K)
    touched = np.unique(ids_o)
    up, down = synth.make_experts(0, experts=touched)
    pos = {int(e): i for i, e in enumerate(touched)}
    bank = om.ExpertBank({e: up[i] for e, i in pos.items()}, {e: down[i] for e, i in pos.items()},
                         fmt)
    # repeat the sample until about ten seconds of CPU work have been timed
    spent, done_tokens, passes = 0.0, 0, 0
    y_o = ids_o = g_o = gap = None
    while spent < 10.0 and passes < 100:
        t0 = time.perf_counter()
        ids_o, g_o, gap, _ = om.route(xs, w_r.numpy(), b.numpy(), synth.TOP_K)
        y_o = om.forward(xs, ids_o, g_o, bank)
        spent += time.perf_counter() - t0
        done_tokens += n
        passes += 1
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    base = {"value": round(done_tokens / spent, 3), "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"{passes} pass(es) over {n} tokens of the {T}-token batch (float64 NumPy, "
                      f"one layer, {fmt} weights dequantised by the oracle), {spent:.1f}s"}
    if whole_batch_only and n < T:
        return base, {"tokens": 0, "skipped": "fp8/nvfp4 scales are per tensor over the whole "
                      f"{T}-token batch; a {n}-token oracle run quantises with other scales "
                      "(the whole-batch comparison runs in the GPU tests)"}
    # parity of the timed run's output on the sample
    ids_g = state["ids"].cpu().numpy()[sample]
    y_g = state["y"].double().cpu().numpy()[sample]
    near = gap < om.NEAR_TIE
    same = np.array([sorted(p_) == sorted(q_) for p_, q_ in zip(ids_g, ids_o)])
    rms = float(np.sqrt(np.mean(y_o[same] ** 2))) if same.any() else float("nan")
    err = float(np.abs(y_g[same] - y_o[same]).max() / rms) if same.any() else float("nan")
    tol = {"bf16": 2e-2, "fp8": 5e-2, "nvfp4": 1e-1}[fmt]
    parity = {"tokens": int(n), "max_abs_delta_over_rms": err, "tolerance": tol,
              "within_tolerance": bool(err <= tol), "near_ties": int(near.sum()),
              "id_set_mismatches": int((~same & ~near).sum()),
              "near_tie_mismatches": int((~same & near).sum()),
              "compared": "fp32 y of the timed run vs the float64 oracle (own routing and gates)"}
    return base, parity


if __name__ == "__main__":
    main()
