#!/usr/bin/env python3
"""Throughput of the Stable LatentMoE FFN layer forward on one MI355X.

One step = one moe_layer_forward call (all steps of the layer) over one batch of
synthetic tokens already resident in HBM.  Prints one JSON line.

Default workload: the K3-shaped layer at decode batch 1 (d 7168, latent 3584, 896 MXFP4
experts top-16, 3072-wide experts, merged 6144-wide shared expert).  Three copies of the
dense weights (3 x 380 MB) and 64 distinct token batches rotate so that the 256 MB
last-level cache cannot hold what a step reads.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "LatentMoE layer tokens/s (decode B=1/64, prefill 8k) + % HBM / MFMA peak"
HBM_PEAK_GBS = 8000.0     # MI355X HBM3E, published


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def expert_weight_bytes(cfg):
    """(gate/up, down) bytes of one routed expert in its storage format."""
    l, m = cfg.l or cfg.d, cfg.m
    if cfg.expert_fmt == "mxfp4":
        return 2 * m * (l // 2 + l // 32), l * (m // 2 + m // 32)
    if cfg.expert_fmt == "fp8b128":
        cd = lambda a, b: (a + b - 1) // b  # noqa: E731
        return 2 * m * l + 4 * cd(2 * m, 128) * cd(l, 128), l * m + 4 * cd(l, 128) * cd(m, 128)
    return 2 * m * l * 2, l * m * 2


def algorithmic_bytes(cfg, T, D):
    """Compulsory HBM bytes of each step for T tokens touching D distinct experts."""
    d, E, k, m, ms = cfg.d, cfg.E, cfg.k, cfg.m, cfg.ms
    l = cfg.l or cfg.d           # the experts' width (the token itself without a latent)
    gu_w, dn_w = expert_weight_bytes(cfg)
    tk = T * k
    small = T <= 3   # the route and the dispatch run inside the IN launch
    mx8 = getattr(cfg, "precision", "fp32") == "mx8"
    ab = 4 if not mx8 else 1 + 1 / 32   # bytes per activation element of the expert inputs
    if mx8:
        # one IN product (router logits, x^c fp32, h_s bf16), then x^c to MXFP8
        router = T * d * 2 + (E + cfg.l + 2 * ms) * d * 2 + T * (E * 4 + cfg.l * 4 + ms * 2)
        in_ = T * cfg.l * 4 + T * cfg.l * ab
    else:
        # W_down_latent rides in the ROUTER launch for a few tokens, in the IN launch otherwise
        ldn = cfg.l if small else 0
        router = T * d * 2 + (E + ldn) * d * 2 + T * (E + ldn) * 4
        in_ = (T * d * 2 + (cfg.l - ldn + 2 * ms) * d * 2 + T * (cfg.l - ldn + ms) * 4
               + ((T * E * 4 + E * 4 + tk * 16 + E * 8) if small else 0))
    return {
        "router": router,
        "in": in_,
        "route": 0 if small else T * E * 4 + E * 4 + tk * 8,
        "dispatch": 0 if small else tk * 4 * 4 + E * 8,
        "expert_gu": D * gu_w + T * l * ab + tk * m * ab,
        "expert_down": D * dn_w + tk * m * ab + tk * l * 4,
        # (mx8: one pass to u_hat in bf16, u itself is not stored)
        "combine": tk * l * 4 + tk * 8 + T * l * (2 if mx8 else 4),
        "out": d * (cfg.l + ms) * 2 + cfg.l * 2 + T * (l + ms) * (2 if mx8 else 4) + T * d * 4,
    }

def algorithmic_flops(cfg, T):
    """Multiply-add flops (2 per product) of each step for T tokens."""
    d, l, E, k, m, ms = cfg.d, cfg.l, cfg.E, cfg.k, cfg.m, cfg.ms
    tk = T * k
    lx = l or d                  # the experts' width (the token itself without a latent)
    return {"router": 2 * T * d * (E + l + 2 * ms), "in": 0, "route": 0, "dispatch": 0,
            "expert_gu": 2 * tk * lx * 2 * m, "expert_down": 2 * tk * m * lx, "combine": 2 * tk * lx,
            "out": 2 * T * (l + ms) * d}


# matrix-core peaks of MI355X (dense, published), TFLOP/s
MFMA_PEAK = {"bf16": 2500.0, "fp8": 5000.0, "fp4": 10100.0}


def weight_bytes(cfg, D):
    """Weights (and the fp32 bias) one call reads: the layer's algorithmic byte count."""
    d, l, E, ms = cfg.d, cfg.l, cfg.E, cfg.ms
    return (E * d + 2 * l * d + l + 3 * ms * d) * 2 + E * 4 + D * sum(expert_weight_bytes(cfg))


# The kernels of each step's launches: (kernel name, a word its template arguments must
# hold, or None).  Kernels of no step (the one-time packing, the QB statistics) map to None.
STEP_KERNELS = {"router": [("k_router", None), ("k_router_tt", None), ("k_token_rows", None)],
                "in": [("k_in", None), ("k_in_tt", None)],
                "route": [("k_route", None)],
                "dispatch": [("k_disp_count", None), ("k_disp_scan", None), ("k_disp_scatter", None)],
                "expert_gu": [("k_exp", "true"), ("k_exp_tt", "true")],
                "expert_down": [("k_exp", "false"), ("k_exp_tt", "false")],
                "combine": [("k_combine", None), ("k_norm", None)],
                "out": [("k_out", None), ("k_out_tt", None)]}
STEP_KERNELS_MX8 = {"router": [("k_pf_dense", "true")], "in": [("k_pf_quant", None)],
                    "route": [("k_route", None)],
                    "dispatch": [("k_disp_count", None), ("k_disp_scan", None), ("k_disp_scatter", None)],
                    "expert_gu": [("k_pf_exp", "true")], "expert_down": [("k_pf_exp", "false")],
                    "combine": [("k_pf_combine_norm", None), ("k_combine", None), ("k_pf_norm", None)],
                    "out": [("k_pf_dense", "false")]}


def step_of_kernel(name, kernels):
    """The step whose launches include the kernel `name` (a rocprofv3 symbol or its short
    form `k_name<args>`), or None."""
    import re
    m = re.search(r"(k_\w+)(<[^>]*>)?", name)
    if not m:
        return None
    base, targs = m.group(1), m.group(2) or ""
    for step, alts in kernels.items():
        if any(base == b and (w is None or w in targs) for b, w in alts):
            return step
    return None


def kernel_sources_sha():
    import glob
    import hashlib
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "sparse_moe_layer_amd", "csrc", "*"))):
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, step, kernels=None):
    """HBM bytes per launch of `step` from the committed rocprofv3 counter summary, or None
    when there is none or the kernel sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"{workload}_hbm_traffic.md")
    if not os.path.exists(path):
        return None
    for line in open(path):
        if line.startswith("traffic_json: "):
            rec = json.loads(line[len("traffic_json: "):])
            if rec.get("src_sha") != kernel_sources_sha():
                return None
            # a step may take more than one launch (the token-tiled expert steps launch the
            # kernel for short units and the one for long units): their bytes add up
            hits = [v for name, v in rec["bytes_per_launch"].items()
                    if step_of_kernel(name, kernels or STEP_KERNELS) == step]
            return sum(hits) if hits else None
    return None


class HipEvents:
    """hipEvent_t handles through the HIP runtime that torch has loaded."""

    def __init__(self):
        self.h = ctypes.CDLL("libamdhip64.so.7")
        self.h.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                               ctypes.c_void_p]
        self.h.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        out = []
        for _ in range(n):
            e = ctypes.c_void_p()
            if self.h.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            out.append(e.value)
        return out

    def ms(self, a, b):
        v = ctypes.c_float()
        if self.h.hipEventElapsedTime(ctypes.byref(v), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return v.value

    def destroy(self, evs):
        for e in evs:
            self.h.hipEventDestroy(e)


def measured_hbm_rates(torch, dev, gib=2, reps=5):
    """What torch's own generic kernels reach on this GPU's HBM: a sum over `gib` GiB (read)
    and a copy of `gib` GiB (read + write), best of `reps`, in GB/s.  Context beside the
    nominal 8 TB/s peak that the roofline fractions use; not an achievable-peak probe."""
    n = gib << 30
    src = torch.empty(n // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    out = {}
    for name, fn, nbytes in (("torch_sum_read_GBps", lambda: src.sum(), n),
                             ("torch_copy_GBps", lambda: dst.copy_(src), 2 * n)):
        fn()
        best = None
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1)
            best = ms if best is None else min(best, ms)
        out[name] = nbytes / (best * 1e-3) / 1e9
    del src, dst
    return out


def percentiles_us(durations_ms):
    import numpy as np
    d = np.asarray(durations_ms, dtype=np.float64) * 1e3
    return {"median_us": float(np.median(d)), "p10_us": float(np.percentile(d, 10)),
            "p90_us": float(np.percentile(d, 90))}


def graph_replay(layers, xs, bufs, rotate, batches, K, warmup):
    """The forward captured as HIP graphs, one per (dense copy, token batch) pair of the
    rotation (at most 16), replayed in turn on torch's current stream.

    Returns the mean over K back-to-back replays, the median / p10 / p90 of single replays
    (one event between consecutive replays, so each figure carries one event record), the
    same percentiles for eager forwards, and whether a replay gives the eager bits."""
    import torch
    G = max(rotate, min(batches, 16))
    pairs = [(j % rotate, j % batches) for j in range(G)]
    graphs = []
    for li, xi in pairs:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            layers[li].forward(xs[xi], *bufs)
        graphs.append(g)
    torch.cuda.synchronize()
    for i in range(max(G, warmup)):
        graphs[i % G].replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(K):
        graphs[i % G].replay()
    e1.record()
    torch.cuda.synchronize()
    mean_ms = e0.elapsed_time(e1) / K

    def per_step(run):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
        evs[0].record()
        for i in range(K):
            run(i)
            evs[i + 1].record()
        torch.cuda.synchronize()
        return [evs[i].elapsed_time(evs[i + 1]) for i in range(K)]
    g_ms = per_step(lambda i: graphs[i % G].replay())
    e_ms = per_step(lambda i: layers[pairs[i % G][0]].forward(xs[pairs[i % G][1]], *bufs))
    # bits: a replay against an eager forward of the same pair, on buffers of its own
    graphs[1 % G].replay()
    got = [t.clone() for t in bufs[:3]]
    li, xi = pairs[1 % G]
    ref = layers[li].forward(xs[xi])
    torch.cuda.synchronize()
    same = all(torch.equal(a, b) for a, b in zip(got, ref))
    del graphs
    return {"graphs": G, "us_per_step": mean_ms * 1e3, "tokens_per_s": None,
            **percentiles_us(g_ms), "eager": percentiles_us(e_ms),
            "bits_equal_eager": same}


def cpu_baseline(cfg, dense, seconds, sample_tokens=None):
    """The float64 CPU oracle, as it is, on a bounded sample of the same workload
    (batches of the workload's size, or of `sample_tokens` tokens for large batches)."""
    import numpy as np
    import oracle
    import synth
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = 1
    OL = oracle.OracleLayer.from_synth(cfg, dense)
    tb = cfg.tokens if sample_tokens is None else min(cfg.tokens, sample_tokens)
    n, t0 = 0, time.perf_counter()
    while True:
        x = synth.tokens(cfg, batch=5000 + n, T=tb)
        oracle.forward(OL, x)
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds or n >= 64:
            break
    tps = n * tb / el
    return {"value": tps, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{n} batch(es) of {tb} token(s) of the workload, {el:.1f} s, float64 numpy "
                      f"oracle in the {getattr(cfg, 'precision', 'fp32')} profile (BLAS threads "
                      f"{cores}), each touched expert regenerated and dequantised per batch"}


def qb_stats(layer, x, cfg, K, dev):
    """Time the Quantile Balancing statistics of one token batch: moe_qb_histogram (router
    launch, cutoffs, counts) and moe_qb_readout, K of each back to back between events."""
    import torch
    T, bins = x.shape[0], 1000
    hist = torch.zeros((cfg.E, bins), dtype=torch.int32, device=dev)
    for _ in range(3):
        layer.qb_readout(layer.qb_histogram(x, n_bins=bins, hist=hist), T)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    ev[0].record()
    for _ in range(K):
        layer.qb_histogram(x, n_bins=bins, hist=hist)
    ev[1].record()
    for _ in range(K):
        layer.qb_readout(hist, T)
    ev[2].record()
    torch.cuda.synchronize()
    h_us = ev[0].elapsed_time(ev[1]) / K * 1e3
    r_us = ev[1].elapsed_time(ev[2]) / K * 1e3
    log(f"[bench] qb statistics: histogram {h_us:.1f} us, readout {r_us:.1f} us per call")
    return {"tokens": T, "bins": bins, "histogram_us": h_us, "readout_us": r_us,
            "tokens_per_s": T / ((h_us + r_us) * 1e-6)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="k3_latent_moe_decode_b1")
    ap.add_argument("--rotate", type=int, default=3, help="dense weight copies rotated")
    ap.add_argument("--batches", type=int, default=64, help="distinct token batches rotated")
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="end with a 1 GiB device copy (scale for HBM byte counters)")
    ap.add_argument("--qb-stats", action="store_true",
                    help="also time the Quantile Balancing statistics step on the workload's "
                         "token batch (1000 bins): adds a qb_stats object")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world})", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import sparse_moe_layer_amd as moe
    import synth

    cfg = synth.PRESETS[args.workload]
    dev = torch.device("cuda:0")
    T = cfg.tokens
    mcfg = moe.config_from(cfg)
    log(f"[bench] workload {cfg.name}: generating and uploading the layer")
    t0 = time.perf_counter()
    dense0 = synth.dense_weights(cfg)
    chunk = 64
    staging = {}

    def slice_fn(a, b):
        if b - a == chunk and "s" in staging:
            return synth.expert_slice(cfg, a, b, out=staging["s"])
        sl = synth.expert_slice(cfg, a, b)
        if b - a == chunk:
            staging["s"] = sl
        return sl
    layer0 = moe.Layer.upload(mcfg, dense0, slice_fn, cfg.E, device=dev, chunk=chunk)
    staging.clear()
    layers = [layer0] + [layer0.with_dense(synth.dense_weights(cfg, copy=c)) for c in range(1, args.rotate)]
    xs = [torch.from_numpy(synth.tokens(cfg, batch=1000 + b).view(np.int16)).to(dev)
          for b in range(args.batches)]
    torch.cuda.synchronize()
    log(f"[bench] layer ready in {time.perf_counter() - t0:.1f} s")

    delta = torch.empty((T, cfg.d), dtype=torch.float32, device=dev)
    idx = torch.empty((T, cfg.k), dtype=torch.int32, device=dev)
    gw = torch.empty((T, cfg.k), dtype=torch.float32, device=dev)
    ws = layer0.workspace(T)

    # distinct experts per batch (for the byte count of the timed steps)
    D = []
    for b in range(args.batches):
        layers[0].forward(xs[b], delta, idx, gw, ws)
        D.append(len(np.unique(idx.cpu().numpy())))
    for i in range(args.warmup):
        layers[i % args.rotate].forward(xs[i % args.batches], delta, idx, gw, ws)
    torch.cuda.synchronize()

    # timed region: K whole forwards back to back
    K = args.steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(K):
        layers[i % args.rotate].forward(xs[i % args.batches], delta, idx, gw, ws)
    e1.record()
    torch.cuda.synchronize()
    ms_total = e0.elapsed_time(e1)
    ms_step = ms_total / K
    log(f"[bench] {K} steps: {ms_step * 1e3:.1f} us/step")
    graph = graph_replay(layers, xs, (delta, idx, gw, ws), args.rotate, args.batches, K,
                         args.warmup)
    graph["tokens_per_s"] = T / (graph["us_per_step"] * 1e-6)
    log(f"[bench] hipGraph replay: {graph['us_per_step']:.1f} us/step over {K} replays; single "
        f"replays median {graph['median_us']:.1f} (p10 {graph['p10_us']:.1f}, p90 "
        f"{graph['p90_us']:.1f}); eager median {graph['eager']['median_us']:.1f}; "
        f"bits equal eager: {graph['bits_equal_eager']}")

    # per-step durations: the same forwards with in-stream events between the steps.  An
    # event record costs a few microseconds of GPU time, so this pass only ranks the steps;
    # the dominant step is then timed with events around it alone.
    hip = HipEvents()
    nst = len(moe.STEPS)
    evs = hip.create(K * (nst + 1))
    for i in range(K):
        layers[i % args.rotate].forward_timed(xs[i % args.batches], evs[i * (nst + 1):(i + 1) * (nst + 1)],
                                              delta, idx, gw, ws)
    torch.cuda.synchronize()
    step_ms = np.zeros(nst)
    for i in range(K):
        base = i * (nst + 1)
        for s_ in range(nst):
            step_ms[s_] += hip.ms(evs[base + s_], evs[base + s_ + 1])
    step_ms /= K
    hip.destroy(evs)
    steps_us = {n: round(float(v) * 1e3, 2) for n, v in zip(moe.STEPS, step_ms)}
    log(f"[bench] per step with events at every boundary (us): {steps_us}")
    dom = max(("router", "in", "expert_gu", "expert_down", "out"),
              key=lambda n: step_ms[moe.STEPS.index(n)])
    mx8 = getattr(cfg, "precision", "fp32") == "mx8"
    # The dominant step alone, K launches back to back between two events.  Each launch
    # works on the buffers of an earlier full forward; R sets of buffers (different tokens,
    # so different experts, and different dense copies) rotate past the last-level cache.
    si = moe.STEPS.index(dom)
    R = 8
    sets = []
    for r in range(R):
        bufs = (torch.empty_like(delta), torch.empty_like(idx), torch.empty_like(gw),
                moe.new_workspace(mcfg, T, dev))
        layers[r % args.rotate].forward(xs[r % args.batches], *bufs[:3], workspace=bufs[3])
        sets.append(bufs)
    for r in range(R):
        layers[r % args.rotate].forward_steps(xs[r % args.batches], si, si + 1, *sets[r])
    torch.cuda.synchronize()
    e2, e3 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e2.record()
    for i in range(K):
        r = i % R
        layers[r % args.rotate].forward_steps(xs[r % args.batches], si, si + 1, *sets[r])
    e3.record()
    torch.cuda.synchronize()
    dom_s = e2.elapsed_time(e3) / K * 1e-3
    del sets
    log(f"[bench] {dom}: {dom_s * 1e6:.2f} us per launch ({K} launches back to back)")
    if args.copy_calibration:
        # a plain device copy of known size, for scaling HBM byte counters
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] calibration copy: 1 GiB read + 1 GiB written")

    # (not in the counter runs: their calibration is the last large device copy of the run)
    measured = None if args.copy_calibration else measured_hbm_rates(torch, dev)
    log(f"[bench] torch's generic kernels on the same HBM (context): {measured}")
    Dm = float(np.mean([D[i % args.batches] for i in range(K)]))
    ab = algorithmic_bytes(cfg, T, Dm)
    af = algorithmic_flops(cfg, T)
    layer_bytes = weight_bytes(cfg, Dm)
    layer_gbs = layer_bytes / (ms_step * 1e-3) / 1e9
    layer_tflops = sum(af.values()) / (ms_step * 1e-3) / 1e12
    if mx8:
        # compute-bound: the expert products on the scaled FP8 x FP4 matrix cores (they run
        # at the FP8 rate), the dense products on bf16 ones
        dtype_peak = "fp8" if dom.startswith("expert") else "bf16"
        achieved = af[dom] / dom_s / 1e12
        roofline = {"bound": "mfma", "kernel": dom, "achieved": achieved,
                    "peak": MFMA_PEAK[dtype_peak], "unit": "TFLOP/s",
                    "frac": achieved / MFMA_PEAK[dtype_peak],
                    "traffic": measured_traffic(cfg.name, dom, STEP_KERNELS_MX8),
                    "algorithmic_flops": af[dom], "avg_us": dom_s * 1e6,
                    "peak_dtype": "fp8 x fp4 (fp8 rate)" if dtype_peak == "fp8" else "bf16",
                    "frac_of_mxfp4_peak": achieved / MFMA_PEAK["fp4"] if dtype_peak == "fp8" else None}
    else:
        achieved = ab[dom] / dom_s / 1e9
        roofline = {"bound": "hbm", "kernel": dom, "achieved": achieved, "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                    "traffic": measured_traffic(cfg.name, dom),
                    "algorithmic_bytes": ab[dom], "avg_us": dom_s * 1e6}

    out = {
        "metric": METRIC,
        "value": T / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8xfp4+bf16" if mx8 else "f32",
        "data": "synthetic",
        "config": {"workload": cfg.name, "tokens_per_step": T, "d": cfg.d, "latent": cfg.l,
                   "experts": cfg.E, "top_k": cfg.k, "expert_hidden": cfg.m,
                   "shared_hidden": cfg.ms, "expert_weights": cfg.expert_fmt,
                   "precision_profile": getattr(cfg, "precision", "fp32"),
                   "dense_weight_copies": args.rotate, "token_batches": args.batches,
                   "distinct_experts_per_step": Dm},
        "roofline": roofline,
        "hipgraph": graph,
        "measured_hbm": measured,
        "layer": {"algorithmic_bytes": layer_bytes, "achieved_GBps": layer_gbs,
                  "hbm_frac": layer_gbs / HBM_PEAK_GBS,
                  "algorithmic_flops": sum(af.values()), "achieved_TFLOPs": layer_tflops,
                  "steps_us_with_event_per_boundary": steps_us},
    }
    if args.qb_stats:
        out["qb_stats"] = qb_stats(layers[0], xs[0], cfg, K, dev)
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle")
        out["cpu_baseline"] = cpu_baseline(cfg, dense0, args.cpu_seconds,
                                           sample_tokens=8 if T > 64 else None)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
