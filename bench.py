#!/usr/bin/env python3
"""Throughput of the Stable LatentMoE FFN layer forward on one MI355X.

One step = one moe_layer_forward call (all steps of the layer) over one batch of
synthetic tokens already resident in HBM.  Prints one JSON line.

By default it measures the three configurations of the metric, each with its roofline, its
CPU oracle baseline and a parity sample: the K3-shaped layer (d 7168, latent 3584, 896 MXFP4
experts top-16, 3072-wide experts, merged 6144-wide shared expert) at decode batch 1 (the
headline: `value` and the top-level fields), at decode batch 64 under a Zipf(1.0) load, and at
prefill of 8192 tokens in the mx8 profile and in the fp32 profile (under "workloads"), with the
mx4 variant of the prefill (MXFP4 activations on the FP4 x FP4 matrix cores) reported beside
them.  Three
copies of the dense weights and distinct token batches rotate at decode so that the 256 MB
last-level cache cannot hold what a step reads.  Measured peaks (an HBM read stream, loops of
each matrix-core instruction) are reported beside the published ones.
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
    prof = getattr(cfg, "precision", "fp32")
    mx = prof in ("mx8", "mx4")        # the mx launches
    # bytes per activation element of the expert inputs (MX: codes plus one scale byte per 32)
    ab = {"mx8": 1 + 1 / 32, "mx4": 0.5 + 1 / 32}.get(prof, 4)
    if mx:
        # one IN product (router logits, x^c fp32, h_s bf16), then x^c to MX
        router = T * d * 2 + (E + cfg.l + 2 * ms) * d * 2 + T * (E * 4 + cfg.l * 4 + ms * 2)
        in_ = T * cfg.l * 4 + T * cfg.l * ab
    elif small and cfg.l:
        # a few tokens of a latent layer: one IN launch takes the router, W_down_latent and the
        # shared gate/up (and the route); W_shared_down rides in the expert down launch
        router = 0
        in_ = (T * d * 2 + (E + cfg.l + 2 * ms) * d * 2 + T * (E + cfg.l + ms) * 4
               + T * E * 4 + E * 4 + tk * 16 + E * 8)
    else:
        # W_down_latent rides in the ROUTER launch for a few tokens, in the IN launch otherwise
        ldn = cfg.l if small else 0
        router = T * d * 2 + (E + ldn) * d * 2 + T * (E + ldn) * 4
        in_ = (T * d * 2 + (cfg.l - ldn + 2 * ms) * d * 2 + T * (cfg.l - ldn + ms) * 4
               + ((T * E * 4 + E * 4 + tk * 16 + E * 8) if small else 0))
    if not mx and small and cfg.l and ms:
        # the four partial sums of h_s W_shared_down, written by the down launch, read by OUT
        sd = ms * d * 2 + T * ms * 4 + 4 * T * d * 8
        down = D * dn_w + tk * m * ab + tk * l * 4 + sd
        out = d * cfg.l * 2 + cfg.l * 2 + T * l * 4 + 4 * T * d * 8 + T * d * 4
    else:
        down = D * dn_w + tk * m * ab + tk * l * 4
        out = d * (cfg.l + ms) * 2 + cfg.l * 2 + T * (l + ms) * (2 if mx else 4) + T * d * 4
    return {
        "router": router,
        "in": in_,
        "route": 0 if small else T * E * 4 + E * 4 + tk * 8,
        "dispatch": 0 if small else tk * 4 * 4 + E * 8,
        "expert_gu": D * gu_w + T * l * ab + tk * m * ab,
        "expert_down": down,
        # (mx: one pass to u_hat in bf16, u itself is not stored)
        "combine": tk * l * 4 + tk * 8 + T * l * (2 if mx else 4),
        "out": out,
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
STEP_KERNELS_MX = {"router": [("k_pf_pack_x", None), ("k_pf_gemm", "true")], "in": [("k_pf_quant", None)],
                    "route": [("k_route", None)],
                    "dispatch": [("k_disp_count", None), ("k_disp_scan", None), ("k_disp_scatter", None)],
                    "expert_gu": [("k_pf_exp", "true")], "expert_down": [("k_pf_exp", "false")],
                    "combine": [("k_pf_combine_norm", None), ("k_combine", None), ("k_pf_norm", None)],
                    "out": [("k_pf_gemm", "false")]}


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


def chain_timing(layers, xs, K, warmup):
    """Decode through a chain of decoder MoE blocks: the layers in turn on one token, each
    adding its Delta into the residual stream and handing the bf16 residual to the next
    (moe_layer_forward_residual), against the same chain where each call's last launch also
    reads the next layer's first-launch weights (moe_layer_forward_residual_prefetch).  The two
    variants alternate in rounds of K calls; returns microseconds per layer of each (median of
    the rounds)."""
    import numpy as np
    import torch
    L = len(layers)
    T, d = xs[0].shape
    x = xs[0].clone()
    res = torch.zeros((T, d), dtype=torch.float32, device=x.device)
    k = layers[0].cfg.top_k
    idx = torch.empty((T, k), dtype=torch.int32, device=x.device)
    w = torch.empty((T, k), dtype=torch.float32, device=x.device)
    ws = layers[0].workspace(T)

    def run(n, prefetch):
        for i in range(n):
            j = i % L
            if prefetch:
                layers[j].forward_residual_prefetch(x, res, layers[(j + 1) % L], x_next=x, idx=idx,
                                                    w=w, workspace=ws)
            else:
                layers[j].forward_residual(x, res, x_next=x, idx=idx, w=w, workspace=ws)
    run(warmup * L, False)
    run(warmup * L, True)
    torch.cuda.synchronize()
    times = {False: [], True: []}
    n = max(L, (K // L) * L)
    for _ in range(5):
        for pf in (False, True):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            run(n, pf)
            e1.record()
            torch.cuda.synchronize()
            times[pf].append(e0.elapsed_time(e1) * 1e3 / n)
    plain, pref = float(np.median(times[False])), float(np.median(times[True]))
    log(f"[bench] chain of {L} layers at batch {T}: {plain:.1f} us per layer, {pref:.1f} with the "
        f"next layer's router and W_down_latent prefetched in the tail")
    return {"layers": L, "calls_per_round": n, "rounds": 5, "us_per_layer": plain,
            "us_per_layer_prefetch": pref, "rounds_us": {"plain": times[False], "prefetch": times[True]}}


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


# ---- measured peaks -----------------------------------------------------------------------

PEAK_KINDS = {"bf16_16x16x32": 0, "bf16_32x32x16": 1, "fp8_16x16x128": 2, "fp8xfp4_16x16x128": 3,
              "fp4_16x16x128": 4, "fp8_32x32x64": 5, "fp4_32x32x64": 6}


def measured_peaks(torch, dev, reps=3):
    """What this GPU reaches at all: a non-temporal HBM read stream over 4 GiB (best grid of
    five) and loops of each matrix-core instruction with register operands (libmoe_peaks.so,
    include/moe_peaks.h).  The roofline fractions are quoted against these and against the
    published peaks."""
    from sparse_moe_layer_amd import peaks as pk
    L = pk.lib()
    st = torch.cuda.current_stream(dev)
    out = torch.empty(16384 * 256, dtype=torch.int32, device=dev)
    src = torch.zeros(4 << 30, dtype=torch.uint8, device=dev)

    def timed(launch):
        best = None
        for _ in range(reps + 1):       # the first launch warms up
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(st)
            launch()
            e1.record(st)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1)
            best = ms if best is None else min(best, ms)
        return best

    read = {}
    for grid in (1024, 2048, 4096, 8192, 16384):
        ms = timed(lambda: pk.check(L.moe_peak_read(src.data_ptr(), src.numel(), out.data_ptr(),
                                                          out.numel(), grid, st.cuda_stream)))
        read[grid] = src.numel() / (ms * 1e-3) / 1e9
    del src
    mfma = {}
    for name, kind in PEAK_KINDS.items():
        flops = ctypes.c_double()
        ms = timed(lambda: pk.check(L.moe_peak_mfma(kind, 2048, 4000, out.data_ptr(), out.numel(),
                                                          ctypes.byref(flops), st.cuda_stream)))
        mfma[name] = flops.value / (ms * 1e-3) / 1e12
    torch.cuda.synchronize()
    res = {"hbm_read_GBps": max(read.values()),
           "hbm_read_GBps_by_grid": {str(g): round(v, 1) for g, v in read.items()},
           "mfma_TFLOPs": {k: round(v, 1) for k, v in mfma.items()},
           "published": {"hbm_GBps": HBM_PEAK_GBS, **{f"{k}_TFLOPs": v for k, v in MFMA_PEAK.items()}}}
    res["by_dtype_TFLOPs"] = {"bf16": max(mfma["bf16_16x16x32"], mfma["bf16_32x32x16"]),
                              "fp8": max(mfma["fp8_16x16x128"], mfma["fp8_32x32x64"]),
                              "fp8xfp4": mfma["fp8xfp4_16x16x128"],
                              "fp4": max(mfma["fp4_16x16x128"], mfma["fp4_32x32x64"])}
    log(f"[bench] measured peaks: HBM read {res['hbm_read_GBps']:.0f} GB/s; matrix cores "
        f"{ {k: round(v) for k, v in res['by_dtype_TFLOPs'].items()} } TFLOP/s")
    return res


# ---- the CPU oracle beside the GPU -----------------------------------------------------------

def host_info():
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    n = os.cpu_count() or 1
    try:
        n_aff = len(os.sched_getaffinity(0))
    except AttributeError:
        n_aff = n
    return model, n, n_aff


def cpu_baseline(cfg, dense, x, rows, gpu, xcq=None, other_precision=None, cache=None):
    """The float64 CPU oracle as it is, timed on the host on a bounded sample of the workload:
    tokens `rows` of the batch x (bf16 [T, d]).  The canonical expert bytes those tokens
    route to are generated before the clock starts; the oracle dequantises them itself inside
    the timed forward (its own work).  Returns (cpu_baseline object, parity sample object):
    the GPU outputs gpu = (delta, idx, w) of x against the oracle on the same tokens in the
    workload's profile (tests/parity.py's rule, the bars reported, not asserted), and, with
    other_precision, against the oracle in that profile too (informational)."""
    import numpy as np
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import oracle
    import parity
    import synth
    model, n_cpu, n_aff = host_info()
    prof = getattr(cfg, "precision", "fp32")
    xs = x[rows]
    key = (cfg.seed, cfg.E, tuple(int(r) for r in rows[:4]), len(rows), x.shape[0])
    OL0 = oracle.OracleLayer.from_synth(cfg, dense)
    # which experts the sample routes to (the oracle's own router), their bytes generated now
    s = oracle.router_scores(oracle.bf16_to_f64(xs), OL0.router)
    idx0, _, _ = oracle.select_and_weight(s, OL0.bias, cfg.k, cfg.route_scale)
    t0 = time.perf_counter()
    slices = {int(e): synth.expert_slice(cfg, int(e), int(e) + 1) for e in np.unique(idx0)}
    gen_s = time.perf_counter() - t0
    OL = oracle.OracleLayer.from_synth(cfg, dense, preload=False, expert_slice=lambda c, a, b: slices[a])
    workers = oracle.moe_oracle._workers(OL, None)

    def timed(precision):
        ck = (key, precision)
        if cache is not None and ck in cache:
            return cache[ck]
        t = time.perf_counter()
        r = oracle.forward(OL, xs, precision=precision)
        out = (r, time.perf_counter() - t)
        if cache is not None:
            cache[ck] = out
        return out
    ref, secs = timed(prof)
    d, i, w = (a[rows] for a in gpu)
    qsel = None if xcq is None else (xcq[0][rows], xcq[1][rows])
    step = int(rows[1] - rows[0]) if len(rows) > 1 else 1
    par = {"tokens": len(rows), "rows": "every token" if step == 1 else f"one token in every {step}"}
    try:
        r = parity.compare(OL, xs, d, i, w, precision=prof, ref=ref, xcq=qsel, bars=False, log=log)
        par["vs_oracle_" + prof] = {"rel_l2": r["rel_l2"], "max_abs_over_rms": r["max_abs_over_rms"],
                                    "near_tie_tokens": r["near_tie_tokens"],
                                    "recomputed_tokens": r["recomputed_tokens"],
                                    "within_bars": r["rel_l2"] <= parity.REL_L2 and
                                    r["max_abs_over_rms"] <= parity.MAX_ABS_RMS}
    except parity.ParityError as e:
        par["vs_oracle_" + prof] = {"error": str(e)}
    if other_precision:
        ref2, secs2 = timed(other_precision)
        try:
            r2 = parity.compare(OL, xs, d, i, w, precision=other_precision, ref=ref2, bars=False, log=log)
            par["vs_oracle_" + other_precision] = {"rel_l2": r2["rel_l2"],
                                                   "max_abs_over_rms": r2["max_abs_over_rms"],
                                                   "informational": True}
        except parity.ParityError as e:
            par["vs_oracle_" + other_precision] = {"error": str(e)}
    base = {"value": len(rows) / secs, "unit": "tokens/s", "cores": int(workers), "kind": "oracle",
            "sample": f"{len(rows)} token(s) of the workload's first timed batches ({par['rows']}), "
                      f"{secs:.1f} s: the float64 numpy oracle in the {prof} profile, experts "
                      f"evaluated by {workers} threads (BLAS 1 thread each; the dense products "
                      f"with BLAS on all cores); the {len(slices)} touched experts' canonical bytes "
                      f"generated before the clock ({gen_s:.1f} s), dequantised inside it",
            "host": {"cpu_model": model, "nproc": n_cpu, "affinity_cpus": n_aff}}
    log(f"[bench] cpu oracle: {base['value']:.3f} tokens/s ({secs:.1f} s for {len(rows)} tokens)")
    return base, par


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


DEFAULT_WORKLOADS = ("k3_latent_moe_decode_b1", "k3_latent_moe_decode_b64_zipf1.0",
                     "k3_latent_moe_prefill_8192", "k3_latent_moe_prefill_8192_fp32",
                     "k3_latent_moe_prefill_8192_mx4")
# per workload: (dense weight copies rotated, distinct token batches rotated, CPU-baseline sample
# as (batches of the rotation, tokens per batch taken one every `stride`))
ROTATION = {"k3_latent_moe_decode_b1": (3, 64), "k3_latent_moe_decode_b64_zipf1.0": (3, 16),
            "k3_latent_moe_prefill_8192": (1, 2), "k3_latent_moe_prefill_8192_fp32": (1, 2),
            "k3_latent_moe_prefill_8192_mx4": (1, 2),
            "k2_moe_1024_zipf1.2": (3, 8), "k3_ep_share_112x1170": (1, 2)}
CPU_SAMPLE = {"k3_latent_moe_decode_b1": (16, 1), "k3_latent_moe_decode_b64_zipf1.0": (1, 1),
              "k3_latent_moe_prefill_8192": (1, 128), "k3_latent_moe_prefill_8192_fp32": (1, 128),
              "k3_latent_moe_prefill_8192_mx4": (1, 128),
              "k2_moe_1024_zipf1.2": (1, 16), "k3_ep_share_112x1170": (1, 128)}


def layer_key(cfg):
    """Workloads that differ only in name, tokens and profile share one uploaded layer."""
    return cfg.with_(name="", tokens=0, precision="fp32")


def run_workload(cfg, args, peaks, store, cpu_cache):
    import numpy as np
    import torch

    import sparse_moe_layer_amd as moe
    import synth

    dev = torch.device("cuda:0")
    T = cfg.tokens
    mcfg = moe.config_from(cfg)
    rot, nb = ROTATION.get(cfg.name, (3, 16))
    rotate = args.rotate if args.rotate is not None else rot
    batches = args.batches if args.batches is not None else nb
    key = layer_key(cfg)
    if store.get("key") != key or len(store.get("layers", [])) < rotate:
        store.clear()
        torch.cuda.empty_cache()
        log(f"[bench] workload {cfg.name}: generating and uploading the layer")
        t0 = time.perf_counter()
        dense0 = synth.dense_weights(cfg)
        chunk, staging = 64, {}

        def slice_fn(a, b):
            if b - a == chunk and "s" in staging:
                return synth.expert_slice(cfg, a, b, out=staging["s"])
            sl = synth.expert_slice(cfg, a, b)
            if b - a == chunk:
                staging["s"] = sl
            return sl
        l0 = moe.Layer.upload(mcfg, dense0, slice_fn, cfg.E, device=dev, chunk=chunk)
        staging.clear()
        store.update(key=key, dense0=dense0,
                     layers=[l0] + [l0.with_dense(synth.dense_weights(cfg, copy=c)) for c in range(1, rotate)])
        torch.cuda.synchronize()
        log(f"[bench] layer ready in {time.perf_counter() - t0:.1f} s")
    else:
        log(f"[bench] workload {cfg.name}: the layer of the previous workload, profile "
            f"{getattr(cfg, 'precision', 'fp32')}")
    dense0 = store["dense0"]
    # the uploaded weights under this workload's config (the profile may differ)
    layers = [moe.Layer(mcfg, L.dense, L.bias, L.experts) for L in store["layers"][:rotate]]
    xs_h = [synth.tokens(cfg, batch=1000 + b) for b in range(batches)]
    xs = [torch.from_numpy(x.view(np.int16)).to(dev) for x in xs_h]
    delta = torch.empty((T, cfg.d), dtype=torch.float32, device=dev)
    idx = torch.empty((T, cfg.k), dtype=torch.int32, device=dev)
    gw = torch.empty((T, cfg.k), dtype=torch.float32, device=dev)
    ws = layers[0].workspace(T)

    # distinct experts per batch (for the byte count of the timed steps)
    D = []
    for b in range(batches):
        layers[0].forward(xs[b], delta, idx, gw, ws)
        D.append(len(np.unique(idx.cpu().numpy())))
    for i in range(args.warmup):
        layers[i % rotate].forward(xs[i % batches], delta, idx, gw, ws)
    torch.cuda.synchronize()

    # timed region: K whole forwards back to back
    K = args.steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(K):
        layers[i % rotate].forward(xs[i % batches], delta, idx, gw, ws)
    e1.record()
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / K
    log(f"[bench] {cfg.name}: {K} steps, {ms_step * 1e3:.1f} us/step, {T / (ms_step * 1e-3):.0f} tokens/s")
    graph = None
    if T <= 64:     # decode: the captured forward as a serving loop would replay it
        graph = graph_replay(layers, xs, (delta, idx, gw, ws), rotate, batches, K, args.warmup)
        graph["tokens_per_s"] = T / (graph["us_per_step"] * 1e-6)
        log(f"[bench] hipGraph replay: {graph['us_per_step']:.1f} us/step over {K} replays; single "
            f"replays median {graph['median_us']:.1f} (p10 {graph['p10_us']:.1f}, p90 "
            f"{graph['p90_us']:.1f}); eager median {graph['eager']['median_us']:.1f}; "
            f"bits equal eager: {graph['bits_equal_eager']}")

    chain = chain_timing(layers, xs, K, args.warmup) if (T <= 4 and rotate > 1) else None

    # per-step durations: the same forwards with in-stream events between the steps (an event
    # record costs a few microseconds of GPU time, so this pass only ranks the steps)
    hip = HipEvents()
    nst = len(moe.STEPS)
    evs = hip.create(K * (nst + 1))
    for i in range(K):
        layers[i % rotate].forward_timed(xs[i % batches], evs[i * (nst + 1):(i + 1) * (nst + 1)],
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
    prof = getattr(cfg, "precision", "fp32")
    mx = prof in ("mx8", "mx4")     # the mx launches
    # The dominant step alone, K launches back to back between two events, each on the
    # buffers of an earlier full forward; R sets of buffers (different tokens, so different
    # experts, and different dense copies) rotate past the last-level cache.
    si = moe.STEPS.index(dom)
    R = 8 if T <= 64 else 2
    sets = []
    for r in range(R):
        bufs = (torch.empty_like(delta), torch.empty_like(idx), torch.empty_like(gw),
                moe.new_workspace(mcfg, T, dev))
        layers[r % rotate].forward(xs[r % batches], *bufs[:3], workspace=bufs[3])
        sets.append(bufs)
    for r in range(R):
        layers[r % rotate].forward_steps(xs[r % batches], si, si + 1, *sets[r])
    torch.cuda.synchronize()
    e2, e3 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e2.record()
    for i in range(K):
        r = i % R
        layers[r % rotate].forward_steps(xs[r % batches], si, si + 1, *sets[r])
    e3.record()
    torch.cuda.synchronize()
    dom_s = e2.elapsed_time(e3) / K * 1e-3
    del sets
    log(f"[bench] {dom}: {dom_s * 1e6:.2f} us per launch ({K} launches back to back)")

    Dm = float(np.mean([D[i % batches] for i in range(K)]))
    ab = algorithmic_bytes(cfg, T, Dm)
    af = algorithmic_flops(cfg, T)
    layer_bytes = weight_bytes(cfg, Dm)
    layer_gbs = layer_bytes / (ms_step * 1e-3) / 1e9
    layer_tflops = sum(af.values()) / (ms_step * 1e-3) / 1e12
    kernels = STEP_KERNELS_MX if mx else STEP_KERNELS
    traffic = measured_traffic(cfg.name, dom, kernels)
    # the bound of the dominant step: its algorithmic bytes at the HBM peak against its flops
    # at the matrix-core rate of its operands (mx8 experts: the FP8 x FP4 instruction runs at
    # the FP8 rate; mx4 experts: FP4 x FP4; everything else: bf16 operands, fp32 activations
    # as bf16 pairs)
    dtype_peak = ({"mx8": "fp8", "mx4": "fp4"}[prof] if (mx and dom.startswith("expert"))
                  else "bf16")
    t_mem = ab[dom] / (HBM_PEAK_GBS * 1e9)
    t_mma = af[dom] / (MFMA_PEAK[dtype_peak] * 1e12)
    meas = peaks or {}
    if t_mma > t_mem:
        achieved = af[dom] / dom_s / 1e12
        mpk = meas.get("by_dtype_TFLOPs", {}).get({"fp8": "fp8xfp4"}.get(dtype_peak, dtype_peak))
        roofline = {"bound": "mfma", "kernel": dom, "achieved": achieved,
                    "peak": MFMA_PEAK[dtype_peak], "unit": "TFLOP/s",
                    "frac": achieved / MFMA_PEAK[dtype_peak],
                    "traffic": traffic, "traffic_over_algorithmic": (traffic / ab[dom]) if traffic else None,
                    "algorithmic_flops": af[dom], "algorithmic_bytes": ab[dom], "avg_us": dom_s * 1e6,
                    "peak_dtype": {"fp8": "fp8 x fp4 (fp8 rate)", "fp4": "fp4 x fp4"}.get(dtype_peak, "bf16"),
                    "measured_peak": mpk, "frac_of_measured": (achieved / mpk) if mpk else None,
                    "frac_of_mxfp4_peak": achieved / MFMA_PEAK["fp4"] if dtype_peak != "bf16" else None}
    else:
        achieved = ab[dom] / dom_s / 1e9
        mpk = meas.get("hbm_read_GBps")
        roofline = {"bound": "hbm", "kernel": dom, "achieved": achieved, "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                    "traffic": traffic, "traffic_over_algorithmic": (traffic / ab[dom]) if traffic else None,
                    "algorithmic_bytes": ab[dom], "avg_us": dom_s * 1e6,
                    "measured_peak": mpk, "frac_of_measured": (achieved / mpk) if mpk else None}
    res = {
        "value": T / (ms_step * 1e-3), "unit": "tokens/s", "ms_per_step": ms_step, "steps": K,
        "warmup": args.warmup,
        "dtype": {"mx8": "fp8xfp4+bf16", "mx4": "fp4xfp4+bf16"}.get(prof, "f32"),
        "config": {"workload": cfg.name, "tokens_per_step": T, "d": cfg.d, "latent": cfg.l,
                   "experts": cfg.E, "top_k": cfg.k, "expert_hidden": cfg.m,
                   "shared_hidden": cfg.ms, "expert_weights": cfg.expert_fmt,
                   "precision_profile": getattr(cfg, "precision", "fp32"),
                   "dense_weight_copies": rotate, "token_batches": batches,
                   "distinct_experts_per_step": Dm},
        "roofline": roofline,
        "layer": {"algorithmic_bytes": layer_bytes, "achieved_GBps": layer_gbs,
                  "hbm_frac": layer_gbs / HBM_PEAK_GBS,
                  "hbm_frac_of_measured": (layer_gbs / meas["hbm_read_GBps"]) if meas else None,
                  "algorithmic_flops": sum(af.values()), "achieved_TFLOPs": layer_tflops,
                  "steps_us_with_event_per_boundary": steps_us},
    }
    if graph is not None:
        res["hipgraph"] = graph
    if chain is not None:
        res["chain"] = chain
    if args.qb_stats:
        res["qb_stats"] = qb_stats(layers[0], xs[0], cfg, K, dev)
    if not args.no_cpu_baseline:
        log(f"[bench] {cfg.name}: the CPU oracle on a sample of the workload")
        nbat, stride = CPU_SAMPLE.get(cfg.name, (1, max(1, T // 64)))
        # the sample's batches, each once more through the GPU (their outputs for the parity
        # sample; the last forward's workspace holds the mx x^c codes)
        xh = np.concatenate([xs_h[b] for b in range(min(nbat, batches))])
        outs = []
        for b in range(min(nbat, batches)):
            d_, i_, w_ = layers[0].forward(xs[b])
            outs.append((d_.cpu().numpy().astype(np.float64), i_.cpu().numpy(),
                         w_.cpu().numpy().astype(np.float64)))
        torch.cuda.synchronize()
        gpu = tuple(np.concatenate([o[j] for o in outs]) for j in range(3))
        xcq = None
        if mx and nbat == 1:
            inter = layers[0].intermediates(T)
            xcq = (inter["xq"].cpu().numpy(), inter["xs"].cpu().numpy())
        rows = np.arange(0, xh.shape[0], stride)
        res["cpu_baseline"], res["parity_sample"] = cpu_baseline(
            cfg, dense0, xh, rows, gpu, xcq=xcq, other_precision="fp32" if mx else None,
            cache=cpu_cache)
    del layers, xs, ws
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=None,
                    help="one workload (synth preset) instead of the default set: K3 decode B=1 "
                         "(the headline), decode B=64 Zipf(1.0), prefill 8192 in the mx8, "
                         "fp32 and mx4 profiles")
    ap.add_argument("--rotate", type=int, default=None, help="dense weight copies rotated")
    ap.add_argument("--batches", type=int, default=None, help="distinct token batches rotated")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-peaks", action="store_true", help="skip the measured-peak probes")
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

    import torch

    import synth

    dev = torch.device("cuda:0")
    names = [args.workload] if args.workload else list(DEFAULT_WORKLOADS)
    peaks = None if (args.no_peaks or args.copy_calibration) else measured_peaks(torch, dev)
    store, cpu_cache, results = {}, {}, {}
    for name in names:
        results[name] = run_workload(synth.PRESETS[name], args, peaks, store, cpu_cache)
    store.clear()
    torch.cuda.empty_cache()
    if args.copy_calibration:
        # a plain device copy of known size, for scaling HBM byte counters
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] calibration copy: 1 GiB read + 1 GiB written")

    head = results[names[0]]
    out = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["dtype"],
        "data": "synthetic",
        "config": head["config"],
        "roofline": head["roofline"],
    }
    for k in ("cpu_baseline", "parity_sample", "hipgraph", "chain", "layer", "qb_stats"):
        if k in head:
            out[k] = head[k]
    if peaks is not None:
        out["measured_peaks"] = peaks
    if len(names) > 1:
        out["workloads"] = {n: results[n] for n in names[1:]}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
