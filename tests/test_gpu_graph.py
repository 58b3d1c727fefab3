"""GPU: the forward captured in a HIP graph (torch.cuda.CUDAGraph) and replayed.

A forward launches kernels on the caller's stream and nothing else: no allocation, no
memset, no copy to the host, no host synchronisation (its grids are sized for the worst
case, not from device data).  So a serving loop can capture it once per token count and
replay it.  Each replay here runs on new inputs copied into the captured input buffer,
with eager work on the same stream between replays, and must give the bits of the eager
forward on those inputs (Delta, indices, weights).  The residual entry point is captured
too: replaying it is a chain of blocks that all have the same weights.
"""
import functools

import numpy as np
import pytest
import torch

import sparse_moe_layer_amd as moe
import synth

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")

TINY = synth.LayerConfig(name="tiny_graph", d=64, l=32, E=8, k=2, m=32, ms=64, tokens=5, seed=650,
                         expert_fmt="mxfp4", bias_kind="uniform", bias_a=-0.01, bias_b=0.01,
                         e8m0_lo=125, e8m0_hi=128)
CASES = {
    "few_tokens": (TINY, 3),
    "token_tiled": (TINY, 40),
    "mx8": (TINY.with_(name="tiny_graph_mx8", d=128, l=64, m=64, precision="mx8"), 40),
    "non_latent_fp8": (synth.LayerConfig(name="tiny_graph_k2", d=160, l=0, E=6, k=2, m=48, ms=32,
                                         tokens=5, seed=651, expert_fmt="fp8b128", act="swiglu",
                                         route_scale=2.827, use_norm=False, bias_kind="uniform",
                                         bias_a=-0.01, bias_b=0.01), 33),
}


def log(msg):
    print(msg, flush=True)


@functools.lru_cache(maxsize=8)
def device_layer(cfg):
    dense = synth.dense_weights(cfg)
    lay = moe.Layer.upload(moe.config_from(cfg), dense, lambda a, b: synth.expert_slice(cfg, a, b),
                           cfg.E, device=DEV, chunk=32)
    torch.cuda.synchronize()
    return lay


def to_dev(x):
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(DEV)


@pytest.mark.parametrize("case", list(CASES))
def test_graph_replays_give_the_eager_bits(case):
    cfg, T = CASES[case]
    log(f"[graph] {case}: T={T}")
    lay = device_layer(cfg)
    xs = [to_dev(synth.tokens(cfg, batch=b, T=T)) for b in range(4)]
    x = xs[0].clone()
    delta = torch.empty((T, cfg.d), dtype=torch.float32, device=DEV)
    idx = torch.empty((T, cfg.k), dtype=torch.int32, device=DEV)
    w = torch.empty((T, cfg.k), dtype=torch.float32, device=DEV)
    ws = moe.new_workspace(lay.cfg, T, DEV)
    lay.forward(x, delta, idx, w, ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        lay.forward(x, delta, idx, w, ws)
    torch.cuda.synchronize()
    ws2 = moe.new_workspace(lay.cfg, T, DEV)
    for b in (1, 2, 3, 1, 0):
        x.copy_(xs[b])
        g.replay()
        got = (delta.clone(), idx.clone(), w.clone())
        ref = lay.forward(xs[b], workspace=ws2)          # eager, between replays
        torch.cuda.synchronize()
        for a, r in zip(got, ref):
            assert torch.equal(a, r), (case, b)


def test_captured_residual_chain():
    """Replaying forward_residual(x, res, x_next=x) n times = n eager calls in a row."""
    T = 24
    lay = device_layer(TINY)
    x0 = to_dev(synth.tokens(TINY, batch=9, T=T))
    r0 = x0.view(torch.bfloat16).float()
    xg, rg = x0.clone(), r0.clone()
    ws = moe.new_workspace(lay.cfg, T, DEV)
    lay.forward_residual(xg.clone(), rg.clone(), workspace=ws)     # warm-up, own copies
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        lay.forward_residual(xg, rg, x_next=xg, workspace=ws)
    torch.cuda.synchronize()
    # capture ran nothing: the buffers still hold the inputs
    assert torch.equal(xg, x0) and torch.equal(rg, r0)
    xe, re_ = x0.clone(), r0.clone()
    for _ in range(3):
        g.replay()
        lay.forward_residual(xe, re_, x_next=xe)
    torch.cuda.synchronize()
    assert torch.equal(rg, re_) and torch.equal(xg, xe)
    assert not torch.equal(rg, r0)
