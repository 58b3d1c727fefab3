"""GPU: the residual add fused into the last step (moe_layer_forward_residual) and a chain
of decoder MoE blocks, through the C ABI.

- Against the library's own forward: the new residual is bit for bit the float32 sum of
  the old one and the Delta that moe_layer_forward returns, and x_next its bf16 rounding
  (every launch path: few tokens, token-tiled, mx8, non-latent).
- Against the oracle: a chain of three layers, each taking the previous one's x_next;
  the oracle runs the same chain on its own values (oracle.residual_add).
"""
import functools

import numpy as np
import pytest
import torch

import oracle as O
import sparse_moe_layer_amd as moe
import synth

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")

TINY = synth.LayerConfig(name="tiny_res", d=64, l=32, E=8, k=2, m=32, ms=64, tokens=5, seed=640,
                         expert_fmt="mxfp4", bias_kind="uniform", bias_a=-0.01, bias_b=0.01,
                         e8m0_lo=125, e8m0_hi=128)
CASES = {
    "few_tokens": (TINY, 3),
    "token_tiled": (TINY, 40),
    "mx8": (TINY.with_(name="tiny_res_mx8", d=128, l=64, m=64, precision="mx8"), 40),
    "non_latent_fp8": (synth.LayerConfig(name="tiny_res_k2", d=160, l=0, E=6, k=2, m=48, ms=32,
                                         tokens=5, seed=641, expert_fmt="fp8b128", act="swiglu",
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
    return lay, dense


def to_dev(x):
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(DEV)


@pytest.mark.parametrize("case", list(CASES))
def test_residual_equals_the_forward_plus_delta(case):
    cfg, T = CASES[case]
    lay, _ = device_layer(cfg)
    x = to_dev(synth.tokens(cfg, batch=T, T=T))
    res0 = torch.randn((T, cfg.d), dtype=torch.float32, device=DEV,
                       generator=torch.Generator(device=DEV).manual_seed(T))
    delta, idx, w = lay.forward(x)
    res = res0.clone()
    xn = torch.empty_like(x)
    d2 = torch.empty_like(delta)
    i2, w2 = lay.forward_residual(x, res, x_next=xn, delta=d2)
    torch.cuda.synchronize()
    assert torch.equal(d2, delta) and torch.equal(i2, idx) and torch.equal(w2, w)
    assert torch.equal(res, res0 + delta)
    assert torch.equal(xn, res.to(torch.bfloat16).view(torch.int16))
    # Delta not stored, x_next written over x itself
    res = res0.clone()
    xin = x.clone()
    lay.forward_residual(xin, res, x_next=xin)
    torch.cuda.synchronize()
    assert torch.equal(res, res0 + delta) and torch.equal(xin, xn)


def test_three_layer_chain_against_the_oracle():
    """x_{l+1} = bf16(h_l + Delta_l), h_0 = x_0: three different layers back to back."""
    cfgs = [TINY.with_(name=f"tiny_chain{i}", seed=700 + i) for i in range(3)]
    T = 24
    x0 = synth.tokens(cfgs[0], batch=1, T=T)
    # GPU chain
    xg = to_dev(x0)
    rg = torch.from_numpy(O.bf16_to_f64(x0).astype(np.float32)).to(DEV)
    for cfg in cfgs:
        lay, _ = device_layer(cfg)
        lay.forward_residual(xg, rg, x_next=xg)
    torch.cuda.synchronize()
    # oracle chain on its own values
    xo = x0
    ro = O.bf16_to_f64(x0)
    for cfg in cfgs:
        _, dense = device_layer(cfg)
        r = O.forward(O.OracleLayer.from_synth(cfg, dense), xo)
        ro, xo = O.residual_add(ro, r.delta)
    got = rg.cpu().numpy().astype(np.float64)
    x1 = O.bf16_to_f64(x0)
    # the blocks' summed contribution h_3 - h_0, compared as a Delta
    rel = np.linalg.norm((got - x1) - (ro - x1)) / np.linalg.norm(ro - x1)
    log(f"[chain] rel-L2 of the three blocks' sum: {rel:.2e}")
    assert rel <= 2e-3
    # the bf16 inputs agree except within rounding distance of a bf16 midpoint
    xg_np = O.bf16_to_f64(xg.cpu().numpy().view(np.uint16))
    xo_np = O.bf16_to_f64(xo)
    diff = xg_np != xo_np
    assert diff.mean() < 1e-2, diff.mean()


@pytest.mark.parametrize("T", [1, 3, 40])
def test_residual_with_next_layer_prefetch_gives_the_same_bits(T):
    """moe_layer_forward_residual_prefetch: with few tokens the last launch also reads the next
    layer's first-launch weight bytes; the results are those of the plain residual forward
    (larger batches ignore the next layer)."""
    cfg = TINY
    lay, _ = device_layer(cfg)
    nxt, _ = device_layer(cfg.with_(name="tiny_res_next", seed=642))
    x = to_dev(synth.tokens(cfg, batch=50 + T, T=T))
    res0 = torch.randn((T, cfg.d), dtype=torch.float32, device=DEV,
                       generator=torch.Generator(device=DEV).manual_seed(7 + T))
    r1, r2 = res0.clone(), res0.clone()
    xn1 = torch.empty_like(x)
    xn2 = torch.empty_like(x)
    i1, w1 = lay.forward_residual(x, r1, x_next=xn1)
    i2, w2 = lay.forward_residual_prefetch(x, r2, nxt, x_next=xn2)
    i3, w3 = lay.forward_residual_prefetch(x, res0.clone(), None)
    torch.cuda.synchronize()
    assert torch.equal(r1, r2) and torch.equal(xn1, xn2)
    assert torch.equal(i1, i2) and torch.equal(w1, w2) and torch.equal(i1, i3)
