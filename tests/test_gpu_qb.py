"""GPU parity of the Quantile Balancing statistics (moe_qb_histogram, moe_qb_readout)
through the C ABI, against the oracle (oracle/qb.py).

- Counts: every token contributes one count per expert; the GPU takes each bin decision
  in float32 on its own scores, the oracle on its float64 router rounded to float32, so a
  value within rounding distance of a bin edge may fall on either side.  The check is
  exact with that allowance: for every expert and bin, the GPU's cumulative count lies
  between the oracle's counts with every r moved down and up by TOL_R.
- Readout: on the same seeded counts, GPU (float32) and oracle (float64) within 1e-5 of
  the range width.
- End to end: the GPU's new biases within one bin width (plus the rounding allowance) of
  the exact order statistic, the walkthrough's bound for its histogram estimate.
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
TOL_R = 2e-5      # |r_gpu - r_oracle|: float32 logit sums and sigmoid against float64
                  # (1% of the bin width of the K3 biases with 1000 bins)

TINY = synth.LayerConfig(name="tiny_qb", d=64, l=32, E=12, k=3, m=32, ms=32, tokens=40,
                         seed=515, expert_fmt="mxfp4", bias_kind="uniform", bias_a=-0.05,
                         bias_b=0.05, e8m0_lo=125, e8m0_hi=128)


def log(msg):
    print(msg, flush=True)


@functools.lru_cache(maxsize=3)
def device_layer(cfg):
    log(f"[upload] {cfg.name}")
    dense = synth.dense_weights(cfg)
    lay = moe.Layer.upload(moe.config_from(cfg), dense, lambda a, b: synth.expert_slice(cfg, a, b),
                           cfg.E, device=DEV, chunk=32)
    torch.cuda.synchronize()
    return lay, dense


def to_dev(x):
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(DEV)


def oracle_scores(cfg, dense, x):
    return O.router_scores(O.bf16_to_f64(x), O.bf16_to_f64(dense.router))


def check_counts(hist, s, bias, k, n_bins):
    """GPU counts [E, B] against the oracle's r with the rounding allowance."""
    r = O.qb_required_bias(s, bias, k).astype(np.float64)
    lo, hi = O.qb_range(bias)
    t_lo = O.qb_bins((r - TOL_R).astype(np.float32), lo, hi, n_bins)
    t_hi = O.qb_bins((r + TOL_R).astype(np.float32), lo, hi, n_bins)
    T, E = r.shape
    assert np.all(hist.sum(axis=1) == T)
    cum = np.cumsum(hist, axis=1)
    for e in range(E):
        most = np.cumsum(np.bincount(t_lo[:, e], minlength=n_bins))    # r moved down
        least = np.cumsum(np.bincount(t_hi[:, e], minlength=n_bins))   # r moved up
        assert np.all(least <= cum[e]) and np.all(cum[e] <= most), e
    exact = int((t_lo == t_hi).sum())
    return exact / r.size


@pytest.mark.parametrize("T,bins", [(1, 16), (40, 50), (300, 1000)])
def test_qb_counts_tiny(T, bins):
    lay, dense = device_layer(TINY)
    x = synth.tokens(TINY, batch=T, T=T)
    h = lay.qb_histogram(to_dev(x), n_bins=bins).cpu().numpy()
    torch.cuda.synchronize()
    frac = check_counts(h, oracle_scores(TINY, dense, x), dense.bias, TINY.k, bins)
    log(f"[qb tiny] T={T} bins={bins}: {frac:.4%} of the values away from a bin edge")


def test_qb_counts_accumulate_over_micro_batches_and_repeat():
    lay, _ = device_layer(TINY)
    x = to_dev(synth.tokens(TINY, batch=3, T=200))
    whole = lay.qb_histogram(x, n_bins=200)
    parts = lay.qb_histogram(x[:77].contiguous(), n_bins=200)
    lay.qb_histogram(x[77:].contiguous(), n_bins=200, hist=parts)
    again = lay.qb_histogram(x, n_bins=200)
    assert torch.equal(whole, parts) and torch.equal(whole, again)


@pytest.mark.parametrize("E,k,bins", [(12, 3, 1000), (5, 4, 7), (896, 16, 1000), (70, 1, 1)])
def test_qb_readout_on_seeded_counts(E, k, bins):
    """The readout alone, on counts drawn by a seeded generator (both sides read the same
    integers), including empty bins, a single bin and E = k + 1."""
    rng = np.random.default_rng(1000 + E + bins)
    T = 3000
    hist = np.zeros((E, bins), dtype=np.int32)
    for e in range(E):
        p = rng.dirichlet(np.full(bins, 0.3))
        hist[e] = rng.multinomial(T, p)
    bias = rng.normal(0, 0.02, E).astype(np.float32)
    cfg = moe.config_from(synth.TOY)
    cfg.n_experts, cfg.top_k = E, k
    out = torch.empty(E, dtype=torch.float32, device=DEV)
    b_dev = torch.from_numpy(bias).to(DEV)
    h_dev = torch.from_numpy(hist).to(DEV)
    import ctypes
    st = moe.lib().moe_qb_readout(ctypes.byref(cfg), b_dev.data_ptr(), bins, h_dev.data_ptr(), T,
                                  out.data_ptr(), None)
    assert st == moe.MOE_OK
    torch.cuda.synchronize()
    ref = O.qb_readout(hist, bias, T, k)
    lo, hi = (float(v) for v in O.qb_range(bias))
    got = out.cpu().numpy().astype(np.float64)
    assert np.max(np.abs(got - ref)) <= 1e-5 * (hi - lo), np.max(np.abs(got - ref))


@pytest.mark.parametrize("T", [64, 8192])
def test_qb_step_on_k3_batches(T):
    """The full K3 router (E = 896, k = 16, 1000 bins) at decode and prefill batch sizes:
    counts against the oracle, and the new biases within one bin width of the exact order
    statistic."""
    cfg = synth.K3_DECODE_B1
    lay, dense = device_layer(cfg)
    x = synth.tokens(cfg, batch=7, T=T)
    log(f"[qb k3] T={T}")
    h_dev = lay.qb_histogram(to_dev(x), n_bins=1000)
    nb = lay.qb_readout(h_dev, T).cpu().numpy().astype(np.float64)
    h = h_dev.cpu().numpy()
    s = oracle_scores(cfg, dense, x)
    frac = check_counts(h, s, dense.bias, cfg.k, 1000)
    exact = O.qb_exact(s, dense.bias, cfg.k)
    lo, hi = (float(v) for v in O.qb_range(dense.bias))
    w = (hi - lo) / 1000
    err = np.max(np.abs(nb - exact))
    log(f"[qb k3] T={T}: {frac:.4%} away from bin edges; max |new b - exact| = {err:.3e} "
        f"(bin width {w:.3e})")
    assert err <= w + 2 * TOL_R
    assert abs(float(nb.mean())) < 1e-6
    # time of one QB step (histogram with its router launch, and the readout)
    xd = to_dev(x)
    for _ in range(2):
        lay.qb_readout(lay.qb_histogram(xd, n_bins=1000), T)
    torch.cuda.synchronize()
    e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    hh = torch.zeros((cfg.E, 1000), dtype=torch.int32, device=DEV)
    e[0].record()
    for _ in range(10):
        lay.qb_histogram(xd, n_bins=1000, hist=hh)
    e[1].record()
    for _ in range(10):
        lay.qb_readout(hh, T)
    e[2].record()
    torch.cuda.synchronize()
    log(f"[qb k3] T={T}: histogram (router launch + counts) {e[0].elapsed_time(e[1]) * 100:.1f} us, "
        f"readout {e[1].elapsed_time(e[2]) * 100:.1f} us")
