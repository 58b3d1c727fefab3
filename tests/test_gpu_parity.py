"""GPU parity: the HIP path through the C ABI against the float64 CPU oracle.

The rule (indices on clear margins, gate weights to 1e-6, Delta within rel-L2 2e-3 and
max-abs 1e-2 rms, near ties and MXFP8 boundary decisions compared with the oracle taking the
GPU's choice) is implemented once in tests/parity.py.
"""
import functools
import time

import numpy as np
import pytest
import torch

import oracle as O
import parity as P
import sparse_moe_layer_amd as moe
import synth

pytestmark = pytest.mark.gpu

MARGIN = P.MARGIN
DEV = torch.device("cuda:0")

TINY = synth.LayerConfig(name="tiny_mxfp4", d=64, l=32, E=8, k=2, m=32, ms=64, tokens=5,
                         seed=77, expert_fmt="mxfp4", bias_kind="uniform", bias_a=-0.01,
                         bias_b=0.01, e8m0_lo=125, e8m0_hi=128)
# widths that leave ragged chunks in every kernel (d/8 = 25, l/8 = 12, E not a multiple of 64)
RAGGED = synth.LayerConfig(name="ragged_mxfp4", d=200, l=96, E=70, k=5, m=64, ms=40, tokens=37,
                           seed=91, expert_fmt="mxfp4", bias_kind="uniform", bias_a=-0.01,
                           bias_b=0.01, e8m0_lo=122, e8m0_hi=127)


def log(msg):
    print(msg, flush=True)


@functools.lru_cache(maxsize=4)
def device_layer(cfg):
    log(f"[upload] {cfg.name}")
    dense = synth.dense_weights(cfg)
    lay = moe.Layer.upload(moe.config_from(cfg), dense, lambda a, b: synth.expert_slice(cfg, a, b),
                           cfg.E, device=DEV, chunk=32)
    torch.cuda.synchronize()
    return lay, dense


@functools.lru_cache(maxsize=4)
def oracle_layer(cfg):
    _, dense = device_layer(cfg)
    return O.OracleLayer.from_synth(cfg, dense)


def to_dev(x):
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(DEV)


def run(lay, x):
    d, i, w = lay.forward(to_dev(x))
    torch.cuda.synchronize()
    return d.cpu().numpy().astype(np.float64), i.cpu().numpy(), w.cpu().numpy().astype(np.float64)


def assert_routing(idx, ridx, kap, margin):
    return P.routing(idx, ridx, kap, margin, log)


def gpu_xc_codes(lay, T):
    """The MX code rows and scale bytes of x^c that the last mx forward of `lay` left in its
    workspace (numpy uint8 [T, 128 ks] in mx8 or [T, 64 ks] in mx4, and [T, 4 ks])."""
    inter = lay.intermediates(T)
    return inter["xq"].cpu().numpy(), inter["xs"].cpu().numpy()


def check(cfg, x, delta, idx, w, rows=None, precision=None, ref=None, bars=True, xcq=None):
    """Compare GPU outputs for tokens `rows` of x against the oracle in `precision` (the
    layer's own profile by default; `ref`: that oracle's result for those rows) by the rule
    of tests/parity.py.  xcq: the GPU's MX x^c (code rows, scale bytes) of all of x, in an
    mx profile.  Returns (rel-L2, max-abs / rms, the oracle's result)."""
    rows = np.arange(x.shape[0]) if rows is None else np.asarray(rows)
    r = P.compare(oracle_layer(cfg), x[rows], delta[rows], idx[rows], w[rows], precision=precision,
                  ref=ref, xcq=None if xcq is None else (xcq[0][rows], xcq[1][rows]), bars=bars,
                  log=log)
    return r["rel_l2"], r["max_abs_over_rms"], r["ref"]


def test_toy_layer_full():
    cfg = synth.TOY
    lay, _ = device_layer(cfg)
    x = synth.tokens(cfg)
    delta, idx, w = run(lay, x)
    rel, _, ref = check(cfg, x, delta, idx, w)
    assert rel < 1e-5        # fp32 activations throughout: far inside the bar
    inter = {k: v.cpu().numpy().astype(np.float64) for k, v in lay.intermediates(cfg.tokens).items()}
    for name, want in (("xc", ref.xc), ("u", ref.u), ("hs", None)):
        if want is None:
            OL = oracle_layer(cfg)
            xf = O.bf16_to_f64(x)
            g = xf @ OL.shared_gu[: cfg.ms].T
            u = xf @ OL.shared_gu[cfg.ms:].T
            want = O.situ(g, u)
        got = inter[name]
        assert np.linalg.norm(got - want) <= 1e-5 * np.linalg.norm(want), name


def test_toy_layer_is_deterministic():
    cfg = synth.TOY
    lay, _ = device_layer(cfg)
    x = to_dev(synth.tokens(cfg, batch=3))
    a = [t.cpu().clone() for t in lay.forward(x)]
    b = [t.cpu().clone() for t in lay.forward(x)]
    for p, q in zip(a, b):
        assert torch.equal(p, q)


@pytest.mark.parametrize("T", [1, 2, 3, 5, 16, 33])
def test_tiny_mxfp4_ragged_token_counts(T):
    cfg = TINY.with_(tokens=T)
    lay, _ = device_layer(TINY)
    x = synth.tokens(cfg, batch=T)
    check(TINY, x, *run(lay, x))


def test_ragged_widths_and_expert_count():
    cfg = RAGGED
    lay, _ = device_layer(cfg)
    x = synth.tokens(cfg)
    check(cfg, x, *run(lay, x))


def test_ragged_router_tiles_at_600_tokens():
    """From 512 tokens on, the token-tiled router gives each wavefront two tile rows.  Here
    70 experts fill 5 of the 8 tile rows of its one group (the dead rows read tile row 0
    and are not written), and d = 1800 gives two logit planes whose last K-step is partial.
    Indices of every token through moe_route and through the forward (they must agree),
    and Delta of every token against the oracle."""
    cfg = RAGGED.with_(name="ragged_wide_router", d=1800, tokens=600)
    lay, _ = device_layer(cfg)
    x = synth.tokens(cfg)
    ri, rw = lay.route(to_dev(x))
    torch.cuda.synchronize()
    delta, idx, w = run(lay, x)
    assert np.array_equal(ri.cpu().numpy(), idx)
    assert np.array_equal(rw.cpu().numpy().astype(np.float64), w)
    check(cfg, x, delta, idx, w)


def test_all_experts_selected():
    cfg = TINY.with_(name="tiny_k_eq_E", k=8)
    lay, _ = device_layer(cfg)
    x = synth.tokens(cfg)
    delta, idx, w = run(lay, x)
    assert np.array_equal(np.sort(idx, axis=1), np.tile(np.arange(8), (cfg.tokens, 1)))
    check(cfg, x, delta, idx, w)


@pytest.mark.parametrize("variant", ["swiglu", "no_norm", "no_shared", "bf16_experts"])
def test_layer_variants(variant):
    kw = {"swiglu": dict(act="swiglu"), "no_norm": dict(use_norm=False),
          "no_shared": dict(ms=0), "bf16_experts": dict(expert_fmt="bf16")}[variant]
    cfg = TINY.with_(name=f"tiny_{variant}", **kw)
    lay, _ = device_layer(cfg)
    x = synth.tokens(cfg)
    check(cfg, x, *run(lay, x))


def test_zero_tokens_is_a_no_op():
    lay, _ = device_layer(TINY)
    x = torch.empty((0, TINY.d), dtype=torch.int16, device=DEV)
    d, i, w = lay.forward(x)
    torch.cuda.synchronize()
    assert d.shape == (0, TINY.d) and i.shape == (0, TINY.k)


# 3001 x 16 and 5000 x 8: 188 and 157 dispatch chunks, past the scan's groups of 32 with a
# ragged last group
@pytest.mark.parametrize("T,E,k", [(1, 896, 16), (37, 896, 16), (100, 64, 2), (300, 70, 5),
                                   (3001, 896, 16), (5000, 384, 8)])
def test_dispatch_bit_exact(T, E, k):
    rng = np.random.default_rng(T * 1000 + E)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    cfg = synth.TOY.with_(E=E, k=k)
    lay = moe.Layer(moe.config_from(cfg), torch.empty(1, device=DEV), None, None)
    got = [t.cpu().numpy() for t in lay.dispatch(torch.from_numpy(idx).to(DEV))]
    want = O.dispatch(idx, E)
    for g, wv, name in zip(got, want, ("counts", "offsets", "perm", "inv")):
        assert np.array_equal(g, wv), name


def k3_layer():
    return device_layer(synth.K3_DECODE_B1)


def test_k3_decode_b1_layer():
    cfg = synth.K3_DECODE_B1
    lay, _ = k3_layer()
    for b in range(3):
        x = synth.tokens(cfg, batch=b)
        log(f"[k3 b1] batch {b}")
        rel, _, _ = check(cfg, x, *run(lay, x))
        assert rel < 1e-4


def test_k3_decode_b64_all_tokens():
    """The K3 layer at 64 tokens under near-uniform routing (about 600 distinct experts,
    units of one or two positions): indices, weights and Delta of every token."""
    cfg = synth.K3_DECODE_B1
    lay, _ = k3_layer()
    x = synth.tokens(cfg, batch=100, T=64)
    delta, idx, w = run(lay, x)
    log(f"[k3 b64] distinct experts {len(np.unique(idx))}")
    rel, _, _ = check(cfg, x, delta, idx, w)
    assert rel < 1e-4
    # per-token independence: the same tokens alone or in twos and threes (the few-token
    # launches: router rows in the IN launch, W_shared_down partial sums in the down launch)
    # give the same Delta bits as in the token-tiled batch
    for lo, hi in ((21, 22), (10, 12), (40, 43)):
        d1, i1, w1 = run(lay, x[lo:hi])
        assert np.array_equal(i1, idx[lo:hi]) and np.array_equal(d1, delta[lo:hi]), (lo, hi)
    # the route's wait for the router workgroups ended by their arrivals (the counter is back
    # at zero, and no wait reached its spin limit)
    ctrl = lay.workspace(1)[:256].view(torch.int32).cpu().numpy()
    assert ctrl[32] == 0 and ctrl[33] == 0, ctrl[32:34]


def test_k3_decode_b64_zipf_layer():
    """The Zipf-loaded B=64 layer: two experts take every token, so their 64 positions
    are split over several units of the expert launches, next to many single-token units.
    Indices, weights and Delta of every token."""
    cfg = synth.K3_DECODE_B64_ZIPF
    lay, _ = device_layer(cfg)
    x = synth.tokens(cfg, batch=1000)
    log(f"[k3 zipf] T={x.shape[0]}")
    delta, idx, w = run(lay, x)
    OL = oracle_layer(cfg)
    s = O.router_scores(O.bf16_to_f64(x), OL.router)
    ridx, G, margin = O.select_and_weight(s, OL.bias, cfg.k)
    assert_routing(idx, ridx, O.selection_kappa(s, OL.bias, cfg.k), margin)
    load = np.bincount(idx.reshape(-1), minlength=cfg.E)
    assert int((load == x.shape[0]).sum()) == 2
    log(f"[k3 zipf] distinct experts {int((load > 0).sum())}")
    rel, _, _ = check(cfg, x, delta, idx, w)      # every token
    assert rel < 1e-4
    d1, i1, w1 = run(lay, x[31:32])
    assert np.array_equal(i1[0], idx[31]) and np.array_equal(d1[0], delta[31])


def test_step_ranges_and_timed_forward_match_the_forward():
    cfg = TINY.with_(tokens=3)
    lay, _ = device_layer(TINY)
    x = to_dev(synth.tokens(cfg, batch=7))
    ref = [t.cpu().clone() for t in lay.forward(x)]
    T = x.shape[0]
    ws = torch.zeros(moe.workspace_size(lay.cfg, T), dtype=torch.uint8, device=DEV)
    d = torch.empty((T, TINY.d), dtype=torch.float32, device=DEV)
    i = torch.empty((T, TINY.k), dtype=torch.int32, device=DEV)
    w = torch.empty((T, TINY.k), dtype=torch.float32, device=DEV)
    lay.forward_steps(x, 0, 4, d, i, w, ws)
    lay.forward_steps(x, 4, len(moe.STEPS), d, i, w, ws)
    for p, q in zip(ref, (d, i, w)):
        assert torch.equal(p, q.cpu())
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so.7")
    evs = []
    for _ in range(len(moe.STEPS) + 1):
        e = ctypes.c_void_p()
        assert hip.hipEventCreate(ctypes.byref(e)) == 0
        evs.append(e.value)
    d2, i2, w2 = torch.empty_like(d), torch.empty_like(i), torch.empty_like(w)
    lay.forward_timed(x, evs, d2, i2, w2)
    torch.cuda.synchronize()
    for p, q in zip(ref, (d2, i2, w2)):
        assert torch.equal(p, q.cpu())
    for e in evs:
        hip.hipEventDestroy(ctypes.c_void_p(e))


# ---- the mx8 profile (MXFP8 expert inputs on the scaled FP8 x FP4 matrix cores) --------
# Compared with the oracle run in the same profile; the kernels and the oracle take each
# rounding decision on their own fp32 / float64 values, so a value within rounding
# distance of an E4M3 or bf16 midpoint may round to the neighbour: rare, and far inside
# the bar.

TINY_MX8 = TINY.with_(name="tiny_mx8", precision="mx8")
RAGGED_MX8 = RAGGED.with_(name="ragged_mx8", precision="mx8")


@pytest.mark.parametrize("T", [1, 5, 33, 100])
def test_mx8_tiny_token_counts(T):
    lay, _ = device_layer(TINY_MX8)
    x = synth.tokens(TINY_MX8, batch=T, T=T)
    out = run(lay, x)
    check(TINY_MX8, x, *out, xcq=gpu_xc_codes(lay, T))


def test_mx8_ragged_widths_and_expert_count():
    lay, _ = device_layer(RAGGED_MX8)
    x = synth.tokens(RAGGED_MX8)
    out = run(lay, x)
    check(RAGGED_MX8, x, *out, xcq=gpu_xc_codes(lay, x.shape[0]))


@pytest.mark.parametrize("variant", ["swiglu", "no_norm", "no_shared"])
def test_mx8_layer_variants(variant):
    kw = {"swiglu": dict(act="swiglu"), "no_norm": dict(use_norm=False), "no_shared": dict(ms=0)}[variant]
    cfg = TINY_MX8.with_(name=f"tiny_mx8_{variant}", tokens=20, **kw)
    lay, _ = device_layer(cfg)
    x = synth.tokens(cfg)
    out = run(lay, x)
    check(cfg, x, *out, xcq=gpu_xc_codes(lay, x.shape[0]))


def test_mx8_is_deterministic_and_token_independent():
    lay, _ = device_layer(TINY_MX8)
    x = to_dev(synth.tokens(TINY_MX8, batch=11, T=70))
    a = [t.cpu().clone() for t in lay.forward(x)]
    b = [t.cpu().clone() for t in lay.forward(x)]
    for p, q in zip(a, b):
        assert torch.equal(p, q)
    one = [t.cpu().clone() for t in lay.forward(x[40:41].contiguous())]
    assert torch.equal(one[1][0], a[1][40]) and torch.equal(one[0][0], a[0][40])


def test_k3_prefill_8192_all_tokens_both_profiles():
    """The K3 layer at prefill size, every one of the 8192 tokens (all 86 token tiles of the
    dense products, every unit of the expert launches):
      - the mx8 launches against the oracle in the mx8 profile (the bars);
      - the fp32 launches (token-tiled) on the same packed weights against the plain
        oracle (the bars, unmodified);
      - informational: the mx8 Delta against the plain oracle (the cost of the declared
        MXFP8 / bf16 rounding points)."""
    cfg = synth.K3_PREFILL_8K
    lay, _ = device_layer(cfg)
    x = synth.tokens(cfg, batch=0)
    log(f"[k3 prefill] T={x.shape[0]} mx8 launches")
    delta, idx, w = run(lay, x)
    assert np.all(np.isfinite(delta))
    xcq = gpu_xc_codes(lay, x.shape[0])
    rel, mxr, _ = check(cfg, x, delta, idx, w, xcq=xcq)
    assert rel < 1e-3
    # the same layer through the fp32 launches (only the precision field differs)
    lay32 = moe.Layer(moe.config_from(cfg.with_(precision="fp32")), lay.dense, lay.bias, lay.experts)
    log("[k3 prefill] fp32 launches")
    d32, i32, w32 = run(lay32, x)
    del lay32
    rel32, mxr32, ref32 = check(cfg, x, d32, i32, w32, precision="fp32")
    assert rel32 < 1e-4
    # informational: the mx8 profile's distance from the plain oracle (near-tie tokens
    # against the oracle on the mx8 launches' own selection)
    relq, mxq, _ = check(cfg, x, delta, idx, w, precision="fp32", ref=ref32, bars=False)
    log(f"[k3 prefill] mx8 launches against the plain (fp32) oracle: rel-L2 {relq:.3e} "
        f"max-abs/rms {mxq:.3e} (informational; the declared rounding points)")
    assert relq < 0.1


def test_k3_ep_share_all_tokens():
    """One GPU's expert-parallel share (112 experts, about 1,170 rows each) in the mx8
    profile: indices, weights and Delta of all 8192 tokens (every unit of 64 positions of
    every expert, every token tile)."""
    cfg = synth.K3_EP_SHARE
    lay, _ = device_layer(cfg)
    x = synth.tokens(cfg, batch=0)
    log(f"[ep share] T={x.shape[0]} E={cfg.E}")
    delta, idx, w = run(lay, x)
    counts = np.bincount(idx.reshape(-1), minlength=cfg.E)
    log(f"[ep share] rows per expert min {counts.min()} max {counts.max()}")
    assert counts.sum() == cfg.tokens * cfg.k and counts.min() > 0
    assert np.all(np.isfinite(delta))
    rel, mxr, _ = check(cfg, x, delta, idx, w, xcq=gpu_xc_codes(lay, x.shape[0]))
    assert rel < 1e-3


# ---- the mx4 profile (MXFP4 expert inputs on the scaled FP4 x FP4 matrix cores) ---------
# The same rule against the oracle in the mx4 profile.  E2M1 keeps two significant bits, so a
# value of h that the GPU rounds to the other neighbour moves its product by up to a quarter
# of the block's largest value: rare (h agrees to about 1e-6), and inside the bar.

TINY_MX4 = TINY.with_(name="tiny_mx4", precision="mx4")
RAGGED_MX4 = RAGGED.with_(name="ragged_mx4", precision="mx4")


@pytest.mark.parametrize("T", [1, 5, 33, 100])
def test_mx4_tiny_token_counts(T):
    lay, _ = device_layer(TINY_MX4)
    x = synth.tokens(TINY_MX4, batch=T, T=T)
    out = run(lay, x)
    check(TINY_MX4, x, *out, xcq=gpu_xc_codes(lay, T))


@pytest.mark.parametrize("variant", ["ragged", "swiglu", "no_norm", "no_shared"])
def test_mx4_widths_and_layer_variants(variant):
    if variant == "ragged":
        cfg = RAGGED_MX4
    else:
        kw = {"swiglu": dict(act="swiglu"), "no_norm": dict(use_norm=False), "no_shared": dict(ms=0)}[variant]
        cfg = TINY_MX4.with_(name=f"tiny_mx4_{variant}", tokens=20, **kw)
    lay, _ = device_layer(cfg)
    x = synth.tokens(cfg)
    out = run(lay, x)
    check(cfg, x, *out, xcq=gpu_xc_codes(lay, x.shape[0]))


def test_mx4_is_deterministic_and_token_independent():
    lay, _ = device_layer(TINY_MX4)
    x = to_dev(synth.tokens(TINY_MX4, batch=11, T=70))
    a = [t.cpu().clone() for t in lay.forward(x)]
    b = [t.cpu().clone() for t in lay.forward(x)]
    for p, q in zip(a, b):
        assert torch.equal(p, q)
    one = [t.cpu().clone() for t in lay.forward(x[40:41].contiguous())]
    assert torch.equal(one[1][0], a[1][40]) and torch.equal(one[0][0], a[0][40])


def test_k3_prefill_8192_mx4_sampled_tokens():
    """The K3 layer at prefill size in the mx4 profile: all 8192 tokens through the launches,
    every 8th token (12 of each 96-token tile of the dense products) against the oracle in
    the mx4 profile (the bars), and, informational, against the plain oracle."""
    cfg = synth.K3_PREFILL_8K
    lay8, _ = device_layer(cfg)
    # the same packed weights through the mx4 launches (only the precision field differs)
    lay = moe.Layer(moe.config_from(synth.K3_PREFILL_8K_MX4), lay8.dense, lay8.bias, lay8.experts)
    x = synth.tokens(cfg, batch=0)
    log(f"[k3 prefill mx4] T={x.shape[0]}")
    delta, idx, w = run(lay, x)
    assert np.all(np.isfinite(delta))
    xcq = gpu_xc_codes(lay, x.shape[0])
    del lay
    rows = np.arange(0, x.shape[0], 8)
    check(cfg, x, delta, idx, w, rows=rows, precision="mx4", xcq=xcq)
    relq, mxq, _ = check(cfg, x, delta, idx, w, rows=rows, precision="fp32", bars=False)
    log(f"[k3 prefill mx4] against the plain (fp32) oracle: rel-L2 {relq:.3e} max-abs/rms "
        f"{mxq:.3e} (informational; the declared rounding points)")
    assert relq < 0.3


# ---- the K2-style non-latent block: FP8 E4M3 block-128 experts, SwiGLU, gate scale 2.827 --

TINY_K2 = synth.LayerConfig(name="tiny_k2", d=160, l=0, E=6, k=2, m=48, ms=32, tokens=5,
                            seed=4242, expert_fmt="fp8b128", act="swiglu", route_scale=2.827,
                            use_norm=False, bias_kind="uniform", bias_a=-0.01, bias_b=0.01)


@pytest.mark.parametrize("T", [1, 3, 5, 33, 100])
def test_nonlatent_fp8_tiny_token_counts(T):
    lay, _ = device_layer(TINY_K2)
    x = synth.tokens(TINY_K2, batch=T, T=T)
    rel, _, _ = check(TINY_K2, x, *run(lay, x))
    assert rel < 1e-5


@pytest.mark.parametrize("fmt", ["mxfp4", "bf16"])
def test_nonlatent_mxfp4_and_bf16_experts_long_units(fmt):
    """Without a latent the token-tiled gate/up reads one bf16 row per position: every
    weight format, with units long enough for the K-step kernel (T * k / E ~ 33)."""
    cfg = TINY_K2.with_(name=f"tiny_k2_{fmt}", expert_fmt=fmt, m=64, tokens=100)
    lay, _ = device_layer(cfg)
    x = synth.tokens(cfg)
    rel, _, _ = check(cfg, x, *run(lay, x))
    assert rel < 1e-5
    one = [t.cpu().clone() for t in lay.forward(to_dev(x[57:58]))]
    full = [t.cpu().clone() for t in lay.forward(to_dev(x))]
    assert torch.equal(one[0][0], full[0][57]) and torch.equal(one[1][0], full[1][57])


def test_latent_layer_with_fp8_block_experts():
    cfg = TINY.with_(name="tiny_latent_fp8", expert_fmt="fp8b128", d=200, l=136, m=40, tokens=9)
    lay, _ = device_layer(cfg)
    x = synth.tokens(cfg)
    rel, _, _ = check(cfg, x, *run(lay, x))
    assert rel < 1e-5


def test_k2_block_1024_all_tokens():
    """The K2-style block at 1024 tokens under the Zipf(1.2) load: indices, weights and
    Delta of every token (all 16 token tiles; every token also routes to the saturated
    expert, whose 1024 positions fill 16 units of 64)."""
    cfg = synth.K2_MOE_1024_ZIPF
    lay, _ = device_layer(cfg)
    x = synth.tokens(cfg, batch=0)
    log(f"[k2] T={x.shape[0]}")
    delta, idx, w = run(lay, x)
    load = np.bincount(idx.reshape(-1), minlength=cfg.E)
    assert int((load == x.shape[0]).sum()) >= 1
    assert np.all(np.isfinite(delta))
    rel, _, _ = check(cfg, x, delta, idx, w)
    assert rel < 1e-4
    # few-token launches on the same layer: the same Delta bits for a token alone
    d1, i1, w1 = run(lay, x[511:512])
    assert np.array_equal(i1[0], idx[511]) and np.array_equal(d1[0], delta[511])
