"""Pins of the oracle on the K2-style non-latent block (CPU only): the K2 block card's
parameter counts, the FP8 E4M3 block-128 dequantisation, the synthetic FP8 weights, a
scalar brute force of a tiny non-latent SwiGLU layer with the 2.827 gate scale, and the
Zipf(1.2) router bias of the 1024-token workload."""
import math

import numpy as np
import pytest

import oracle as O
import synth
from synth import calibrate_zipf as cz

K2 = synth.K2_MOE_1024_ZIPF
TINY_K2 = synth.LayerConfig(name="tiny_k2", d=160, l=0, E=6, k=2, m=48, ms=32, tokens=3,
                            seed=4242, expert_fmt="fp8b128", act="swiglu", route_scale=2.827,
                            use_norm=False, bias_kind="uniform", bias_a=-0.01, bias_b=0.01)


def test_k2_parameter_counts_match_block_card_table():
    s = synth.param_shapes(K2)
    router = np.prod(s["router"]) + np.prod(s["bias"])
    expert = (np.prod(s["expert_gu"]) + np.prod(s["expert_down"])) // K2.E
    shared = np.prod(s["shared_gu"]) + np.prod(s["shared_down"])
    assert router == 2_752_896
    assert expert == 44_040_192 == shared
    assert router + K2.E * expert + shared == 16_958_226_816
    assert "w_down_latent" not in s and "norm_gamma" not in s


def test_fp8_block128_dequant_on_a_hand_built_matrix():
    codes = np.zeros((130, 200), np.uint8)
    scales = np.array([[0.5, 4.0], [2.0, 0.25]], np.float32)
    codes[0, 0] = 0x38          # 1.0 in block (0, 0)
    codes[5, 150] = 0xB8        # -1.0 in block (0, 1)
    codes[129, 0] = 0x7E        # 448 in block (1, 0)
    codes[128, 199] = 0x01      # 2^-9 in block (1, 1)
    w = O.dequant_fp8_block128(codes, scales)
    assert w.shape == (130, 200)
    assert w[0, 0] == 0.5 and w[5, 150] == -4.0 and w[129, 0] == 896.0
    assert w[128, 199] == 0.25 * 2.0 ** -9
    assert np.count_nonzero(w) == 4


def test_synthetic_fp8_experts_fill_each_block_and_have_the_target_spread():
    sl = synth.expert_slice(TINY_K2.with_(d=300, m=200), 0, 2)
    for codes, scales in ((sl.gu, sl.gu_scale), (sl.down, sl.down_scale)):
        v = O.e4m3_decode(codes)
        assert not np.isnan(v).any()
        rows, cols = codes.shape[1:]
        for b in np.ndindex(scales.shape[1:]):
            blk = v[:, 128 * b[0]:128 * (b[0] + 1), 128 * b[1]:128 * (b[1] + 1)]
            assert np.all(np.max(np.abs(blk), axis=(1, 2)) == 448.0)    # amax lands on 448
        w = O.dequant_fp8_block128(codes, scales)
        assert abs(w.std() / 0.02 - 1) < 0.05


def _brute_force_nonlatent(cfg, dense, sl, x_bits):
    """Scalar loops over the [out, in] storage of a non-latent SwiGLU block."""
    f = O.bf16_to_f64
    Wr, Sg, Sd = f(dense.router), f(dense.shared_gu), f(dense.shared_down)
    lut = [O.e4m3_decode(np.array([c]))[0] for c in range(256)]

    def deq(codes, scales):
        out = np.zeros(codes.shape)
        for idx in np.ndindex(codes.shape):
            e, r, c = idx
            out[idx] = lut[int(codes[idx])] * float(scales[e, r // 128, c // 128])
        return out
    EGU, EDN = deq(sl.gu, sl.gu_scale), deq(sl.down, sl.down_scale)
    sig = lambda z: 1 / (1 + math.exp(-z)) if z >= 0 else math.exp(z) / (1 + math.exp(z))  # noqa: E731
    X = f(x_bits)
    T, d = X.shape
    out = np.zeros((T, d))
    for t in range(T):
        xt = X[t]
        s = [sig(sum(xt[c] * Wr[e, c] for c in range(d))) for e in range(cfg.E)]
        kap = [float(np.float32(s[e]) + np.float32(dense.bias[e])) for e in range(cfg.E)]
        sel = sorted(range(cfg.E), key=lambda e: (-kap[e], e))[: cfg.k]
        tot = sum(s[e] for e in sel)
        for e in sel:
            h = []
            for i in range(cfg.m):
                g = sum(xt[c] * EGU[e, i, c] for c in range(d))
                u = sum(xt[c] * EGU[e, cfg.m + i, c] for c in range(d))
                h.append(g * sig(g) * u)
            for r in range(d):
                out[t, r] += cfg.route_scale * s[e] / tot * sum(h[i] * EDN[e, r, i] for i in range(cfg.m))
        hs = []
        for i in range(cfg.ms):
            g = sum(xt[c] * Sg[i, c] for c in range(d))
            u = sum(xt[c] * Sg[cfg.ms + i, c] for c in range(d))
            hs.append(g * sig(g) * u)
        for r in range(d):
            out[t, r] += sum(hs[i] * Sd[r, i] for i in range(cfg.ms))
    return out


def test_nonlatent_fp8_layer_against_scalar_brute_force():
    cfg = TINY_K2
    dense = synth.dense_weights(cfg)
    sl = synth.expert_slice(cfg, 0, cfg.E)
    x = synth.tokens(cfg)
    r = O.forward(O.OracleLayer.from_synth(cfg, dense), x)
    assert np.allclose(r.G.sum(axis=1), 2.827, rtol=0, atol=1e-12)
    bf = _brute_force_nonlatent(cfg, dense, sl, x)
    assert np.max(np.abs(r.delta - bf)) <= 1e-12 * np.max(np.abs(bf))


def test_k2_zipf_bias_targets_and_held_out_load():
    pi, rank, c = cz.zipf_targets(K2.E, K2.k, cz.K2_ZIPF_S, np.random.default_rng(cz.PERM_SEED))
    assert abs(pi.sum() - 8) < 1e-9 and abs(c - 2.279) < 1e-3 and int((pi >= 1).sum()) == 1
    dense = synth.dense_weights(K2)
    x = synth.tokens(K2, batch=1000)          # the bench's first batch, held out
    s = O.router_scores(O.bf16_to_f64(x), O.bf16_to_f64(dense.router))
    idx, _, _ = O.select_and_weight(s, dense.bias, K2.k, K2.route_scale)
    load = np.bincount(idx.reshape(-1), minlength=K2.E)
    by_rank = load[np.argsort(rank)]
    assert by_rank[0] == K2.tokens                  # the saturated expert takes every token
    D = int((load > 0).sum())
    assert 355 <= D <= 384, D                       # E[D] ~ 369 under the capped Zipf(1.2)
