"""Pins of the oracle's "mx8" precision profile (CPU only).

The profile inserts the rounding points of a compute-bound path: MXFP8-E4M3 conversion
of the experts' input x^c and hidden h (the walkthrough's deployment recipe: MXFP4
weights, MXFP8 activations), bf16 rounding of u_hat and h_s.  The element format and
the conversion rule are the OCP 8-bit floating point (E4M3) and OCP MX v1.0 definitions;
the pages only name the formats.  Independent references used here: torch's
float8_e4m3fn and bfloat16 conversions (library routines), hand-computed values, and a
scalar brute force of the layer.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
import oracle.moe_oracle as OM
import synth

TINY = synth.LayerConfig(name="tiny_mx8", d=64, l=64, E=8, k=2, m=64, ms=64, tokens=5,
                         seed=1234, expert_fmt="mxfp4", bias_kind="uniform", bias_a=-0.01,
                         bias_b=0.01, e8m0_lo=125, e8m0_hi=128, precision="mx8")


def test_e4m3_all_256_codes():
    v = O.e4m3_decode(np.arange(256))
    nan = np.isnan(v)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert v[0x00] == 0.0 and v[0x80] == 0.0 and math.copysign(1, v[0x80]) < 0
    assert v[0x7E] == 448.0 == O.E4M3_MAX
    assert v[0x01] == 2.0 ** -9 and v[0x08] == 2.0 ** -6 and v[0x38] == 1.0
    pos = v[:0x7F]
    assert np.all(np.diff(pos) > 0)                      # codes 0..126 increase
    assert np.array_equal(v[0x80:0xFF], -v[:0x7F])       # sign bit
    for e in range(-6, 9):     # 8 values per normal binade; the top one loses 480 to NaN
        assert np.sum((pos >= 2.0 ** e) & (pos < 2.0 ** (e + 1))) == (8 if e < 8 else 7)
    lib = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.nan_to_num(lib, nan=-1e9), np.nan_to_num(v, nan=-1e9))


def test_round_e4m3_matches_torch_float8_on_fp32_inputs():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(100000) * np.exp2(rng.integers(-14, 9, 100000))).astype(np.float32)
    x = np.clip(x, -448, 448)
    lib = torch.from_numpy(x).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(O.round_e4m3(x.astype(np.float64)), lib)


def test_round_e4m3_ties_and_saturation():
    r = O.round_e4m3
    assert r(1 + 1 / 16) == 1.0 and r(1 + 3 / 16) == 1.25      # halves go to the even mantissa
    assert r(-(1 + 3 / 16)) == -1.25
    assert r(2 ** -10) == 0.0 and r(3 * 2 ** -11) == 2 ** -9   # subnormal spacing 2^-9
    assert r(1.97) == 2.0                                       # rounding into the next binade
    assert r(464.0) == 448.0 and r(465.0) == 448.0 and r(1e9) == 448.0 and r(-1e9) == -448.0


def test_mx8_scale_rule_on_hand_computed_blocks():
    v = np.zeros(64)
    v[0], v[1], v[2] = 1.0, 0.3, -0.6     # block 0: amax 1 -> X = 0 - 8
    v[32] = 1.9                            # block 1: amax 1.9 -> X = -8, 1.9*256 = 486.4 saturates
    v[33] = 1.0
    deq, q, sc = O.quantize_mx8(v)
    assert sc.tolist() == [119, 119]
    # 0.3 * 256 = 76.8 lies in [64, 128): spacing 8, nearest 80; 0.6 * 256 = 153.6 lies in
    # [128, 256): spacing 16, nearest 160
    assert deq[0] == 1.0 and deq[1] == 80 / 256 and deq[2] == -160 / 256
    assert q[32] == 448.0 and deq[32] == 1.75 and deq[33] == 1.0
    z, _, sz = O.quantize_mx8(np.zeros(32))
    assert sz.tolist() == [0] and np.all(z == 0)
    for k in (-20, -3, 0, 5, 30):          # amax = 2^k exactly: X = k - 8
        _, _, s = O.quantize_mx8(np.full(32, 2.0 ** k))
        assert int(s[0]) == 127 + k - 8


def test_mx8_error_bound_idempotence_and_block_independence():
    rng = np.random.default_rng(9)
    v = rng.standard_normal((50, 256)) * np.exp2(rng.integers(-8, 8, (50, 1)))
    deq, q, sc = O.quantize_mx8(v)
    X = sc.astype(np.int64) - 127
    scale = np.repeat(np.ldexp(1.0, X), 32, axis=-1)
    y = np.abs(v) / scale
    normal = (y >= 2.0 ** -6) & (y <= 448)
    assert np.all(np.abs(deq - v)[normal] <= 2.0 ** -4 * np.abs(v)[normal])
    assert np.all(np.abs(deq - v)[y < 2.0 ** -6] <= 2.0 ** -10 * scale[y < 2.0 ** -6])
    assert np.all(y < 512)                 # the scale puts every block's amax below 2^9
    assert np.array_equal(O.quantize_mx8(deq)[0], deq)
    w = v.copy()
    w[:, 40] *= 3.0                        # block 1 only
    d2 = O.quantize_mx8(w)[0]
    assert np.array_equal(np.delete(d2, np.s_[32:64], axis=1), np.delete(deq, np.s_[32:64], axis=1))


def test_round_bf16_matches_torch_on_fp32_inputs():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(100000) * np.exp2(rng.integers(-60, 60, 100000))).astype(np.float32)
    lib = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(O.round_bf16(x.astype(np.float64)), lib)
    assert O.round_bf16(1 + 2 ** -8) == 1.0 and O.round_bf16(1 + 3 * 2 ** -8) == 1 + 2 ** -6


def test_mx8_profile_inserts_only_its_declared_points(monkeypatch):
    cfg = TINY
    L = O.OracleLayer.from_synth(cfg)
    x = synth.tokens(cfg)
    ref = O.forward(L, x, precision="fp32")
    monkeypatch.setattr(OM, "quantize_mx8", lambda v, block=32: (np.asarray(v, np.float64), None, None))
    monkeypatch.setattr(OM, "round_bf16", lambda v: np.asarray(v, np.float64))
    same = O.forward(L, x, precision="mx8")
    assert np.array_equal(same.delta, ref.delta)


def _brute_force_mx8(cfg, dense, sl, x_bits):
    """Scalar loops with the profile's rounding points; elements through torch's float8 and
    bfloat16 conversions, the block exponent from math.frexp."""
    f = O.bf16_to_f64
    Wr, Wd, Wu, gam = f(dense.router), f(dense.w_down_latent), f(dense.w_up_latent), f(dense.norm_gamma)
    Sg, Sd = f(dense.shared_gu), f(dense.shared_down)
    EGU, EDN = O.dequant_mxfp4(sl.gu, sl.gu_scale), O.dequant_mxfp4(sl.down, sl.down_scale)

    def q8(vals):
        out = []
        for b0 in range(0, len(vals), 32):
            blk = vals[b0:b0 + 32]
            amax = max(abs(v) for v in blk)
            X = (math.frexp(amax)[1] - 1 - 8) if amax > 0 else -127
            y = torch.tensor([min(max(v / 2.0 ** X, -448.0), 448.0) for v in blk], dtype=torch.float64)
            # torch may pass through float32 on the way to float8; the double rounding this
            # allows changes a result only for values within 2^-24 of an E4M3 midpoint
            e = y.to(torch.float8_e4m3fn).to(torch.float64).tolist()
            out += [c * 2.0 ** X for c in e]
        return out

    def bf(v):
        return torch.tensor(v, dtype=torch.float64).to(torch.bfloat16).to(torch.float64).tolist()
    sig = lambda z: 1 / (1 + math.exp(-z)) if z >= 0 else math.exp(z) / (1 + math.exp(z))  # noqa: E731

    def act(g, u):
        return 4 * math.tanh(g / 4) * sig(g) * 25 * math.tanh(u / 25)
    X = f(x_bits)
    T, d = X.shape
    out = np.zeros((T, d))
    for t in range(T):
        xt = X[t]
        s = [sig(sum(xt[c] * Wr[e, c] for c in range(d))) for e in range(cfg.E)]
        kap = [float(np.float32(s[e]) + np.float32(dense.bias[e])) for e in range(cfg.E)]
        sel = sorted(range(cfg.E), key=lambda e: (-kap[e], e))[: cfg.k]
        tot = sum(s[e] for e in sel)
        xc = q8([sum(xt[c] * Wd[r, c] for c in range(d)) for r in range(cfg.l)])
        u = [0.0] * cfg.l
        for e in sel:
            h = q8([act(sum(xc[c] * EGU[e, i, c] for c in range(cfg.l)),
                        sum(xc[c] * EGU[e, cfg.m + i, c] for c in range(cfg.l))) for i in range(cfg.m)])
            for r in range(cfg.l):
                u[r] += s[e] / tot * sum(h[i] * EDN[e, r, i] for i in range(cfg.m))
        rms = math.sqrt(sum(v * v for v in u) / cfg.l + cfg.eps)
        uh = bf([u[r] / rms * gam[r] for r in range(cfg.l)])
        hs = bf([act(sum(xt[c] * Sg[i, c] for c in range(d)), sum(xt[c] * Sg[cfg.ms + i, c] for c in range(d)))
                 for i in range(cfg.ms)])
        for o in range(d):
            out[t, o] = sum(uh[r] * Wu[o, r] for r in range(cfg.l)) + sum(hs[i] * Sd[o, i] for i in range(cfg.ms))
    return out


def test_mx8_layer_against_scalar_brute_force():
    cfg = TINY.with_(tokens=2)
    dense = synth.dense_weights(cfg)
    sl = synth.expert_slice(cfg, 0, cfg.E)
    x = synth.tokens(cfg)
    r = O.forward(O.OracleLayer.from_synth(cfg, dense), x)
    bf = _brute_force_mx8(cfg, dense, sl, x)
    # the two sides agree up to summation order, except where a value lands within
    # rounding distance of an E4M3 or bf16 midpoint; on these inputs none does
    assert np.max(np.abs(r.delta - bf)) <= 1e-10 * np.max(np.abs(bf))


def test_mx8_moves_delta_by_the_expected_quantisation_noise():
    cfg = TINY.with_(tokens=16)
    L = O.OracleLayer.from_synth(cfg)
    x = synth.tokens(cfg)
    a = O.forward(L, x, precision="fp32").delta
    b = O.forward(L, x, precision="mx8").delta
    rel = np.linalg.norm(a - b) / np.linalg.norm(a)
    # E4M3 keeps 4 significant bits: each converted value moves by about 2^-5 relative
    # (uniform rounding error, rms ~ 2^-4 / sqrt(12) x the element), diluted by the sums
    assert 3e-3 < rel < 6e-2, rel
