"""Pins of the oracle's "mx8" and "mx4" precision profiles (CPU only).

The profiles insert the rounding points of a compute-bound path: MX conversion of the
experts' input x^c and hidden h (mx8: MXFP8-E4M3, the walkthrough's deployment recipe of
MXFP4 weights with MXFP8 activations; mx4: MXFP4-E2M1, the weights' own format), bf16
rounding of u_hat and h_s.  The element formats and the conversion rule are the OCP 8-bit
floating point (E4M3) and OCP MX v1.0 definitions; the pages only name the formats.
Independent references used here: torch's float8_e4m3fn and bfloat16 conversions (library
routines), an exhaustive nearest-value search over the E2M1 grid as OCP MX v1.0 prints it
(torch has no conversion to its FP4 type), hand-computed values, and a scalar brute force
of the layer.
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


@pytest.mark.parametrize("profile", ["mx8", "mx4"])
def test_mx_profile_inserts_only_its_declared_points(monkeypatch, profile):
    cfg = TINY
    L = O.OracleLayer.from_synth(cfg)
    x = synth.tokens(cfg)
    ref = O.forward(L, x, precision="fp32")
    monkeypatch.setattr(OM, "quantize_mx", lambda v, elem, block=32, flip=None, scale_flip=None:
                        (np.asarray(v, np.float64), None, None))
    monkeypatch.setattr(OM, "round_bf16", lambda v: np.asarray(v, np.float64))
    same = O.forward(L, x, precision=profile)
    assert np.array_equal(same.delta, ref.delta)


def _e2m1_nearest(y):
    """The E2M1 value nearest y by exhaustive search over the printed grid (ties: the value
    whose code is even, i.e. whose mantissa bit is 0), saturated to +-6."""
    grid = O.E2M1_GRID
    a = min(abs(y), grid[-1])
    best = min(range(8), key=lambda i: (abs(grid[i] - a), i % 2))
    return math.copysign(grid[best], y)


def _brute_force_mx8(cfg, dense, sl, x_bits, elem="e4m3"):
    """Scalar loops with the profile's rounding points; E4M3 elements through torch's float8
    conversion, E2M1 elements by exhaustive search (_e2m1_nearest), bf16 through torch, the
    block exponent from math.frexp."""
    f = O.bf16_to_f64
    Wr, Wd, Wu, gam = f(dense.router), f(dense.w_down_latent), f(dense.w_up_latent), f(dense.norm_gamma)
    Sg, Sd = f(dense.shared_gu), f(dense.shared_down)
    EGU, EDN = O.dequant_mxfp4(sl.gu, sl.gu_scale), O.dequant_mxfp4(sl.down, sl.down_scale)

    def q8(vals):
        out = []
        emax = 8 if elem == "e4m3" else 2
        for b0 in range(0, len(vals), 32):
            blk = vals[b0:b0 + 32]
            amax = max(abs(v) for v in blk)
            X = (math.frexp(amax)[1] - 1 - emax) if amax > 0 else -127
            if elem == "e2m1":
                out += [_e2m1_nearest(v / 2.0 ** X) * 2.0 ** X for v in blk]
                continue
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


@pytest.mark.parametrize("profile", ["mx8", "mx4"])
def test_mx_layer_against_scalar_brute_force(profile):
    cfg = TINY.with_(tokens=2, precision=profile)
    dense = synth.dense_weights(cfg)
    sl = synth.expert_slice(cfg, 0, cfg.E)
    x = synth.tokens(cfg)
    r = O.forward(O.OracleLayer.from_synth(cfg, dense), x)
    bf = _brute_force_mx8(cfg, dense, sl, x, O.MX_PROFILE_ELEMENT[profile])
    # the two sides agree up to summation order, except where a value lands within
    # rounding distance of an E4M3, E2M1 or bf16 midpoint; on these inputs none does
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
    c = O.forward(L, x, precision="mx4").delta
    rel4 = np.linalg.norm(a - c) / np.linalg.norm(a)
    # E2M1 keeps 2 significant bits: about 4 times E4M3's relative rounding error per value
    assert 2 * rel < rel4 < 0.4, (rel, rel4)


# ---- decisions on a conversion boundary (the other valid rounding) ---------------------------
# A value computed to fp32 accuracy that lies within that accuracy of an MX conversion boundary
# may convert either way; the oracle can take the other decision where it marks one.

def test_mx8_flips_off_change_nothing():
    v = np.random.default_rng(7).normal(size=(9, 96)) * 3.0
    base = O.quantize_mx8(v)
    off = O.quantize_mx8(v, flip=np.zeros(v.shape, bool), scale_flip=np.zeros((9, 3), bool))
    for a, b in zip(base, off):
        assert np.array_equal(a, b)


def test_mx8_scale_flip_on_hand_computed_blocks():
    # amax just above 4 = 2^2: exponent 2 - 8 = -6 (byte 121); the other side is -7 (byte 120),
    # where 4.000000004 / 2^-7 = 512.0000005 saturates to 448 and 1.0 / 2^-7 = 128 exactly
    b = np.zeros((1, 32)); b[0, 0] = 4 * (1 + 1e-9); b[0, 1] = 1.0
    _, q0, s0 = O.quantize_mx8(b)
    _, q1, s1 = O.quantize_mx8(b, scale_flip=np.array([[True]]))
    assert s0[0, 0] == 121 and s1[0, 0] == 120
    assert q0[0, 0] == 256.0 and q0[0, 1] == 64.0
    assert q1[0, 0] == 448.0 and q1[0, 1] == 128.0
    # amax just below 8 = 2^3: exponent 2 - 8 = -6; the other side is -5
    c = np.zeros((1, 32)); c[0, 0] = 8 * (1 - 1e-9)
    assert O.quantize_mx8(c)[2][0, 0] == 121
    assert O.quantize_mx8(c, scale_flip=np.array([[True]]))[2][0, 0] == 122
    # both blocks are marked ambiguous at eta = 1e-6; a block with amax 5 is not
    d = np.zeros((1, 32)); d[0, 0] = 5.0
    for blk, want in ((b, True), (c, True), (d, False)):
        assert O.mx8_ambiguous(blk, 1e-6)[1][0, 0] == want


def test_mx8_element_flip_takes_the_other_neighbour():
    # block amax 300 (exponent 8 - 8 = 0; 300 itself is 4 from the midpoint 304 of 288 and
    # 320): 1.0625 is the midpoint of 1.0 and 1.125 (quantum 1/8); just above it rounds up,
    # the other decision is 1.0; 40.5 (quantum 4 in [32, 64)) is 0.375 quanta from the
    # midpoint 42 and is not marked at eta = 1e-6
    e = np.zeros((1, 32)); e[0, 0] = 300.0; e[0, 1] = 1.0625 * (1 + 1e-7); e[0, 2] = 40.5
    flip = np.zeros((1, 32), bool); flip[0, 1] = True
    assert O.quantize_mx8(e)[1][0, 1] == 1.125
    assert O.quantize_mx8(e, flip=flip)[1][0, 1] == 1.0
    el, blk = O.mx8_ambiguous(e, 1e-6)
    assert el[0, 1] and not el[0, 2] and not el[0, 0] and not blk[0, 0]
    # a subnormal midpoint: 2.5 * 2^-9 between 2 and 3 * 2^-9 (ties to even: 2 * 2^-9)
    s = np.zeros((1, 32)); s[0, 0] = 300.0; s[0, 1] = 2.5 * 2.0 ** -9
    f1 = np.zeros((1, 32), bool); f1[0, 1] = True
    assert O.quantize_mx8(s)[1][0, 1] == 2 * 2.0 ** -9
    assert O.quantize_mx8(s, flip=f1)[1][0, 1] == 3 * 2.0 ** -9


def test_mx8_every_flip_is_the_other_neighbour_and_never_past_448():
    rng = np.random.default_rng(11)
    v = rng.normal(size=(64, 128)) * np.exp(rng.normal(size=(64, 1)))
    _, q, sb = O.quantize_mx8(v)
    _, qf, sbf = O.quantize_mx8(v, flip=np.ones(v.shape, bool))
    assert np.array_equal(sb, sbf)
    y = (v.reshape(64, 4, 32) * np.ldexp(1.0, 127 - sb.astype(np.int64))[..., None]).reshape(v.shape)
    # brute force: the two representable E4M3 values bracketing |y|
    grid = O.e4m3_decode(np.arange(0, 0x7F))
    hi_i = np.searchsorted(grid, np.abs(y), side="right")
    lo = grid[hi_i - 1]
    hi = np.where(hi_i < len(grid), grid[np.minimum(hi_i, len(grid) - 1)], np.inf)
    aq, aqf = np.abs(q), np.abs(qf)
    inside = hi <= 448.0
    assert np.all(np.isin(aq[inside], [0.0]) | (aq[inside] == lo[inside]) | (aq[inside] == hi[inside]))
    assert np.all((aqf[inside] == lo[inside]) | (aqf[inside] == hi[inside]))
    assert np.all(aqf[inside] != aq[inside])
    assert np.all(aqf <= 448.0) and np.array_equal(qf[~inside], q[~inside])
    assert np.all(np.sign(qf[qf != 0]) == np.sign(y[qf != 0]))


# ---- MXFP4-E2M1 activations (the "mx4" profile) ----------------------------------------------

def test_e2m1_codes_decode_to_the_printed_grid():
    v = O.e2m1_decode(np.arange(16))
    assert v[:8].tolist() == list(O.E2M1_GRID) and O.E2M1_MAX == 6.0 == v[7]
    assert np.array_equal(v[8:], -v[:8])


def test_round_e2m1_hand_computed_ties_and_saturation():
    r = O.round_e2m1
    # the midpoints of the grid 0 0.5 1 1.5 2 3 4 6 go to the value with the even code
    ties = {0.25: 0.0, 0.75: 1.0, 1.25: 1.0, 1.75: 2.0, 2.5: 2.0, 3.5: 4.0, 5.0: 4.0}
    for y, want in ties.items():
        assert r(y) == want and r(-y) == -want, y
    assert r(0.26) == 0.5 and r(0.74) == 0.5 and r(2.51) == 3.0 and r(5.01) == 6.0
    assert r(6.0) == 6.0 and r(7.0) == 6.0 and r(7.99) == 6.0 and r(1e9) == 6.0 and r(-1e9) == -6.0


def test_round_e2m1_matches_an_exhaustive_search():
    rng = np.random.default_rng(21)
    y = np.concatenate([rng.uniform(-9, 9, 20000), np.arange(-36, 37) / 4.0])   # every quarter
    want = np.array([_e2m1_nearest(float(v)) for v in y])
    assert np.array_equal(O.round_e2m1(y), want)


def test_mx4_scale_rule_on_hand_computed_blocks():
    v = np.zeros(64)
    v[0], v[1], v[2] = 1.0, 0.3, -0.6     # block 0: amax 1 -> X = 0 - 2; 0.3 * 4 = 1.2 -> 1.0,
    v[32], v[33] = 1.9, 0.5                # -0.6 * 4 = -2.4 -> -2; block 1: X = -2, 7.6 -> 6
    deq, q, sc = O.quantize_mx4(v)
    assert sc.tolist() == [125, 125]
    assert q[:3].tolist() == [4.0, 1.0, -2.0] and deq[1] == 0.25 and deq[2] == -0.5
    assert q[32] == 6.0 and deq[32] == 1.5 and q[33] == 2.0
    _, _, sz = O.quantize_mx4(np.zeros(32))
    assert sz.tolist() == [0]
    for k in (-20, -3, 0, 5, 30):          # amax = 2^k exactly: X = k - 2, the element 4
        _, qk, s = O.quantize_mx4(np.full(32, 2.0 ** k))
        assert int(s[0]) == 127 + k - 2 and qk[0] == 4.0


def test_mx4_error_bound_idempotence_and_block_independence():
    rng = np.random.default_rng(19)
    v = rng.standard_normal((50, 256)) * np.exp2(rng.integers(-8, 8, (50, 1)))
    deq, q, sc = O.quantize_mx4(v)
    scale = np.repeat(np.ldexp(1.0, sc.astype(np.int64) - 127), 32, axis=-1)
    y = np.abs(v) / scale
    assert np.all(y < 8) and np.all(np.max(y.reshape(50, 8, 32), -1) >= 4)   # amax lands in [4, 8)
    normal = (y >= 1) & (y <= 6)
    assert np.all(np.abs(deq - v)[normal] <= 0.25 * np.abs(v)[normal])  # half a spacing of 2^(e-1)
    assert np.all(np.abs(deq - v)[y < 1] <= 0.25 * scale[y < 1])
    assert np.all(np.abs(deq - v)[y > 6] <= 2 * scale[y > 6])           # saturation below 8
    assert np.array_equal(O.quantize_mx4(deq)[0], deq)
    w = v.copy()
    w[:, 100] *= 3.0                       # block 3 only
    d2 = O.quantize_mx4(w)[0]
    assert np.array_equal(np.delete(d2, np.s_[96:128], axis=1), np.delete(deq, np.s_[96:128], axis=1))


def test_mx4_decisions_on_a_boundary():
    # block amax 7.5 (exponent 2 - 2 = 0): 0.75 (1 + 1e-7) lies just above the midpoint of 0.5
    # and 1 and rounds to 1; the other decision is 0.5.  2.2 is 0.3 from the midpoint 2.5 and
    # is not marked; 7 (past 6) has no decision to take
    e = np.zeros((1, 32)); e[0, 0] = 7.5; e[0, 1] = 0.75 * (1 + 1e-7); e[0, 2] = 2.2; e[0, 3] = -7.0
    flip = np.zeros((1, 32), bool); flip[0, 1] = True; flip[0, 3] = True
    _, q, sb = O.quantize_mx4(e)
    assert sb[0, 0] == 127 and q[0, 1] == 1.0 and q[0, 2] == 2.0 and q[0, 3] == -6.0 and q[0, 0] == 6.0
    _, qf, _ = O.quantize_mx4(e, flip=flip)
    assert qf[0, 1] == 0.5 and qf[0, 3] == -6.0
    el, blk = O.mx_ambiguous(e, "e2m1", 1e-6)
    assert el[0, 1] and not el[0, 2] and not el[0, 3] and not el[0, 0] and not blk[0, 0]
    # amax just above 4: exponent 0 (byte 127); the other side is -1, where it saturates
    b = np.zeros((1, 32)); b[0, 0] = 4 * (1 + 1e-9); b[0, 1] = 1.0
    _, q1, s1 = O.quantize_mx4(b, scale_flip=np.array([[True]]))
    assert O.quantize_mx4(b)[2][0, 0] == 127 and s1[0, 0] == 126
    assert q1[0, 0] == 6.0 and q1[0, 1] == 2.0
    assert O.mx_ambiguous(b, "e2m1", 1e-6)[1][0, 0]


def test_mx4_every_flip_is_the_other_neighbour_and_never_past_6():
    rng = np.random.default_rng(13)
    v = rng.normal(size=(64, 128)) * np.exp(rng.normal(size=(64, 1)))
    _, q, sb = O.quantize_mx4(v)
    _, qf, sbf = O.quantize_mx4(v, flip=np.ones(v.shape, bool))
    assert np.array_equal(sb, sbf)
    y = (v.reshape(64, 4, 32) * np.ldexp(1.0, 127 - sb.astype(np.int64))[..., None]).reshape(v.shape)
    grid = np.array(O.E2M1_GRID)
    hi_i = np.searchsorted(grid, np.abs(y), side="right")
    lo = grid[hi_i - 1]
    hi = np.where(hi_i < len(grid), grid[np.minimum(hi_i, len(grid) - 1)], np.inf)
    aq, aqf = np.abs(q), np.abs(qf)
    inside = hi <= 6.0
    assert np.all((aq[inside] == lo[inside]) | (aq[inside] == hi[inside]))
    assert np.all((aqf[inside] == lo[inside]) | (aqf[inside] == hi[inside]))
    assert np.all(aqf[inside] != aq[inside])
    assert np.all(aqf <= 6.0) and np.array_equal(qf[~inside], q[~inside])
