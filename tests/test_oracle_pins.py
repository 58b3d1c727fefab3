"""Pins of the CPU oracle against what the pages and the mathematics fix (CPU only).

Each test names its source.  None of them re-types an oracle formula and compares the
oracle with itself: they use values printed on the pages, closed forms, limits,
invariants, special cases, and brute force on tiny inputs.
"""
import math

import numpy as np
import pytest

import oracle as O
import synth

# ------------------------------------------------------------------------------------
# Shapes: the K3 latent-MoE block card's exact per-instance parameter table.
# ------------------------------------------------------------------------------------


def test_k3_parameter_counts_match_block_card_table():
    s = synth.param_shapes(synth.K3_DECODE_B1)
    n = {k: int(np.prod(v)) for k, v in s.items()}
    assert n["router"] + n["bias"] == 6_423_424                  # Router row of the table
    assert n["w_down_latent"] == 25_690_112                       # 7,168 x 3,584
    per_expert = (n["expert_gu"] + n["expert_down"]) // 896
    assert per_expert == 33_030_144                               # Routed expert, per expert
    assert n["expert_gu"] + n["expert_down"] == 29_595_009_024    # x 896
    assert n["norm_gamma"] == 3_584                               # Latent RMSNorm
    assert n["w_up_latent"] == 25_690_112                         # Latent up-projection
    assert n["shared_gu"] + n["shared_down"] == 132_120_576       # Shared experts
    assert sum(n.values()) == 29_784_936_832                      # Per-instance total
    # walkthrough's active-parameter account: 16 experts ~ 528M, shared 132M, projections 51M
    assert 16 * per_expert == 528_482_304
    assert round((n["w_down_latent"] + n["w_up_latent"]) / 1e6) == 51


def test_all_k3_presets_share_the_layer_shape():
    ref = synth.param_shapes(synth.K3_DECODE_B1)
    for cfg in (synth.K3_DECODE_B64_ZIPF, synth.K3_PREFILL_8K):
        assert synth.param_shapes(cfg) == ref


def test_toy_shapes():
    c = synth.TOY
    assert (c.d, c.l, c.E, c.k, c.m, c.ms, c.tokens) == (640, 320, 64, 2, 256, 512, 16)
    assert c.ms == 2 * c.m   # two shared experts merged into one wider MLP


# ------------------------------------------------------------------------------------
# MXFP4 = E2M1 elements + one E8M0 scale per 32 (OCP MX v1.0 definitions).
# ------------------------------------------------------------------------------------


def test_e2m1_all_16_codes():
    v = O.e2m1_decode(np.arange(16))
    assert list(v[:8]) == list(O.E2M1_GRID)
    assert list(v[8:]) == [-g for g in O.E2M1_GRID]
    assert math.copysign(1.0, v[8]) == -1.0          # code 8 is negative zero
    # E2M1's largest normal is 6 = 2^2 * 1.5, its smallest subnormal 0.5 = 2^0 * 0.5
    assert v.max() == 6.0 and v[1] == 0.5


def test_e8m0_all_256_bytes():
    v = O.e8m0_decode(np.arange(256))
    assert np.isnan(v[255])
    for b in range(255):
        m, e = math.frexp(v[b])          # v = m * 2^e with m in [0.5, 1)
        assert m == 0.5 and e - 1 == b - 127
    assert v[127] == 1.0


def test_mxfp4_nibble_order_and_block_scale():
    codes = np.zeros((1, 16), np.uint8)
    codes[0, 0] = 0x2F          # column 0 <- code 0xF (-6), column 1 <- code 0x2 (+1)
    codes[0, 15] = 0x71         # column 30 <- code 0x1 (0.5), column 31 <- code 0x7 (6)
    scales = np.array([[128]], np.uint8)          # 2^1
    w = O.dequant_mxfp4(codes, scales)
    assert w.shape == (1, 32)
    assert w[0, 0] == -12.0 and w[0, 1] == 2.0 and w[0, 30] == 1.0 and w[0, 31] == 12.0
    assert np.all(w[0, 2:30] == 0.0)


def test_mxfp4_dequant_exact_in_fp32_and_bf16():
    # every product code * 2^(b-127) is an fp32 (and bf16) value while it stays below the
    # fp32 overflow: 6 * 2^(b-127) < 2^128 holds up to b = 252
    codes = np.arange(256, dtype=np.uint8).reshape(1, 256)
    for sb in range(0, 253):
        w = O.dequant_mxfp4(codes, np.full((1, 16), sb, np.uint8))
        f32 = w.astype(np.float32)
        assert np.array_equal(f32.astype(np.float64), w)
        bits = f32.view(np.uint32)
        assert np.all(bits & 0xFFFF == 0)            # representable in bf16 as well


def test_synthetic_mxfp4_expert_weight_rms():
    # E2M1 codes uniform over 16: E[q^2] = sum(grid^2)/8; scales uniform over 2^-8..2^-4.
    eq2 = sum(g * g for g in O.E2M1_GRID) / 8
    es2 = sum(2.0 ** (2 * e) for e in range(-8, -3)) / 5
    want = math.sqrt(eq2 * es2)
    assert abs(want - 0.0944) < 5e-4
    sl = synth.expert_slice(synth.K3_DECODE_B1, 5, 6)
    w = O.dequant_mxfp4(sl.gu[0, :256], sl.gu_scale[0, :256])
    assert abs(np.sqrt(np.mean(w * w)) / want - 1) < 0.02


# ------------------------------------------------------------------------------------
# Router: the toy chapter's worked example, and brute force.
# ------------------------------------------------------------------------------------


def test_router_worked_example_from_toy_chapter():
    s = np.array([[0.90, 0.80, 0.65, 0.20]])
    idx, G, _ = O.select_and_weight(s, np.zeros(4), k=2)
    assert list(idx[0]) == [0, 1]                       # no adjustment: first two
    b = np.array([-0.40, 0.0, 0.25, 0.0])               # selection scores 0.50 0.80 0.90 0.20
    idx, G, margin = O.select_and_weight(s, b, k=2)
    assert list(idx[0]) == [2, 1]                       # the third and second experts
    assert abs(G[0, 0] - 0.65 / 1.45) < 1e-12 and abs(G[0, 1] - 0.80 / 1.45) < 1e-12
    assert round(100 * G[0, 0]) == 45 and round(100 * G[0, 1]) == 55   # "about 45% and 55%"
    assert abs(margin[0] - (0.80 - 0.50)) < 1e-6


def test_topk_matches_a_full_sort_brute_force():
    rng = np.random.default_rng(0)
    for _ in range(200):
        E, k = int(rng.integers(2, 12)), 0
        k = int(rng.integers(1, E + 1))
        s = rng.random((3, E))
        b = (rng.random(E) - 0.5) * 0.2
        if rng.random() < 0.3:        # force exact ties in kappa
            s[:, : E // 2] = 0.5
            b[: E // 2] = 0.0
        idx, G, _ = O.select_and_weight(s, b, k)
        for t in range(3):
            kap = [float(np.float32(s[t, e]) + np.float32(b[e])) for e in range(E)]
            want = sorted(range(E), key=lambda e: (-kap[e], e))[:k]
            assert list(idx[t]) == want
            ssel = [s[t, e] for e in want]
            assert np.allclose(G[t], [v / sum(ssel) for v in ssel], rtol=0, atol=1e-15)


def test_gate_weights_sum_to_route_scale():
    rng = np.random.default_rng(1)
    s = O.sigmoid(rng.normal(size=(50, 896)) * 2)
    b = rng.normal(size=896) * 0.03
    _, G, _ = O.select_and_weight(s, b, 16)
    assert np.all(np.abs(G.sum(1) - 1) < 1e-12)
    _, G2, _ = O.select_and_weight(s, b, 16, route_scale=2.827)   # K2 card's 2.827
    assert np.all(np.abs(G2.sum(1) - 2.827) < 1e-12)


def test_bias_picks_but_does_not_weight():
    rng = np.random.default_rng(2)
    s = O.sigmoid(rng.normal(size=(64, 40)))
    b1 = rng.normal(size=40) * 0.05
    idx1, G1, m1 = O.select_and_weight(s, b1, 4)
    # a common offset of the bias does not change the selection (centering is harmless)
    idx2, G2, _ = O.select_and_weight(s, b1 + 0.125, 4)
    ok = m1 > 1e-6
    assert np.array_equal(idx1[ok], idx2[ok])
    # for a fixed selection, the weights do not depend on the bias at all
    b3 = rng.normal(size=40)
    _, G3, _ = O.select_and_weight(s, b3, 4, forced_idx=idx1)
    assert np.array_equal(G1, G3)
    # a large bias on one expert invites it everywhere; its weight stays its raw share
    b4 = b1.copy()
    b4[7] = 10.0
    idx4, G4, _ = O.select_and_weight(s, b4, 4)
    assert np.all(idx4[:, 0] == 7)
    for t in range(64):
        assert abs(G4[t, 0] - s[t, 7] / s[t, idx4[t]].sum()) < 1e-15


# ------------------------------------------------------------------------------------
# SiTU-GLU (walkthrough, Appendix B properties; port notes' formula).
# ------------------------------------------------------------------------------------


def test_situ_bounded_by_beta_product():
    g = np.concatenate([-np.logspace(-3, 4, 200), [0.0], np.logspace(-3, 4, 200)])
    G, U = np.meshgrid(g, g)
    h = O.situ(G, U)
    assert np.all(np.isfinite(h))
    # |tanh| < 1 and 0 < sigma < 1: no coordinate exceeds beta_gate * beta_lin = 100
    assert np.max(np.abs(h)) <= 100.0
    small = (np.abs(G) < 50) & (np.abs(U) < 50)
    assert np.max(np.abs(h[small])) < 100.0
    # sup |h| = beta_gate * beta_lin = 100, approached as g, u -> +inf
    assert abs(O.situ(np.array(60.0), np.array(1e3)) - 100.0) < 1e-9
    inf = O.situ(np.array([np.inf, -np.inf, 5.0]), np.array([np.inf, 3.0, -np.inf]))
    assert inf[0] == 100.0 and inf[1] == 0.0 and inf[2] == pytest.approx(-25 * 4 * math.tanh(1.25) / (1 + math.exp(-5)))


def test_situ_first_order_equals_swiglu_near_zero():
    # beta tanh(z/beta) = z - z^3/(3 beta^2) + O(z^5), so SiTU/SwiGLU = 1 - g^2/48 - u^2/1875 + O(z^4)
    for g, u in [(1e-3, 2e-3), (-2e-3, 1e-3), (3e-3, -3e-3)]:
        r = O.situ(np.array(g), np.array(u)) / O.swiglu(np.array(g), np.array(u))
        assert abs(r - (1 - g * g / 48 - u * u / 1875)) < 1e-10
    # relative gap shrinks like z^2
    z = np.array([1e-1, 1e-2])
    gap = np.abs(O.situ(z, z) / O.swiglu(z, z) - 1)
    assert 90 < gap[0] / gap[1] < 110


def test_situ_converges_to_swiglu_as_betas_grow():
    rng = np.random.default_rng(3)
    g, u = rng.normal(size=1000) * 3, rng.normal(size=1000) * 3
    h = O.situ(g, u, 1e6, 1e6)
    sw = O.swiglu(g, u)
    assert np.max(np.abs(h - sw) / (np.abs(sw) + 1e-300)) < 1e-6


def test_situ_sigmoid_acts_on_raw_gate():
    # with sigma of the raw gate, a(g) -> beta_gate for large g; sigma of the capped gate
    # would give beta_gate * sigma(beta_gate) = 3.93 instead
    a = O.situ(np.array(50.0), np.array(25.0 * np.arctanh(0.999999)))
    assert abs(a / (25 * 0.999999) - 4.0) < 1e-9
    # negative half: response tends to zero (Swish shape kept)
    assert abs(O.situ(np.array(-40.0), np.array(1.0))) < 1e-15
    assert O.sigmoid(np.array([-1e4, 0.0, 1e4])).tolist() == [0.0, 0.5, 1.0]


# ------------------------------------------------------------------------------------
# Whole-layer pins on small synthetic layers.
# ------------------------------------------------------------------------------------

TINY = synth.LayerConfig(name="tiny", d=64, l=32, E=8, k=2, m=32, ms=64, tokens=5, seed=77,
                         expert_fmt="mxfp4", bias_kind="uniform", bias_a=-0.01, bias_b=0.01,
                         e8m0_lo=125, e8m0_hi=128)


def _layer(cfg):
    return O.OracleLayer.from_synth(cfg)


def test_shared_merge_equals_sum_of_two_experts():
    rng = np.random.default_rng(4)
    d, m = 48, 16
    x = rng.normal(size=(7, d))
    wg1, wu1, wd1 = rng.normal(size=(m, d)), rng.normal(size=(m, d)), rng.normal(size=(d, m))
    wg2, wu2, wd2 = rng.normal(size=(m, d)), rng.normal(size=(m, d)), rng.normal(size=(d, m))
    merged = O.glu(x, np.vstack([wg1, wg2, wu1, wu2]), np.hstack([wd1, wd2]), O.situ)
    two = O.glu(x, np.vstack([wg1, wu1]), wd1, O.situ) + O.glu(x, np.vstack([wg2, wu2]), wd2, O.situ)
    assert np.max(np.abs(merged - two)) <= 1e-12 * np.max(np.abs(two))


def test_sort_dispatch_equals_dense_mask_definition():
    for fmt in ("mxfp4", "bf16"):
        cfg = TINY.with_(expert_fmt=fmt)
        L = _layer(cfg)
        x = synth.tokens(cfg)
        r = O.forward(L, x)
        Gd = np.zeros((cfg.tokens, cfg.E))
        for t in range(cfg.tokens):
            Gd[t, r.idx[t]] = r.G[t]
        u = O.routed_sum_dense_mask(L, r.xc, Gd)
        assert np.max(np.abs(u - r.u)) <= 1e-13 * np.max(np.abs(u))


def test_single_expert_top1_has_unit_gate():
    cfg = TINY.with_(E=1, k=1)
    r = O.forward(_layer(cfg), synth.tokens(cfg))
    assert np.all(r.idx == 0) and np.all(r.G == 1.0)
    assert np.all(np.isinf(r.margin))


def _brute_force_layer(cfg, dense, sl, x_bits):
    """Pure-Python loops over the [out, in] storage, one scalar at a time."""
    f = lambda a: O.bf16_to_f64(a)  # noqa: E731
    Wr, Wd, Wu, gam = f(dense.router), f(dense.w_down_latent), f(dense.w_up_latent), f(dense.norm_gamma)
    Sg, Sd = f(dense.shared_gu), f(dense.shared_down)
    if sl.fmt == "bf16":
        EGU, EDN = f(sl.gu), f(sl.down)
    else:
        lut = O.E2M1_GRID + tuple(-v for v in O.E2M1_GRID)

        def deq(codes, scales):
            rows, half = codes.shape[-2:]
            out = np.zeros(codes.shape[:-2] + (rows, 2 * half))
            for idx in np.ndindex(codes.shape[:-1]):
                for c in range(2 * half):
                    byte = int(codes[idx + (c // 2,)])
                    q = lut[(byte >> 4) if c % 2 else (byte & 15)]
                    out[idx + (c,)] = q * 2.0 ** (int(scales[idx + (c // 32,)]) - 127)
            return out
        EGU, EDN = deq(sl.gu, sl.gu_scale), deq(sl.down, sl.down_scale)
    X = f(x_bits)
    T, d = X.shape
    sig = lambda z: 1 / (1 + math.exp(-z)) if z >= 0 else math.exp(z) / (1 + math.exp(z))  # noqa: E731

    def act(g, u):
        return 4 * math.tanh(g / 4) * sig(g) * 25 * math.tanh(u / 25)
    out = np.zeros((T, d))
    for t in range(T):
        xt = X[t]
        s = [sig(sum(xt[c] * Wr[e, c] for c in range(d))) for e in range(cfg.E)]
        kap = [float(np.float32(s[e]) + np.float32(dense.bias[e])) for e in range(cfg.E)]
        sel = sorted(range(cfg.E), key=lambda e: (-kap[e], e))[: cfg.k]
        tot = sum(s[e] for e in sel)
        xc = [sum(xt[c] * Wd[r, c] for c in range(d)) for r in range(cfg.l)]
        u = [0.0] * cfg.l
        for e in sel:
            h = [act(sum(xc[c] * EGU[e, i, c] for c in range(cfg.l)),
                     sum(xc[c] * EGU[e, cfg.m + i, c] for c in range(cfg.l))) for i in range(cfg.m)]
            for r in range(cfg.l):
                u[r] += s[e] / tot * sum(h[i] * EDN[e, r, i] for i in range(cfg.m))
        rms = math.sqrt(sum(v * v for v in u) / cfg.l + cfg.eps)
        uh = [u[r] / rms * gam[r] for r in range(cfg.l)]
        hs = [act(sum(xt[c] * Sg[i, c] for c in range(d)), sum(xt[c] * Sg[cfg.ms + i, c] for c in range(d)))
              for i in range(cfg.ms)]
        for o in range(d):
            out[t, o] = sum(uh[r] * Wu[o, r] for r in range(cfg.l)) + sum(hs[i] * Sd[o, i] for i in range(cfg.ms))
    return out


@pytest.mark.parametrize("fmt", ["mxfp4", "bf16"])
def test_layer_against_scalar_brute_force(fmt):
    cfg = TINY.with_(expert_fmt=fmt, tokens=3)
    dense = synth.dense_weights(cfg)
    sl = synth.expert_slice(cfg, 0, cfg.E)
    x = synth.tokens(cfg)
    r = O.forward(O.OracleLayer.from_synth(cfg, dense), x)
    bf = _brute_force_layer(cfg, dense, sl, x)
    assert np.max(np.abs(r.delta - bf)) <= 1e-12 * np.max(np.abs(bf))


def test_rmsnorm_makes_routed_path_scale_invariant():
    # multiply every expert's W_down by 2^p (an exact E8M0 +p): u scales, u_hat does not.
    # With eps = 0 the norm is exactly scale invariant; with eps > 0 the output moves by
    # about eps / (2 mean(u^2)) of y_routed (the toy's u is small, so eps is visible there).
    cfg = synth.TOY.with_(eps=0.0)
    L = _layer(cfg)
    x = synth.tokens(cfg)
    r0 = O.forward(L, x)
    gu, dn = L._experts
    L2 = O.OracleLayer(cfg, synth.dense_weights(cfg), experts=(gu, dn * 8.0))
    r1 = O.forward(L2, x)
    assert np.array_equal(r0.idx, r1.idx)
    assert np.max(np.abs(r1.u - 8 * r0.u)) <= 1e-14 * np.max(np.abs(r1.u))
    assert np.max(np.abs(r1.delta - r0.delta)) <= 1e-12 * np.max(np.abs(r0.delta))
    ce = synth.TOY
    a = O.forward(O.OracleLayer(ce, synth.dense_weights(ce), experts=(gu, dn)), x)
    b = O.forward(O.OracleLayer(ce, synth.dense_weights(ce), experts=(gu, dn * 8.0)), x)
    ms = np.mean(a.u ** 2, axis=1, keepdims=True)
    bound = 0.6 * ce.eps / ms * np.max(np.abs(a.y_routed), axis=1, keepdims=True)
    assert np.all(np.abs(b.delta - a.delta) <= bound)
    # without the norm the same change moves the output: the check has teeth
    c3 = cfg.with_(use_norm=False)
    r2 = O.forward(O.OracleLayer(c3, synth.dense_weights(cfg), experts=(gu, dn)), x)
    r3 = O.forward(O.OracleLayer(c3, synth.dense_weights(cfg), experts=(gu, dn * 8.0)), x)
    assert np.max(np.abs(r3.delta - r2.delta)) > 1e-3 * np.max(np.abs(r2.delta))


def test_normalised_latent_has_unit_rms_and_expected_up_projection_scale():
    cfg = synth.TOY
    L = _layer(cfg)
    r = O.forward(L, synth.tokens(cfg))
    uh = O.rmsnorm(r.u, L.gamma, cfg.eps)
    ms = np.mean(r.u ** 2, axis=1)
    # gamma = 1: mean(u_hat^2) = mean(u^2) / (mean(u^2) + eps), which is 1 when eps = 0
    assert np.all(np.abs(np.mean(uh * uh, axis=1) - ms / (ms + cfg.eps)) < 1e-12)
    uh0 = O.rmsnorm(r.u, L.gamma, 0.0)
    assert np.all(np.abs(np.mean(uh0 * uh0, axis=1) - 1) < 1e-12)
    # W_up ~ N(0, 0.02^2) and an input of rms sqrt(ms/(ms+eps)): rms(y_routed) ~ 0.02 sqrt(l)
    want = 0.02 * math.sqrt(cfg.l) * np.sqrt(np.mean(ms / (ms + cfg.eps)))
    assert abs(np.sqrt(np.mean(r.y_routed ** 2)) / want - 1) < 0.05


def test_token_permutation_equivariance():
    cfg = synth.TOY
    L = _layer(cfg)
    x = synth.tokens(cfg)
    perm = np.random.default_rng(5).permutation(cfg.tokens)
    a, b = O.forward(L, x), O.forward(L, x[perm])
    assert np.array_equal(a.idx[perm], b.idx)
    assert np.max(np.abs(a.delta[perm] - b.delta)) <= 1e-13 * np.max(np.abs(a.delta))


def test_expert_permutation_equivariance():
    cfg = synth.TOY
    dense = synth.dense_weights(cfg)
    L = _layer(cfg)
    x = synth.tokens(cfg)
    p = np.random.default_rng(6).permutation(cfg.E)       # new expert i = old expert p[i]
    d2 = synth.DenseWeights(dense.router[p], dense.w_down_latent, dense.w_up_latent,
                            dense.norm_gamma, dense.shared_gu, dense.shared_down, dense.bias[p])
    gu, dn = L._experts
    L2 = O.OracleLayer(cfg, d2, experts=(gu[p], dn[p]))
    a, b = O.forward(L, x), O.forward(L2, x)
    inv = np.argsort(p)
    assert np.array_equal(inv[a.idx], b.idx)
    assert np.max(np.abs(a.delta - b.delta)) <= 1e-13 * np.max(np.abs(a.delta))


def test_forced_routing_reproduces_free_routing():
    cfg = synth.TOY
    L = _layer(cfg)
    x = synth.tokens(cfg)
    a = O.forward(L, x)
    b = O.forward(L, x, forced_idx=a.idx)
    assert np.array_equal(a.delta, b.delta)


# ------------------------------------------------------------------------------------
# The generator: slices regenerate independently, streams differ.
# ------------------------------------------------------------------------------------


def test_generator_slices_are_independent_of_range():
    cfg = TINY
    a = synth.expert_slice(cfg, 0, 8)
    b = synth.expert_slice(cfg, 3, 6)
    assert np.array_equal(a.gu[3:6], b.gu) and np.array_equal(a.down_scale[3:6], b.down_scale)
    assert np.all((a.gu_scale >= 125) & (a.gu_scale <= 128))
    x0, x1 = synth.tokens(cfg, 0), synth.tokens(cfg, 1)
    assert not np.array_equal(x0, x1)
    xf = O.bf16_to_f64(synth.tokens(synth.TOY.with_(tokens=512)))
    assert abs(xf.mean()) < 0.01 and abs(xf.std() - 1) < 0.01


def test_dispatch_bookkeeping_brute_force():
    rng = np.random.default_rng(8)
    for _ in range(20):
        E, k, T = int(rng.integers(1, 40)), 0, int(rng.integers(1, 30))
        k = int(rng.integers(1, E + 1))
        idx = np.stack([rng.permutation(E)[:k] for _ in range(T)])
        counts, offs, perm, inv = O.dispatch(idx, E)
        flat = idx.reshape(-1)
        order = [a for e in range(E) for a in range(T * k) if flat[a] == e]
        assert list(perm) == order
        assert [sum(flat == e) for e in range(E)] == list(counts)
        assert offs[0] == 0 and offs[-1] == T * k and np.all(np.diff(offs) == counts)
        assert all(perm[inv[a]] == a for a in range(T * k))


def test_selection_kappa_ranks_and_gives_the_margin():
    rng = np.random.default_rng(4)
    s = O.sigmoid(rng.standard_normal((40, 30)))
    b = rng.uniform(-0.1, 0.1, 30).astype(np.float32)
    idx, G, margin = O.select_and_weight(s, b, 6)
    kap = O.selection_kappa(s, b, 6)
    assert kap.shape == (40, 7) and np.all(np.diff(kap, axis=1) <= 0)
    assert np.array_equal(kap[:, 5] - kap[:, 6], margin)
    # brute force: the kappas of the selected experts, in selection order
    want = np.float32(s).astype(np.float64)[np.arange(40)[:, None], idx] + b[idx]
    assert np.allclose(kap[:, :6], want, rtol=0, atol=1e-7)
    full = O.selection_kappa(s[:, :6], b[:6], 6)    # E == k
    assert full.shape == (40, 7) and np.all(np.isneginf(full[:, 6]))


def test_residual_add_rounds_the_new_stream_to_bf16():
    """residual_add: the sum, and the next input as the bf16 patterns of that sum (against
    torch's bfloat16 conversion; a zero Delta returns a bf16 residual unchanged)."""
    import torch
    rng = np.random.default_rng(21)
    res = (rng.standard_normal((6, 40)) * 3).astype(np.float32).astype(np.float64)
    d = rng.standard_normal((6, 40)) * 1e-2
    new, xb = O.residual_add(res, d)
    assert np.array_equal(new, res + d)
    lib = torch.from_numpy(new.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(xb, lib)
    x = O.bf16_to_f64(xb)
    _, again = O.residual_add(x, np.zeros_like(x))
    assert np.array_equal(again, xb)
