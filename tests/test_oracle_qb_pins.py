"""Pins of the oracle's Quantile Balancing statistics (CPU only).

The QB step has no printed worked example on the pages.  It is pinned here by what they
state about it and by independent computations: the cutoff against a brute-force sort,
bin membership against the bin edges, the readout within one bin width of the exact order
statistic (the walkthrough's error bound), the load each new bias gives its expert against
the fixed cutoffs, invariance to a common bias offset, and balancing within a few steps.
"""
import math

import numpy as np
import pytest

import oracle as O


def _scores(T, E, seed, spread=2.0):
    rng = np.random.default_rng(seed)
    return 1.0 / (1.0 + np.exp(-spread * rng.standard_normal((T, E))))


def test_alpha_is_the_k_plus_first_biased_score_by_brute_force():
    s = _scores(7, 9, 1)
    b = np.random.default_rng(2).normal(0, 0.05, 9)
    for k in (1, 3, 8):
        a = O.qb_alpha(s, b, k)
        for i in range(7):
            kap = sorted((float(np.float32(s[i, e]) + np.float32(b[e])) for e in range(9)), reverse=True)
            assert a[i] == np.float32(kap[k])
    with pytest.raises(ValueError):
        O.qb_alpha(s, b, 9)          # E == k has no cutoff


def test_required_bias_selects_exactly_the_top_k():
    """Token i takes expert j exactly when b_j > r_ij (the walkthrough's equivalence)."""
    s = _scores(40, 12, 3)
    b = np.random.default_rng(4).normal(0, 0.03, 12)
    k = 4
    r = O.qb_required_bias(s, b, k)
    idx, _, margin = O.select_and_weight(s, b, k)
    chosen = np.zeros_like(r, dtype=bool)
    np.put_along_axis(chosen, idx.astype(np.int64), True, axis=1)
    # away from the cutoff itself (the (k+1)-th expert has r = b up to rounding)
    clear = (margin > 1e-6)[:, None] & (np.abs(np.float32(b)[None, :] - r) > 1e-6)
    assert clear.mean() > 0.9
    assert np.array_equal((np.float32(b)[None, :] > r)[clear], chosen[clear])


def test_histogram_counts_range_and_edges():
    s = _scores(300, 10, 5)
    b = np.random.default_rng(6).normal(0, 0.1, 10)
    k, B = 3, 50
    h = O.qb_histogram(s, b, k, B)
    assert h.shape == (10, B) and np.all(h.sum(axis=1) == 300)     # one r per (token, expert)
    r = O.qb_required_bias(s, b, k).astype(np.float64)
    lo, hi = (float(v) for v in O.qb_range(b))
    assert lo < r.min() and r.max() < hi                            # r in (b_min - 1, b_max + 1)
    # membership against the bin edges, independently of the index formula
    edges = lo + (hi - lo) * np.arange(B + 1) / B
    t = O.qb_bins(r, lo, hi, B)
    w = (hi - lo) / B
    assert np.all(r >= edges[t] - 1e-5 * w) and np.all(r < edges[t + 1] + 1e-5 * w)
    for e in range(10):
        assert np.array_equal(h[e], np.bincount(t[:, e], minlength=B))


def test_readout_closed_forms():
    b = np.zeros(4)
    lo, hi = -1.0, 1.0
    B = 10                      # bin width 0.2
    h = np.zeros((4, B), dtype=np.int64)
    h[:, 3] = 8                 # every count in bin 3 = [-0.4, -0.2)
    # n_tokens 8, k 2, E 4: ceil(q) = 4 -> half way through bin 3
    v = O.qb_readout(h, b, 8, 2, centre=False)
    assert np.allclose(v, lo + 0.2 * (3 + 4 / 8))
    # uniform counts: the readout is the linear quantile of a uniform distribution
    h = np.full((4, B), 3, dtype=np.int64)
    v = O.qb_readout(h, b, 30, 2, centre=False)          # ceil(q) = 15 of 30: the middle
    assert np.allclose(v, 0.0)
    v = O.qb_readout(h, b, 30, 1, centre=False)          # ceil(30/4) = 8: bin 2, 2 of 3
    assert np.allclose(v, lo + 0.2 * (2 + 2 / 3))
    # centring: a common shift of every expert's value disappears
    h2 = np.zeros((4, B), dtype=np.int64)
    h2[0, 2] = h2[1, 5] = h2[2, 7] = h2[3, 0] = 30
    c = O.qb_readout(h2, b, 30, 1)
    u = O.qb_readout(h2, b, 30, 1, centre=False)
    assert abs(c.sum()) < 1e-12 and np.allclose(c, u - u.mean())


@pytest.mark.parametrize("B", [100, 1000])
def test_readout_within_one_bin_of_the_exact_quantile(B):
    """The walkthrough's bound: the histogram estimate is off by at most one bin width."""
    s = _scores(2000, 64, 7)
    b = np.random.default_rng(8).normal(0, 0.02, 64)
    k = 6
    est = O.qb_readout(O.qb_histogram(s, b, k, B), b, 2000, k, centre=False)
    exact = O.qb_exact(s, b, k, centre=False)
    lo, hi = (float(v) for v in O.qb_range(b))
    assert np.max(np.abs(est - exact)) <= (hi - lo) / B * (1 + 1e-6)


def test_new_bias_gives_each_expert_its_share_against_the_fixed_cutoffs():
    """Against the batch's cutoffs, expert j's new (uncentred) bias admits ceil(q) tokens,
    up to the tokens inside the bin that was interpolated."""
    T, E, k, B = 1600, 32, 4, 1000
    s = _scores(T, E, 9)
    b = np.random.default_rng(10).normal(0, 0.05, E)
    h = O.qb_histogram(s, b, k, B)
    v = O.qb_readout(h, b, T, k, centre=False)
    r = O.qb_required_bias(s, b, k).astype(np.float64)
    qc = O.qb_target(T, k, E)
    lo, hi = (float(x) for x in O.qb_range(b))
    t = np.floor((v - lo) / ((hi - lo) / B)).astype(int)
    for e in range(E):
        admitted = int((r[:, e] < v[e]).sum())
        assert abs(admitted - qc) <= h[e, min(t[e], B - 1)]
    exact = O.qb_exact(s, b, k, centre=False)
    assert all(int((r[:, e] <= exact[e]).sum()) >= qc for e in range(E))


def test_common_bias_offset_changes_nothing():
    s = _scores(500, 16, 11)
    b = np.random.default_rng(12).normal(0, 0.05, 16)
    k = 3
    a = O.qb_exact(s, b, k)
    c = O.qb_exact(s, b + 0.25, k)      # 0.25 is exact in float32: every kappa shifts alike
    assert np.max(np.abs(a - c)) < 1e-6
    x = O.qb_update(s, b, k, 1000)
    y = O.qb_update(s, b + 0.25, k, 1000)
    lo, hi = (float(v) for v in O.qb_range(b))
    assert np.max(np.abs(x - y)) <= 2 * (hi - lo) / 1000


def test_qb_balances_a_skewed_router_in_a_few_steps():
    """The walkthrough: QB jumps to the exact coordinate minimum, so even many experts
    balance in a few steps (here a batch routed with its own updated biases)."""
    T, E, k = 4096, 128, 8
    rng = np.random.default_rng(13)
    # experts of unequal appeal: a per-expert offset on the logits
    s = 1.0 / (1.0 + np.exp(-(rng.standard_normal((T, E)) + rng.normal(0, 1.0, E)[None, :])))
    b = np.zeros(E)

    def load(bias):
        idx, _, _ = O.select_and_weight(s, bias, k)
        return np.bincount(idx.reshape(-1), minlength=E)

    mean = T * k / E
    before = load(b).max() / mean
    for _ in range(3):
        b = O.qb_update(s, b, k, 1000)
    after = load(b)
    assert before > 3.0
    assert after.max() / mean < 1.15 and after.min() / mean > 0.85
    assert math.isclose(float(b.mean()), 0.0, abs_tol=1e-12)
