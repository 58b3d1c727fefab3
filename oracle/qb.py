"""Quantile Balancing statistics of the router (test infrastructure only).

Parity unpinned: none.  What it computes, from two pages:

- the toy chapter, section "Quantile Balancing: giving every expert a fair shot": per token
  the biased score of the expert that just misses the top-k is a cutoff (the (k+1)-th
  largest of s + b); per expert, the extra bias it would need to cross each token's cutoff
  is cutoff - s; the expert's new bias is the quantile of that quantity over the tokens at
  the level that gives it its share of the assignments (a fraction k/E of the tokens), and
  the new biases are centred (their mean subtracted: a common offset does not change any
  selection);
- the walkthrough, "Stable 之三：Quantile Balancing" and its histogram estimate: route with
  the top-(k+1) to get alpha_i; count r_ij = alpha_i - s_ij into an E x B histogram of B
  uniform bins over [min(b) - 1, max(b) + 1] (r lies there because s is in (0, 1) and alpha
  is some expert's biased score); counts add over micro-batches; the readout per expert is
  the first bin where the cumulative count reaches ceil(q), q = m k / E for m tokens,
  interpolated linearly inside the bin, so the error is at most one bin width.

Readings where the pages leave a step open (listed in the design notes):
- the linear interpolation: with C the count below bin t and c_t the bin's count, the value
  is lo + w (t + (ceil(q) - C) / c_t), w = (hi - lo) / B;
- the range ends are formed in float32 from the float32 biases, and alpha_i, r_ij and the bin
  index in float32, because that is the precision in which the kernel takes the integer
  decision (bin = floor((r - lo) * (B / (hi - lo))), clamped to [0, B - 1]).
The exact quantile (an order statistic of r, no histogram) is given as well: it is what the
histogram estimates, within one bin width.
"""
from __future__ import annotations

import numpy as np

__all__ = ["qb_alpha", "qb_required_bias", "qb_range", "qb_bins", "qb_histogram", "qb_target",
           "qb_readout", "qb_exact", "qb_update"]


def qb_alpha(s: np.ndarray, bias: np.ndarray, k: int) -> np.ndarray:
    """alpha_i = the (k+1)-th largest biased score float32(s_i) + float32(b) of token i, as a
    float32 value (walkthrough step 1: route with top-(k+1), the last one is the cutoff)."""
    kappa = np.asarray(s, dtype=np.float64).astype(np.float32) + np.asarray(bias, dtype=np.float32)[None, :]
    E = kappa.shape[1]
    if not 0 <= k < E:
        raise ValueError("QB needs k < E (the (k+1)-th score is the cutoff)")
    return -np.sort(-kappa, axis=1)[:, k]


def qb_required_bias(s: np.ndarray, bias: np.ndarray, k: int) -> np.ndarray:
    """r_ij = alpha_i - s_ij in float32: the bias expert j needs to make token i's top-k
    (token i takes j exactly when s_ij + b_j > alpha_i)."""
    a = qb_alpha(s, bias, k)
    return a[:, None] - np.asarray(s, dtype=np.float64).astype(np.float32)


def qb_range(bias: np.ndarray):
    """(lo, hi) = (min b - 1, max b + 1) in float32."""
    b = np.asarray(bias, dtype=np.float32)
    return np.float32(b.min()) - np.float32(1.0), np.float32(b.max()) + np.float32(1.0)


def qb_bins(r: np.ndarray, lo, hi, n_bins: int) -> np.ndarray:
    """Bin of each r among n_bins uniform bins over [lo, hi]; float32 arithmetic."""
    r = np.asarray(r, dtype=np.float32)
    inv_w = np.float32(n_bins) / (np.float32(hi) - np.float32(lo))
    t = np.floor((r - np.float32(lo)) * inv_w).astype(np.int64)
    return np.clip(t, 0, n_bins - 1)


def qb_histogram(s: np.ndarray, bias: np.ndarray, k: int, n_bins: int) -> np.ndarray:
    """counts [E, n_bins] of r_ij over the tokens (walkthrough: the n x B count matrix)."""
    r = qb_required_bias(s, bias, k)
    lo, hi = qb_range(bias)
    t = qb_bins(r, lo, hi, n_bins)
    T, E = t.shape
    hist = np.zeros((E, n_bins), dtype=np.int64)
    np.add.at(hist, (np.broadcast_to(np.arange(E), (T, E)), t), 1)
    return hist


def qb_target(n_tokens: int, k: int, E: int) -> int:
    """ceil(q), q = m k / E: the assignments per expert of a uniform load."""
    return -(-(int(n_tokens) * int(k)) // int(E))


def qb_readout(hist: np.ndarray, bias: np.ndarray, n_tokens: int, k: int,
               centre: bool = True) -> np.ndarray:
    """New biases from the counts (float64): per expert the first bin whose cumulative count
    reaches ceil(q), linearly interpolated inside it; then the mean over experts removed."""
    hist = np.asarray(hist, dtype=np.int64)
    E, n_bins = hist.shape
    lo, hi = (float(v) for v in qb_range(bias))
    w = (hi - lo) / n_bins
    qc = qb_target(n_tokens, k, E)
    out = np.empty(E)
    for e in range(E):
        cum = 0
        val = hi
        for t in range(n_bins):
            c = int(hist[e, t])
            if c > 0 and cum + c >= qc:
                val = lo + w * (t + (qc - cum) / c)
                break
            cum += c
        out[e] = val
    return out - out.mean() if centre else out


def qb_exact(s: np.ndarray, bias: np.ndarray, k: int, centre: bool = True) -> np.ndarray:
    """The quantity the histogram estimates, without bins: per expert the ceil(q)-th
    smallest r_ij (so that ceil(q) tokens need less bias than it), centred."""
    r = qb_required_bias(s, bias, k).astype(np.float64)
    T, E = r.shape
    qc = qb_target(T, k, E)
    out = np.sort(r, axis=0)[qc - 1]
    return out - out.mean() if centre else out


def qb_update(s: np.ndarray, bias: np.ndarray, k: int, n_bins: int = 1000) -> np.ndarray:
    """One QB step on one batch: histogram of r, readout, centring."""
    return qb_readout(qb_histogram(s, bias, k, n_bins), bias, np.asarray(s).shape[0], k)
