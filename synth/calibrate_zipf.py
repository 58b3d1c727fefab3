"""Router biases with expert load shaped as a capped Zipf(s).

Writes synth/data/k3_zipf1.0_bias.f32 (the K3 decode B=64 workload, Zipf(1.0)) or, with
the argument "k2", synth/data/k2_zipf1.2_bias.f32 (the K2-style block, Zipf(1.2)): E
little-endian float32, the input the presets load.  Input tooling, run offline once:

    python -m synth.calibrate_zipf [k2]

It calls the float64 oracle's router for the scores and nothing of the HIP path.

Target.  A token picks k distinct experts, so a literal Zipf over experts is infeasible
at the head.  Expert j, ranked r_j = 1..E by a seeded permutation, is picked by a
fraction pi_j = min(1, c / r_j^s) of the tokens, with c solved so that sum_j pi_j = k
(so q_j = M pi_j of the M calibration tokens pick it).

Bias.  The quantile-balancing coordinate step of the K3 walkthrough (Kimi K3 模型结构
（5）, section "Stable 之三：Quantile Balancing"), with the per-expert targets q_j in
place of the uniform M k / E and beta = -b:
    alpha_i = the (k+1)-th largest of s_i - beta          (token side)
    beta_j  = the (q_j+1)-th largest of s_{:,j} - alpha   (expert side)
iterated to a fixed point of the selection; experts with pi_j = 1 (picked by every
token) are left out of the expert step and get b = +2.  At inference the bias is frozen
and the top-k of s + b reproduces the calibrated load (the walkthrough's closing remark
on the dual solution).
"""
from __future__ import annotations

import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))

import oracle  # noqa: E402
import synth  # noqa: E402

ZIPF_S = 1.0
K2_ZIPF_S = 1.2
CAL_TOKENS = 16384
CAL_BATCH = 900_000          # token stream of the calibration batch (never timed)
PERM_SEED = 20_251           # seeds the expert ranking
SATURATED_BIAS = 2.0


def zipf_targets(E: int, k: int, s: float, rng: np.random.Generator):
    """pi_j = min(1, c / r_j^s) with sum pi = k; returns (pi, rank, c)."""
    rank = np.empty(E, dtype=np.int64)
    rank[rng.permutation(E)] = np.arange(1, E + 1)
    base = rank.astype(np.float64) ** -s
    lo, hi = 0.0, float(E) ** s * k
    for _ in range(200):
        c = 0.5 * (lo + hi)
        if np.minimum(1.0, c * base).sum() < k:
            lo = c
        else:
            hi = c
    c = 0.5 * (lo + hi)
    return np.minimum(1.0, c * base), rank, c


def kth_largest(a: np.ndarray, n: int, axis: int) -> np.ndarray:
    """The n-th largest (1-based) along `axis`."""
    m = a.shape[axis]
    return np.take(np.partition(a, m - n, axis=axis), m - n, axis=axis)


def qb_bias(s: np.ndarray, k: int, q: np.ndarray, saturated: np.ndarray, iters: int = 60):
    M, E = s.shape
    beta = np.zeros(E)
    beta[saturated] = -SATURATED_BIAS
    qi = np.clip(np.round(q).astype(np.int64), 1, M - 1)
    prev = None
    for it in range(iters):
        alpha = kth_largest(s - beta, k + 1, axis=1)                     # [M]
        margin = s - alpha[:, None]                                       # [M, E]
        for j in np.nonzero(~saturated)[0]:
            beta[j] = kth_largest(margin[:, j], int(qi[j]) + 1, axis=0)
        sel = np.argpartition(-(s - beta), k, axis=1)[:, :k]
        load = np.bincount(sel.ravel(), minlength=E)
        if prev is not None and np.array_equal(load, prev):
            break
        prev = load
    return -beta, load, it + 1


def main(cfg=None, zipf_s=None):
    cfg = synth.K3_DECODE_B64_ZIPF if cfg is None else cfg
    zipf_s = ZIPF_S if zipf_s is None else zipf_s
    dense = synth.dense_weights(cfg.with_(bias_kind="normal", bias_a=0.0, bias_b=0.0))
    w_r = oracle.bf16_to_f64(dense.router)
    rng = np.random.default_rng(PERM_SEED)
    pi, rank, c = zipf_targets(cfg.E, cfg.k, zipf_s, rng)
    saturated = pi >= 1.0
    print(f"c = {c:.4f}, saturated experts {int(saturated.sum())}, sum pi = {pi.sum():.6f}")
    s = np.empty((CAL_TOKENS, cfg.E))
    for t0 in range(0, CAL_TOKENS, 2048):
        x = synth.tokens(cfg, batch=CAL_BATCH + t0 // 2048, T=2048)
        s[t0:t0 + 2048] = oracle.router_scores(oracle.bf16_to_f64(x), w_r)
    b, load, n_it = qb_bias(s, cfg.k, CAL_TOKENS * pi, saturated)
    print(f"QB fixed point after {n_it} iterations; calibration load: max {load.max()} "
          f"(target {CAL_TOKENS * pi.max():.0f}), tail min {load.min()}")
    out = os.path.join(HERE, "data", cfg.bias_file)
    os.makedirs(os.path.dirname(out), exist_ok=True)
    b.astype("<f4").tofile(out)
    print(f"wrote {out}")


if __name__ == "__main__":
    # default: the K3 decode B=64 layer, Zipf(1.0); "k2": the K2-style block, Zipf(1.2)
    if len(sys.argv) > 1 and sys.argv[1] == "k2":
        main(synth.K2_MOE_1024_ZIPF, K2_ZIPF_S)
    else:
        main()
