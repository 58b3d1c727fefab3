"""The calibrated router bias of the K3 decode B=64 workload (synth/calibrate_zipf.py):
its targets and the load it produces on held-out token batches, routed by the oracle."""
import numpy as np
import pytest

import oracle as O
import synth
from synth import calibrate_zipf as cz


def test_capped_zipf_targets():
    # pi_j = min(1, c / r_j) summing to k = 16 over 896 experts: c ~ 2.383, two saturated
    pi, rank, c = cz.zipf_targets(896, 16, 1.0, np.random.default_rng(cz.PERM_SEED))
    assert abs(pi.sum() - 16) < 1e-9
    assert abs(c - 2.383) < 1e-3
    assert int((pi >= 1).sum()) == 2
    assert sorted(rank.tolist()) == list(range(1, 897))
    # E[distinct experts] of 64 independent tokens under these marginals (~348)
    ed = np.sum(1 - (1 - pi) ** 64)
    assert 340 < ed < 356


@pytest.fixture(scope="module")
def routed():
    cfg = synth.K3_DECODE_B64_ZIPF
    dense = synth.dense_weights(cfg)
    w_r = O.bf16_to_f64(dense.router)
    out = []
    for b in range(8):      # the bench's first token batches (held out from the calibration)
        x = synth.tokens(cfg, batch=1000 + b)
        s = O.router_scores(O.bf16_to_f64(x), w_r)
        idx, _, _ = O.select_and_weight(s, dense.bias, cfg.k)
        out.append(idx)
    return cfg, np.stack(out)


def test_held_out_load_follows_the_targets(routed):
    cfg, idx = routed
    pi, rank, _ = cz.zipf_targets(cfg.E, cfg.k, cz.ZIPF_S, np.random.default_rng(cz.PERM_SEED))
    n_tok = idx.shape[0] * idx.shape[1]
    load = np.bincount(idx.reshape(-1), minlength=cfg.E)
    by_rank = load[np.argsort(rank)]
    assert by_rank[0] == by_rank[1] == n_tok          # the saturated experts take every token
    for r in range(2, 8):                              # the head within 4 binomial std
        p = pi[np.argsort(rank)][r]
        assert abs(by_rank[r] - n_tok * p) <= 4 * np.sqrt(n_tok * p * (1 - p)) + 1
    D = [len(np.unique(b)) for b in idx]
    assert 320 <= np.mean(D) <= 375                    # distinct experts per 64-token batch
