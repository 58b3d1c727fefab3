"""bench.py on the host (no GPU needed): the one-GPU rule, and its byte and flop model against
the parameter counts it is built from."""
import os
import subprocess
import sys

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_b1_bytes_are_the_layer_weights():
    # at one token every weight is read once: the steps' weight bytes add up to the layer's
    cfg = synth.K3_DECODE_B1
    ab = bench.algorithmic_bytes(cfg, 1, 16)
    gu, dn = bench.expert_weight_bytes(cfg)
    assert gu == 11_698_176 and dn == 5_849_088          # MXFP4: 4.25 bits per weight
    assert bench.weight_bytes(cfg, 16) == 660_613_632     # the K3 layer at B=1
    # IN rows (router, W_down_latent, shared gate/up), the experts, OUT rows ([W_up_latent |
    # W_shared_down]) and gamma
    weights_in_steps = (cfg.E + cfg.l + 2 * cfg.ms) * cfg.d * 2 + 16 * (gu + dn) \
        + cfg.d * (cfg.l + cfg.ms) * 2 + cfg.l * 2
    activations = sum(ab.values()) - weights_in_steps
    assert 0 < activations < 2_000_000                   # x, z, x^c, h_s, h, E, u, Delta


def test_prefill_flops():
    cfg = synth.K3_PREFILL_8K
    af = bench.algorithmic_flops(cfg, 8192)
    expert = af["expert_gu"] + af["expert_down"]
    assert expert == 2 * 8192 * 16 * 3 * 3584 * 3072        # 8.659 TFLOP
    assert abs(sum(af.values()) - 11.770e12) / 11.770e12 < 1e-3
