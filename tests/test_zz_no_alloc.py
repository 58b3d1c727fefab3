"""GPU: moe_layer_forward_noalloc (the forward with its intermediates in the library's own
per-GPU buffer instead of a caller's workspace) against moe_layer_forward.

Both run the same launches, so the outputs must be the same bits.  Each case makes two
calls in a row, the second with fewer tokens than the first, so that the second runs on a
buffer that still holds the first call's intermediates.  A batch whose workspace exceeds
the buffer is refused before anything runs.
"""
import functools

import numpy as np
import pytest
import torch

import oracle as O
import sparse_moe_layer_amd as moe
import synth

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")

TINY_MX8 = synth.LayerConfig(name="tiny_noalloc_mx8", d=128, l=64, E=8, k=2, m=64, ms=64,
                             tokens=100, seed=78, expert_fmt="mxfp4", bias_kind="uniform",
                             bias_a=-0.01, bias_b=0.01, e8m0_lo=125, e8m0_hi=128, precision="mx8")
# (layer, first token count, second token count): the few-token launches, the token-tiled
# launches, the mx8 launches, and the K3 layer at decode batch 64 then 1
CASES = {
    "toy_16_then_5": (synth.TOY, 16, 5),
    "toy_16_then_2": (synth.TOY, 16, 2),
    "mx8_100_then_33": (TINY_MX8, 100, 33),
    "k3_64_then_1": (synth.K3_DECODE_B1, 64, 1),
}


def log(msg):
    print(msg, flush=True)


@functools.lru_cache(maxsize=2)
def device_layer(cfg):
    log(f"[upload] {cfg.name}")
    dense = synth.dense_weights(cfg)
    lay = moe.Layer.upload(moe.config_from(cfg), dense, lambda a, b: synth.expert_slice(cfg, a, b),
                           cfg.E, device=DEV, chunk=32)
    torch.cuda.synchronize()
    return lay, dense


def outputs(lay, T):
    c = lay.cfg
    return (torch.full((T, c.d_model), float("nan"), dtype=torch.float32, device=DEV),
            torch.full((T, c.top_k), -1, dtype=torch.int32, device=DEV),
            torch.full((T, c.top_k), float("nan"), dtype=torch.float32, device=DEV))


@pytest.mark.parametrize("case", list(CASES))
def test_noalloc_matches_the_workspace_forward(case):
    cfg, t1, t2 = CASES[case]
    lay, dense = device_layer(cfg)
    for call, T in enumerate((t1, t2)):
        log(f"[noalloc] {case}: call {call}, {T} tokens")
        xh = synth.tokens(cfg, batch=300 + call, T=T)
        x = torch.from_numpy(xh.view(np.int16)).to(DEV)
        got = lay.forward_noalloc(x, *outputs(lay, T))
        ref = lay.forward(x, *outputs(lay, T))
        torch.cuda.synchronize()
        for a, b, name in zip(got, ref, ("delta", "topk_idx", "topk_w")):
            assert torch.equal(a, b), f"{name} differs from moe_layer_forward"
        if cfg.E <= 64 and cfg.precision == "fp32":   # small layers: also the oracle's bars
            res = O.forward(O.OracleLayer.from_synth(cfg, dense), xh)
            d = got[0].cpu().numpy().astype(np.float64)
            assert np.array_equal(got[1].cpu().numpy(), res.idx)
            rel = np.linalg.norm(d - res.delta) / np.linalg.norm(res.delta)
            rms = np.sqrt(np.mean(res.delta ** 2))
            assert rel <= 2e-3 and np.max(np.abs(d - res.delta)) <= 1e-2 * rms


def test_noalloc_refuses_a_batch_past_its_buffer():
    cfg = synth.K3_DECODE_B1
    lay, _ = device_layer(cfg)
    T = 128   # the K3 workspace of 128 tokens is about 94 MiB
    assert moe.workspace_size(lay.cfg, T) > moe.STATIC_WORKSPACE_BYTES
    assert moe.workspace_size(lay.cfg, 64) <= moe.STATIC_WORKSPACE_BYTES
    x = torch.zeros((T, cfg.d), dtype=torch.int16, device=DEV)
    with pytest.raises(moe.MoeError) as e:
        lay.forward_noalloc(x, *outputs(lay, T))
    assert e.value.status == moe.MOE_ERR_WORKSPACE
