"""The C ABI on the host (no GPU needed): the library loads, exports every declared entry
point, sizes buffers as documented, and rejects bad arguments before any launch."""
import ctypes
import os
import re

import pytest

import sparse_moe_layer_amd as moe
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(moe.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return moe.lib()


def _declared():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported(L):
    names = _declared()
    assert len(names) >= 9
    assert sorted(names) == sorted(moe.EXPORTS)
    for n in names:
        assert hasattr(L, n), n


def test_peak_probe_library_exports_its_header():
    from sparse_moe_layer_amd import peaks
    if not os.path.exists(peaks.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    src = open(os.path.join(ROOT, "include", "moe_peaks.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src)))
    assert names == sorted(peaks.EXPORTS)
    P = peaks.lib()
    for n in names:
        assert hasattr(P, n), n
    # argument checks happen before any launch (no GPU needed for these)
    import ctypes
    f = ctypes.c_double()
    assert P.moe_peak_mfma(99, 1, 1, 16, 4096, ctypes.byref(f), None) == 1
    assert P.moe_peak_mfma(0, 4, 1, 16, 256, ctypes.byref(f), None) == 1     # out too small
    assert P.moe_peak_read(None, 1024, 16, 4096, 1, None) == 1
    assert P.moe_peak_read(32, 1000, 16, 4096, 1, None) == 1                  # not 16-byte sized


def test_version_and_status_strings(L):
    assert L.moe_abi_version() == 7 == moe.ABI_VERSION
    assert moe.status_str(0) == "MOE_OK"
    assert moe.status_str(3) == "MOE_ERR_WORKSPACE"
    assert moe.status_str(99) == "MOE_ERR_UNKNOWN"


def test_packed_expert_bytes_equal_mxfp4_storage(L):
    # MXFP4 packing moves bytes, it adds none: 4.25 bits per weight for the K3 experts
    cfg = moe.config_from(synth.K3_DECODE_B1)
    assert moe.packed_experts_size(cfg) == 896 * 17_547_264
    assert 17_547_264 * 8 == 33_030_144 * 4.25
    # toy bf16 experts: gate/up input columns 320 padded to 3 K-steps of 128
    toy = moe.config_from(synth.TOY)
    assert moe.packed_experts_size(toy) == 64 * (2 * 256 * 384 * 2 + 320 * 256 * 2)


def test_packed_dense_bytes_equal_bf16_storage(L):
    # K3 widths are multiples of 128: the tiles hold exactly the canonical bytes + gamma
    cfg = moe.config_from(synth.K3_DECODE_B1)
    d, l, E, ms = 7168, 3584, 896, 6144
    canonical = (E * d + l * d + 2 * ms * d + d * l + d * ms) * 2
    assert moe.packed_dense_size(cfg) == canonical + l * 2
    assert canonical == 379_846_656


@pytest.mark.parametrize("preset", [synth.K3_DECODE_B1, synth.K3_PREFILL_8K])
def test_workspace_layout_is_ordered_and_aligned(L, preset):
    cfg = moe.config_from(preset)
    for T in (1, 64, 8192):
        off = moe.workspace_layout(cfg, T)
        vals = [off[k] for k in moe.WS_SLOTS]
        assert vals == sorted(vals) and all(v % 256 == 0 for v in vals)
        assert moe.workspace_size(cfg, T) >= vals[-1]
    assert moe.workspace_size(cfg, 64) > moe.workspace_size(cfg, 1)


def _bad(**kw):
    c = moe.config_from(synth.TOY)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


@pytest.mark.parametrize("field,value,status", [
    ("top_k", 65, moe.MOE_ERR_INVALID_ARG),          # k > E
    ("top_k", 0, moe.MOE_ERR_INVALID_ARG),
    ("d_model", 644, moe.MOE_ERR_INVALID_ARG),       # not a multiple of 8
    ("d_model", 16384, moe.MOE_ERR_UNSUPPORTED),     # wider than the shapes built
    ("n_experts", 2048, moe.MOE_ERR_UNSUPPORTED),
    ("act", 7, moe.MOE_ERR_INVALID_ARG),
    ("expert_wfmt", 5, moe.MOE_ERR_INVALID_ARG),
    ("precision", 1, moe.MOE_ERR_UNSUPPORTED),       # mx8 needs MXFP4 experts (toy: bf16)
    ("precision", 2, moe.MOE_ERR_UNSUPPORTED),       # so does mx4
    ("precision", 3, moe.MOE_ERR_INVALID_ARG),
    ("d_shared", 0, moe.MOE_OK),                      # latent block without shared: fine
    ("expert_wfmt", 2, moe.MOE_OK),                   # FP8 block-128 experts
    ("rms_eps", float("nan"), moe.MOE_ERR_INVALID_ARG),
    ("beta_gate", 0.0, moe.MOE_ERR_INVALID_ARG),
])
def test_invalid_configs(L, field, value, status):
    n = ctypes.c_size_t()
    assert L.moe_workspace_size(ctypes.byref(_bad(**{field: value})), 4, ctypes.byref(n)) == status


def test_mxfp4_needs_blocks_of_32(L):
    n = ctypes.c_size_t()
    c = _bad(expert_wfmt=1, d_latent=328)
    assert L.moe_packed_experts_size(ctypes.byref(c), ctypes.byref(n)) == moe.MOE_ERR_INVALID_ARG


def test_forward_rejects_bad_arguments_before_launch(L):
    cfg = moe.config_from(synth.TOY)
    A = 1 << 20          # a 256-aligned non-null address; never dereferenced on error paths
    W = moe.MoeWeights(A, A)
    f = L.moe_layer_forward
    ok = dict(bias=A, x=A, T=4, delta=A, idx=A, w=A, ws=A, wsb=1 << 40)

    def call(**kw):
        a = {**ok, **kw}
        return f(ctypes.byref(cfg), ctypes.byref(a.get("W", W)), a["bias"], a["x"], a["T"],
                 a["delta"], a["idx"], a["w"], a["ws"], a["wsb"], None)
    assert call(x=None) == moe.MOE_ERR_INVALID_ARG
    assert call(delta=A + 4) == moe.MOE_ERR_INVALID_ARG          # misaligned output
    assert call(ws=A + 64) == moe.MOE_ERR_INVALID_ARG            # workspace not 256-aligned
    assert call(T=-1) == moe.MOE_ERR_INVALID_ARG
    assert call(wsb=16) == moe.MOE_ERR_WORKSPACE
    assert call(W=moe.MoeWeights(A, None)) == moe.MOE_ERR_INVALID_ARG
    assert call(W=moe.MoeWeights(A + 16, A)) == moe.MOE_ERR_INVALID_ARG   # packed: 256-aligned
    assert call(T=0) == moe.MOE_OK                               # nothing to do, no launch
    assert call(T=0, x=None, delta=None, W=moe.MoeWeights()) == moe.MOE_OK
    assert f(None, ctypes.byref(W), A, A, 1, A, A, A, A, 1 << 40, None) == moe.MOE_ERR_INVALID_ARG


def test_qb_statistics_reject_bad_arguments_before_launch(L):
    cfg = moe.config_from(synth.TOY)
    A = 1 << 20
    W = moe.MoeWeights(A, A)
    h = L.moe_qb_histogram
    ok = dict(bias=A, x=A, T=4, bins=1000, hist=A, ws=A, wsb=1 << 40)

    def hist(c=cfg, **kw):
        a = {**ok, **kw}
        return h(ctypes.byref(c), ctypes.byref(W), a["bias"], a["x"], a["T"], a["bins"],
                 a["hist"], a["ws"], a["wsb"], None)
    assert hist(bins=0) == moe.MOE_ERR_INVALID_ARG
    assert hist(bins=16385) == moe.MOE_ERR_INVALID_ARG
    assert hist(hist=None) == moe.MOE_ERR_INVALID_ARG
    assert hist(hist=A + 2) == moe.MOE_ERR_INVALID_ARG
    assert hist(T=-1) == moe.MOE_ERR_INVALID_ARG
    assert hist(x=None) == moe.MOE_ERR_INVALID_ARG
    assert hist(wsb=16) == moe.MOE_ERR_WORKSPACE
    assert hist(T=0) == moe.MOE_OK
    full = moe.config_from(synth.TOY)
    full.top_k = full.n_experts                 # no (k+1)-th score: no cutoff
    assert hist(c=full) == moe.MOE_ERR_INVALID_ARG
    r = L.moe_qb_readout
    assert r(ctypes.byref(cfg), None, 1000, A, 16, A, None) == moe.MOE_ERR_INVALID_ARG
    assert r(ctypes.byref(cfg), A, 1000, A, 0, A, None) == moe.MOE_ERR_INVALID_ARG
    assert r(ctypes.byref(cfg), A, 0, A, 16, A, None) == moe.MOE_ERR_INVALID_ARG
    assert r(ctypes.byref(cfg), A, 1000, A, 16, A + 2, None) == moe.MOE_ERR_INVALID_ARG
    assert r(ctypes.byref(full), A, 1000, A, 16, A, None) == moe.MOE_ERR_INVALID_ARG


def test_pack_and_dispatch_reject_bad_ranges(L):
    cfg = moe.config_from(synth.TOY)
    A = 1 << 20
    src = moe.MoeExpertSrc(A, A, A, A)
    size = moe.packed_experts_size(cfg)
    assert L.moe_pack_experts(ctypes.byref(cfg), ctypes.byref(src), 60, 5, A, size, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_pack_experts(ctypes.byref(cfg), ctypes.byref(src), 0, 4, A, size - 1, None) == moe.MOE_ERR_WORKSPACE
    assert L.moe_pack_experts(ctypes.byref(cfg), ctypes.byref(src), 3, 0, A, size, None) == moe.MOE_OK
    dsrc = moe.MoeDenseSrc(A, A, A, A, A, A)
    dsize = moe.packed_dense_size(cfg)
    assert L.moe_pack_dense(ctypes.byref(cfg), ctypes.byref(dsrc), A, dsize - 1, None) == moe.MOE_ERR_WORKSPACE
    assert L.moe_pack_dense(ctypes.byref(cfg), ctypes.byref(dsrc), A + 16, dsize, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_pack_dense(ctypes.byref(cfg), ctypes.byref(moe.MoeDenseSrc(A, None, A, A, A, A)), A,
                            dsize, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_dispatch(ctypes.byref(cfg), A, 8, A, A, A, A, A, 8, None) == moe.MOE_ERR_WORKSPACE
    assert L.moe_dispatch(ctypes.byref(cfg), None, 8, A, A, A, A, A, 1 << 40, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_dispatch(ctypes.byref(cfg), None, 0, None, None, None, None, None, 0, None) == moe.MOE_OK


def test_nonlatent_blocks_need_a_shared_expert(L):
    n = ctypes.c_size_t()
    ok = _bad(d_latent=0, use_latent_norm=0)
    assert L.moe_workspace_size(ctypes.byref(ok), 4, ctypes.byref(n)) == moe.MOE_OK
    no_shared = _bad(d_latent=0, d_shared=0)
    assert L.moe_workspace_size(ctypes.byref(no_shared), 4, ctypes.byref(n)) == moe.MOE_ERR_UNSUPPORTED
    k2 = moe.config_from(synth.K2_MOE_1024_ZIPF)
    assert L.moe_packed_experts_size(ctypes.byref(k2), ctypes.byref(n)) == moe.MOE_OK
    # 384 experts of 256 + 448 tile rows x (56 / 16 K-steps) x (2048 codes + 16 scale bytes)
    assert n.value == 384 * (256 * 56 + 448 * 16) * 2064
