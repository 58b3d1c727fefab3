"""Seeded synthetic layers and token batches for the Stable LatentMoE FFN layer.

This module is the only code shared by the CPU oracle and the HIP path.  It
holds none of the layer's arithmetic: it produces the canonical bytes of a
layer (bf16 weights as uint16 arrays, MXFP4 weights as code bytes plus E8M0
scale bytes, the fp32 router bias) and bf16 token batches, each element a pure
function of (seed, stream, index) so that any slice regenerates on its own.

Canonical storage (both sides read exactly these arrays):
  router        [E, d]        bf16   (nn.Linear [out, in])
  w_down_latent [l, d]        bf16   (W_down, d -> l)
  w_up_latent   [d, l]        bf16   (W_up,   l -> d)
  norm_gamma    [l]           bf16   (all ones)
  shared_gu     [2*ms, d]     bf16   (gate rows first, then up rows)
  shared_down   [d, ms]       bf16
  expert gate/up [E, 2*m, l] and down [E, l, m]:
     bf16 layers: uint16 arrays of those shapes;
     MXFP4 layers: codes [E, rows, cols/2] uint8 (low nibble = even column)
                   plus E8M0 scales [E, rows, cols/32] uint8, blocks of 32
                   along the input (reduction) axis.
     FP8 block-128 layers: E4M3 codes [E, rows, cols] uint8 plus fp32 scales
                   [E, ceil(rows/128), ceil(cols/128)], one per 128 x 128 block.
  bias          [E]           fp32
  x             [T, d]        bf16
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field, replace

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile synth.c into libsynth.so with gcc (-O2, OpenMP, no fast-math)."""
    src = os.path.join(_HERE, "synth.c")
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", tmp, src, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build(force=False)
    lib = ctypes.CDLL(_LIB_PATH)
    u64 = ctypes.c_uint64
    vp = ctypes.c_void_p
    lib.synth_word.restype = u64
    lib.synth_word.argtypes = [u64, u64, u64]
    lib.synth_normal_bf16.argtypes = [u64, u64, u64, u64, ctypes.c_double, ctypes.c_double, vp]
    lib.synth_normal_f32.argtypes = [u64, u64, u64, u64, ctypes.c_double, ctypes.c_double, vp]
    lib.synth_uniform_f32.argtypes = [u64, u64, u64, u64, ctypes.c_double, ctypes.c_double, vp]
    lib.synth_bytes.argtypes = [u64, u64, u64, u64, vp]
    lib.synth_uniform_int_u8.argtypes = [u64, u64, u64, u64, ctypes.c_uint32, ctypes.c_uint32, vp]
    lib.synth_fp8_block128.argtypes = [u64, u64, u64, ctypes.c_int64, ctypes.c_int64,
                                       ctypes.c_double, vp, vp]
    for f in ("synth_normal_bf16", "synth_normal_f32", "synth_uniform_f32", "synth_bytes",
              "synth_uniform_int_u8", "synth_fp8_block128"):
        getattr(lib, f).restype = None
    _lib = lib
    return lib


def stream_id(name: str) -> int:
    """64-bit FNV-1a of a tensor name: the stream a tensor's elements come from."""
    h = 0xCBF29CE484222325
    for b in name.encode():
        h ^= b
        h = (h * 0x100000001B3) & 0xFFFFFFFFFFFFFFFF
    return h


def word(seed: int, stream: int, i: int) -> int:
    return int(_load().synth_word(seed, stream, i))


def normal_bf16(seed, name, start, shape, std, mean=0.0, out=None):
    n = int(np.prod(shape))
    out = np.empty(shape, np.uint16) if out is None else out
    _load().synth_normal_bf16(seed, stream_id(name), start, n, mean, std, out.ctypes.data)
    return out


def normal_f32(seed, name, start, shape, std, mean=0.0):
    out = np.empty(shape, np.float32)
    _load().synth_normal_f32(seed, stream_id(name), start, int(np.prod(shape)), mean, std,
                             out.ctypes.data)
    return out


def uniform_f32(seed, name, start, shape, lo, hi):
    out = np.empty(shape, np.float32)
    _load().synth_uniform_f32(seed, stream_id(name), start, int(np.prod(shape)), lo, hi,
                              out.ctypes.data)
    return out


def random_bytes(seed, name, start, shape, out=None):
    out = np.empty(shape, np.uint8) if out is None else out
    _load().synth_bytes(seed, stream_id(name), start, int(np.prod(shape)), out.ctypes.data)
    return out


def uniform_int_u8(seed, name, start, shape, lo, hi, out=None):
    out = np.empty(shape, np.uint8) if out is None else out
    _load().synth_uniform_int_u8(seed, stream_id(name), start, int(np.prod(shape)), lo, hi,
                                 out.ctypes.data)
    return out


def fp8_block128(seed, name, start, rows, cols, std, codes_out=None, scales_out=None):
    """One [rows, cols] matrix as FP8 E4M3 codes with an fp32 scale per 128 x 128 block
    (scale = block max |w| / 448; w = std x a unit-variance Irwin-Hall(4) draw, close to
    N(0, std^2), from stream `name` at `start`)."""
    codes = np.empty((rows, cols), np.uint8) if codes_out is None else codes_out
    scales = (np.empty(((rows + 127) // 128, (cols + 127) // 128), np.float32)
              if scales_out is None else scales_out)
    assert codes.flags.c_contiguous and scales.flags.c_contiguous
    _load().synth_fp8_block128(seed, stream_id(name), start, rows, cols, std, codes.ctypes.data,
                               scales.ctypes.data)
    return codes, scales


# --------------------------------------------------------------------------------------
# Layer presets.  Shapes follow the Kimi K3 latent-MoE block card (parameter table) and
# the toy reproduction chapter (640 -> 320 latent, 64 experts, top-2, merged 2x256 shared).
# --------------------------------------------------------------------------------------

BF16_ONE = 0x3F80
WEIGHT_STD = 0.02


@dataclass(frozen=True)
class LayerConfig:
    name: str
    d: int            # model width
    l: int            # latent width (0: non-latent)
    E: int            # routed experts
    k: int            # experts per token
    m: int            # routed expert hidden width
    ms: int           # shared hidden width (merged shared experts)
    tokens: int       # tokens per call of the workload
    seed: int
    expert_fmt: str = "mxfp4"        # "bf16" | "mxfp4" | "fp8b128"
    act: str = "situ"                # "situ" | "swiglu"
    route_scale: float = 1.0
    use_norm: bool = True
    eps: float = 1e-6
    beta_gate: float = 4.0
    beta_lin: float = 25.0
    bias_kind: str = "normal"        # "uniform" | "normal" | "file"
    bias_a: float = 0.0              # uniform: lo, normal: mean
    bias_b: float = 0.0              # uniform: hi, normal: std
    bias_file: str = ""
    e8m0_lo: int = 119               # E8M0 scale bytes uniform in [lo, hi]
    e8m0_hi: int = 123
    precision: str = "fp32"          # rounding profile of the forward: "fp32" | "mx8" | "mx4"

    def with_(self, **kw) -> "LayerConfig":
        return replace(self, **kw)


TOY = LayerConfig(
    name="toy_latent_moe_d640_l320_e64k2_t16", d=640, l=320, E=64, k=2, m=256, ms=512,
    tokens=16, seed=1001, expert_fmt="bf16", bias_kind="uniform", bias_a=-0.01, bias_b=0.01)

# Router bias N(0, 1e-3): the second argument is read as the standard deviation.  The
# prefill workload is described as near-uniform routing under this bias, which holds for a
# spread of 1e-3 (every expert used, per-expert load within about +-11%) but not for a
# variance of 1e-3 (std 0.032 outweighs the gaps between the top sigmoid scores: a fifth of
# the experts never chosen, others taking six times the mean).
_K3 = dict(d=7168, l=3584, E=896, k=16, m=3072, ms=6144, expert_fmt="mxfp4",
           bias_kind="normal", bias_a=0.0, bias_b=1e-3)
K3_DECODE_B1 = LayerConfig(name="k3_latent_moe_decode_b1", tokens=1, seed=1002, **_K3)
K3_DECODE_B64_ZIPF = LayerConfig(
    name="k3_latent_moe_decode_b64_zipf1.0", tokens=64, seed=1003,
    **{**_K3, "bias_kind": "file", "bias_file": "k3_zipf1.0_bias.f32"})
# prefill: MXFP4 weights against MXFP8 activations on the matrix cores ("mx8" profile)
K3_PREFILL_8K = LayerConfig(name="k3_latent_moe_prefill_8192", tokens=8192, seed=1004,
                            precision="mx8", **_K3)
# the same layer and tokens through the fp32-activation launches (no declared rounding)
K3_PREFILL_8K_FP32 = K3_PREFILL_8K.with_(name="k3_latent_moe_prefill_8192_fp32", precision="fp32")
# the same layer with MXFP4 activations too (FP4 x FP4 matrix cores; a reported variant)
K3_PREFILL_8K_MX4 = K3_PREFILL_8K.with_(name="k3_latent_moe_prefill_8192_mx4", precision="mx4")

# The K2 block card's non-latent MoE block on the same kernels: 384 SwiGLU experts top-8,
# gate weights renormalised and scaled by 2.827, one shared 2048-wide expert, FP8 E4M3
# experts with 128 x 128 fp32 block scales, 1024 tokens with Zipf(1.2)-loaded routing.
K2_MOE_1024_ZIPF = LayerConfig(
    name="k2_moe_1024_zipf1.2", d=7168, l=0, E=384, k=8, m=2048, ms=2048, tokens=1024, seed=1005,
    expert_fmt="fp8b128", act="swiglu", route_scale=2.827, use_norm=False,
    bias_kind="file", bias_file="k2_zipf1.2_bias.f32")

# One GPU's share of an expert-parallel prefill: 65,536 tokens over 8 GPUs send each GPU's
# 112 experts about 1,170 rows apiece (65,536 x 16 / 896).  The same row count comes from
# 8192 tokens routed top-16 over 112 experts, the regime where the expert products are
# bound by the matrix cores rather than by the weight stream.
K3_EP_SHARE = LayerConfig(name="k3_ep_share_112x1170", tokens=8192, seed=1006, precision="mx8",
                          **{**_K3, "E": 112})

PRESETS = {c.name: c for c in (TOY, K3_DECODE_B1, K3_DECODE_B64_ZIPF, K3_PREFILL_8K,
                               K3_PREFILL_8K_FP32, K3_PREFILL_8K_MX4, K2_MOE_1024_ZIPF, K3_EP_SHARE)}


def param_shapes(cfg: LayerConfig) -> dict:
    """Logical parameter shapes of one layer ([out, in] for every matrix)."""
    s = {"router": (cfg.E, cfg.d), "bias": (cfg.E,)}
    if cfg.l:
        s["w_down_latent"] = (cfg.l, cfg.d)
        s["w_up_latent"] = (cfg.d, cfg.l)
        if cfg.use_norm:
            s["norm_gamma"] = (cfg.l,)
    lin = cfg.l if cfg.l else cfg.d
    s["expert_gu"] = (cfg.E, 2 * cfg.m, lin)
    s["expert_down"] = (cfg.E, lin, cfg.m)
    if cfg.ms:
        s["shared_gu"] = (2 * cfg.ms, cfg.d)
        s["shared_down"] = (cfg.d, cfg.ms)
    return s


@dataclass
class DenseWeights:
    router: np.ndarray
    w_down_latent: np.ndarray
    w_up_latent: np.ndarray
    norm_gamma: np.ndarray
    shared_gu: np.ndarray
    shared_down: np.ndarray
    bias: np.ndarray


def dense_weights(cfg: LayerConfig, copy: int = 0) -> DenseWeights:
    """bf16 router, latent projections, norm gain, shared expert; fp32 bias.

    `copy` selects an independent copy of the dense weights (copy 0 is the
    layer; other copies exist only so that a benchmark can rotate weight sets
    larger than the last-level cache)."""
    seed = cfg.seed + 7919 * copy
    sfx = "" if copy == 0 else f"#copy{copy}"
    std = WEIGHT_STD
    router = normal_bf16(seed, "router" + sfx, 0, (cfg.E, cfg.d), std)
    wdn = normal_bf16(seed, "w_down_latent" + sfx, 0, (cfg.l, cfg.d), std)
    wup = normal_bf16(seed, "w_up_latent" + sfx, 0, (cfg.d, cfg.l), std)
    gamma = np.full((cfg.l,), BF16_ONE, np.uint16)
    sgu = normal_bf16(seed, "shared_gu" + sfx, 0, (2 * cfg.ms, cfg.d), std)
    sdn = normal_bf16(seed, "shared_down" + sfx, 0, (cfg.d, cfg.ms), std)
    return DenseWeights(router, wdn, wup, gamma, sgu, sdn, router_bias(cfg))


def router_bias(cfg: LayerConfig) -> np.ndarray:
    if cfg.bias_kind == "uniform":
        return uniform_f32(cfg.seed, "bias", 0, (cfg.E,), cfg.bias_a, cfg.bias_b)
    if cfg.bias_kind == "normal":
        return normal_f32(cfg.seed, "bias", 0, (cfg.E,), cfg.bias_b, cfg.bias_a)
    if cfg.bias_kind == "file":
        path = os.path.join(_HERE, "data", cfg.bias_file)
        b = np.fromfile(path, dtype="<f4")
        if b.shape != (cfg.E,):
            raise ValueError(f"bias file {path} holds {b.shape} values, expected {cfg.E}")
        return b
    raise ValueError(cfg.bias_kind)


@dataclass
class ExpertSlice:
    """Experts e0..e1-1 in canonical storage."""
    e0: int
    e1: int
    fmt: str
    gu: np.ndarray               # bf16 [n, 2m, l] or codes [n, 2m, l/2] (fp8: [n, 2m, l])
    down: np.ndarray             # bf16 [n, l, m]  or codes [n, l, m/2] (fp8: [n, l, m])
    gu_scale: np.ndarray | None = None    # [n, 2m, l/32] (fp8: fp32 [n, 2m/128, l/128])
    down_scale: np.ndarray | None = None  # [n, l, m/32] (fp8: fp32 [n, l/128, m/128])


def expert_slice(cfg: LayerConfig, e0: int, e1: int, out: ExpertSlice | None = None) -> ExpertSlice:
    """Regenerate experts e0..e1-1 (any range, independently of the others)."""
    n = e1 - e0
    lin = cfg.l if cfg.l else cfg.d
    r_gu, c_gu = 2 * cfg.m, lin
    r_dn, c_dn = lin, cfg.m
    if cfg.expert_fmt == "bf16":
        gu = normal_bf16(cfg.seed, "expert_gu", e0 * r_gu * c_gu, (n, r_gu, c_gu), WEIGHT_STD,
                         out=None if out is None else out.gu)
        dn = normal_bf16(cfg.seed, "expert_down", e0 * r_dn * c_dn, (n, r_dn, c_dn), WEIGHT_STD,
                         out=None if out is None else out.down)
        return ExpertSlice(e0, e1, "bf16", gu, dn)
    if cfg.expert_fmt == "mxfp4":
        if c_gu % 32 or c_dn % 32:
            raise ValueError("MXFP4 needs reduction widths divisible by 32")
        gu = random_bytes(cfg.seed, "expert_gu_codes", e0 * r_gu * (c_gu // 2),
                          (n, r_gu, c_gu // 2), out=None if out is None else out.gu)
        gus = uniform_int_u8(cfg.seed, "expert_gu_scales", e0 * r_gu * (c_gu // 32),
                             (n, r_gu, c_gu // 32), cfg.e8m0_lo, cfg.e8m0_hi,
                             out=None if out is None else out.gu_scale)
        dn = random_bytes(cfg.seed, "expert_down_codes", e0 * r_dn * (c_dn // 2),
                          (n, r_dn, c_dn // 2), out=None if out is None else out.down)
        dns = uniform_int_u8(cfg.seed, "expert_down_scales", e0 * r_dn * (c_dn // 32),
                             (n, r_dn, c_dn // 32), cfg.e8m0_lo, cfg.e8m0_hi,
                             out=None if out is None else out.down_scale)
        return ExpertSlice(e0, e1, "mxfp4", gu, dn, gus, dns)
    if cfg.expert_fmt == "fp8b128":
        gu = np.empty((n, r_gu, c_gu), np.uint8) if out is None else out.gu
        dn = np.empty((n, r_dn, c_dn), np.uint8) if out is None else out.down
        gus = (np.empty((n, (r_gu + 127) // 128, (c_gu + 127) // 128), np.float32)
               if out is None else out.gu_scale)
        dns = (np.empty((n, (r_dn + 127) // 128, (c_dn + 127) // 128), np.float32)
               if out is None else out.down_scale)
        for i in range(n):
            e = e0 + i
            fp8_block128(cfg.seed, "expert_gu", e * r_gu * c_gu, r_gu, c_gu, WEIGHT_STD, gu[i], gus[i])
            fp8_block128(cfg.seed, "expert_down", e * r_dn * c_dn, r_dn, c_dn, WEIGHT_STD, dn[i], dns[i])
        return ExpertSlice(e0, e1, "fp8b128", gu, dn, gus, dns)
    raise ValueError(cfg.expert_fmt)


def tokens(cfg: LayerConfig, batch: int = 0, T: int | None = None) -> np.ndarray:
    """bf16 token batch x [T, d] ~ N(0, 1); each batch index is its own stream."""
    T = cfg.tokens if T is None else T
    return normal_bf16(cfg.seed, f"x#{batch}", 0, (T, cfg.d), 1.0)

