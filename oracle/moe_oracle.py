"""Float64 CPU oracle of the Stable LatentMoE FFN layer forward (test infrastructure only).

What it computes, per token t (the K3 latent-MoE block card, "All 23 steps";
the same order as the card's code excerpt of `KimiSparseMoeBlock.forward`):

  router      z = x W_r,  s = sigmoid(z)                       (card: Router)
  selection   I = top_k(s + b), descending, ties to the lower index
  weights     G_j = route_scale * s_{I_j} / sum_j' s_{I_j'}     (card: G_i; K3 has no scale,
                                                               the K2 card multiplies by 2.827)
  latent      x^c = x W_down_latent                            (card: x^c)
  experts     g = x^c W_gate, u = x^c W_up,
              h = 4 tanh(g/4) sigmoid(g) * 25 tanh(u/25),      (card: Routed expert; the
              E_j = h W_down                                    walkthrough's SituAndMul)
  combine     u = sum_j G_j E_j                                (card: u = sum_i G_i E_i)
  norm        u_hat = u / sqrt(mean(u^2) + eps) * gamma        (card code: routed_expert_norm
                                                               between the sum and W_up)
  up          y_routed = u_hat W_up_latent
  shared      y_shared = SiTU-GLU(x) at full width (merged 2 x 3072 = 6144 hidden)
  output      Delta = y_routed + y_shared

Precision: every continuous quantity is float64 on exactly dequantised weights
(bf16 and MXFP4 values are exact in float64).  The one place where floating
point decides an integer, the top-k selection, is taken in float32 as the
kernel takes it: kappa = float32(s) + float32(b).

Precision profiles.  "fp32" (the default) rounds nothing.  "mx8" inserts exactly
the rounding points that a compute-bound path declares, and nothing else:
  - the experts' input x^c and their hidden h are converted to MXFP8-E4M3
    (the walkthrough's deployment recipe: MXFP4 weights with MXFP8 activations),
    blocks of 32 along the reduction axis, by the OCP MX conversion rule;
  - the normalised latent u_hat and the shared hidden h_s are rounded to bf16
    (nearest, ties to even) before their products with W_up and W_shared_down.
"mx4" is "mx8" with MXFP4-E2M1 in place of MXFP8-E4M3 for x^c and h (the same OCP MX
rule with the E2M1 element: scale exponent floor(log2 amax) - 2, saturation at 6): both
operands of the expert products in the walkthrough's MXFP4 weight format.  It is a
reported variant, not a default: its error against "fp32" is about ten times mx8's.

Readings of points the pages leave open are listed in the repository's design
notes; the ones that change arithmetic are stated where they act below.
"""
from __future__ import annotations

import math
import os
from dataclasses import dataclass
from typing import Callable

import numpy as np

__all__ = [
    "bf16_to_f64", "e2m1_decode", "e8m0_decode", "dequant_mxfp4", "E2M1_GRID",
    "e4m3_decode", "round_e4m3", "E4M3_MAX", "quantize_mx8", "mx8_ambiguous", "round_bf16",
    "round_e2m1", "E2M1_MAX", "round_elem", "quantize_mx", "quantize_mx4", "mx_ambiguous",
    "MX_ELEMENTS", "MX_PROFILE_ELEMENT", "PRECISIONS",
    "dequant_fp8_block128",
    "sigmoid", "select_and_weight", "selection_kappa", "router_scores", "situ", "swiglu", "glu", "rmsnorm",
    "OracleLayer", "forward", "routed_sum_dense_mask", "Result", "dispatch", "residual_add",
]

# ----------------------------------------------------------------------------------------
# Formats.  The card states that routed experts are MXFP4 with one scale per 32 weights, and
# the port notes ("Notes from an NVFP4 port of Kimi K3", paragraph "Architecture facts") name
# the element as E2M1 and the scale as an E8M0 byte over each run of 32 columns.  The element and scale
# encodings are those of the OCP Microscaling Formats (MX) v1.0 specification:
#   E2M1: 1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit; exponent field 0 is
#         subnormal (value = mantissa * 0.5).
#   E8M0: unsigned 8-bit exponent, value 2^(e - 127); 0xFF encodes NaN.
# ----------------------------------------------------------------------------------------

#: Magnitudes of the eight non-negative E2M1 codes 0..7 as printed in OCP MX v1.0.
E2M1_GRID = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def bf16_to_f64(a: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly (bf16 is the top half of fp32)."""
    return (np.asarray(a).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def e2m1_decode(codes: np.ndarray) -> np.ndarray:
    """4-bit E2M1 codes (0..15) -> float64 from the field definition."""
    c = np.asarray(codes).astype(np.int64) & 0xF
    sign = np.where(c & 0x8, -1.0, 1.0)
    e = (c >> 1) & 0x3
    mant = (c & 0x1).astype(np.float64)
    mag = np.where(e == 0, 0.5 * mant, np.ldexp(1.0 + 0.5 * mant, (e - 1).astype(np.int64)))
    return sign * mag


def e8m0_decode(b: np.ndarray) -> np.ndarray:
    """E8M0 scale bytes -> float64: 2^(b-127), NaN for 0xFF."""
    b = np.asarray(b).astype(np.int64)
    v = np.ldexp(1.0, b - 127)
    return np.where(b == 0xFF, np.nan, v)


def dequant_mxfp4(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """MXFP4 block [.., rows, cols/2] codes + [.., rows, cols/32] E8M0 -> float64 [.., rows, cols].

    Two codes per byte, the low nibble holding the even column (storage convention of
    the synthetic layers); one scale per 32 consecutive columns of a row (the blocks run
    along the input axis, as the port notes' "Architecture facts" place them)."""
    codes = np.asarray(codes)
    lut = e2m1_decode(np.arange(16))
    cols = codes.shape[-1] * 2
    q = np.empty(codes.shape[:-1] + (cols,), np.float64)
    q[..., 0::2] = lut[codes & 0xF]
    q[..., 1::2] = lut[codes >> 4]
    s = e8m0_decode(scales)
    if s.shape[-1] * 32 != cols:
        raise ValueError("scale count does not match the block size of 32")
    q = q.reshape(q.shape[:-1] + (cols // 32, 32)) * s[..., None]
    return q.reshape(q.shape[:-2] + (cols,))


# FP8 E4M3 (the OCP 8-bit floating point formats, E4M3 variant; also the element format
# of MXFP8 in OCP MX v1.0): 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits;
# exponent field 0 is subnormal (value = mantissa/8 * 2^-6); S.1111.111 is NaN; there is
# no infinity, so the largest finite magnitude is 1.75 * 2^8 = 448.
E4M3_MAX = 448.0
#: Largest E2M1 magnitude (1.5 * 2^2).
E2M1_MAX = 6.0

#: Where the "mx8" and "mx4" profiles round (see the module docstring).
PRECISIONS = ("fp32", "mx8", "mx4")

#: Element formats of the MX conversions, from their field layouts: (largest exponent of a
#: normal value emax, largest magnitude, mantissa bits, exponent of the smallest normal).
#:   E4M3: normals 2^-6 .. 1.75 * 2^8, 3 mantissa bits;
#:   E2M1: normals 2^0 .. 1.5 * 2^2, 1 mantissa bit (0.5 is its one subnormal).
MX_ELEMENTS = {"e4m3": (8, E4M3_MAX, 3, -6), "e2m1": (2, E2M1_MAX, 1, 0)}
#: The element format of each MX profile.
MX_PROFILE_ELEMENT = {"mx8": "e4m3", "mx4": "e2m1"}


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """8-bit E4M3 codes -> float64 from the field definition (NaN for S.1111.111)."""
    c = np.asarray(codes).astype(np.int64) & 0xFF
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    mant = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, mant / 8.0 * 2.0 ** -6, np.ldexp(1.0 + mant / 8.0, (e - 7).astype(np.int64)))
    return np.where((c & 0x7F) == 0x7F, np.nan, sign * mag)


def dequant_fp8_block128(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """FP8 E4M3 codes [.., rows, cols] with one fp32 scale per 128 x 128 block
    [.., ceil(rows/128), ceil(cols/128)] -> float64: code value times its block's scale
    (the K2 block card's expert weights: FP8 with 128 x 128 block scales)."""
    codes = np.asarray(codes)
    rows, cols = codes.shape[-2:]
    s = np.asarray(scales, dtype=np.float64)
    full = np.repeat(np.repeat(s, 128, axis=-2), 128, axis=-1)[..., :rows, :cols]
    return e4m3_decode(codes) * full


def _binade(a: np.ndarray) -> np.ndarray:
    """floor(log2(a)) for a > 0 (exact, from the binary exponent); 0 where a == 0."""
    _, ex = np.frexp(a)
    return np.where(a > 0, ex - 1, 0).astype(np.int64)


def _quantum(a: np.ndarray, elem: str) -> np.ndarray:
    """Spacing of the element format's values around magnitude a: 2^(e - mantissa bits)
    in binade e, the subnormal spacing below the smallest normal."""
    _, _, mbits, emin = MX_ELEMENTS[elem]
    return np.ldexp(1.0, np.maximum(_binade(a), emin) - mbits)


def round_elem(y: np.ndarray, elem: str) -> np.ndarray:
    """The nearest value of the element format (ties to the even mantissa), saturated to
    its largest magnitude (the OCP MX conversion clamps values past the largest normal)."""
    y = np.asarray(y, dtype=np.float64)
    a = np.abs(y)
    quantum = _quantum(a, elem)
    r = np.round(a / quantum) * quantum        # numpy rounds halves to even
    return np.copysign(np.minimum(r, MX_ELEMENTS[elem][1]), y)


def round_e4m3(y: np.ndarray) -> np.ndarray:
    """The nearest E4M3 value (ties to the even mantissa), saturated to +-448: normal binade
    2^e (e >= -6) holds 8 values spaced 2^(e-3); below 2^-6 the subnormals are spaced 2^-9."""
    return round_elem(y, "e4m3")


def round_e2m1(y: np.ndarray) -> np.ndarray:
    """The nearest E2M1 value (ties to the even mantissa), saturated to +-6: binade 2^e
    (e >= 0) holds 2 values spaced 2^(e-1); below 1 the values 0 and 0.5."""
    return round_elem(y, "e2m1")


def _mx_exponent(amax: np.ndarray, emax: int, scale_flip: np.ndarray | None) -> np.ndarray:
    """Block exponent X = floor(log2(amax)) - emax (-127 for amax = 0); where `scale_flip` is
    set, the exponent of the other side of the power of two nearest amax (mx_ambiguous)."""
    X = np.where(amax > 0, _binade(amax) - emax, -127)
    if scale_flip is not None:
        # amax in [2^(X+emax), 2^(X+emax+1)): the nearer end decides which side is the other one
        upper = amax >= np.ldexp(np.sqrt(2.0), (X + emax).astype(np.int64))
        X = np.where(np.asarray(scale_flip, bool) & (amax > 0), np.where(upper, X + 1, X - 1), X)
    return np.clip(X, -127, 127)


def _neighbours(y: np.ndarray, elem: str):
    """The two element-format magnitudes around |y| (lo <= |y| < hi, spaced by the quantum
    of |y|'s binade)."""
    a = np.abs(y)
    quantum = _quantum(a, elem)
    lo = np.floor(a / quantum) * quantum
    return lo, lo + quantum


def quantize_mx(v: np.ndarray, elem: str, block: int = 32, flip: np.ndarray | None = None,
                scale_flip: np.ndarray | None = None):
    """MX conversion (one E8M0 scale per `block` values along the last axis) to element format
    `elem` ("e4m3": MXFP8, "e2m1": MXFP4), by the OCP MX v1.0 rule: X = floor(log2(max |v|))
    - emax per block (emax: the element format's largest normal exponent), -127 for an
    all-zero block, clamped to the E8M0 range; elements are v / 2^X rounded to the element
    format (round_elem).

    `scale_flip` (bool per block) and `flip` (bool per element) take the other valid decision
    where a value sits on a decision boundary (mx_ambiguous): the block exponent of the other
    side of the nearest power of two, or the other of the element's two neighbours (never
    past the largest magnitude).  Both are correct conversions of a value known only to the
    accuracy with which it was computed.

    Returns (dequantised values, element values, scale bytes X + 127)."""
    emax, vmax = MX_ELEMENTS[elem][:2]
    v = np.asarray(v, dtype=np.float64)
    shp = v.shape
    if shp[-1] % block:
        raise ValueError("the last axis must be a multiple of the block size")
    vb = v.reshape(shp[:-1] + (shp[-1] // block, block))
    amax = np.max(np.abs(vb), axis=-1)
    X = _mx_exponent(amax, emax, scale_flip)
    y = vb * np.ldexp(1.0, -X)[..., None]
    q = round_elem(y, elem)
    if flip is not None:
        lo, hi = _neighbours(y, elem)
        other = np.copysign(np.where(np.abs(q) == lo, hi, lo), y)
        take = np.asarray(flip, bool).reshape(q.shape) & (hi <= vmax)
        q = np.where(take, other, q)
    deq = q * np.ldexp(1.0, X)[..., None]
    return deq.reshape(shp), q.reshape(shp), (X + 127).astype(np.uint8)


def quantize_mx8(v: np.ndarray, block: int = 32, flip: np.ndarray | None = None,
                 scale_flip: np.ndarray | None = None):
    """MXFP8: quantize_mx with E4M3 elements (X = floor(log2 amax) - 8, saturation at 448)."""
    return quantize_mx(v, "e4m3", block, flip, scale_flip)


def quantize_mx4(v: np.ndarray, block: int = 32, flip: np.ndarray | None = None,
                 scale_flip: np.ndarray | None = None):
    """MXFP4: quantize_mx with E2M1 elements (X = floor(log2 amax) - 2, saturation at 6)."""
    return quantize_mx(v, "e2m1", block, flip, scale_flip)


def mx_ambiguous(v: np.ndarray, elem: str, eta: float, block: int = 32,
                 scale_flip: np.ndarray | None = None):
    """Where the MX conversion of v to `elem` takes a decision on a boundary, to within eta:
      - blocks whose amax lies within a relative eta of a power of two (the block exponent
        could fall on either side);
      - elements whose scaled value lies within eta * (the block's largest scaled magnitude)
        of the midpoint of its two neighbours (it could round either way), with the block
        exponents of `scale_flip` applied; midpoints past the largest magnitude are none
        (everything there saturates).
    A value computed with an error below those distances may legitimately convert to either
    decision.  Returns (element mask, block mask)."""
    emax, vmax = MX_ELEMENTS[elem][:2]
    v = np.asarray(v, dtype=np.float64)
    shp = v.shape
    vb = v.reshape(shp[:-1] + (shp[-1] // block, block))
    amax = np.max(np.abs(vb), axis=-1)
    p2 = np.ldexp(1.0, np.round(np.log2(np.where(amax > 0, amax, 1.0))).astype(np.int64))
    blk = (amax > 0) & (np.abs(amax / p2 - 1.0) <= eta)
    X = _mx_exponent(amax, emax, scale_flip)
    y = vb * np.ldexp(1.0, -X)[..., None]
    lo, hi = _neighbours(y, elem)
    ymax = (amax * np.ldexp(1.0, -X))[..., None]
    el = (np.abs(np.abs(y) - 0.5 * (lo + hi)) <= eta * ymax) & (hi <= vmax)
    return el.reshape(shp), blk


def mx8_ambiguous(v: np.ndarray, eta: float, block: int = 32, scale_flip: np.ndarray | None = None):
    """mx_ambiguous for the MXFP8 conversion."""
    return mx_ambiguous(v, "e4m3", eta, block, scale_flip)


def round_bf16(v: np.ndarray) -> np.ndarray:
    """The nearest bf16 value (ties to even) of float64 values: 8 significant bits over the
    fp32 exponent range (bf16 is the upper half of an fp32; subnormals below 2^-126)."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    e = np.maximum(_binade(a), -126)
    quantum = np.ldexp(1.0, e - 7)
    return np.copysign(np.round(a / quantum) * quantum, v)


# ----------------------------------------------------------------------------------------
# Router (block card: z = x W_r, s = sigmoid(z), selection by top_k(s + b), weights from the
# raw s renormalised; toy chapter: the bias decides who is invited, not how much each
# answer counts; port notes item (3)).
# ----------------------------------------------------------------------------------------

def sigmoid(z: np.ndarray) -> np.ndarray:
    """Logistic function in a form that is finite for every finite input."""
    z = np.asarray(z, dtype=np.float64)
    out = np.empty_like(z)
    pos = z >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-z[pos]))
    ez = np.exp(z[~pos])
    out[~pos] = ez / (1.0 + ez)
    return out


def router_scores(x: np.ndarray, w_router: np.ndarray) -> np.ndarray:
    """s[t, e] = sigmoid(sum_c x[t, c] W_r[e, c]), full model width (not the latent)."""
    return sigmoid(x @ w_router.T)


def select_and_weight(s: np.ndarray, bias: np.ndarray, k: int, route_scale: float = 1.0,
                      forced_idx: np.ndarray | None = None):
    """Top-k of kappa = s + b and the renormalised raw-score weights.

    Returns (idx [T, k] int32 in descending kappa order, ties to the lower expert index;
    G [T, k] float64; margin [T] = kappa_(k) - kappa_(k+1), +inf when E == k).
    kappa is formed in float32 (float32(s) + float32(b)) because that is the precision in
    which the kernel takes the same integer decision.  With `forced_idx` the selection
    is taken from the caller and only the weights are computed from s."""
    s = np.asarray(s, dtype=np.float64)
    T, E = s.shape
    kappa = s.astype(np.float32) + np.asarray(bias, dtype=np.float32)[None, :]
    order = np.argsort(-kappa, axis=1, kind="stable")
    if forced_idx is None:
        idx = order[:, :k]
    else:
        idx = np.asarray(forced_idx, dtype=np.int64)
    rows = np.arange(T)[:, None]
    ssel = s[rows, idx]
    G = route_scale * ssel / ssel.sum(axis=1, keepdims=True)
    if E > k:
        kk = kappa[rows[:, 0], order[:, k - 1]].astype(np.float64)
        k1 = kappa[rows[:, 0], order[:, k]].astype(np.float64)
        margin = kk - k1
    else:
        margin = np.full(T, np.inf)
    return idx.astype(np.int32), G, margin


def selection_kappa(s: np.ndarray, bias: np.ndarray, k: int) -> np.ndarray:
    """kappa = float32(s) + float32(b) of the k + 1 largest, in selection order [T, k+1]
    (as select_and_weight forms it), for the gaps between neighbours of the ranking; the
    (k+1)-th is -inf when E == k."""
    kappa = np.asarray(s, dtype=np.float64).astype(np.float32) + np.asarray(bias, dtype=np.float32)[None, :]
    order = np.argsort(-kappa, axis=1, kind="stable")[:, : k + 1]
    out = np.take_along_axis(kappa, order, axis=1).astype(np.float64)
    if out.shape[1] == k:     # E == k: no (k+1)-th expert, the margin is unbounded
        out = np.concatenate([out, np.full((out.shape[0], 1), -np.inf)], axis=1)
    return out


# ----------------------------------------------------------------------------------------
# Activations.  SiTU-GLU (walkthrough, Stable #2 and its SituAndMul excerpt; card: a, u-bar,
# h): the Swish gate's linear factor and the up branch are each soft-capped,
# softcap(z, beta) = beta tanh(z / beta); the sigmoid acts on the raw gate value.
# SwiGLU (K2 card): g sigmoid(g) * u.
# ----------------------------------------------------------------------------------------

def situ(g: np.ndarray, u: np.ndarray, beta_gate: float = 4.0, beta_lin: float = 25.0) -> np.ndarray:
    g = np.asarray(g, dtype=np.float64)
    u = np.asarray(u, dtype=np.float64)
    a = beta_gate * np.tanh(g / beta_gate) * sigmoid(g)
    ubar = beta_lin * np.tanh(u / beta_lin)
    return a * ubar


def swiglu(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    g = np.asarray(g, dtype=np.float64)
    return g * sigmoid(g) * np.asarray(u, dtype=np.float64)


def _act(cfg, g, u):
    if cfg.act == "situ":
        return situ(g, u, cfg.beta_gate, cfg.beta_lin)
    if cfg.act == "swiglu":
        return swiglu(g, u)
    raise ValueError(cfg.act)


def glu(xin: np.ndarray, w_gu: np.ndarray, w_down: np.ndarray, act: Callable,
        hidden_round: Callable | None = None) -> np.ndarray:
    """Three-matrix gated MLP: h = act(x W_gate, x W_up), out = h W_down.

    w_gu is [2m, K] with the gate rows first and the up rows second (the walkthrough's
    SituAndMul splits the last axis in half, gate then up); w_down is [K_out, m].
    `hidden_round`, when given, is applied to h before the down product (a declared
    rounding point of a precision profile)."""
    m = w_gu.shape[0] // 2
    g = xin @ w_gu[:m].T
    u = xin @ w_gu[m:].T
    h = act(g, u)
    if hidden_round is not None:
        h = hidden_round(h)
    return h @ w_down.T


def rmsnorm(u: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """u / sqrt(mean(u^2) + eps) * gamma over the last axis."""
    ms = np.mean(u * u, axis=-1, keepdims=True)
    return u / np.sqrt(ms + eps) * gamma


# ----------------------------------------------------------------------------------------
# The layer
# ----------------------------------------------------------------------------------------

class OracleLayer:
    """A layer in float64, built from the canonical bytes of `synth`.

    Dense weights are widened once; experts are dequantised on demand (one expert of the
    K3 layer is 132 MB in float64, the whole set would be 118 GB)."""

    def __init__(self, cfg, dense, expert_fn: Callable[[int], tuple] | None = None,
                 experts: tuple | None = None):
        self.cfg = cfg
        self.router = bf16_to_f64(dense.router)
        self.bias = np.asarray(dense.bias, dtype=np.float32)
        self.w_down_latent = bf16_to_f64(dense.w_down_latent) if cfg.l else None
        self.w_up_latent = bf16_to_f64(dense.w_up_latent) if cfg.l else None
        self.gamma = bf16_to_f64(dense.norm_gamma) if cfg.l and cfg.use_norm else None
        self.shared_gu = bf16_to_f64(dense.shared_gu) if cfg.ms else None
        self.shared_down = bf16_to_f64(dense.shared_down) if cfg.ms else None
        self._expert_fn = expert_fn
        self._experts = experts   # optional fully materialised (w_gu [E,2m,K], w_down [E,K,m])

    @classmethod
    def from_synth(cls, cfg, dense=None, preload: bool | None = None, expert_slice=None):
        """The layer of a `synth` config.  expert_slice(cfg, e0, e1): where the canonical
        expert bytes come from (synth.expert_slice by default; a caller may hand over bytes
        it generated beforehand).  The oracle dequantises them itself."""
        import synth
        dense = synth.dense_weights(cfg) if dense is None else dense
        small = cfg.E * 3 * cfg.m * (cfg.l or cfg.d) <= 64 * 1024 * 1024
        preload = small if preload is None else preload
        source = synth.expert_slice if expert_slice is None else expert_slice

        def expert_fn(e):
            return _expert_from_slice(source(cfg, e, e + 1), 0)

        experts = None
        if preload:
            sl = source(cfg, 0, cfg.E)
            gu, dn = _slice_to_f64(sl)
            experts = (gu, dn)
        return cls(cfg, dense, expert_fn, experts)

    def expert(self, e: int):
        """(w_gu [2m, K], w_down [K, m]) of expert e in float64."""
        if self._experts is not None:
            return self._experts[0][e], self._experts[1][e]
        return self._expert_fn(int(e))


def _slice_to_f64(sl):
    if sl.fmt == "bf16":
        return bf16_to_f64(sl.gu), bf16_to_f64(sl.down)
    if sl.fmt == "fp8b128":
        return dequant_fp8_block128(sl.gu, sl.gu_scale), dequant_fp8_block128(sl.down, sl.down_scale)
    return dequant_mxfp4(sl.gu, sl.gu_scale), dequant_mxfp4(sl.down, sl.down_scale)


def _expert_from_slice(sl, i):
    gu, dn = _slice_to_f64(sl)
    return gu[i], dn[i]


def _workers(layer: OracleLayer, workers: int | None) -> int:
    if workers is not None:
        return max(1, int(workers))
    if layer._experts is not None:      # small, preloaded layers: nothing to gain
        return 1
    return max(1, min(16, os.cpu_count() or 1))


def _map_ordered(fn, items, workers: int):
    """fn over items, results yielded in the order of items.  With several workers the
    calls run in a thread pool (numpy releases the interpreter lock in its array work) with
    the BLAS library held to one thread per call."""
    items = list(items)
    if workers <= 1 or len(items) <= 1:
        for it in items:
            yield fn(it)
        return
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1, user_api="blas"), ThreadPoolExecutor(workers) as ex:
        # at most 2 x workers calls submitted ahead of the one being consumed: each holds
        # one dequantised expert while it runs
        pending = []
        it = iter(items)
        for x in it:
            pending.append(ex.submit(fn, x))
            if len(pending) >= 2 * workers:
                break
        while pending:
            res = pending.pop(0).result()
            nxt = next(it, None)
            if nxt is not None:
                pending.append(ex.submit(fn, nxt))
            yield res


@dataclass
class Result:
    delta: np.ndarray      # [T, d] float64
    idx: np.ndarray        # [T, k] int32
    G: np.ndarray          # [T, k] float64
    margin: np.ndarray     # [T]
    xc: np.ndarray         # [T, l] latent input of the experts
    u: np.ndarray          # [T, l] gated sum before the norm
    y_routed: np.ndarray   # [T, d]
    y_shared: np.ndarray   # [T, d]


def forward(layer: OracleLayer, x_bf16: np.ndarray, forced_idx: np.ndarray | None = None,
            precision: str | None = None, workers: int | None = None,
            xc_flip: np.ndarray | None = None, xc_scale_flip: np.ndarray | None = None) -> Result:
    """The layer forward for tokens x [T, d] (bf16 bit patterns or float64 values).

    The routed sum is organised as the block card's `moe_infer` does it: assignments are
    grouped by expert, each expert runs once on the tokens that chose it, and each result
    is weighted by its G and added into its token's sum.  `forced_idx` replaces the
    selection (used for tokens whose top-k margin is a near tie).  `precision` is a
    profile of PRECISIONS (default: the layer config's `precision`, else "fp32").
    `workers`: threads that evaluate experts side by side (default: one per host core for
    layers whose experts are dequantised on demand, else 1); the result is the same.
    `xc_flip`, `xc_scale_flip` (mx profiles): take the other valid MX decision at the
    marked elements / blocks of x^c (quantize_mx), for tokens whose x^c has a value on a
    conversion boundary (mx_ambiguous), as forced routing does for top-k near ties."""
    cfg = layer.cfg
    precision = precision or getattr(cfg, "precision", "fp32")
    if precision not in PRECISIONS:
        raise ValueError(precision)
    elem = MX_PROFILE_ELEMENT.get(precision)          # None in "fp32"
    mx = elem is not None                             # the mx profiles' rounding points
    qmx = (lambda v: quantize_mx(v, elem)[0]) if mx else None  # noqa: E731
    x = bf16_to_f64(x_bf16) if np.asarray(x_bf16).dtype == np.uint16 else np.asarray(x_bf16, np.float64)
    T = x.shape[0]
    s = router_scores(x, layer.router)
    idx, G, margin = select_and_weight(s, layer.bias, cfg.k, cfg.route_scale, forced_idx)

    xc = x @ layer.w_down_latent.T if cfg.l else x
    xe = quantize_mx(xc, elem, flip=xc_flip, scale_flip=xc_scale_flip)[0] if mx else xc  # the experts' input
    lat = xc.shape[1]
    u = np.zeros((T, lat), np.float64)
    act = lambda g, v: _act(cfg, g, v)  # noqa: E731
    flat = idx.reshape(-1)

    def run_expert(e):
        tj = np.nonzero(flat == e)[0]
        t_rows, j_cols = tj // cfg.k, tj % cfg.k
        w_gu, w_dn = layer.expert(int(e))
        return t_rows, j_cols, glu(xe[t_rows], w_gu, w_dn, act, qmx)

    # The experts' outputs may be evaluated concurrently (each is a pure function of its
    # expert and rows); they are added into the sums one expert at a time in increasing
    # expert order either way, so the result does not depend on `workers`.
    for t_rows, j_cols, out in _map_ordered(run_expert, np.unique(flat), _workers(layer, workers)):
        u[t_rows] += G[t_rows, j_cols][:, None] * out   # one (t, e) pair per token at most

    if cfg.l:
        u_hat = rmsnorm(u, layer.gamma, cfg.eps) if cfg.use_norm else u
        if mx:
            u_hat = round_bf16(u_hat)
        y_r = u_hat @ layer.w_up_latent.T
    else:
        y_r = u
    if cfg.ms:
        y_s = glu(x, layer.shared_gu, layer.shared_down, act, round_bf16 if mx else None)
    else:
        y_s = np.zeros_like(y_r)
    return Result(y_r + y_s, idx, G, margin, xc, u, y_r, y_s)


def routed_sum_dense_mask(layer: OracleLayer, xc: np.ndarray, G_dense: np.ndarray) -> np.ndarray:
    """The card's definition u = sum_{i=1}^{E} G_i E_i with G_i = 0 off the selection:
    every expert is evaluated on every token (tiny shapes only)."""
    cfg = layer.cfg
    act = lambda g, v: _act(cfg, g, v)  # noqa: E731
    u = np.zeros((xc.shape[0], xc.shape[1]), np.float64)
    for e in range(cfg.E):
        w_gu, w_dn = layer.expert(e)
        u += G_dense[:, e:e + 1] * glu(xc, w_gu, w_dn, act)
    return u


def dispatch(idx: np.ndarray, n_experts: int):
    """The block card's moe_infer bookkeeping for the flattened assignments a = t*k + j:
    tokens_per_expert (a histogram of the selected ids), the argsort of the ids (stable, so
    assignments of one expert keep increasing a), and its inverse.

    Returns (counts [E], offsets [E+1] = exclusive scan of counts, perm [T*k], inv [T*k])."""
    flat = np.asarray(idx, dtype=np.int64).reshape(-1)
    counts = np.bincount(flat, minlength=n_experts).astype(np.int32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    perm = np.argsort(flat, kind="stable").astype(np.int32)
    inv = np.empty_like(perm)
    inv[perm] = np.arange(perm.size, dtype=np.int32)
    return counts, offsets, perm, inv


def residual_add(residual: np.ndarray, delta: np.ndarray):
    """The block's output joins the residual stream (the block card: the FFN returns
    Delta_ffn, the decoder layer adds it to its hidden state, h <- h + Delta): the new
    residual (float64) and its bf16 rounding, the next layer's input (uint16 patterns)."""
    new = np.asarray(residual, dtype=np.float64) + np.asarray(delta, dtype=np.float64)
    xb = round_bf16(new).astype(np.float32).view(np.uint32) >> 16
    return new, xb.astype(np.uint16)

