"""The parity rule between the HIP path's outputs and the CPU oracle's (test infrastructure,
shared by the GPU tests and the benchmark's CPU-baseline leg; it calls the oracle only).

Bars (restating the layer's acceptance rule):
  - on every token whose oracle top-k margin kappa_(k) - kappa_(k+1) is >= MARGIN, the
    oracle's set of experts, in the oracle's order wherever neighbouring kappas are
    >= MARGIN apart (near ties are reported, and their Delta is compared with the oracle
    run on the GPU's own selection);
  - gate weights within 1e-6 of the oracle's G where the indices agree;
  - Delta: relative L2 error <= REL_L2 and max abs error <= MAX_ABS_RMS * rms(Delta_oracle).
In the mx profiles the MX conversion of x^c (MXFP8-E4M3 in mx8, MXFP4-E2M1 in mx4) takes
integer decisions (block exponents, element codes) on computed values: the GPU's decisions
must equal the oracle's except where the oracle marks one as on a boundary (within MX8_ETA),
and tokens where the GPU took the other valid decision are compared with the oracle taking
it too.
"""
from __future__ import annotations

import time

import numpy as np

import oracle as O

REL_L2 = 2e-3
MAX_ABS_RMS = 1e-2
MARGIN = 1e-5
MX8_ETA = 1e-4   # relative to the block's largest magnitude (O.mx_ambiguous), both mx profiles


class ParityError(AssertionError):
    pass


def _need(ok: bool, msg: str):
    if not ok:
        raise ParityError(msg)


def routing(idx, ridx, kap, margin, log=print):
    """The index rule.  On every token whose margin is >= MARGIN the GPU selects the oracle's
    set of experts, and the oracle's expert at every rank whose kappa is at least MARGIN
    away from both neighbours (experts whose kappas lie closer than that may come out in
    either order).  Raises ParityError otherwise; returns the mask of clear tokens."""
    clear = margin >= MARGIN
    _need(np.array_equal(np.sort(idx[clear], 1), np.sort(ridx[clear], 1)),
          "expert sets differ on clear margins")
    k = idx.shape[1]
    gaps = kap[:, :-1] - kap[:, 1:]                 # rank j to j + 1, j = 0..k-1
    left = np.concatenate([np.full((len(kap), 1), np.inf), gaps[:, : k - 1]], axis=1)
    pinned = (left >= MARGIN) & (gaps >= MARGIN)
    bad = clear[:, None] & pinned & (idx != ridx)
    _need(not bad.any(), f"rank order differs at clear gaps on tokens {np.nonzero(bad.any(1))[0][:8]}")
    swapped = clear & np.any(idx != ridx, axis=1)
    if swapped.any():
        log(f"tokens with near-equal neighbours ranked in the other order: {int(swapped.sum())}")
    return clear


def by_expert(idx, w):
    """Weights reordered by expert id (for comparing tokens whose ranking differs only
    between near-equal neighbours)."""
    o = np.argsort(idx, axis=1)
    return np.take_along_axis(idx, o, 1), np.take_along_axis(w, o, 1)


def gpu_codes(xq, elem):
    """Element values of GPU code rows: E4M3 bytes, or bytes of two E2M1 codes (the low
    nibble holding the even column)."""
    xq = np.asarray(xq)
    if elem == "e4m3":
        return O.e4m3_decode(xq)
    nib = np.empty(xq.shape[:-1] + (2 * xq.shape[-1],), np.uint8)
    nib[..., 0::2] = xq & 0xF
    nib[..., 1::2] = xq >> 4
    return O.e2m1_decode(nib)


def mx_decisions(xc, xq, xs, elem="e4m3", log=print):
    """The GPU's MX decisions on x^c (code rows [T, ...] uint8, scale bytes [T, >= l/32])
    against the oracle's (x^c float64 [T, l]) for element format `elem`: they must agree
    except where the oracle marks a boundary.  Returns (element mask, block mask) of the
    other decisions the GPU took."""
    l = xc.shape[1]
    gq = gpu_codes(xq, elem)[:, :l]
    gs = xs[:, : l // 32]
    _, _, osb = O.quantize_mx(xc, elem)
    _, blk_amb = O.mx_ambiguous(xc, elem, MX8_ETA)
    sflip = gs != osb
    _need(not np.any(sflip & ~blk_amb),
          f"x^c block exponents differ away from a power of two on tokens "
          f"{np.nonzero((sflip & ~blk_amb).any(1))[0][:8]}")
    _, oq, _ = O.quantize_mx(xc, elem, scale_flip=sflip)
    el_amb, _ = O.mx_ambiguous(xc, elem, MX8_ETA, scale_flip=sflip)
    eflip = gq != oq
    _need(not np.any(eflip & ~el_amb),
          f"x^c codes differ away from an {elem.upper()} midpoint on tokens "
          f"{np.nonzero((eflip & ~el_amb).any(1))[0][:8]}")
    log(f"x^c MX ({elem}) decisions on a boundary taken the other way: {int(eflip.sum())} codes, "
        f"{int(sflip.sum())} block exponents, on {int((eflip.any(1) | sflip.any(1)).sum())} tokens "
        f"(oracle-marked boundary values: {int(el_amb.sum())} codes, {int(blk_amb.sum())} blocks)")
    return eflip, sflip


def compare(OL, x, delta, idx, w, precision=None, ref=None, xcq=None, bars=True, log=print):
    """Compare GPU outputs (delta [T, d], idx and w [T, k], numpy) for the tokens x [T, d]
    (bf16 patterns) with the oracle layer OL in `precision` (the layer's own profile by
    default; `ref`: that oracle's result for x, when already computed).  xcq: the GPU's MX
    x^c (code rows, scale bytes) in an mx profile.  Raises ParityError when the index rule,
    the gate weights or (with `bars`) the Delta bars fail.  Returns a dict of the errors and
    the oracle's result under "ref"."""
    cfg = OL.cfg
    prof = precision or getattr(cfg, "precision", "fp32")
    t0 = time.perf_counter()
    if ref is None:
        ref = O.forward(OL, x, precision=precision)
    near = ref.margin < MARGIN
    kap = O.selection_kappa(O.router_scores(O.bf16_to_f64(x), OL.router), OL.bias, cfg.k)
    routing(idx, ref.idx, kap, ref.margin, log)
    gi, gw = by_expert(idx, w)
    ri, rg = by_expert(ref.idx, ref.G)
    same = np.all(gi == ri, axis=1)
    _need(np.max(np.abs(gw[same] - rg[same]), initial=0.0) <= 1e-6, "gate weights differ by more than 1e-6")
    ref_delta = ref.delta.copy()
    redo = ~same
    eflip = sflip = None
    if prof in O.MX_PROFILE_ELEMENT and xcq is not None:
        eflip, sflip = mx_decisions(ref.xc, xcq[0], xcq[1], O.MX_PROFILE_ELEMENT[prof], log)
        redo = redo | eflip.any(1) | sflip.any(1)
    if np.any(~same):
        log(f"near-tie tokens {np.nonzero(~same)[0].tolist()[:16]} margins {ref.margin[~same].tolist()[:16]}")
    if np.any(redo):   # the oracle on the GPU's selection and boundary decisions
        forced = O.forward(OL, x[redo], forced_idx=idx[redo], precision=precision,
                           xc_flip=None if eflip is None else eflip[redo],
                           xc_scale_flip=None if sflip is None else sflip[redo])
        ref_delta[redo] = forced.delta
    err = delta - ref_delta
    rel = float(np.linalg.norm(err) / np.linalg.norm(ref_delta))
    rms = float(np.sqrt(np.mean(ref_delta ** 2)))
    mx = float(np.max(np.abs(err)))
    out = {"tokens": int(x.shape[0]), "profile": prof, "rel_l2": rel, "max_abs_over_rms": mx / rms,
           "near_tie_tokens": int(near.sum()), "recomputed_tokens": int(redo.sum()),
           "seconds": time.perf_counter() - t0, "ref": ref}
    log(f"{cfg.name} [oracle {prof}]: tokens {x.shape[0]} rel-L2 {rel:.3e} "
        f"max-abs/rms {mx / rms:.3e} near-ties {int(near.sum())} ({out['seconds']:.0f} s on the host)")
    if bars:
        _need(rel <= REL_L2, f"rel-L2 {rel:.3e} > {REL_L2}")
        _need(mx <= MAX_ABS_RMS * rms,
              f"max-abs/rms {mx / rms:.3e} on token {int(np.argmax(np.max(np.abs(err), 1)))}")
    return out
