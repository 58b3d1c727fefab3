"""Python binding of libmoe.so, the gfx950 Stable LatentMoE FFN layer library.

Argument marshalling only: every step of the layer runs in the HIP kernels behind the
C ABI declared in include/moe.h.  PyTorch provides device memory and the current stream.
The binding refuses to run if libmoe.so has not been built (there is no fallback).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
ACT = {"situ": 0, "swiglu": 1}
WFMT = {"bf16": 0, "mxfp4": 1, "fp8b128": 2}
PREC = {"fp32": 0, "mx8": 1, "mx4": 2}
WS_SLOTS = ("ctrl", "xc", "hs", "h", "eo", "u", "uh", "hl", "perm", "inv", "counts", "offsets", "z",
            "chunk_hist", "units")

EXPORTS = ("moe_abi_version", "moe_status_str", "moe_packed_dense_size", "moe_pack_dense",
           "moe_packed_experts_size", "moe_pack_experts", "moe_workspace_size",
           "moe_workspace_layout", "moe_layer_forward",
           "moe_layer_forward_timed", "moe_layer_forward_steps", "moe_route", "moe_dispatch",
           "moe_qb_histogram", "moe_qb_readout", "moe_layer_forward_residual",
           "moe_layer_forward_noalloc", "moe_layer_forward_residual_prefetch")
STEPS = ("router", "in", "route", "dispatch", "expert_gu", "expert_down", "combine", "out")
ABI_VERSION = 7
STATIC_WORKSPACE_BYTES = 64 << 20   # MOE_STATIC_WORKSPACE_BYTES


class MoeConfig(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int32), ("d_latent", ctypes.c_int32),
                ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("d_expert", ctypes.c_int32), ("d_shared", ctypes.c_int32),
                ("use_latent_norm", ctypes.c_int32), ("rms_eps", ctypes.c_float),
                ("route_scale", ctypes.c_float), ("beta_gate", ctypes.c_float),
                ("beta_lin", ctypes.c_float), ("act", ctypes.c_int32),
                ("expert_wfmt", ctypes.c_int32), ("precision", ctypes.c_int32)]


class MoeWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("dense", "experts")]


class MoeDenseSrc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("router", "w_down_latent", "w_up_latent",
                                                "norm_gamma", "shared_gu", "shared_down")]


class MoeExpertSrc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("gu", "gu_scale", "down", "down_scale")]


class MoeError(RuntimeError):
    def __init__(self, what: str, status: int):
        super().__init__(f"{what} failed: {status_str(status)} ({status})")
        self.status = status


_lib = None


def lib():
    """The loaded libmoe.so (raises if it was not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                           "(hipcc, gfx950); there is no fallback path")
    try:   # load torch's HIP runtime first so that both share one runtime (same soname)
        import torch  # noqa: F401
    except ImportError:
        pass
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    vp, i64, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
    L.moe_abi_version.restype = ctypes.c_int
    L.moe_status_str.restype = ctypes.c_char_p
    L.moe_status_str.argtypes = [ctypes.c_int]
    L.moe_packed_dense_size.argtypes = [P(MoeConfig), P(sz)]
    L.moe_pack_dense.argtypes = [P(MoeConfig), P(MoeDenseSrc), vp, sz, vp]
    L.moe_packed_experts_size.argtypes = [P(MoeConfig), P(sz)]
    L.moe_pack_experts.argtypes = [P(MoeConfig), P(MoeExpertSrc), ctypes.c_int32, ctypes.c_int32,
                                   vp, sz, vp]
    L.moe_workspace_size.argtypes = [P(MoeConfig), i64, P(sz)]
    L.moe_workspace_layout.argtypes = [P(MoeConfig), i64, P(sz)]
    L.moe_layer_forward.argtypes = [P(MoeConfig), P(MoeWeights), vp, vp, i64, vp, vp, vp, vp, sz, vp]
    L.moe_layer_forward_timed.argtypes = [P(MoeConfig), P(MoeWeights), vp, vp, i64, vp, vp, vp,
                                          vp, sz, vp, vp]
    L.moe_layer_forward_steps.argtypes = [P(MoeConfig), P(MoeWeights), vp, vp, i64, vp, vp, vp,
                                          vp, sz, ctypes.c_int32, ctypes.c_int32, vp]
    L.moe_route.argtypes = [P(MoeConfig), P(MoeWeights), vp, vp, i64, vp, vp, vp, sz, vp]
    L.moe_dispatch.argtypes = [P(MoeConfig), vp, i64, vp, vp, vp, vp, vp, sz, vp]
    i32 = ctypes.c_int32
    L.moe_qb_histogram.argtypes = [P(MoeConfig), P(MoeWeights), vp, vp, i64, i32, vp, vp, sz, vp]
    L.moe_qb_readout.argtypes = [P(MoeConfig), vp, i32, vp, i64, vp, vp]
    L.moe_layer_forward_residual.argtypes = [P(MoeConfig), P(MoeWeights), vp, vp, i64, vp, vp, vp,
                                             vp, vp, vp, sz, vp]
    L.moe_layer_forward_noalloc.argtypes = [P(MoeConfig), P(MoeWeights), vp, vp, i64, vp, vp, vp, vp]
    L.moe_layer_forward_residual_prefetch.argtypes = [P(MoeConfig), P(MoeWeights), vp, vp, i64, vp,
                                                      vp, vp, vp, vp, vp, sz, P(MoeWeights), vp]
    for f in EXPORTS[2:]:
        getattr(L, f).restype = ctypes.c_int
    if L.moe_abi_version() != ABI_VERSION:
        raise RuntimeError(f"{LIB_PATH} has ABI {L.moe_abi_version()}, the binding expects "
                           f"{ABI_VERSION}: rebuild it")
    _lib = L
    return L


def status_str(s: int) -> str:
    return lib().moe_status_str(int(s)).decode()


def _check(st: int, what: str):
    if st != MOE_OK:
        raise MoeError(what, st)


def make_config(d, l, E, k, m, ms, expert_fmt="mxfp4", act="situ", route_scale=1.0,
                use_norm=True, eps=1e-6, beta_gate=4.0, beta_lin=25.0,
                precision="fp32") -> MoeConfig:
    return MoeConfig(d, l, E, k, m, ms, 1 if use_norm else 0, eps, route_scale, beta_gate,
                     beta_lin, ACT[act], WFMT[expert_fmt], PREC[precision])


def config_from(c) -> MoeConfig:
    """MoeConfig from any object with the layer-config attribute names."""
    return make_config(c.d, c.l, c.E, c.k, c.m, c.ms, c.expert_fmt, c.act, c.route_scale,
                       c.use_norm, c.eps, c.beta_gate, c.beta_lin,
                       getattr(c, "precision", "fp32"))


def workspace_size(cfg: MoeConfig, max_tokens: int) -> int:
    n = ctypes.c_size_t()
    _check(lib().moe_workspace_size(ctypes.byref(cfg), int(max_tokens), ctypes.byref(n)),
           "moe_workspace_size")
    return n.value


def workspace_layout(cfg: MoeConfig, n_tokens: int) -> dict:
    off = (ctypes.c_size_t * len(WS_SLOTS))()
    _check(lib().moe_workspace_layout(ctypes.byref(cfg), int(n_tokens), off), "moe_workspace_layout")
    return dict(zip(WS_SLOTS, list(off)))


def packed_dense_size(cfg: MoeConfig) -> int:
    n = ctypes.c_size_t()
    _check(lib().moe_packed_dense_size(ctypes.byref(cfg), ctypes.byref(n)), "moe_packed_dense_size")
    return n.value


def new_workspace(cfg: MoeConfig, max_tokens: int, device):
    """A device workspace for up to max_tokens tokens, its control words zeroed (as a
    workspace must start; the calls leave them so)."""
    import torch
    ws = torch.empty(max(workspace_size(cfg, max_tokens), 256), dtype=torch.uint8, device=device)
    ws[:256].zero_()
    return ws


def packed_experts_size(cfg: MoeConfig) -> int:
    n = ctypes.c_size_t()
    _check(lib().moe_packed_experts_size(ctypes.byref(cfg), ctypes.byref(n)),
           "moe_packed_experts_size")
    return n.value


def _stream(stream=None) -> int:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _dev_u16(a, device):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device)


def _dev_u8(a, device):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def pack_dense(cfg: MoeConfig, dense, device="cuda"):
    """Upload canonical dense weights (numpy, bf16 patterns) and pack them on the device."""
    import torch
    t = [_dev_u16(getattr(dense, n), device) if getattr(dense, n) is not None else None
         for n in ("router", "w_down_latent", "w_up_latent", "norm_gamma", "shared_gu",
                   "shared_down")]
    packed = torch.empty(packed_dense_size(cfg), dtype=torch.uint8, device=device)
    stream = torch.cuda.current_stream(device)
    src = MoeDenseSrc(*[_ptr(v) for v in t])
    _check(lib().moe_pack_dense(ctypes.byref(cfg), ctypes.byref(src), packed.data_ptr(),
                                packed.numel(), stream.cuda_stream), "moe_pack_dense")
    stream.synchronize()   # the canonical staging tensors are released on return
    return packed


class Layer:
    """One layer resident on the device: the packed dense weights (moe_pack_dense), the
    fp32 bias and the routed experts packed by moe_pack_experts (torch device tensors)."""

    def __init__(self, cfg: MoeConfig, dense, bias, experts):
        self.cfg = cfg
        self.dense, self.bias, self.experts = dense, bias, experts
        self._ws = None

    @property
    def device(self):
        return self.dense.device

    def weights_struct(self) -> MoeWeights:
        return MoeWeights(_ptr(self.dense), _ptr(self.experts))

    def with_dense(self, dense, device=None) -> "Layer":
        """The same packed experts with another set of dense weights (numpy canonical)."""
        device = self.device if device is None else device
        return Layer(self.cfg, pack_dense(self.cfg, dense, device), self.bias, self.experts)

    @classmethod
    def upload(cls, cfg: MoeConfig, dense, expert_slice, n_experts: int, device="cuda",
               chunk: int = 64) -> "Layer":
        """Upload canonical numpy arrays and pack the dense weights and the experts on the
        device.

        dense: object with router, w_down_latent, w_up_latent, norm_gamma, shared_gu,
        shared_down (uint16 bf16 patterns) and bias (float32).  expert_slice(e0, e1) returns
        an object with gu, down (and gu_scale, down_scale for MXFP4) for experts e0..e1-1."""
        import torch
        experts = torch.empty(packed_experts_size(cfg), dtype=torch.uint8, device=device)
        stream = torch.cuda.current_stream(device)
        for e0 in range(0, n_experts, chunk):
            e1 = min(n_experts, e0 + chunk)
            sl = expert_slice(e0, e1)
            if cfg.expert_wfmt == WFMT["mxfp4"]:
                t = [_dev_u8(sl.gu, device), _dev_u8(sl.gu_scale, device),
                     _dev_u8(sl.down, device), _dev_u8(sl.down_scale, device)]
            elif cfg.expert_wfmt == WFMT["fp8b128"]:
                t = [_dev_u8(sl.gu, device), _dev_u8(np.ascontiguousarray(sl.gu_scale, np.float32).view(np.uint8), device),
                     _dev_u8(sl.down, device), _dev_u8(np.ascontiguousarray(sl.down_scale, np.float32).view(np.uint8), device)]
            else:
                t = [_dev_u16(sl.gu, device), None, _dev_u16(sl.down, device), None]
            src = MoeExpertSrc(*[_ptr(v) for v in t])
            _check(lib().moe_pack_experts(ctypes.byref(cfg), ctypes.byref(src), e0, e1 - e0,
                                          experts.data_ptr(), experts.numel(), stream.cuda_stream),
                   "moe_pack_experts")
            stream.synchronize()   # staging tensors are released at the next iteration
        bias = torch.from_numpy(np.ascontiguousarray(dense.bias, dtype=np.float32)).to(device)
        return cls(cfg, pack_dense(cfg, dense, device), bias, experts)

    def workspace(self, n_tokens: int):
        need = workspace_size(self.cfg, n_tokens)
        if self._ws is None or self._ws.numel() < need:
            self._ws = new_workspace(self.cfg, n_tokens, self.device)
        return self._ws

    def forward(self, x, delta=None, idx=None, w=None, workspace=None, stream=None):
        """x: [T, d] bf16 patterns (torch int16/uint16/bfloat16 on the device).
        Returns (delta [T, d] fp32, topk_idx [T, k] int32, topk_w [T, k] fp32)."""
        import torch
        T = x.shape[0]
        c = self.cfg
        dev = self.device
        delta = torch.empty((T, c.d_model), dtype=torch.float32, device=dev) if delta is None else delta
        idx = torch.empty((T, c.top_k), dtype=torch.int32, device=dev) if idx is None else idx
        w = torch.empty((T, c.top_k), dtype=torch.float32, device=dev) if w is None else w
        ws = self.workspace(T) if workspace is None else workspace
        W = self.weights_struct()
        _check(lib().moe_layer_forward(ctypes.byref(c), ctypes.byref(W), self.bias.data_ptr(),
                                       x.data_ptr(), T, delta.data_ptr(), idx.data_ptr(),
                                       w.data_ptr(), ws.data_ptr(), ws.numel(), _stream(stream)),
               "moe_layer_forward")
        return delta, idx, w

    def forward_noalloc(self, x, delta, idx, w, stream=None):
        """forward() through moe_layer_forward_noalloc: the intermediates in the library's
        own per-GPU buffer (no workspace).  delta, idx, w: preallocated outputs."""
        W = self.weights_struct()
        _check(lib().moe_layer_forward_noalloc(ctypes.byref(self.cfg), ctypes.byref(W),
                                               self.bias.data_ptr(), x.data_ptr(), x.shape[0],
                                               delta.data_ptr(), idx.data_ptr(), w.data_ptr(),
                                               _stream(stream)), "moe_layer_forward_noalloc")
        return delta, idx, w

    def forward_residual(self, x, residual, x_next=None, delta=None, idx=None, w=None,
                         workspace=None, stream=None):
        """forward() with residual += Delta fused into the last step (residual fp32 [T, d]
        on the device, updated in place) and, when x_next is given (bf16 patterns [T, d],
        may be x itself), the updated residual rounded to bf16.  Returns (idx, w)."""
        import torch
        T = x.shape[0]
        c = self.cfg
        idx = torch.empty((T, c.top_k), dtype=torch.int32, device=self.device) if idx is None else idx
        w = torch.empty((T, c.top_k), dtype=torch.float32, device=self.device) if w is None else w
        ws = self.workspace(T) if workspace is None else workspace
        W = self.weights_struct()
        _check(lib().moe_layer_forward_residual(
            ctypes.byref(c), ctypes.byref(W), self.bias.data_ptr(), x.data_ptr(), T,
            residual.data_ptr(), None if x_next is None else x_next.data_ptr(),
            None if delta is None else delta.data_ptr(), idx.data_ptr(), w.data_ptr(),
            ws.data_ptr(), ws.numel(), _stream(stream)), "moe_layer_forward_residual")
        return idx, w

    def forward_residual_prefetch(self, x, residual, next_layer, x_next=None, delta=None, idx=None,
                                  w=None, workspace=None, stream=None):
        """forward_residual() that also reads, in its last launch, the weight bytes the next
        layer's first launch reads (next_layer: a Layer of the same config, or None)."""
        import torch
        T = x.shape[0]
        c = self.cfg
        idx = torch.empty((T, c.top_k), dtype=torch.int32, device=self.device) if idx is None else idx
        w = torch.empty((T, c.top_k), dtype=torch.float32, device=self.device) if w is None else w
        ws = self.workspace(T) if workspace is None else workspace
        W = self.weights_struct()
        N = None if next_layer is None else ctypes.byref(next_layer.weights_struct())
        _check(lib().moe_layer_forward_residual_prefetch(
            ctypes.byref(c), ctypes.byref(W), self.bias.data_ptr(), x.data_ptr(), T,
            residual.data_ptr(), None if x_next is None else x_next.data_ptr(),
            None if delta is None else delta.data_ptr(), idx.data_ptr(), w.data_ptr(),
            ws.data_ptr(), ws.numel(), N, _stream(stream)), "moe_layer_forward_residual_prefetch")
        return idx, w

    def forward_timed(self, x, events, delta, idx, w, workspace=None, stream=None):
        """forward() that also records events[s] (hipEvent_t handles, len(STEPS) + 1) on the
        stream before each step and after the last."""
        c = self.cfg
        T = x.shape[0]
        ws = self.workspace(T) if workspace is None else workspace
        W = self.weights_struct()
        ev = (ctypes.c_void_p * (len(STEPS) + 1))(*events)
        _check(lib().moe_layer_forward_timed(ctypes.byref(c), ctypes.byref(W), self.bias.data_ptr(),
                                             x.data_ptr(), T, delta.data_ptr(), idx.data_ptr(),
                                             w.data_ptr(), ws.data_ptr(), ws.numel(), ev,
                                             _stream(stream)), "moe_layer_forward_timed")
        return delta, idx, w

    def forward_steps(self, x, begin, end, delta, idx, w, workspace, stream=None):
        """Steps begin..end-1 of the forward on the buffers of an earlier call."""
        W = self.weights_struct()
        _check(lib().moe_layer_forward_steps(ctypes.byref(self.cfg), ctypes.byref(W),
                                             self.bias.data_ptr(), x.data_ptr(), x.shape[0],
                                             delta.data_ptr(), idx.data_ptr(), w.data_ptr(),
                                             workspace.data_ptr(), workspace.numel(), begin, end,
                                             _stream(stream)), "moe_layer_forward_steps")

    def route(self, x, stream=None):
        import torch
        T = x.shape[0]
        c = self.cfg
        idx = torch.empty((T, c.top_k), dtype=torch.int32, device=self.device)
        w = torch.empty((T, c.top_k), dtype=torch.float32, device=self.device)
        ws = self.workspace(T)
        W = self.weights_struct()
        _check(lib().moe_route(ctypes.byref(c), ctypes.byref(W), self.bias.data_ptr(),
                               x.data_ptr(), T, idx.data_ptr(), w.data_ptr(), ws.data_ptr(),
                               ws.numel(), _stream(stream)), "moe_route")
        return idx, w

    def qb_histogram(self, x, n_bins=1000, hist=None, stream=None):
        """Quantile Balancing counts of the tokens x under the layer's biases, added to
        hist (int32 [E, n_bins] on the device; a zeroed one when None)."""
        import torch
        T = x.shape[0]
        c = self.cfg
        if hist is None:
            hist = torch.zeros((c.n_experts, n_bins), dtype=torch.int32, device=self.device)
        ws = self.workspace(T)
        W = self.weights_struct()
        _check(lib().moe_qb_histogram(ctypes.byref(c), ctypes.byref(W), self.bias.data_ptr(),
                                      x.data_ptr(), T, n_bins, hist.data_ptr(), ws.data_ptr(),
                                      ws.numel(), _stream(stream)), "moe_qb_histogram")
        return hist

    def qb_readout(self, hist, n_tokens, bias=None, stream=None):
        """The centred Quantile Balancing biases from counts over n_tokens tokens (taken
        with `bias`, the layer's own by default)."""
        import torch
        c = self.cfg
        b = self.bias if bias is None else bias
        out = torch.empty(c.n_experts, dtype=torch.float32, device=self.device)
        _check(lib().moe_qb_readout(ctypes.byref(c), b.data_ptr(), hist.shape[1], hist.data_ptr(),
                                    n_tokens, out.data_ptr(), _stream(stream)), "moe_qb_readout")
        return out

    def dispatch(self, idx, stream=None):
        import torch
        T = idx.shape[0]
        c = self.cfg
        dev = self.device
        counts = torch.empty(c.n_experts, dtype=torch.int32, device=dev)
        offs = torch.empty(c.n_experts + 1, dtype=torch.int32, device=dev)
        perm = torch.empty(T * c.top_k, dtype=torch.int32, device=dev)
        inv = torch.empty(T * c.top_k, dtype=torch.int32, device=dev)
        ws = self.workspace(T)
        _check(lib().moe_dispatch(ctypes.byref(c), idx.data_ptr(), T, counts.data_ptr(),
                                  offs.data_ptr(), perm.data_ptr(), inv.data_ptr(), ws.data_ptr(),
                                  ws.numel(), _stream(stream)), "moe_dispatch")
        return counts, offs, perm, inv

    def intermediates(self, n_tokens: int, workspace=None) -> dict:
        """Views of the step outputs left in the workspace by the last forward."""
        import torch
        c = self.cfg
        ws = self.workspace(n_tokens) if workspace is None else workspace
        off = workspace_layout(c, n_tokens)
        T, k = n_tokens, c.top_k
        shapes = {"ctrl": (64,), "xc": (T, c.d_latent), "hs": (T, c.d_shared),
                  "h": (T * k, c.d_expert), "eo": (T * k, c.d_latent), "u": (T, c.d_latent),
                  "uh": (T, c.d_latent),
                  "perm": (T * k,), "inv": (T * k,), "counts": (c.n_experts,),
                  "offsets": (c.n_experts + 1,), "z": (T, c.n_experts)}
        out = {}
        for name, shp in shapes.items():
            n = int(np.prod(shp))
            dt = torch.int32 if name in ("ctrl", "perm", "inv", "counts", "offsets") else torch.float32
            out[name] = ws[off[name]: off[name] + 4 * n].view(dt).view(shp)
        if c.precision in (PREC["mx8"], PREC["mx4"]):
            # the experts' input x^c in MX form: code rows of 128 E4M3 bytes (mx8) or 64 bytes of
            # E2M1 pairs (mx4) per K-step of 128 columns (padded) and E8M0 scale bytes [T][4 ks],
            # the first parts of slot [7] (whose code part is sized for E4M3)
            ks = -(-c.d_latent // 128)
            row = (128 if c.precision == PREC["mx8"] else 64) * ks
            o = off["hl"]
            out["xq"] = ws[o: o + T * row].view(T, row)
            o += (T * 128 * ks + 255) & ~255
            out["xs"] = ws[o: o + T * 4 * ks].view(T, 4 * ks)
        return out
