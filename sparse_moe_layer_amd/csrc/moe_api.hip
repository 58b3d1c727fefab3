// C ABI of libmoe.so: argument validation, workspace layout and the launch sequence of
// the Stable LatentMoE FFN forward.  Declarations and the contract are in include/moe.h.
#include <hip/hip_runtime.h>

#include <mutex>

#include "moe.h"
#include "moe_internal.hpp"

#define MOE_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

using moe::Shape;

inline int64_t cdiv64(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }
inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

moe_status make_shape(const moe_config* c, Shape* s) {
  if (!c || !s) return MOE_ERR_INVALID_ARG;
  if (c->d_model <= 0 || c->d_latent < 0 || c->n_experts <= 0 || c->top_k <= 0 ||
      c->d_expert <= 0 || c->d_shared < 0)
    return MOE_ERR_INVALID_ARG;
  if (c->top_k > c->n_experts) return MOE_ERR_INVALID_ARG;
  if (c->act != MOE_ACT_SITU && c->act != MOE_ACT_SWIGLU) return MOE_ERR_INVALID_ARG;
  if (c->expert_wfmt != MOE_WFMT_BF16 && c->expert_wfmt != MOE_WFMT_MXFP4 &&
      c->expert_wfmt != MOE_WFMT_FP8_B128)
    return MOE_ERR_INVALID_ARG;
  if (!(c->rms_eps >= 0.f) || !(c->route_scale == c->route_scale)) return MOE_ERR_INVALID_ARG;
  if (c->act == MOE_ACT_SITU && !(c->beta_gate > 0.f && c->beta_lin > 0.f)) return MOE_ERR_INVALID_ARG;
  if (c->d_model % 8 || c->d_latent % 8 || c->d_expert % 8 || c->d_shared % 8)
    return MOE_ERR_INVALID_ARG;
  const int32_t lin = c->d_latent > 0 ? c->d_latent : c->d_model;   // the experts' input width
  if (c->expert_wfmt == MOE_WFMT_MXFP4 && (lin % 32 || c->d_expert % 32)) return MOE_ERR_INVALID_ARG;
  if (c->precision != MOE_PREC_FP32 && c->precision != MOE_PREC_MX8 && c->precision != MOE_PREC_MX4)
    return MOE_ERR_INVALID_ARG;
  const bool mx = c->precision != MOE_PREC_FP32;
  if (mx && c->expert_wfmt != MOE_WFMT_MXFP4) return MOE_ERR_UNSUPPORTED;
  if (c->d_latent == 0 && c->d_shared == 0) return MOE_ERR_UNSUPPORTED;  // non-latent needs a shared expert
  if (c->d_latent == 0 && mx) return MOE_ERR_UNSUPPORTED;
  if (c->n_experts > 1024 || c->top_k > 64) return MOE_ERR_UNSUPPORTED;
  if (c->d_model > 8192 || c->d_latent > 8192 || c->d_expert > 8192 || c->d_shared > 8192)
    return MOE_ERR_UNSUPPORTED;
  s->d = c->d_model;
  s->latent = c->d_latent > 0 ? 1 : 0;
  s->l = lin;   // the width the experts read and write (the token itself without a latent)
  s->E = c->n_experts;
  s->k = c->top_k;
  s->m = c->d_expert;
  s->ms = c->d_shared;
  s->use_norm = (c->use_latent_norm && s->latent) ? 1 : 0;
  s->eps = c->rms_eps;
  s->route_scale = c->route_scale;
  s->beta_gate = c->beta_gate;
  s->beta_lin = c->beta_lin;
  s->act = c->act;
  s->wfmt = c->expert_wfmt;
  s->prec = c->precision == MOE_PREC_MX8 ? 1 : c->precision == MOE_PREC_MX4 ? 2 : 0;
  // packed dense weights
  s->ks_in = moe::cdiv(s->d, moe::kStepK);
  s->tr_r = moe::cdiv(s->E, moe::kTileRows);
  s->tr_dn = s->latent ? moe::cdiv(s->l, moe::kTileRows) : 0;
  s->tr_sh = moe::cdiv(s->ms, moe::kTileRows / 2);
  s->tr_in = s->tr_r + s->tr_dn + s->tr_sh;
  // Router logits as partial planes over K-ranges of at least 28 K-steps (2 at d = 7168):
  // with few tokens the router workgroups of the IN launch then finish well before its
  // stream does (so the route that waits for them is hidden) without crowding the
  // launch's first wave (8 planes: 2.5 us per token slower at B = 1, 0.6% faster at 64).
  s->zplanes = moe::clampi(s->ks_in / 28, 1, 8);
  s->ks_l = s->latent ? moe::cdiv(s->l, moe::kStepK) : 0;   // OUT's u_hat segment
  s->ks_ms = moe::cdiv(s->ms, moe::kStepK);
  s->ks_out = s->ks_l + s->ks_ms;
  s->tr_out = moe::cdiv(s->d, moe::kTileRows);
  s->in_bytes = (size_t)s->tr_in * s->ks_in * moe::kBf16StepBytes;
  s->out_bytes = (size_t)s->tr_out * s->ks_out * moe::kBf16StepBytes;
  s->gamma_off = s->in_bytes + s->out_bytes;
  s->dense_bytes = align256(s->gamma_off + (size_t)s->l * 2);
  // packed experts
  s->ks_gu = moe::cdiv(s->l, moe::kStepK);
  s->tr_gu = moe::cdiv(s->m, moe::kTileRows / 2);
  s->ks_edn = moe::cdiv(s->m, moe::kStepK);
  s->tr_edn = moe::cdiv(s->l, moe::kTileRows);
  s->step_bytes = s->wfmt == MOE_WFMT_MXFP4 ? moe::kFp4StepBytes
                : s->wfmt == MOE_WFMT_FP8_B128 ? moe::kFp8StepBytes : moe::kBf16StepBytes;
  s->gu_bytes = (size_t)s->tr_gu * s->ks_gu * s->step_bytes;
  s->expert_bytes = align256(s->gu_bytes + (size_t)s->tr_edn * s->ks_edn * s->step_bytes);
  return MOE_OK;
}

// Slot [7].  FP32: x^c, h_s, h and u_hat as bf16 row pairs.  MX8 / MX4: the MX codes and
// scales of x^c and h (MX4 uses the first half of each code row), u_hat and h_s in bf16.
// Each part 256-aligned.
constexpr int kHiloParts = 6;
size_t hilo_part(const Shape& s, int64_t T, int part) {
  if (moe::mx_profile(s)) {
    const int64_t rows[6] = {T, T, T * s.k, T * s.k, T, T};
    if (part == 4) return align256(moe::pf_packed_bytes(s, T, true));
    if (part == 5) return align256(moe::pf_packed_bytes(s, T, false));
    const int64_t bytes[4] = {128LL * s.ks_gu, 4LL * s.ks_gu, 128LL * s.ks_edn, 4LL * s.ks_edn};
    return align256((size_t)(rows[part] * bytes[part]));
  }
  if (part >= 4) return 0;
  const int64_t rows[4] = {T, T, T * s.k, T};
  const int64_t width[4] = {s.l, s.ms, s.m, s.l};
  return align256((size_t)rows[part] * 2 * width[part] * 2);
}
size_t hilo_bytes(const Shape& s, int64_t T) {
  size_t n = 0;
  for (int i = 0; i < kHiloParts; ++i) n += hilo_part(s, T, i);
  return n;
}
// The few-token launches use slot [7] for the shared down-projection's partial sums.
size_t slot7_bytes(const Shape& s, int64_t T) {
  const size_t h = hilo_bytes(s, T), y = moe::sd_partial_bytes(s, T);
  return h > y ? h : y;
}

// Workspace slots in the order of moe_workspace_layout.
void layout(const Shape& s, int64_t T, size_t off[MOE_WS_NUM_SLOTS], size_t* total) {
  const int64_t tk = T * s.k;
  const int64_t nch = cdiv64(T, moe::dispatch_chunk_tokens(s.k));
  const size_t sz[MOE_WS_NUM_SLOTS] = {
      (size_t)moe::kCtrlWords * 4,          // control words (unit count)
      (size_t)T * s.l * 4,                  // x^c
      (size_t)T * s.ms * 4,                 // h_s
      (size_t)tk * s.m * 4,                 // h
      (size_t)tk * s.l * 4,                 // E
      (size_t)T * s.l * 4,                  // u
      (size_t)T * s.l * 4,                  // u_hat
      slot7_bytes(s, T),                    // hi/lo rows of the token-tiled launches
      (size_t)tk * 4,                       // perm
      (size_t)tk * 4,                       // inv
      (size_t)s.E * 4,                      // counts
      (size_t)(s.E + 1) * 4,                // offsets
      (size_t)s.zplanes * moe::kZSub * T * s.E * 4,   // z (partial planes, their parts)
      (size_t)nch * s.E * 4,                // chunk histograms
      (size_t)moe::max_units(s, T) * 16,    // unit table
  };
  size_t o = 0;
  for (int i = 0; i < MOE_WS_NUM_SLOTS; ++i) {
    off[i] = o;
    o += align256(sz[i]);
  }
  *total = o;
}

moe::Work make_work(const Shape& s, int64_t T, void* ws, const size_t off[MOE_WS_NUM_SLOTS]) {
  char* b = static_cast<char*>(ws);
  moe::Work w;
  w.ctrl = reinterpret_cast<int32_t*>(b + off[0]);
  w.xc = reinterpret_cast<float*>(b + off[1]);
  w.hs = reinterpret_cast<float*>(b + off[2]);
  w.h = reinterpret_cast<float*>(b + off[3]);
  w.eo = reinterpret_cast<float*>(b + off[4]);
  w.u = reinterpret_cast<float*>(b + off[5]);
  w.uh = reinterpret_cast<float*>(b + off[6]);
  {
    char* p = b + off[7];
    void* parts[kHiloParts];
    for (int i = 0; i < kHiloParts; ++i) {
      parts[i] = p;
      p += hilo_part(s, T, i);
    }
    w.xc_hl = static_cast<uint16_t*>(parts[0]);
    w.hs_hl = static_cast<uint16_t*>(parts[1]);
    w.h_hl = static_cast<uint16_t*>(parts[2]);
    w.uh_hl = static_cast<uint16_t*>(parts[3]);
    w.pf.xq = static_cast<uint8_t*>(parts[0]);
    w.pf.xs = static_cast<uint8_t*>(parts[1]);
    w.pf.hq = static_cast<uint8_t*>(parts[2]);
    w.pf.hsc = static_cast<uint8_t*>(parts[3]);
    w.pf.ao = static_cast<uint8_t*>(parts[4]);
    w.pf.ax = static_cast<uint8_t*>(parts[5]);
    w.ys = reinterpret_cast<float2*>(b + off[7]);
  }
  w.perm = reinterpret_cast<int32_t*>(b + off[8]);
  w.inv = reinterpret_cast<int32_t*>(b + off[9]);
  w.counts = reinterpret_cast<int32_t*>(b + off[10]);
  w.offs = reinterpret_cast<int32_t*>(b + off[11]);
  w.z = reinterpret_cast<float*>(b + off[12]);
  w.chunk_hist = reinterpret_cast<int32_t*>(b + off[13]);
  w.units = reinterpret_cast<int32_t*>(b + off[14]);
  return w;
}

moe_status check_weights(const moe_weights* w) {
  if (!w || !w->dense || !w->experts || !aligned(w->dense, 256) || !aligned(w->experts, 256))
    return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

inline moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

}  // namespace

MOE_EXPORT int moe_abi_version(void) { return MOE_ABI_VERSION; }

MOE_EXPORT const char* moe_status_str(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
  }
  return "MOE_ERR_UNKNOWN";
}

MOE_EXPORT moe_status moe_packed_dense_size(const moe_config* cfg, size_t* bytes) {
  Shape s;
  moe_status st = make_shape(cfg, &s);
  if (st != MOE_OK) return st;
  if (!bytes) return MOE_ERR_INVALID_ARG;
  *bytes = s.dense_bytes;
  return MOE_OK;
}

MOE_EXPORT moe_status moe_pack_dense(const moe_config* cfg, const moe_dense_src* src, void* packed,
                                     size_t packed_bytes, moe_stream_t stream) {
  Shape s;
  moe_status st = make_shape(cfg, &s);
  if (st != MOE_OK) return st;
  if (!src || !packed || !src->router || !aligned(packed, 256)) return MOE_ERR_INVALID_ARG;
  if (s.latent && (!src->w_down_latent || !src->w_up_latent || !src->norm_gamma))
    return MOE_ERR_INVALID_ARG;
  if (s.ms > 0 && (!src->shared_gu || !src->shared_down)) return MOE_ERR_INVALID_ARG;
  const void* ptrs[6] = {src->router, src->w_down_latent, src->w_up_latent, src->norm_gamma,
                         src->shared_gu, src->shared_down};
  for (const void* p : ptrs)
    if (p && !aligned(p, 16)) return MOE_ERR_INVALID_ARG;
  if (packed_bytes < s.dense_bytes) return MOE_ERR_WORKSPACE;
  moe::DenseSrc d;
  d.router = static_cast<const uint16_t*>(src->router);
  d.wdn = static_cast<const uint16_t*>(src->w_down_latent);
  d.wup = static_cast<const uint16_t*>(src->w_up_latent);
  d.gamma = static_cast<const uint16_t*>(src->norm_gamma);
  d.sgu = static_cast<const uint16_t*>(src->shared_gu);
  d.sdn = static_cast<const uint16_t*>(src->shared_down);
  return hip_status(moe::launch_pack_dense(s, d, static_cast<uint8_t*>(packed), (hipStream_t)stream));
}

MOE_EXPORT moe_status moe_packed_experts_size(const moe_config* cfg, size_t* bytes) {
  Shape s;
  moe_status st = make_shape(cfg, &s);
  if (st != MOE_OK) return st;
  if (!bytes) return MOE_ERR_INVALID_ARG;
  *bytes = s.expert_bytes * (size_t)s.E;
  return MOE_OK;
}

MOE_EXPORT moe_status moe_pack_experts(const moe_config* cfg, const moe_expert_src* src,
                                       int32_t e0, int32_t n, void* packed, size_t packed_bytes,
                                       moe_stream_t stream) {
  Shape s;
  moe_status st = make_shape(cfg, &s);
  if (st != MOE_OK) return st;
  if (!src || !packed || !src->gu || !src->down || !aligned(packed, 256)) return MOE_ERR_INVALID_ARG;
  if (s.wfmt == MOE_WFMT_MXFP4 &&
      (!src->gu_scale || !src->down_scale || !aligned(src->gu, 4) || !aligned(src->down, 4)))
    return MOE_ERR_INVALID_ARG;
  if (s.wfmt == MOE_WFMT_BF16 && (!aligned(src->gu, 16) || !aligned(src->down, 16)))
    return MOE_ERR_INVALID_ARG;
  if (s.wfmt == MOE_WFMT_FP8_B128 &&
      (!src->gu_scale || !src->down_scale || !aligned(src->gu, 8) || !aligned(src->down, 8) ||
       !aligned(src->gu_scale, 4) || !aligned(src->down_scale, 4)))
    return MOE_ERR_INVALID_ARG;
  if (e0 < 0 || n < 0 || (int64_t)e0 + n > s.E) return MOE_ERR_INVALID_ARG;
  if (packed_bytes < s.expert_bytes * (size_t)s.E) return MOE_ERR_WORKSPACE;
  if (n == 0) return MOE_OK;
  return hip_status(moe::launch_pack_experts(s, src->gu, src->gu_scale, src->down, src->down_scale,
                                             e0, n, static_cast<uint8_t*>(packed),
                                             (hipStream_t)stream));
}

MOE_EXPORT moe_status moe_workspace_size(const moe_config* cfg, int64_t max_tokens, size_t* bytes) {
  Shape s;
  moe_status st = make_shape(cfg, &s);
  if (st != MOE_OK) return st;
  if (!bytes || max_tokens < 0) return MOE_ERR_INVALID_ARG;
  size_t off[MOE_WS_NUM_SLOTS];
  layout(s, max_tokens, off, bytes);
  return MOE_OK;
}

MOE_EXPORT moe_status moe_workspace_layout(const moe_config* cfg, int64_t n_tokens,
                                           size_t offsets[MOE_WS_NUM_SLOTS]) {
  Shape s;
  moe_status st = make_shape(cfg, &s);
  if (st != MOE_OK) return st;
  if (!offsets || n_tokens < 0) return MOE_ERR_INVALID_ARG;
  size_t total;
  layout(s, n_tokens, offsets, &total);
  return MOE_OK;
}

namespace {

moe_status check_call(const Shape& s, const moe_weights* w, const float* bias, const void* x,
                      int64_t n_tokens, void* workspace, size_t workspace_bytes,
                      size_t off[MOE_WS_NUM_SLOTS]) {
  moe_status st;
  if ((st = check_weights(w)) != MOE_OK) return st;
  if (!bias || !x || !workspace) return MOE_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(workspace, 256) || !aligned(bias, 4)) return MOE_ERR_INVALID_ARG;
  size_t need;
  layout(s, n_tokens, off, &need);
  if (workspace_bytes < need) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

moe_status forward_impl(const moe_config* cfg, const moe_weights* w, const float* bias,
                        const void* x, int64_t n_tokens, float* delta, int32_t* topk_idx,
                        float* topk_w, void* workspace, size_t workspace_bytes,
                        void* const* events, int step_begin, int step_end, moe_stream_t stream,
                        float* residual = nullptr, uint16_t* x_next = nullptr,
                        const moe_weights* next = nullptr) {
  Shape s;
  moe_status st = make_shape(cfg, &s);
  if (st != MOE_OK) return st;
  if (n_tokens < 0) return MOE_ERR_INVALID_ARG;
  if (step_begin < 0 || step_end > MOE_NUM_STEPS || step_begin > step_end) return MOE_ERR_INVALID_ARG;
  if (n_tokens == 0) return MOE_OK;  // nothing to read or write: buffers may be empty (null)
  size_t off[MOE_WS_NUM_SLOTS];
  if ((st = check_call(s, w, bias, x, n_tokens, workspace, workspace_bytes, off)) != MOE_OK) return st;
  if ((!delta && !residual) || !topk_idx || !topk_w) return MOE_ERR_INVALID_ARG;
  if (!aligned(delta, 16) || !aligned(topk_idx, 4) || !aligned(topk_w, 4)) return MOE_ERR_INVALID_ARG;
  if (!aligned(residual, 16) || !aligned(x_next, 16) || (x_next && !residual)) return MOE_ERR_INVALID_ARG;
  const moe::OutSink sink{delta, residual, x_next};
  const moe::Work ws = make_work(s, n_tokens, workspace, off);
  const uint8_t* dense = static_cast<const uint8_t*>(w->dense);
  const uint8_t* experts = static_cast<const uint8_t*>(w->experts);
  hipStream_t hs = (hipStream_t)stream;
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  const bool fused = moe::route_fused(s, n_tokens);
  for (int step = step_begin; step < step_end; ++step) {
    if (events && events[step] && hipEventRecord((hipEvent_t)events[step], hs) != hipSuccess)
      return MOE_ERR_HIP;
    hipError_t e = hipSuccess;
    if (moe::mx_profile(s)) {
      switch (step) {
        case MOE_STEP_ROUTER: e = moe::launch_pf_in(s, dense, xb, n_tokens, ws.pf, ws.z, ws.xc, hs); break;
        case MOE_STEP_IN: e = moe::launch_pf_quant(s, ws.xc, n_tokens, ws.pf, hs); break;
        case MOE_STEP_ROUTE: e = moe::launch_route(s, bias, n_tokens, ws, topk_idx, topk_w, hs); break;
        case MOE_STEP_DISPATCH:
          e = moe::launch_dispatch(s, topk_idx, n_tokens, ws.counts, ws.offs, ws.perm, ws.inv,
                                   ws.chunk_hist, ws.units, ws.ctrl, hs);
          break;
        case MOE_STEP_EXPERT_GU: e = moe::launch_pf_expert(s, experts, true, n_tokens, ws, ws.pf, hs); break;
        case MOE_STEP_EXPERT_DOWN: e = moe::launch_pf_expert(s, experts, false, n_tokens, ws, ws.pf, hs); break;
        case MOE_STEP_COMBINE:
          e = moe::launch_pf_combine_norm(s, dense, topk_w, n_tokens, ws, ws.pf, hs);
          break;
        case MOE_STEP_OUT: e = moe::launch_pf_out(s, dense, n_tokens, ws.pf, sink, hs); break;
      }
      if (e != hipSuccess) return MOE_ERR_HIP;
      continue;
    }
    switch (step) {
      case MOE_STEP_ROUTER: e = moe::launch_router(s, dense, xb, n_tokens, false, ws, hs); break;
      case MOE_STEP_IN:
        e = moe::launch_in(s, dense, xb, n_tokens, bias, topk_idx, topk_w, ws, hs);
        break;
      case MOE_STEP_ROUTE:
        if (!fused) e = moe::launch_route(s, bias, n_tokens, ws, topk_idx, topk_w, hs);
        break;
      case MOE_STEP_DISPATCH:
        if (!fused)
          e = moe::launch_dispatch(s, topk_idx, n_tokens, ws.counts, ws.offs, ws.perm, ws.inv,
                                   ws.chunk_hist, ws.units, ws.ctrl, hs);
        break;
      case MOE_STEP_EXPERT_GU: e = moe::launch_expert(s, experts, dense, true, n_tokens, ws, hs); break;
      case MOE_STEP_EXPERT_DOWN: e = moe::launch_expert(s, experts, dense, false, n_tokens, ws, hs); break;
      case MOE_STEP_COMBINE: e = moe::launch_combine(s, dense, topk_w, n_tokens, ws, hs); break;
      case MOE_STEP_OUT: {
        moe::Prefetch pf{};
        if (next && fused) {   // the next layer's first launch reads these bytes
          pf.p = static_cast<const uint8_t*>(next->dense);
          pf.bytes = moe::first_launch_dense_bytes(s);
          pf.sink = reinterpret_cast<uint32_t*>(ws.units);
        }
        e = moe::launch_out(s, dense, n_tokens, ws, sink, hs, pf);
        break;
      }
    }
    if (e != hipSuccess) return MOE_ERR_HIP;
  }
  if (events && step_end == MOE_NUM_STEPS && events[MOE_NUM_STEPS] &&
      hipEventRecord((hipEvent_t)events[MOE_NUM_STEPS], hs) != hipSuccess)
    return MOE_ERR_HIP;
  return MOE_OK;
}

}  // namespace

MOE_EXPORT moe_status moe_layer_forward(const moe_config* cfg, const moe_weights* w,
                                        const float* bias, const void* x, int64_t n_tokens,
                                        float* delta, int32_t* topk_idx, float* topk_w,
                                        void* workspace, size_t workspace_bytes,
                                        moe_stream_t stream) {
  return forward_impl(cfg, w, bias, x, n_tokens, delta, topk_idx, topk_w, workspace,
                      workspace_bytes, nullptr, 0, MOE_NUM_STEPS, stream);
}

// The workspace of moe_layer_forward_noalloc: one copy per GPU in the library's code object.
// Host code never passes `scratch` itself to a kernel (on the host the name is a stand-in,
// not a device address): the address of each device's copy comes from hipGetSymbolAddress.
static __device__ __align__(256) uint8_t scratch[MOE_STATIC_WORKSPACE_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices];   // device address of `scratch` per device, once looked up

// The device address of `scratch` on the current device (looked up on the first call).
moe_status scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return MOE_OK;
}

}  // namespace

MOE_EXPORT moe_status moe_layer_forward_noalloc(const moe_config* cfg, const moe_weights* w,
                                                const float* bias, const void* x, int64_t n_tokens,
                                                float* delta, int32_t* topk_idx, float* topk_w,
                                                moe_stream_t stream) {
  Shape s;
  moe_status st = make_shape(cfg, &s);
  if (st != MOE_OK) return st;
  if (n_tokens < 0) return MOE_ERR_INVALID_ARG;
  if (n_tokens == 0) return MOE_OK;
  size_t off[MOE_WS_NUM_SLOTS], need;
  layout(s, n_tokens, off, &need);
  if (need > MOE_STATIC_WORKSPACE_BYTES) return MOE_ERR_WORKSPACE;
  void* ws = nullptr;
  if ((st = scratch_of_current_device(&ws)) != MOE_OK) return st;
  return forward_impl(cfg, w, bias, x, n_tokens, delta, topk_idx, topk_w, ws,
                      MOE_STATIC_WORKSPACE_BYTES, nullptr, 0, MOE_NUM_STEPS, stream);
}

MOE_EXPORT moe_status moe_layer_forward_residual(const moe_config* cfg, const moe_weights* w,
                                                 const float* bias, const void* x,
                                                 int64_t n_tokens, float* residual, void* x_next,
                                                 float* delta, int32_t* topk_idx, float* topk_w,
                                                 void* workspace, size_t workspace_bytes,
                                                 moe_stream_t stream) {
  if (n_tokens > 0 && !residual) return MOE_ERR_INVALID_ARG;
  return forward_impl(cfg, w, bias, x, n_tokens, delta, topk_idx, topk_w, workspace,
                      workspace_bytes, nullptr, 0, MOE_NUM_STEPS, stream, residual,
                      static_cast<uint16_t*>(x_next));
}

MOE_EXPORT moe_status moe_layer_forward_residual_prefetch(
    const moe_config* cfg, const moe_weights* w, const float* bias, const void* x, int64_t n_tokens,
    float* residual, void* x_next, float* delta, int32_t* topk_idx, float* topk_w, void* workspace,
    size_t workspace_bytes, const moe_weights* next, moe_stream_t stream) {
  if (n_tokens > 0 && !residual) return MOE_ERR_INVALID_ARG;
  if (next && check_weights(next) != MOE_OK) return MOE_ERR_INVALID_ARG;
  return forward_impl(cfg, w, bias, x, n_tokens, delta, topk_idx, topk_w, workspace,
                      workspace_bytes, nullptr, 0, MOE_NUM_STEPS, stream, residual,
                      static_cast<uint16_t*>(x_next), next);
}

MOE_EXPORT moe_status moe_layer_forward_steps(const moe_config* cfg, const moe_weights* w,
                                              const float* bias, const void* x, int64_t n_tokens,
                                              float* delta, int32_t* topk_idx, float* topk_w,
                                              void* workspace, size_t workspace_bytes,
                                              int32_t step_begin, int32_t step_end,
                                              moe_stream_t stream) {
  return forward_impl(cfg, w, bias, x, n_tokens, delta, topk_idx, topk_w, workspace,
                      workspace_bytes, nullptr, step_begin, step_end, stream);
}

MOE_EXPORT moe_status moe_layer_forward_timed(const moe_config* cfg, const moe_weights* w,
                                              const float* bias, const void* x, int64_t n_tokens,
                                              float* delta, int32_t* topk_idx, float* topk_w,
                                              void* workspace, size_t workspace_bytes,
                                              void* const* step_events, moe_stream_t stream) {
  if (!step_events) return MOE_ERR_INVALID_ARG;
  return forward_impl(cfg, w, bias, x, n_tokens, delta, topk_idx, topk_w, workspace,
                      workspace_bytes, step_events, 0, MOE_NUM_STEPS, stream);
}

MOE_EXPORT moe_status moe_route(const moe_config* cfg, const moe_weights* w, const float* bias,
                                const void* x, int64_t n_tokens, int32_t* topk_idx, float* topk_w,
                                void* workspace, size_t workspace_bytes, moe_stream_t stream) {
  Shape s;
  moe_status st = make_shape(cfg, &s);
  if (st != MOE_OK) return st;
  if (n_tokens < 0) return MOE_ERR_INVALID_ARG;
  if (n_tokens == 0) return MOE_OK;
  size_t off[MOE_WS_NUM_SLOTS];
  if ((st = check_call(s, w, bias, x, n_tokens, workspace, workspace_bytes, off)) != MOE_OK) return st;
  if (!topk_idx || !topk_w || !aligned(topk_idx, 4) || !aligned(topk_w, 4)) return MOE_ERR_INVALID_ARG;
  const moe::Work ws = make_work(s, n_tokens, workspace, off);
  hipStream_t hs = (hipStream_t)stream;
  Shape rs = s;     // the router of the FP32 launches (its logit planes fit the z slot)
  rs.prec = 0;
  if (moe::launch_router(rs, static_cast<const uint8_t*>(w->dense), static_cast<const uint16_t*>(x),
                         n_tokens, true, ws, hs) != hipSuccess)
    return MOE_ERR_HIP;
  return hip_status(moe::launch_route(rs, bias, n_tokens, ws, topk_idx, topk_w, hs));
}

MOE_EXPORT moe_status moe_qb_histogram(const moe_config* cfg, const moe_weights* w,
                                       const float* bias, const void* x, int64_t n_tokens,
                                       int32_t n_bins, int32_t* hist, void* workspace,
                                       size_t workspace_bytes, moe_stream_t stream) {
  Shape s;
  moe_status st = make_shape(cfg, &s);
  if (st != MOE_OK) return st;
  if (n_tokens < 0 || n_bins < 1 || n_bins > MOE_QB_MAX_BINS || s.k >= s.E || s.k + 1 > 64)
    return MOE_ERR_INVALID_ARG;
  if (!hist || !aligned(hist, 4)) return MOE_ERR_INVALID_ARG;
  if (n_tokens == 0) return MOE_OK;
  size_t off[MOE_WS_NUM_SLOTS];
  if ((st = check_call(s, w, bias, x, n_tokens, workspace, workspace_bytes, off)) != MOE_OK) return st;
  const moe::Work ws = make_work(s, n_tokens, workspace, off);
  hipStream_t hs = (hipStream_t)stream;
  Shape rs = s;     // the router of the FP32 launches, as in moe_route
  rs.prec = 0;
  if (moe::launch_router(rs, static_cast<const uint8_t*>(w->dense), static_cast<const uint16_t*>(x),
                         n_tokens, true, ws, hs) != hipSuccess)
    return MOE_ERR_HIP;
  return hip_status(moe::launch_qb_hist(rs, bias, n_tokens, n_bins, hist, ws, hs));
}

MOE_EXPORT moe_status moe_qb_readout(const moe_config* cfg, const float* bias, int32_t n_bins,
                                     const int32_t* hist, int64_t n_tokens, float* new_bias,
                                     moe_stream_t stream) {
  Shape s;
  moe_status st = make_shape(cfg, &s);
  if (st != MOE_OK) return st;
  if (n_tokens < 1 || n_bins < 1 || n_bins > MOE_QB_MAX_BINS || s.k >= s.E) return MOE_ERR_INVALID_ARG;
  if (!bias || !hist || !new_bias || !aligned(bias, 4) || !aligned(hist, 4) || !aligned(new_bias, 4))
    return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_qb_readout(s, bias, n_tokens, n_bins, hist, new_bias,
                                           (hipStream_t)stream));
}

MOE_EXPORT moe_status moe_dispatch(const moe_config* cfg, const int32_t* topk_idx, int64_t n_tokens,
                                   int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv,
                                   void* workspace, size_t workspace_bytes, moe_stream_t stream) {
  Shape s;
  moe_status st = make_shape(cfg, &s);
  if (st != MOE_OK) return st;
  if (n_tokens < 0) return MOE_ERR_INVALID_ARG;
  if (n_tokens == 0) return MOE_OK;
  if (!topk_idx || !counts || !offsets || !perm || !inv || !workspace) return MOE_ERR_INVALID_ARG;
  if (!aligned(workspace, 256)) return MOE_ERR_INVALID_ARG;
  size_t off[MOE_WS_NUM_SLOTS], need;
  layout(s, n_tokens, off, &need);
  if (workspace_bytes < need) return MOE_ERR_WORKSPACE;
  const moe::Work ws = make_work(s, n_tokens, workspace, off);
  return hip_status(moe::launch_dispatch(s, topk_idx, n_tokens, counts, offsets, perm, inv,
                                         ws.chunk_hist, ws.units, ws.ctrl, (hipStream_t)stream));
}
