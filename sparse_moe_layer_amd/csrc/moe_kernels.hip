// gfx950 kernels of the Stable LatentMoE FFN layer forward.
//
// Step order follows the Kimi K3 latent mixture-of-experts block card ("All 23 steps"
// and its KimiSparseMoeBlock.forward / moe_infer excerpt):
//   k_in          router logits z = x W_r, latent down x^c = x W_down_latent and the
//                 shared gate/up with its SiTU epilogue, one launch over one packed
//                 matrix; for a few tokens its last router workgroup also takes
//                 s = sigmoid(z), the top_k of s + b, G = s / sum(s) and sorts the
//                 assignments by expert
//   k_route       the same selection in its own launch for larger batches
//   k_disp_*      per-expert histogram -> scan -> stable permutation for larger batches
//                 (moe_infer's scatter_/argsort, kept on the device: no host round trip)
//   k_exp         routed gate/up (+ SiTU) and down, MXFP4 or bf16 weights
//   k_combine     u = sum_j G_j E_j in a fixed order (no atomics)
//   k_out         RMSNorm(u) W_up_latent + h_s W_shared_down -> Delta, one product over
//                 the packed [W_up_latent | W_shared_down] matrix
//
// The weight products run on the matrix cores (v_mfma_f32_16x16x32_bf16) with the
// weights streamed once from HBM as the B operand and the activations staged in LDS as
// the A operand; decode is bound by HBM bandwidth.  Activations are fp32 between the
// steps; where they meet the matrix cores they are carried as exact bf16 hi/lo pairs.
#include <climits>
#include <cmath>

#include "moe_device.hpp"
#include "moe_internal.hpp"

namespace moe {
namespace {

constexpr int kWavesPerBlock = kBlock / kWave;

// ------------------------------------------------------------------------------------
// Step ROUTE: one workgroup (4 wavefronts) per token.  Expert e = (4i + w)*64 + lane
// belongs to wavefront w, slot i.  Each wavefront finds the top-k of its share with k
// rounds of a DPP arg-max over a 64-bit key (order key of kappa = s + b in the high word,
// ~e in the low word: larger kappa first, then the lower index); the 4k candidates are
// then ranked in LDS.  G = route_scale * s / sum(s), the sum in selection order.
// For at most 4 tokens one workgroup handles all of them and then sorts the T*k
// assignments by expert (histogram, scan, stable rank) in LDS and writes the unit table
// of the expert launches.
// ------------------------------------------------------------------------------------
struct RouteArgs {
  float* z;         // zplanes partial planes of zsub parts each [zplanes * zsub][T][E]; the
                    // route leaves their sum in plane 0
  int zplanes, zsub;
  int64_t zplane;   // floats between (sub-)planes
  const float* bias;
  int64_t T;
  int E, k;
  float route_scale;
  int32_t* idx;
  float* gw;
  int32_t* counts;
  int32_t* offs;
  int32_t* perm;
  int32_t* inv;
  int32_t* units;   // unit table of the expert launches (dispatch only)
  int32_t* ctrl;    // ctrl[0] <- number of units, ctrl[1] <- the same (dispatch only)
  int nu;           // positions per unit
  int even;         // units of an expert near-equal (unit_run)
};

constexpr int kRouteSlots = 4;      // E <= 4 slots x 4 wavefronts x 64 lanes = 1024
constexpr int kMaxZPlanes = 8;      // partial logit (sub-)planes of the router launch

// The logit from its partial planes: each plane's parts added in order, then the planes in
// plane order from zero (absent planes add nothing).
// (Compile-time indices only: a register array indexed at run time would live in scratch.)
__device__ __forceinline__ float plane_sum(const float (&zp)[kMaxZPlanes], int planes, int sub) {
  float zv = 0.f, pv = 0.f;
#pragma unroll
  for (int q = 0; q < kMaxZPlanes; ++q) {
    if (q < planes * sub) {
      const int r = q % sub;
      pv = r == 0 ? zp[q] : pv + zp[q];
      if (r == sub - 1) zv += pv;
    }
  }
  return zv;
}

// AGENT: the logit planes come from other workgroups of the same launch (agent-scope loads:
// the XCDs' L2 caches are not coherent with each other within a launch).
template <bool AGENT>
__device__ __forceinline__ void block_route_token(const RouteArgs& a, int64_t t, uint64_t* cand_key,
                                                  float* cand_s, int* sel_e, float* sel_s,
                                                  int* sidx) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x >> 6;
  uint64_t key[kRouteSlots];
  float sv[kRouteSlots];
  // every logit plane and bias value of this lane's experts in flight at once
  float* zr = a.z + t * a.E;
  float zp[kRouteSlots][kMaxZPlanes], bv[kRouteSlots];
  const int np = a.zplanes * a.zsub;
#pragma unroll
  for (int i = 0; i < kRouteSlots; ++i) {
    const int e = (i * kWavesPerBlock + wv) * kWave + lane;
    const bool ok = e < a.E;
#pragma unroll
    for (int p = 0; p < kMaxZPlanes; ++p)
      zp[i][p] = !(ok && p < np) ? 0.f
                 : AGENT ? __hip_atomic_load(zr + p * a.zplane + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                         : zr[p * a.zplane + e];
    bv[i] = ok ? a.bias[e] : 0.f;
  }
#pragma unroll
  for (int i = 0; i < kRouteSlots; ++i) {
    const int e = (i * kWavesPerBlock + wv) * kWave + lane;
    const float zv = plane_sum(zp[i], a.zplanes, a.zsub);
    if (e < a.E) {
      if (np > 1) zr[e] = zv;   // the logits themselves, for inspection
      const float s = sigmoidf_(zv);
      float kk = s + bv[i];
      if (kk != kk) kk = -INFINITY;
      sv[i] = s;
      key[i] = ((uint64_t)float_order_key(kk) << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)e);
    } else {
      sv[i] = 0.f;
      key[i] = 0;
    }
  }
  uint64_t head = 0;
#pragma unroll
  for (int i = 0; i < kRouteSlots; ++i) head = max_u64(head, key[i]);
  for (int j = 0; j < a.k; ++j) {
    const uint64_t m = wave_max_u64(head);
    float s_win = 0.f;
    if (m != 0) {
      const int e = (int)(0xFFFFFFFFu - (uint32_t)m);
      const int owner = e & (kWave - 1);
      const int slot = e >> 8;
      float mine = 0.f;
#pragma unroll
      for (int i = 0; i < kRouteSlots; ++i) mine = (i == slot) ? sv[i] : mine;
      s_win = __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(mine), owner));
      if (lane == owner) {
        head = 0;
#pragma unroll
        for (int i = 0; i < kRouteSlots; ++i) {
          if (i == slot) key[i] = 0;
          head = max_u64(head, key[i]);
        }
      }
    }
    if (lane == 0) {
      cand_key[wv * kMaxK + j] = m;
      cand_s[wv * kMaxK + j] = s_win;
    }
  }
  __syncthreads();
  {
    static_assert(kBlock == kWavesPerBlock * kMaxK, "one thread per candidate");
    const int c = threadIdx.x;  // candidate j = c % kMaxK of wavefront c / kMaxK
    const int j = c & (kMaxK - 1);
    const uint64_t kc = cand_key[c];
    if (j < a.k && kc != 0) {
      int rank = 0;
#pragma unroll
      for (int w = 0; w < kWavesPerBlock; ++w)
        for (int q = 0; q < a.k; ++q) rank += (cand_key[w * kMaxK + q] > kc);
      if (rank < a.k) {
        sel_e[rank] = (int)(0xFFFFFFFFu - (uint32_t)kc);
        sel_s[rank] = cand_s[c];
      }
    }
  }
  __syncthreads();
  if ((int)threadIdx.x < a.k) {
    float tot = 0.f;
    for (int q = 0; q < a.k; ++q) tot += sel_s[q];
    const int j = threadIdx.x;
    a.idx[t * a.k + j] = sel_e[j];
    a.gw[t * a.k + j] = (sel_s[j] / tot) * a.route_scale;
    if (sidx) sidx[t * a.k + j] = sel_e[j];
  }
  __syncthreads();
}

// Unit i of the ceil(tot / nu) units of an expert's tot positions: first position r0 and
// count n.  Full units of nu and a shorter last one, or (even) near-equal runs whose
// counts differ by at most one.
__device__ __forceinline__ void unit_run(int tot, int nu, int even, int i, int& r0, int& n) {
  if (even) {
    const int nun = (tot + nu - 1) / nu, base = tot / nun, rem = tot - base * nun;
    r0 = i * base + min(i, rem);
    n = base + (i < rem ? 1 : 0);
  } else {
    r0 = i * nu;
    n = min(nu, tot - r0);
  }
}

// The route of tokens t_begin..t_end-1 by one workgroup; with `dispatch`, also the
// counting sort of their (at most 256) assignments by expert.
template <bool AGENT = false>
__device__ void route_block(const RouteArgs& a, int64_t t_begin, int64_t t_end, bool dispatch) {
  __shared__ uint64_t cand_key[kWavesPerBlock * kMaxK];
  __shared__ float cand_s[kWavesPerBlock * kMaxK];
  __shared__ int sel_e[kMaxK];
  __shared__ float sel_s[kMaxK];
  __shared__ int sidx[kBlock];
  __shared__ int hist[1024];
  __shared__ int soff[1024];
  __shared__ int part[kBlock];
  __shared__ int upart[kBlock];
  for (int64_t t = t_begin; t < t_end; ++t)
    block_route_token<AGENT>(a, t, cand_key, cand_s, sel_e, sel_s, dispatch ? sidx : nullptr);
  if (!dispatch) return;
  // dispatch of the n = T*k <= 256 assignments
  const int n = (int)(a.T * a.k);
  const int tid = threadIdx.x;
  for (int e = tid; e < a.E; e += kBlock) hist[e] = 0;
  __syncthreads();
  if (tid < n) atomicAdd(&hist[sidx[tid]], 1);
  __syncthreads();
  // exclusive scans over experts (4 consecutive experts per thread, then across threads)
  // of the counts and of the units (runs of at most nu positions of one expert)
  int loc[4], ps = 0, pu = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = tid * 4 + i;
    loc[i] = (e < a.E) ? hist[e] : 0;
    ps += loc[i];
    pu += (loc[i] + a.nu - 1) / a.nu;
  }
  part[tid] = ps;
  upart[tid] = pu;
  __syncthreads();
  for (int o = 1; o < kBlock; o <<= 1) {
    const int v = (tid >= o) ? part[tid - o] : 0;
    const int w = (tid >= o) ? upart[tid - o] : 0;
    __syncthreads();
    part[tid] += v;
    upart[tid] += w;
    __syncthreads();
  }
  int run = part[tid] - ps, urun = upart[tid] - pu;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = tid * 4 + i;
    if (e < a.E) {
      soff[e] = run;
      a.offs[e] = run;
      a.counts[e] = loc[i];
      const int nun = (loc[i] + a.nu - 1) / a.nu;
      for (int j = 0; j < nun; ++j, ++urun) {
        int r0, cnt;
        unit_run(loc[i], a.nu, a.even, j, r0, cnt);
        *reinterpret_cast<int4*>(a.units + 4 * urun) = make_int4(e, run + r0, cnt, 0);
      }
    }
    run += loc[i];
  }
  if (tid == 0) a.offs[a.E] = n;
  if (tid == kBlock - 1) a.ctrl[0] = a.ctrl[1] = upart[tid];
  __syncthreads();
  if (tid < n) {
    const int e = sidx[tid];
    int r = 0;
    for (int q = 0; q < tid; ++q) r += (sidx[q] == e);
    const int pos = soff[e] + r;
    a.perm[pos] = tid;
    a.inv[tid] = pos;
  }
}

// Step ROUTE for larger batches: one workgroup per token, no dispatch.
__global__ __launch_bounds__(kBlock) void k_route(RouteArgs a) {
  route_block(a, blockIdx.x, blockIdx.x + 1, false);
}


// ------------------------------------------------------------------------------------
// Step DISPATCH for larger batches: deterministic counting sort by expert.
//   count:   per-chunk histograms (integer LDS atomics: exact counts)
//   scan:    per-expert prefix over chunks, then the exclusive scan over experts and
//            the unit table of the expert launches (runs of at most nu positions)
//   scatter: position = offsets[e] + chunk prefix + rank among the chunk's earlier
//            assignments of the same expert (stable: increasing t*k+j)
// ------------------------------------------------------------------------------------
__global__ __launch_bounds__(kBlock) void k_disp_count(const int32_t* idx, int64_t n, int E,
                                                       int chunk, int32_t* chunk_hist) {
  __shared__ int hist[1024];
  for (int e = threadIdx.x; e < E; e += kBlock) hist[e] = 0;
  __syncthreads();
  const int64_t a0 = (int64_t)blockIdx.x * chunk;
  const int64_t a1 = min(n, a0 + chunk);
  for (int64_t i = a0 + threadIdx.x; i < a1; i += kBlock) atomicAdd(&hist[idx[i]], 1);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kBlock) chunk_hist[(int64_t)blockIdx.x * E + e] = hist[e];
}

// Units of at most `small` positions come first in the table (ctrl[1] of them), then
// the larger ones; ctrl[0] = all units.  Each list runs in expert order.  (With `even`
// the units of an expert are near-equal, unit_run, and small >= nu: one list.)
__global__ __launch_bounds__(1024) void k_disp_scan(int n_chunks, int E, int nu, int small, int even,
                                                    int32_t* chunk_hist, int32_t* counts,
                                                    int32_t* offs, int32_t* units,
                                                    int32_t* ctrl) {
  __shared__ int sc[1024];
  __shared__ int su[1024];
  __shared__ int sb[1024];
  const int e = threadIdx.x;
  int tot = 0;
  if (e < E) {
    // the chunks' counts in groups of 32 loads in flight, then their exclusive scan in place
    // (a load after each store of the scan would wait out its whole latency)
    constexpr int kGroup = 32;
    for (int c0 = 0; c0 < n_chunks; c0 += kGroup) {
      int v[kGroup];
#pragma unroll
      for (int j = 0; j < kGroup; ++j)
        v[j] = c0 + j < n_chunks ? chunk_hist[(int64_t)(c0 + j) * E + e] : 0;
#pragma unroll
      for (int j = 0; j < kGroup; ++j) {
        if (c0 + j < n_chunks) chunk_hist[(int64_t)(c0 + j) * E + e] = tot;
        tot += v[j];
      }
    }
    counts[e] = tot;
  }
  // this expert's units: tot / nu full ones and a tail of tot % nu positions (or, even,
  // ceil(tot / nu) units of at most nu <= small positions)
  const int full = tot / nu, tail = tot - full * nu;
  const bool full_small = nu <= small;
  const int ns = (e < E) ? (even ? (tot + nu - 1) / nu : (full_small ? full : 0) + (tail > 0 && tail <= small)) : 0;
  const int nb = (e < E && !even) ? (full_small ? 0 : full) + (tail > small) : 0;
  sc[e] = (e < E) ? tot : 0;
  su[e] = ns;
  sb[e] = nb;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int v = (e >= o) ? sc[e - o] : 0;
    const int w = (e >= o) ? su[e - o] : 0;
    const int x = (e >= o) ? sb[e - o] : 0;
    __syncthreads();
    sc[e] += v;
    su[e] += w;
    sb[e] += x;
    __syncthreads();
  }
  const int n_small = su[1023];
  if (e < E) {
    const int off = sc[e] - tot;
    offs[e] = off;
    int us = su[e] - ns, ub = n_small + sb[e] - nb;
    const int nun = (tot + nu - 1) / nu;
    for (int j = 0; j < nun; ++j) {
      int r0, n;
      unit_run(tot, nu, even, j, r0, n);
      const int slot = (even || n <= small) ? us++ : ub++;
      *reinterpret_cast<int4*>(units + 4 * slot) = make_int4(e, off + r0, n, 0);
    }
  }
  if (e == 0) offs[E] = sc[1023];
  if (e == 1023) {
    ctrl[0] = n_small + sb[1023];
    ctrl[1] = n_small;
  }
}

__global__ __launch_bounds__(kBlock) void k_disp_scatter(const int32_t* idx, int64_t n, int E,
                                                         int chunk, const int32_t* chunk_hist,
                                                         const int32_t* offs, int32_t* perm,
                                                         int32_t* inv) {
  __shared__ int se[kBlock];
  const int64_t a0 = (int64_t)blockIdx.x * chunk;
  const int cnt = (int)min((int64_t)chunk, n - a0);
  const int i = threadIdx.x;
  if (i < cnt) se[i] = idx[a0 + i];
  __syncthreads();
  if (i < cnt) {
    const int e = se[i];
    int r = 0;
    for (int q = 0; q < i; ++q) r += (se[q] == e);
    const int pos = offs[e] + chunk_hist[(int64_t)blockIdx.x * E + e] + r;
    perm[pos] = (int32_t)(a0 + i);
    inv[a0 + i] = pos;
  }
}


// ------------------------------------------------------------------------------------
// Quantile Balancing statistics (the toy chapter's "Quantile Balancing"; the walkthrough's
// "Stable 之三" and its histogram estimate).  Per token the cutoff alpha = the (k+1)-th
// largest s + b (route with the top k + 1); per expert e the bias r = alpha - s_e it would
// need to make the token's top k, counted into hist[e][bins] over [min b - 1, max b + 1]
// (integer atomics: the counts do not depend on the order).  The readout takes per expert
// the first bin where the cumulative count reaches ceil(T k / E), interpolates linearly
// inside it, and removes the mean over the experts.
// ------------------------------------------------------------------------------------
struct QbArgs {
  float* z;
  int zplanes, zsub;
  int64_t zplane;
  const float* bias;
  int64_t T;
  int E, k, bins;
  int32_t* hist;
  float* alpha;             // [T] the cutoffs (k_qb_alpha -> k_qb_count)
  int eb, tc;               // k_qb_count: experts and tokens per workgroup
  const int32_t* chist;     // readout: the counts
  float* new_bias;          // readout: the centred biases
};

// (min b - 1, max b + 1) by the whole workgroup, from the float32 biases (E <= 1024).
__device__ __forceinline__ void qb_range(const float* bias, int E, float* red, float& lo,
                                         float& hi) {
  const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x >> 6;
  float mn = INFINITY, mx = -INFINITY;
  for (int e = threadIdx.x; e < E; e += kBlock) {
    mn = fminf(mn, bias[e]);
    mx = fmaxf(mx, bias[e]);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    mn = fminf(mn, __shfl_xor(mn, o));
    mx = fmaxf(mx, __shfl_xor(mx, o));
  }
  if (lane == 0) {
    red[wv] = mn;
    red[kWavesPerBlock + wv] = mx;
  }
  __syncthreads();
  mn = red[0];
  mx = red[kWavesPerBlock];
#pragma unroll
  for (int w = 1; w < kWavesPerBlock; ++w) {
    mn = fminf(mn, red[w]);
    mx = fmaxf(mx, red[kWavesPerBlock + w]);
  }
  __syncthreads();
  lo = mn - 1.0f;
  hi = mx + 1.0f;
}

// The logit of expert e for token t: the partial planes added in plane order (as the
// route adds them), then the float32 sigmoid.
__device__ __forceinline__ float qb_score(const QbArgs& a, int64_t t, int e) {
  const float* zr = a.z + t * a.E + e;
  float zp[kMaxZPlanes];
#pragma unroll
  for (int p = 0; p < kMaxZPlanes; ++p) zp[p] = p < a.zplanes * a.zsub ? zr[p * a.zplane] : 0.f;
  return sigmoidf_(plane_sum(zp, a.zplanes, a.zsub));
}

// alpha[t] = the (k+1)-th largest s + b of token t, one workgroup per token (grid stride);
// the scores s replace the token's logits in plane 0.
__global__ __launch_bounds__(kBlock) void k_qb_alpha(QbArgs a) {
  __shared__ uint64_t cand_key[kWavesPerBlock * kMaxK];
  __shared__ float cand_v[kWavesPerBlock * kMaxK];
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x >> 6;
  const int kk = a.k + 1;   // the cutoff is the (k+1)-th largest
  for (int64_t t = blockIdx.x; t < a.T; t += gridDim.x) {
    uint64_t key[kRouteSlots];
    float kv[kRouteSlots];
#pragma unroll
    for (int i = 0; i < kRouteSlots; ++i) {
      const int e = (i * kWavesPerBlock + wv) * kWave + lane;
      key[i] = 0;
      kv[i] = 0.f;
      if (e < a.E) {
        const float sc = qb_score(a, t, e);
        a.z[t * a.E + e] = sc;     // plane 0 keeps the score for the counts (read above)
        float kap = sc + a.bias[e];
        if (kap != kap) kap = -INFINITY;
        kv[i] = kap;
        key[i] = ((uint64_t)float_order_key(kap) << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)e);
      }
    }
    // the wave's k + 1 largest keys, then their rank among all waves' candidates
    uint64_t head = 0;
#pragma unroll
    for (int i = 0; i < kRouteSlots; ++i) head = max_u64(head, key[i]);
    for (int j = 0; j < kk; ++j) {
      const uint64_t m = wave_max_u64(head);
      float v_win = -INFINITY;
      if (m != 0) {
        const int e = (int)(0xFFFFFFFFu - (uint32_t)m);
        const int owner = e & (kWave - 1);
        const int slot = e >> 8;
        float mine = 0.f;
#pragma unroll
        for (int i = 0; i < kRouteSlots; ++i) mine = (i == slot) ? kv[i] : mine;
        v_win = __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(mine), owner));
        if (lane == owner) {
          head = 0;
#pragma unroll
          for (int i = 0; i < kRouteSlots; ++i) {
            if (i == slot) key[i] = 0;
            head = max_u64(head, key[i]);
          }
        }
      }
      if (lane == 0) {
        cand_key[wv * kMaxK + j] = m;
        cand_v[wv * kMaxK + j] = v_win;
      }
    }
    __syncthreads();
    {
      const int c = threadIdx.x;
      const int j = c & (kMaxK - 1);
      const uint64_t kc = cand_key[c];
      if (j < kk && kc != 0) {
        int rank = 0;
#pragma unroll
        for (int w = 0; w < kWavesPerBlock; ++w)
          for (int q = 0; q < kk; ++q) rank += (cand_key[w * kMaxK + q] > kc);
        if (rank == a.k) a.alpha[t] = cand_v[c];
      }
    }
    __syncthreads();   // the candidate tables are rewritten by the next token
  }
}

// The counts: a workgroup takes eb consecutive experts (their eb x bins counters in LDS)
// and tc consecutive tokens; thread i walks (token, expert) pairs with the expert fastest
// so that a wavefront's plane loads are contiguous runs.  r = alpha - s and the bin in
// float32 (s from plane 0, where k_qb_alpha left it), LDS atomics, then the non-zero
// counters added to the global histogram.
__global__ __launch_bounds__(kBlock) void k_qb_count(QbArgs a) {
  extern __shared__ int32_t cnt[];
  __shared__ float red[2 * kWavesPerBlock];
  float lo, hi;
  qb_range(a.bias, a.E, red, lo, hi);
  const float inv_w = (float)a.bins / (hi - lo);
  const int n_eg = (a.E + a.eb - 1) / a.eb;
  const int eg = blockIdx.x % n_eg;
  const int64_t tb = blockIdx.x / n_eg;
  const int e0 = eg * a.eb, ne = min(a.eb, a.E - e0);
  const int64_t t0 = tb * a.tc;
  const int64_t nt = min((int64_t)a.tc, a.T - t0);
  for (int i = threadIdx.x; i < a.eb * a.bins; i += kBlock) cnt[i] = 0;
  __syncthreads();
  const int64_t n = nt * ne;
  for (int64_t i = threadIdx.x; i < n; i += kBlock) {
    const int64_t t = t0 + i / ne;
    const int el = (int)(i % ne);
    const float r = a.alpha[t] - a.z[t * a.E + e0 + el];
    const float u = (r - lo) * inv_w;
    const int b = (u == u) ? (int)fmaxf(0.f, fminf(floorf(u), (float)(a.bins - 1))) : 0;
    atomicAdd(cnt + el * a.bins + b, 1);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < ne * a.bins; i += kBlock) {
    const int v = cnt[i];
    if (v) atomicAdd(a.hist + (int64_t)(e0 + i / a.bins) * a.bins + i % a.bins, v);
  }
}

// Readout, one workgroup per expert: thread i sums bins [i c, i c + c) (c = ceil(bins /
// 256)), an exclusive scan of those sums finds the thread whose bins reach ceil(T k / E),
// and that thread walks them to the bin and interpolates.  The uncentred value goes to
// new_bias[e]; k_qb_centre removes the mean.
__global__ __launch_bounds__(kBlock) void k_qb_readout(QbArgs a) {
  __shared__ float red[2 * kWavesPerBlock];
  __shared__ int64_t pre[kBlock];
  __shared__ float found;
  const int e = blockIdx.x;
  float lo, hi;
  qb_range(a.bias, a.E, red, lo, hi);
  const float w = (hi - lo) / (float)a.bins;
  const int64_t qc = (a.T * a.k + a.E - 1) / a.E;
  const int32_t* h = a.chist + (int64_t)e * a.bins;
  const int per = (a.bins + kBlock - 1) / kBlock;
  const int t0 = min(a.bins, (int)threadIdx.x * per), t1 = min(a.bins, t0 + per);
  int64_t mine = 0;
  for (int t = t0; t < t1; ++t) mine += h[t];
  pre[threadIdx.x] = mine;
  if (threadIdx.x == 0) found = hi;   // no bin reaches the target: the top of the range
  __syncthreads();
  for (int o = 1; o < kBlock; o <<= 1) {   // inclusive scan
    const int64_t v = (int)threadIdx.x >= o ? pre[threadIdx.x - o] : 0;
    __syncthreads();
    pre[threadIdx.x] += v;
    __syncthreads();
  }
  int64_t cum = pre[threadIdx.x] - mine;
  if (cum < qc && cum + mine >= qc) {
    for (int t = t0; t < t1; ++t) {
      const int64_t c = h[t];
      if (c > 0 && cum + c >= qc) {
        found = lo + w * ((float)t + (float)(qc - cum) / (float)c);
        break;
      }
      cum += c;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) a.new_bias[e] = found;
}

// new_bias -= mean(new_bias) over the experts, one workgroup, a fixed summation order.
__global__ __launch_bounds__(kBlock) void k_qb_centre(QbArgs a) {
  __shared__ float red[kWavesPerBlock];
  const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x >> 6;
  float part = 0.f;
  for (int e = threadIdx.x; e < a.E; e += kBlock) part += a.new_bias[e];   // e = tid, tid + 256, ...
  part = wave_sum(part);
  if (lane == 0) red[wv] = part;
  __syncthreads();
  const float mean = ((red[0] + red[1]) + (red[2] + red[3])) / (float)a.E;
  for (int e = threadIdx.x; e < a.E; e += kBlock) a.new_bias[e] -= mean;
}

// ------------------------------------------------------------------------------------
// Step COMBINE: u[t] = sum_j G[t,j] E[inv[t,j]], j = 0..k-1 in order.
// ------------------------------------------------------------------------------------
__global__ __launch_bounds__(kBlock) void k_combine(const float* __restrict__ gw,
                                                    const int32_t* __restrict__ inv,
                                                    const float* __restrict__ eo, int64_t T,
                                                    int k, int l, int blocks_per_tok,
                                                    float* __restrict__ u) {
  __shared__ float sg[kMaxK];
  __shared__ int si[kMaxK];
  const int64_t t = blockIdx.x / blocks_per_tok;
  const int r = (int)(blockIdx.x - t * blocks_per_tok) * kBlock + threadIdx.x;
  if (t >= T) return;
  if ((int)threadIdx.x < k) {
    sg[threadIdx.x] = gw[t * k + threadIdx.x];
    si[threadIdx.x] = inv[t * k + threadIdx.x];
  }
  __syncthreads();
  if (r >= l) return;
  float acc = 0.f;
  for (int j0 = 0; j0 < k; j0 += 16) {
    float v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = (j0 + i < k) ? eo[(int64_t)si[j0 + i] * l + r] : 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (j0 + i < k) acc = fmaf(sg[j0 + i], v[i], acc);
  }
  u[t * l + r] = acc;
}


// ------------------------------------------------------------------------------------
// Weight streaming on the matrix cores.
//
// Every weight matrix is packed (moe_pack_dense / moe_pack_experts) into tile rows of 16
// output rows; a tile row is a run of K-steps of 128 input columns.  In a bf16 K-step,
// sub-tile s (1 KiB) holds columns 32s..32s+31 with lane l's 16 bytes = row l % 16,
// columns 32s + 8 (l / 16) .. +8: exactly the B operand of v_mfma_f32_16x16x32_bf16, so
// one wavefront load brings 1 KiB of contiguous bytes and feeds one MFMA.  An MXFP4
// K-step is 1 KiB of codes (lane l: the 32 codes of row l % 16, columns 32 (l / 16) ..
// +32, one MX block, as the checkpoint stores them) plus the 16 rows' four scale bytes.
// With few tokens the codes become bf16 operands through v_cvt_scalef32_pk_bf16_fp4
// (exact); on the compute-bound path the same bytes are the B operand of the scaled
// 16x16x128 FP4 MFMA.
//
// The activations form the A operand: up to 16 rows staged once per workgroup in LDS.
// bf16 tokens are rows as they are; fp32 activations are split into a bf16 pair
// hi = bf16(v), lo = bf16(v - hi) in rows 2i, 2i + 1, so that hi + lo carries 16
// significant bits and both MFMA products are exact: D = A W^T then holds fp32-accurate
// dot products (row 2i + row 2i+1 of D).  D row r of the 16x16 block depends on A row r
// alone, so lanes beyond the staged rows read a duplicate row and are ignored.
//
// LDS layout of the staged rows: the 16-byte word (q, j, r) at (16 q + j) nr + r holds
// row r, columns 128 q + 8 j .. +8 (piece j of K-step q; nr = rows staged).
// ------------------------------------------------------------------------------------

// Tokens x (bf16, row stride ld) rows r0..r0+nr-1 into LDS; columns >= n are zero.
__device__ __forceinline__ void stage_bf16(uint4* sm, const uint16_t* x, int64_t ld, int nr,
                                           int n, int ks) {
  const int per_row = ks * 16;
  for (int idx = threadIdx.x; idx < nr * per_row; idx += kBlock) {
    const int r = idx / per_row, j = idx - r * per_row;
    const int col = 8 * j;
    const uint4 v = (col < n) ? *reinterpret_cast<const uint4*>(x + r * ld + col)
                              : make_uint4(0u, 0u, 0u, 0u);
    sm[j * nr + r] = v;  // j = 16 q + piece
  }
}

// One activation row staged from loads issued before the weight stream of the launch (the
// loads complete in issue order, so staging loads issued after the stream would wait for
// it).  Bf16RowPre: stage_bf16 of one row (nr = 1), up to 4 pieces of 8 columns per thread.
constexpr int kPreBf16 = 4;
struct Bf16RowPre {
  uint4 v[kPreBf16];
  static __device__ __forceinline__ bool fits(int ks) { return ks * 16 <= kBlock * kPreBf16; }
  __device__ __forceinline__ void load(const uint16_t* x, int n, int ks) {
#pragma unroll
    for (int m = 0; m < kPreBf16; ++m) {
      const int j = threadIdx.x + kBlock * m;
      if (j < ks * 16)
        v[m] = 8 * j < n ? *reinterpret_cast<const uint4*>(x + 8 * j) : make_uint4(0u, 0u, 0u, 0u);
    }
  }
  __device__ __forceinline__ void commit(uint4* sm, int ks) const {
#pragma unroll
    for (int m = 0; m < kPreBf16; ++m) {
      const int j = threadIdx.x + kBlock * m;
      if (j < ks * 16) sm[j] = v[m];
    }
  }
};

// Eight fp32 values into the hi and lo bf16 words.
__device__ __forceinline__ void split_hilo(const float (&v)[8], uint4& hi, uint4& lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
    const float h0 = bf16_lo(h[i]), h1 = bf16_hi(h[i]);
    l[i] = pack_bf16x2(v[2 * i] - h0, v[2 * i + 1] - h1);
  }
  hi = make_uint4(h[0], h[1], h[2], h[3]);
  lo = make_uint4(l[0], l[1], l[2], l[3]);
}

// An fp32 value as the hi/lo bf16 pair the token-tiled launches read: p[0] = hi, p[ld] = lo
// (the same split as split_hilo).
__device__ __forceinline__ void store_hilo(uint16_t* p, int64_t ld, float v) {
  const uint32_t w = pack_bf16x2(v, 0.f);
  const float h = bf16_lo(w);
  p[0] = (uint16_t)(w & 0xFFFFu);
  p[ld] = (uint16_t)(pack_bf16x2(v - h, 0.f) & 0xFFFFu);
}

// An fp32 activation row for the hi/lo staging: columns [0, n0) from p0 (optionally
// times scale * gamma[c]), columns [c1, c1 + n1) from p1, zero elsewhere.
struct HiloRow {
  const float* p0;
  const float* p1;
  float scale;
};

__device__ __forceinline__ void load8(const float* p, float (&v)[8]) {
  const float4 a = reinterpret_cast<const float4*>(p)[0];
  const float4 b = reinterpret_cast<const float4*>(p)[1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// nt fp32 rows (rows[i], resolved by the caller into the per-row pointers) as 2*nt hi/lo
// rows; gamma (bf16, may be null) multiplies segment 0 with the row's scale.
__device__ __forceinline__ void stage_hilo(uint4* sm, const HiloRow* rows, int nt, int n0,
                                           int c1, int n1, const uint16_t* gamma, int ks) {
  const int per_row = ks * 16;
  const int nr = 2 * nt;
  for (int idx = threadIdx.x; idx < nt * per_row; idx += kBlock) {
    const int i = idx / per_row, j = idx - i * per_row;
    const int col = 8 * j;
    float v[8];
    if (col < n0) {
      load8(rows[i].p0 + col, v);
      if (gamma) {
        const uint4 g = *reinterpret_cast<const uint4*>(gamma + col);
        const float s = rows[i].scale;
        v[0] = v[0] * s * bf16_lo(g.x); v[1] = v[1] * s * bf16_hi(g.x);
        v[2] = v[2] * s * bf16_lo(g.y); v[3] = v[3] * s * bf16_hi(g.y);
        v[4] = v[4] * s * bf16_lo(g.z); v[5] = v[5] * s * bf16_hi(g.z);
        v[6] = v[6] * s * bf16_lo(g.w); v[7] = v[7] * s * bf16_hi(g.w);
      }
    } else if (col >= c1 && col < c1 + n1) {
      load8(rows[i].p1 + (col - c1), v);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = 0.f;
    }
    uint4 hi, lo;
    split_hilo(v, hi, lo);
    sm[j * nr + 2 * i] = hi;
    sm[j * nr + 2 * i + 1] = lo;
  }
}

// stage_hilo of one fp32 row (nt = 1, segment 0 of n0 columns, no gamma) from loads issued
// before the weight stream, up to 2 pieces of 8 columns per thread.
constexpr int kPreHilo = 2;
struct HiloRowPre {
  float4 v[kPreHilo][2];
  static __device__ __forceinline__ bool fits(int ks) { return ks * 16 <= kBlock * kPreHilo; }
  __device__ __forceinline__ void load(const float* p, int n0, int ks) {
#pragma unroll
    for (int m = 0; m < kPreHilo; ++m) {
      const int j = threadIdx.x + kBlock * m;
      if (j < ks * 16 && 8 * j < n0) {
        v[m][0] = reinterpret_cast<const float4*>(p + 8 * j)[0];
        v[m][1] = reinterpret_cast<const float4*>(p + 8 * j)[1];
      }
    }
  }
  __device__ __forceinline__ void commit(uint4* sm, int n0, int ks) const {
#pragma unroll
    for (int m = 0; m < kPreHilo; ++m) {
      const int j = threadIdx.x + kBlock * m;
      if (j >= ks * 16) continue;
      float e[8];
      if (8 * j < n0) {
        e[0] = v[m][0].x; e[1] = v[m][0].y; e[2] = v[m][0].z; e[3] = v[m][0].w;
        e[4] = v[m][1].x; e[5] = v[m][1].y; e[6] = v[m][1].z; e[7] = v[m][1].w;
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) e[i] = 0.f;
      }
      uint4 hi, lo;
      split_hilo(e, hi, lo);
      sm[2 * j] = hi;
      sm[2 * j + 1] = lo;
    }
  }
};

// The weight registers of one tile row in flight: P K-steps, filled by prefetch() before
// the activations are staged (so that the stream starts at once) and consumed by run().
template <int WF, int P>
struct TileStream {
  WeightStep<WF> w[P];
  // K-steps q0 .. q0 + P - 1 (clamped to the last of the n >= 1 steps of the wavefront)
  __device__ __forceinline__ void prefetch(const uint8_t* trow, int q0, int n) {
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int i = 0; i < P; ++i) w[i].load(trow, q0 + min(i, n - 1), lane);
  }
};

// One tile row over K-steps [q0, q0 + n) after prefetch(trow, q0, n): D += A W^T on the
// 16 x 16 block (A = staged rows, W = the tile row's 16 weight rows).  N > 0: n == N at
// compile time, the loop fully unrolled, so every load is unconditional and the waits
// count exactly the loads in flight; N == 0: any n, the loads past the end clamped to
// the last K-step (re-reads that are never used).
// `arow` is the lane's staged row, `nr` the rows staged (word 16 q nr + piece nr + row).
template <int WF, int P, int N>
__device__ __forceinline__ f32x4_t run_tile_row(TileStream<WF, P>& ts, const uint8_t* trow,
                                                int q0, int n, const uint4* sm, int arow,
                                                int nr) {
  const int lane = threadIdx.x & (kWave - 1);
  const int g = lane >> 4;
  const uint4* ap = sm + arow + q0 * 16 * nr;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  if (N > 0) {
#pragma unroll
    for (int q = 0; q < N; ++q) {
      acc = ts.w[q % P].mma(ap + q * 16 * nr, nr, g, acc);
      if (q + P < N) {
        ts.w[q % P].load(trow, q0 + q + P, lane);
        asm volatile("" ::: "memory");
      }
      // FP8: every K-step's products start from zero and only the scaled sums chain the
      // steps; pin each step's sum here, or the compiler defers them all to the end and
      // holds every step's products in registers at once
      if (WeightStep<WF>::kFp8) asm volatile("" : "+v"(acc));
    }
    return acc;
  }
  const int ql = q0 + n - 1;
  for (int j = 0; j < n; j += P) {
#pragma unroll
    for (int i = 0; i < P; ++i) {
      if (j + i < n) acc = ts.w[i].mma(ap + (j + i) * 16 * nr, nr, g, acc);
      ts.w[i].load(trow, min(q0 + j + i + P, ql), lane);
    }
    asm volatile("" ::: "memory");
  }
  return acc;
}

// run_tile_row with the K-step count as a compile-time constant where it is 1..32.
template <int WF, int P>
__device__ __forceinline__ f32x4_t run_tile_row_n(TileStream<WF, P>& ts, const uint8_t* trow,
                                                  int q0, int n, const uint4* sm, int arow,
                                                  int nr) {
  if (n <= 0) return f32x4_t{0.f, 0.f, 0.f, 0.f};
  switch (n) {
#define MOE_N_CASE(N) \
  case N: return run_tile_row<WF, P, N>(ts, trow, q0, n, sm, arow, nr);
    MOE_N_CASE(1) MOE_N_CASE(2) MOE_N_CASE(3) MOE_N_CASE(4) MOE_N_CASE(5) MOE_N_CASE(6)
    MOE_N_CASE(7) MOE_N_CASE(8) MOE_N_CASE(9) MOE_N_CASE(10) MOE_N_CASE(11) MOE_N_CASE(12)
    MOE_N_CASE(13) MOE_N_CASE(14) MOE_N_CASE(15) MOE_N_CASE(16) MOE_N_CASE(17) MOE_N_CASE(18)
    MOE_N_CASE(19) MOE_N_CASE(20) MOE_N_CASE(21) MOE_N_CASE(22) MOE_N_CASE(23) MOE_N_CASE(24)
    MOE_N_CASE(25) MOE_N_CASE(26) MOE_N_CASE(27) MOE_N_CASE(28) MOE_N_CASE(29) MOE_N_CASE(30)
    MOE_N_CASE(31) MOE_N_CASE(32)
#undef MOE_N_CASE
    default: return run_tile_row<WF, P, 0>(ts, trow, q0, n, sm, arow, nr);
  }
}

// run_tile_row for a wavefront whose whole range of n <= P K-steps is in the ring (loaded
// before it stages its activations), unrolled per count (run_tile_row_n's counts above P
// would hold two generations of the ring in registers); P = 3 is run_tile_row_n.
template <int WF, int P>
__device__ __forceinline__ f32x4_t run_tile_row_upto(TileStream<WF, P>& ts, const uint8_t* trow,
                                                     int q0, int n, const uint4* sm, int arow,
                                                     int nr) {
  if constexpr (P == 3) {
    return run_tile_row_n<WF, 3>(ts, trow, q0, n, sm, arow, nr);
  } else {
    static_assert(P <= 8, "counts up to 8");
    switch (n) {
#define MOE_N_CASE(N) \
  case N: if constexpr (N <= P) return run_tile_row<WF, P, N>(ts, trow, q0, n, sm, arow, nr); else break;
      MOE_N_CASE(1) MOE_N_CASE(2) MOE_N_CASE(3) MOE_N_CASE(4) MOE_N_CASE(5) MOE_N_CASE(6)
      MOE_N_CASE(7) MOE_N_CASE(8)
#undef MOE_N_CASE
      default: break;
    }
    return f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
}

// Partial blocks of the K-split: waves kp > 0 of a tile row hand theirs to the wave with
// kp = 0, which adds them in the order kp = 1, 2, ... (a fixed order).
__device__ __forceinline__ f32x4_t reduce_ksplit(f32x4_t acc, f32x4_t (*part)[kWave], int ksplit,
                                                 int kp) {
  if (ksplit == 1) return acc;
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (kp > 0) part[wv][lane] = acc;
  __syncthreads();
  if (kp == 0)
    for (int i = 1; i < ksplit; ++i) acc += part[wv + i][lane];
  return acc;
}

// ------------------------------------------------------------------------------------
// Steps ROUTER and IN: the three products with the token as input, over the packed IN
// matrix [router ; W_down_latent ; shared gate/up]: z = x W_r^T, x^c = x W_down^T and
// h_s = act(x W_sg^T, x W_su^T).  A launch covers a range of tile rows, 4/ksplit tile
// rows per workgroup with K split between ksplit wavefronts, a workgroup staging up to
// ntb tokens (bf16 rows).  The ROUTER launch takes the router (as partial logit planes
// over ranges of K, see in_body) and W_down_latent; the IN launch the shared gate/up,
// and with few tokens its workgroup 0 meanwhile takes the route and the dispatch from the
// logits of the ROUTER launch (hidden behind the stream of the shared weights, which do
// not depend on the route).
// ------------------------------------------------------------------------------------
struct InArgs {
  const uint8_t* w;
  int ks, tr_r, tr_dn, tr_sh, ksplit, ntb;
  int router_wgs, zplanes;    // router K-range workgroups first (per token block) ...
  int tr_first, tr_count;     // ... then the tile rows [tr_first, tr_first + tr_count)
  int wg_per_blk;             // workgroups per token block (route workgroup excluded)
  int n_blk;                  // token blocks
  const uint16_t* x;
  int64_t T;
  int d;
  float* z;
  int E;
  float* xc;
  int l;
  float* hs;
  int ms;
  int act;
  float bg, bl;
  int route;
  RouteArgs ra;
  // n_arrive > 0: the router rows run in this launch too.  Their workgroups store their
  // logits with agent-scope stores and then count themselves in *arrive; workgroup 0 waits
  // for all n_arrive of them (after which it zeroes the counter) before the route.
  int32_t* arrive;
  int n_arrive;
};

// Spin limit of the route's wait for the router workgroups of its launch (each try sleeps
// about 0.1 us); a wait that reaches it goes on (and counts itself in the word after the
// counter) rather than hold the GPU.
constexpr int kRouteSpinLimit = 1 << 22;

__device__ __forceinline__ void in_body(const InArgs& a) {
  extern __shared__ uint4 sm[];
  __shared__ f32x4_t part[kWavesPerBlock][kWave];
  if (a.route) {
    // the logits come from the ROUTER launch; this workgroup's selection runs while the
    // others stream the shared weights
    if (blockIdx.x == 0) {
      if (a.n_arrive > 0) {
        if (threadIdx.x == 0) {
          int n = 0;
          while (__hip_atomic_load(a.arrive, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < a.n_arrive &&
                 ++n < kRouteSpinLimit)
            __builtin_amdgcn_s_sleep(2);
          if (n == kRouteSpinLimit)
            __hip_atomic_fetch_add(a.arrive + 1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_store(a.arrive, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
        route_block<true>(a.ra, 0, a.T, true);
      } else {
        route_block(a.ra, 0, a.T, true);
      }
      return;
    }
  }
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15, g = lane >> 4;
  const int bid = blockIdx.x - a.route;
  int wgi, blk;
  if (!xcd_item(bid, a.wg_per_blk, a.n_blk, wgi, blk)) return;
  const int64_t t0 = (int64_t)blk * a.ntb;
  const int nt = (int)min((int64_t)a.ntb, a.T - t0);
  const bool router = wgi < a.router_wgs;
  int tr, kp, ksplit, q0, q1;
  if (router) {
    // router tile row wgi / zplanes, K-range plane wgi % zplanes split over the 4
    // wavefronts, each of which stores its part as a sub-plane (kZSub = 4); the route adds
    // them
    tr = wgi / a.zplanes;
    const int plane = wgi - tr * a.zplanes;
    const int qpp = cdiv(a.ks, a.zplanes);
    const int r0 = min(a.ks, plane * qpp), r1 = min(a.ks, r0 + qpp);
    const int qw = cdiv(r1 - r0, kWavesPerBlock);
    kp = wv;
    ksplit = kWavesPerBlock;
    q0 = min(r1, r0 + wv * qw);
    q1 = min(r1, q0 + qw);
  } else {
    const int slot = (wgi - a.router_wgs) * kWavesPerBlock + wv;
    ksplit = a.ksplit;
    tr = slot / ksplit;
    kp = slot - tr * ksplit;
    tr = tr < a.tr_count ? a.tr_first + tr : INT_MAX;
    const int qper = cdiv(a.ks, ksplit);
    q0 = min(a.ks, kp * qper);
    q1 = min(a.ks, q0 + qper);
  }
  const bool live = tr != INT_MAX && q1 > q0;
  const uint8_t* trow = a.w + (size_t)(live ? tr : 0) * a.ks * kBf16StepBytes;
  TileStream<0, 3> ts;
  if (nt == 1 && Bf16RowPre::fits(a.ks)) {   // one token: its row first, then the stream
    Bf16RowPre pre;
    pre.load(a.x + t0 * a.d, a.d, a.ks);
    ts.prefetch(trow, live ? q0 : 0, live ? q1 - q0 : 1);   // unconditional: see k_out
    pre.commit(sm, a.ks);
  } else {
    if (live) ts.prefetch(trow, q0, q1 - q0);
    stage_bf16(sm, a.x + t0 * a.d, a.d, nt, a.d, a.ks);
  }
  __syncthreads();
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  if (live) acc = run_tile_row_n<0, 3>(ts, trow, q0, q1 - q0, sm, c % nt, nt);
  static_assert(kZSub == kWavesPerBlock, "a router wavefront per sub-plane");
  if (!router) acc = reduce_ksplit(acc, part, ksplit, kp);
  if (tr != INT_MAX && (router || kp == 0)) {
    // D row 4g + v = token 4g + v of the block, column c = weight row 16 tr + c
    if (router) {
      const int e = 16 * tr + c;
      float* zp = a.z + (int64_t)((wgi - tr * a.zplanes) * kZSub + kp) * a.T * a.E;
#pragma unroll
      for (int v = 0; v < 4; ++v)
        if (4 * g + v < nt && e < a.E) {
          float* o = zp + (t0 + 4 * g + v) * a.E + e;
          if (a.n_arrive > 0) __hip_atomic_store(o, acc[v], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          else *o = acc[v];
        }
    } else if (tr < a.tr_r + a.tr_dn) {
      const int r = 16 * (tr - a.tr_r) + c;
#pragma unroll
      for (int v = 0; v < 4; ++v)
        if (4 * g + v < nt && r < a.l) a.xc[(t0 + 4 * g + v) * a.l + r] = acc[v];
    } else {
      const int r = 8 * (tr - a.tr_r - a.tr_dn) + (c - 8);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float gate = from_gate_lane(acc[v]);
        if (c >= 8 && 4 * g + v < nt && r < a.ms)
          a.hs[(t0 + 4 * g + v) * a.ms + r] = glu_act(gate, acc[v], a.act, a.bg, a.bl);
      }
    }
  }
  if (router && a.n_arrive > 0) {
    // every logit of the workgroup stored before its arrival is counted
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) __hip_atomic_fetch_add(a.arrive, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Entry points over the same body so that profilers tell the launches apart.
__global__ __launch_bounds__(kBlock) void k_router(InArgs a) { in_body(a); }
__global__ __launch_bounds__(kBlock) void k_in(InArgs a) { in_body(a); }

// ------------------------------------------------------------------------------------
// Routed experts.  The unit table lists runs of at most nu dispatch positions of one
// expert; a work item is (unit, group of 4/ksplit tile rows).  Gate/up: the input rows
// are x^c of the positions' tokens and the output h[p] = act(g, u) (tile rows carry 8
// gate and the matching 8 up rows); down: the input rows are h[p], the output E[p].
// The workgroups walk the items with a grid stride (the number of units is known only
// on the device).
// ------------------------------------------------------------------------------------
struct ExpArgs {
  const uint8_t* experts;
  size_t expert_bytes, region_off;
  int ks, n_tr, ksplit, wg_per_unit;
  const int32_t* units;
  const int32_t* ctrl;
  int max_units, nu, E, k;
  int chunk;                // > 0: chunk_item work order (token-tiled launches), else xcd_item
  int64_t n_assign;
  const int32_t* perm;
  const float* xin;
  int kin;
  float* out;
  int n_out;
  int act;
  float bg, bl;
  const uint16_t* xin_hl;   // token-tiled launches: hi/lo input rows [rows][2][kin_ld]
  int kin_ld;
  uint16_t* out_hl;         // and the gate/up output's hi/lo rows [T*k][2][out_ld]
  int out_ld;
  int single;               // 1: the input is bf16 (lo rows zero): the long units read the
                            // hi rows alone, one row per position
  // The down launch of a few tokens of a latent layer also takes the shared down-projection
  // W_sd h_s, in its first sd_wgs workgroups: sd_parts partial products over ranges of
  // sd_qper of the sd_ks K-steps that W_sd's tile rows hold from K-step sd_q0 of the OUT
  // matrix (rows of sd_row K-steps), each written as (hi, lo) row sums [part][T][d].
  const uint8_t* sd_w;
  int sd_wgs, sd_parts, sd_q0, sd_qper, sd_ks, sd_row, sd_ntr;
  const float* sd_hs;
  int sd_ms, sd_T, sd_d;
  float2* sd_out;
};

// Gate/up: h[p] = act(gate, up) (and, with out_hl, its hi/lo row for the token-tiled down
// launch); down: E[p].
// y0, y1 are the sums of positions i0 and i0 + 1 of the unit (position offset p0, n used).
template <bool GU>
__device__ __forceinline__ void exp_store(const ExpArgs& a, int p0, int n, int tr, int c, int i0,
                                          float y0, float y1) {
  const int i1 = i0 + 1;
  if (GU) {
    const float g0 = from_gate_lane(y0), g1 = from_gate_lane(y1);
    const int r = 8 * tr + (c - 8);
    if (c >= 8 && r < a.n_out) {
      if (i0 < n) {
        const float h = glu_act(g0, y0, a.act, a.bg, a.bl);
        a.out[(int64_t)(p0 + i0) * a.n_out + r] = h;
        if (a.out_hl) store_hilo(a.out_hl + (int64_t)(p0 + i0) * 2 * a.out_ld + r, a.out_ld, h);
      }
      if (i1 < n) {
        const float h = glu_act(g1, y1, a.act, a.bg, a.bl);
        a.out[(int64_t)(p0 + i1) * a.n_out + r] = h;
        if (a.out_hl) store_hilo(a.out_hl + (int64_t)(p0 + i1) * 2 * a.out_ld + r, a.out_ld, h);
      }
    }
  } else {
    const int r = 16 * tr + c;
    if (r < a.n_out) {
      if (i0 < n) a.out[(int64_t)(p0 + i0) * a.n_out + r] = y0;
      if (i1 < n) a.out[(int64_t)(p0 + i1) * a.n_out + r] = y1;
    }
  }
}

constexpr int kSdDepth = 3;   // bf16 K-steps in flight per wavefront

// Item bid of the shared down-projection in the down launch: (group of 4 tile rows, K-range
// part), one tile row per wavefront.  The part's h_s columns of the T tokens are staged as
// hi/lo rows, and the partial sums are those the OUT launch would form over the same
// K-steps (run_tile_row from zero; its loop for any count, which keeps the launch's register
// budget that of the expert items).
__device__ __forceinline__ void sd_partial(const ExpArgs& a, int bid, uint4* sm, HiloRow* rows) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15, g = lane >> 4;
  const int grp = bid / a.sd_parts, kp = bid - grp * a.sd_parts;
  const int tr = grp * kWavesPerBlock + wv;
  const int qa = kp * a.sd_qper, n = min(a.sd_ks, qa + a.sd_qper) - qa;
  const bool live = tr < a.sd_ntr && n > 0;
  const uint8_t* trow =
      a.sd_w + ((size_t)(live ? tr : 0) * a.sd_row + a.sd_q0 + (n > 0 ? qa : 0)) * kBf16StepBytes;
  TileStream<0, kSdDepth> ts;
  const int nt = a.sd_T;
  const int n0 = min(n * kStepK, a.sd_ms - qa * kStepK);
  if (nt == 1 && n > 0 && HiloRowPre::fits(n)) {   // one token: its row first, then the stream
    HiloRowPre pre;
    pre.load(a.sd_hs + qa * kStepK, n0, n);
    ts.prefetch(trow, 0, n);   // unconditional (tile row 0 without work): see k_out
    pre.commit(sm, n0, n);
  } else {
    if (live) ts.prefetch(trow, 0, n);
    if ((int)threadIdx.x < nt)
      rows[threadIdx.x] = HiloRow{a.sd_hs + (int64_t)threadIdx.x * a.sd_ms + qa * kStepK, nullptr, 1.f};
    __syncthreads();
    if (n > 0) stage_hilo(sm, rows, nt, n0, 0, 0, nullptr, n);
  }
  __syncthreads();
  if (!live) return;
  const int nr = 2 * nt;
  const f32x4_t acc = run_tile_row<0, kSdDepth, 0>(ts, trow, 0, n, sm, c % nr, nr);
  const int r = 16 * tr + c;
  if (r >= a.sd_d) return;
  // D rows 4g .. 4g + 3 = (hi, lo) of tokens 2g and 2g + 1
  float2* o = a.sd_out + (int64_t)kp * nt * a.sd_d + r;
  if (2 * g < nt) o[(int64_t)(2 * g) * a.sd_d] = make_float2(acc[0], acc[1]);
  if (2 * g + 1 < nt) o[(int64_t)(2 * g + 1) * a.sd_d] = make_float2(acc[2], acc[3]);
}

template <int WF, bool GU>
__global__ __launch_bounds__(kBlock) void k_exp(ExpArgs a) {
  extern __shared__ uint4 sm[];
  __shared__ f32x4_t part[kWavesPerBlock][kWave];
  __shared__ HiloRow rows[8];
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15, g = lane >> 4;
  // the shared down-projection's workgroups first (their items are the longest); sd_wgs is
  // a multiple of the XCD count, so the expert items keep their XCDs
  if (!GU && (int)blockIdx.x < a.sd_wgs) {
    sd_partial(a, blockIdx.x, sm, rows);
    return;
  }
  const int bid = (int)blockIdx.x - (GU ? 0 : a.sd_wgs);
  // one (tile-row group, unit) item per workgroup, the units of a group on one XCD in
  // unit order (so that the units of one expert reuse its weights from that L2)
  const int n_units = min(a.ctrl[0], a.max_units);
  int wgi, u;
  if (a.chunk > 0) {
    if (!chunk_item(bid, n_units, a.wg_per_unit, a.chunk, wgi, u)) return;
  } else if (!xcd_item(bid, a.wg_per_unit, a.max_units, wgi, u) || u >= n_units) {
    return;
  }
  {
    const int4 un = *reinterpret_cast<const int4*>(a.units + 4 * u);
    const int e = un.x, p0 = un.y, n = un.z;
    if (e < 0 || e >= a.E || n < 1 || n > a.nu || p0 < 0 || p0 + n > a.n_assign) return;
    const int nr = 2 * n;
    const int slot = wgi * kWavesPerBlock + wv;
    const int tr = slot / a.ksplit, kp = slot - tr * a.ksplit;
    const int qper = cdiv(a.ks, a.ksplit);
    const int q0 = min(a.ks, kp * qper), q1 = min(a.ks, q0 + qper);
    const bool live = tr < a.n_tr && q1 > q0;
    const uint8_t* trow = a.experts + (size_t)e * a.expert_bytes + a.region_off +
                          (size_t)tr * a.ks * WeightStep<WF>::SB;
    TileStream<WF, WF == 1 ? 4 : 3> ts;
    // one position whose row is known without a load (down: its own row; gate/up with a
    // single token: token 0): the row first, then the stream
    if (n == 1 && (!GU || a.n_assign == a.k) && HiloRowPre::fits(a.ks)) {
      HiloRowPre pre;
      pre.load(a.xin + (GU ? 0 : (int64_t)p0 * a.kin), a.kin, a.ks);
      // unconditional: see k_out
      ts.prefetch(live ? trow : a.experts + (size_t)e * a.expert_bytes + a.region_off,
                  live ? q0 : 0, live ? q1 - q0 : 1);
      pre.commit(sm, a.kin, a.ks);
    } else {
      if (live) ts.prefetch(trow, q0, q1 - q0);
      if ((int)threadIdx.x < n) {
        const int p = p0 + threadIdx.x;
        int64_t src = p;
        if (GU) {
          const int asg = a.perm[p];
          src = (asg >= 0 && asg < a.n_assign) ? asg / a.k : 0;
        }
        rows[threadIdx.x] = HiloRow{a.xin + src * a.kin, nullptr, 1.f};
      }
      __syncthreads();
      stage_hilo(sm, rows, n, a.kin, 0, 0, nullptr, a.ks);
    }
    __syncthreads();
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    if (live) acc = run_tile_row_n<WF, WF == 1 ? 4 : 3>(ts, trow, q0, q1 - q0, sm, c % nr, nr);
    acc = reduce_ksplit(acc, part, a.ksplit, kp);
    // D rows 4g..4g+3 = (hi, lo) of positions 2g and 2g + 1 of the unit
    if (tr < a.n_tr && kp == 0) exp_store<GU>(a, p0, n, tr, c, 2 * g, acc[0] + acc[1], acc[2] + acc[3]);
  }
}

// ------------------------------------------------------------------------------------
// Step OUT: Delta[t] = [W_up_latent | W_shared_down] [RMSNorm(u_t) * gamma ; h_s,t], one
// product over the packed OUT matrix.  The workgroup computes the norm of its tokens'
// u rows and stages [u_hat ; h_s] as hi/lo pairs.  With few tokens of a latent layer the
// h_s segment's partial sums come from the expert down launch (which streams W_shared_down
// beside the experts' down weights), and this launch multiplies the u_hat segment alone.
// ------------------------------------------------------------------------------------
struct OutArgs {
  const uint8_t* w;
  int ks, ks_l, n_tr, ksplit, wg_per_blk, ntb, n_blk;
  int ks_row;           // K-steps of a tile row (ks: those this launch multiplies, from 0)
  const float* u;
  const float* hs;
  const uint16_t* gamma;
  int d, l, ms, norm;
  int n0;               // columns of the u_hat segment (0 without a latent)
  int n1;               // columns of the h_s segment staged (0: its products come from ys)
  const float2* ys;     // [nsd][T][d] (hi, lo) partial sums of W_sd h_s, added in order
  int nsd;
  float eps;
  int64_t T;
  OutSink sink;
  const float* add_u;   // without a latent: Delta = u + the product
  int prod_wgs;         // workgroups of the product; the ones after them prefetch
  Prefetch pf;
  int pf_wgs;
};

constexpr int kOutMaxTokens = 8;
constexpr size_t kPrefetchWgBytes = 64 * 1024;   // bytes read by one prefetch workgroup

// A prefetch workgroup: 16-byte cached loads of its 64 KiB slice of pf, four in flight per
// lane; the XOR of what it read is stored only under a flag the host never sets.
__device__ __forceinline__ void prefetch_slice(const Prefetch& pf, int w) {
  const uint4* p = reinterpret_cast<const uint4*>(pf.p);
  const int64_t n16 = (int64_t)(pf.bytes / 16);
  const int64_t b0 = (int64_t)w * (kPrefetchWgBytes / 16);
  const int64_t b1 = min(n16, b0 + (int64_t)(kPrefetchWgBytes / 16));
  uint32_t acc = 0;
  for (int64_t i = b0 + threadIdx.x; i < b1; i += 4 * kBlock) {
    uint4 v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = i + j * kBlock < b1 ? p[i + j * kBlock] : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int j = 0; j < 4; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
  }
  if (pf.flag) pf.sink[threadIdx.x] = acc;
}

// 1 / sqrt(mean(row^2) + eps) of an fp32 row, by the whole workgroup (fixed order).
__device__ __forceinline__ float row_inv_rms(const float* ur, int l, float eps, float* red) {
  const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x >> 6;
  float ss = 0.f;
  for (int col = threadIdx.x * 4; col < l; col += kBlock * 4) {
    const float4 p = *reinterpret_cast<const float4*>(ur + col);
    ss = fmaf(p.x, p.x, ss); ss = fmaf(p.y, p.y, ss);
    ss = fmaf(p.z, p.z, ss); ss = fmaf(p.w, p.w, ss);
  }
  ss = wave_sum(ss);
  if (lane == 0) red[wv] = ss;
  __syncthreads();
  const float tot = (red[0] + red[1]) + (red[2] + red[3]);
  __syncthreads();
  return 1.0f / sqrtf(tot / (float)l + eps);
}

// One token's u row and gamma, loaded by the OUT launch before its weight stream (the loads
// complete in issue order, so a load issued after the stream would wait for it): thread i
// holds columns 4 i + 1024 c, c < kOutRow4, the order row_inv_rms sums them in.
constexpr int kOutRow4 = 4;   // l <= 4096
struct OutRow {
  float4 u[kOutRow4];
  uint2 g[kOutRow4];
  __device__ __forceinline__ void load(const float* ur, const uint16_t* gamma, int l) {
#pragma unroll
    for (int c = 0; c < kOutRow4; ++c) {
      const int col = 4 * ((int)threadIdx.x + kBlock * c);
      if (col < l) {
        u[c] = *reinterpret_cast<const float4*>(ur + col);
        if (gamma) g[c] = *reinterpret_cast<const uint2*>(gamma + col);
      }
    }
  }
  // row_inv_rms of the row (the same sums in the same order)
  __device__ __forceinline__ float inv_rms(int l, float eps, float* red) const {
    const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x >> 6;
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < kOutRow4; ++c) {
      if (4 * ((int)threadIdx.x + kBlock * c) < l) {
        ss = fmaf(u[c].x, u[c].x, ss); ss = fmaf(u[c].y, u[c].y, ss);
        ss = fmaf(u[c].z, u[c].z, ss); ss = fmaf(u[c].w, u[c].w, ss);
      }
    }
    ss = wave_sum(ss);
    if (lane == 0) red[wv] = ss;
    __syncthreads();
    const float tot = (red[0] + red[1]) + (red[2] + red[3]);
    __syncthreads();
    return 1.0f / sqrtf(tot / (float)l + eps);
  }
  // The hi/lo rows 0 and 1 (nr = 2) of stage_hilo with segment 0 = the row (times scale and
  // gamma when gamma is set), ks K-steps, no segment 1: the same words.
  __device__ __forceinline__ void stage(uint4* sm, int l, float scale, bool gamma, int ks) const {
    uint2* s2 = reinterpret_cast<uint2*>(sm);
#pragma unroll
    for (int c = 0; c < kOutRow4; ++c) {
      const int col = 4 * ((int)threadIdx.x + kBlock * c);
      if (col >= ks * kStepK) continue;
      float v[4] = {0.f, 0.f, 0.f, 0.f};
      if (col < l) {
        v[0] = u[c].x; v[1] = u[c].y; v[2] = u[c].z; v[3] = u[c].w;
        if (gamma) {
          v[0] = v[0] * scale * bf16_lo(g[c].x); v[1] = v[1] * scale * bf16_hi(g[c].x);
          v[2] = v[2] * scale * bf16_lo(g[c].y); v[3] = v[3] * scale * bf16_hi(g[c].y);
        }
      }
      uint32_t h[2], lo[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        h[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
        lo[i] = pack_bf16x2(v[2 * i] - bf16_lo(h[i]), v[2 * i + 1] - bf16_hi(h[i]));
      }
      // piece j = col / 8 holds words 2 j (hi) and 2 j + 1 (lo); this half is (col / 4) % 2
      const int w = 2 * (col >> 3), half = (col >> 2) & 1;
      s2[2 * w + half] = make_uint2(h[0], h[1]);
      s2[2 * (w + 1) + half] = make_uint2(lo[0], lo[1]);
    }
  }
};

// u_hat = u * inv * gamma, one workgroup per token: the same values the OUT launch of a
// few tokens stages itself (the same reduction and the same products).
__global__ __launch_bounds__(kBlock) void k_norm(const float* __restrict__ u,
                                                 const uint16_t* __restrict__ gamma, int l,
                                                 int norm, float eps, float* __restrict__ uhat,
                                                 uint16_t* __restrict__ uhat_hl) {
  __shared__ float red[kWavesPerBlock];
  const int64_t t = blockIdx.x;
  const float* ur = u + t * l;
  const float inv = norm ? row_inv_rms(ur, l, eps, red) : 1.f;
  for (int col = threadIdx.x; col < l; col += kBlock) {
    const float gm = norm ? __uint_as_float((uint32_t)gamma[col] << 16) : 1.f;
    const float v = norm ? ur[col] * inv * gm : ur[col];
    uhat[t * l + col] = v;
    store_hilo(uhat_hl + t * 2 * l + col, l, v);
  }
}

constexpr int kOutDeepRing = 7;

// P: bf16 K-steps in the ring; 7 when every wavefront's range fits it (the whole range is
// then in flight while the workgroup stages its activations), else 3.
template <int P>
__global__ __launch_bounds__(kBlock) void k_out(OutArgs a) {
  extern __shared__ uint4 sm[];
  __shared__ f32x4_t part[kWavesPerBlock][kWave];
  __shared__ HiloRow rows[kOutMaxTokens];
  __shared__ float red[kWavesPerBlock];
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15, g = lane >> 4;
  if ((int)blockIdx.x >= a.prod_wgs) {   // after the product's workgroups: the prefetch
    prefetch_slice(a.pf, blockIdx.x - a.prod_wgs);
    return;
  }
  int wgi, blk;
  if (!xcd_item(blockIdx.x, a.wg_per_blk, a.n_blk, wgi, blk)) return;
  const int64_t t0 = (int64_t)blk * a.ntb;
  const int nt = (int)min((int64_t)a.ntb, a.T - t0);
  const int slot = wgi * kWavesPerBlock + wv;
  const int tr = slot / a.ksplit, kp = slot - tr * a.ksplit;
  const int qper = cdiv(a.ks, a.ksplit);
  const int q0 = min(a.ks, kp * qper), q1 = min(a.ks, q0 + qper);
  const bool live = tr < a.n_tr && q1 > q0;
  const uint8_t* trow = a.w + (size_t)tr * a.ks_row * kBf16StepBytes;
  TileStream<0, P> ts;
  // one token, the u_hat segment alone: its row first, then the weight stream
  const bool one = nt == 1 && a.n1 == 0 && a.n0 == a.l && a.l % 4 == 0 &&
                   a.l <= 4 * kBlock * kOutRow4;
  // with one token, the W_sd partial sums this lane adds (token 0: lanes g = 0 of the
  // wavefront with kp = 0) are loaded with the row too
  float2 ysv[kSdParts];
  const bool ys_lane = one && a.nsd > 0 && a.nsd <= kSdParts && kp == 0 && tr < a.n_tr &&
                       16 * tr + c < a.d && g == 0;
  if (one) {
    OutRow row;
    row.load(a.u + t0 * a.l, a.norm ? a.gamma : nullptr, a.l);
    if (ys_lane) {
#pragma unroll
      for (int p = 0; p < kSdParts; ++p)
        if (p < a.nsd) ysv[p] = a.ys[((int64_t)p * a.T + t0) * a.d + 16 * tr + c];
    }
    // unconditional (a wavefront without work re-reads K-step 0 of tile row 0), so that the
    // wait for the row counts the stream's loads as still in flight
    ts.prefetch(live ? trow : a.w, live ? q0 : 0, live ? q1 - q0 : 1);
    const float inv = a.norm ? row.inv_rms(a.l, a.eps, red) : 1.f;
    row.stage(sm, a.l, inv, a.norm != 0, a.ks);
  } else {
    if (live) ts.prefetch(trow, q0, q1 - q0);
    for (int i = 0; i < nt; ++i) {
      const float* ur = a.u + (t0 + i) * a.l;
      const float inv = a.norm ? row_inv_rms(ur, a.l, a.eps, red) : 1.f;
      if (threadIdx.x == 0) rows[i] = HiloRow{ur, a.hs + (t0 + i) * a.ms, inv};
    }
    __syncthreads();
    stage_hilo(sm, rows, nt, a.n0, a.ks_l * kStepK, a.n1, a.norm ? a.gamma : nullptr, a.ks);
  }
  __syncthreads();
  const int nr = 2 * nt;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  if (live) acc = run_tile_row_upto<0, P>(ts, trow, q0, q1 - q0, sm, c % nr, nr);
  acc = reduce_ksplit(acc, part, a.ksplit, kp);
  if (tr < a.n_tr && kp == 0) {
    const int r = 16 * tr + c;
    if (r < a.d) {
      // the shared down-projection's parts after the K-split's, in part order
      if (ys_lane) {
#pragma unroll
        for (int p = 0; p < kSdParts; ++p)
          if (p < a.nsd) {
            acc[0] += ysv[p].x;
            acc[1] += ysv[p].y;
          }
      }
      for (int p = 0; p < (one ? 0 : a.nsd); ++p) {
        const float2* yp = a.ys + ((int64_t)p * a.T + t0 + 2 * g) * a.d + r;
        if (2 * g < nt) {
          const float2 v = yp[0];
          acc[0] += v.x;
          acc[1] += v.y;
        }
        if (2 * g + 1 < nt) {
          const float2 v = yp[a.d];
          acc[2] += v.x;
          acc[3] += v.y;
        }
      }
    }
    const float y0 = acc[0] + acc[1], y1 = acc[2] + acc[3];
    if (r < a.d) {
      const int64_t i0 = (t0 + 2 * g) * a.d + r, i1 = i0 + a.d;
      if (2 * g < nt) store_out(a.sink, i0, a.add_u ? a.add_u[i0] + y0 : y0);
      if (2 * g + 1 < nt) store_out(a.sink, i1, a.add_u ? a.add_u[i1] + y1 : y1);
    }
  }
}

// ------------------------------------------------------------------------------------
// Larger batches: token-tiled products.  A workgroup takes a tile of up to 16*NB
// activation rows (bf16 tokens, or hi/lo pairs of fp32 rows) and 4 tile rows of weights
// (one per wavefront) and walks K one K-step at a time: the K-step of the tile's rows is
// staged in LDS (double buffer, its loads issued a step ahead) and each wavefront
// multiplies it with its weight K-step, NB MFMA blocks per weight operand, so a weight
// byte is read once per tile instead of once per token block.  The partial sums follow
// the K-split of the launches for a few tokens (a running sum over the same K ranges,
// added in the same order), so a token's result has the same bits in both paths.
// ------------------------------------------------------------------------------------
constexpr int kTTMaxSrc = 64;     // activation rows per tile

// The tile's activation rows, bf16 (tokens as they are, fp32 values as hi/lo row pairs
// written by their producer).  Row r: columns [0, n0) at b0 + 8 o0[r] + col, columns
// [c1, c1 + n1) at b1 + 8 o1[r] + (col - c1) (offsets in 16-byte words), zero elsewhere
// and for rows r >= R.
struct TTRows {
  uint32_t o0[kTTMaxSrc];
  uint32_t o1[kTTMaxSrc];
};
struct TTSrc {
  const uint16_t* b0;
  const uint16_t* b1;
  int R, n0, c1, n1;
};

// A ring of P K-steps of the tile's 16 NB rows in registers, each loaded P K-steps ahead
// of its use and written to the LDS buffer of its K-step one step ahead.  Thread piece i
// is idx = threadIdx + 256 i: row idx / 16, columns 8 (idx % 16) .. + 8 of the K-step,
// so that a wavefront reads 4 rows of 256 contiguous bytes.  The rows' offsets are read
// once; every load is issued (a piece outside the rows reads the first word of b0 and
// is zeroed when it is committed): no branches, so the waits count the loads in
// flight exactly.
template <int P, int NB>
struct TTStage {
  uint4 v[P][NB];
  uint32_t o0[NB], o1[NB];
  bool rv[NB];
  __device__ __forceinline__ void init(const TTRows& rows, const TTSrc& src) {
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int r = (threadIdx.x + i * kBlock) >> 4;
      rv[i] = r < src.R;
      o0[i] = rv[i] ? rows.o0[r] : 0u;
      o1[i] = rv[i] && src.n1 > 0 ? rows.o1[r] : 0u;
    }
  }
  __device__ __forceinline__ bool in0(int i, const TTSrc& src, int col) const {
    return rv[i] && col < src.n0;
  }
  __device__ __forceinline__ bool in1(int i, const TTSrc& src, int col) const {
    return rv[i] && col >= src.c1 && col < src.c1 + src.n1;
  }
  __device__ __forceinline__ int col_of(int i, int q) const {
    return q * kStepK + 8 * ((threadIdx.x + i * kBlock) & 15);
  }
  __device__ __forceinline__ void load(int slot, const TTSrc& src, int q) {
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int col = col_of(i, q);
      const bool a0 = in0(i, src, col), a1 = in1(i, src, col);
      const uint32_t w = a0 ? o0[i] + (col >> 3) : a1 ? o1[i] + ((col - src.c1) >> 3) : 0u;
      const uint4* base = reinterpret_cast<const uint4*>(a1 ? src.b1 : src.b0);
#pragma unroll
      for (int sl = 0; sl < P; ++sl)
        if (sl == slot) v[sl][i] = base[w];
    }
  }
  // Slot `slot` holds K-step q: the pieces outside the rows are zeroed here, where the
  // data is needed anyway (a select at the load would wait for it there).  The LDS
  // buffer holds piece j of row r at word j * 16 NB + (r ^ j): the XOR keeps both these
  // writes and the MFMA operand reads free of bank conflicts.
  __device__ __forceinline__ void commit(int slot, uint4* buf, const TTSrc& src, int q) const {
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int idx = threadIdx.x + i * kBlock;
      const int r = idx >> 4, j = idx & 15;
      const int col = col_of(i, q);
      const bool z = !(in0(i, src, col) || in1(i, src, col));
#pragma unroll
      for (int sl = 0; sl < P; ++sl)
        if (sl == slot) {
          const uint4 x = v[sl][i];
          buf[j * 16 * NB + (r ^ j)] =
              make_uint4(z ? 0u : x.x, z ? 0u : x.y, z ? 0u : x.z, z ? 0u : x.w);
        }
    }
  }
};

// The K loop of a tile: D[t][b] (16 x 16 block b of the tile's rows x this wavefront's tile
// row t, trow[t]) over all ks K-steps.  With PARTS, sums restart every qper K-steps and the
// partial sums are added in order (the K-split of the launches for few tokens); without, one
// running sum over all of K (qper is then ks).  Every wavefront of the workgroup runs it
// (staging and barriers are shared); each trow[t] must be a valid tile row (waves without one
// pass tile row 0 and drop the result).  Each A operand read from LDS feeds the TR tile rows.
// Weights are loaded P K-steps ahead, activations PA (P a multiple of PA).  The loop runs
// whole rounds of P steps: steps past ks re-read the last K-step and are never summed.
template <int WF, int P, int NB, int PA, bool PARTS, int TR>
__device__ __forceinline__ void tt_run_tr(const TTRows& rows, const TTSrc& src,
                                          const uint8_t* const (&trow)[TR], int ks, int qper,
                                          uint4* lds, f32x4_t (&tot)[TR][NB], int kb = -1,
                                          int qper2 = 0) {
  static_assert(P % PA == 0, "the weight ring is a multiple of the activation ring");
  const int lane = threadIdx.x & (kWave - 1);
  const int c = lane & 15, g = lane >> 4;
  constexpr int RB = 16 * NB;
  constexpr int rstride = RB * 16;           // words per buffer (16 pieces x RB rows)
  TileStream<WF, P> ts[TR];
  TTStage<PA, NB> st;
  st.init(rows, src);
#pragma unroll
  for (int i = 0; i < P; ++i) {
#pragma unroll
    for (int t = 0; t < TR; ++t) ts[t].w[i].load(trow[t], min(i, ks - 1), lane);
    if (i < PA) st.load(i, src, min(i, ks - 1));
  }
  asm volatile("" ::: "memory");
  st.commit(0, lds, src, 0);
  __syncthreads();
  f32x4_t cur[TR][NB];
#pragma unroll
  for (int t = 0; t < TR; ++t)
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      cur[t][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      tot[t][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
  bool first = true;
  int in_part = 0;
  const int rounds = cdiv(ks, P);
  for (int j = 0; j < rounds * P; j += P) {
#pragma unroll
    for (int i = 0; i < P; ++i) {
      const int q = j + i;
      // activation slot i % PA held K-step q, committed to LDS at the end of the previous step
      st.load(i % PA, src, min(q + PA, ks - 1));
      const uint4* buf = lds + (q & 1) * rstride;
      constexpr bool kFp8 = WeightStep<WF>::kFp8;
      float scl[TR];
      f32x4_t part[TR][NB];
#pragma unroll
      for (int t = 0; t < TR; ++t) {
        scl[t] = WF ? ts[t].w[i].scale(g) : 0.f;
#pragma unroll
        for (int b = 0; b < NB; ++b) part[t][b] = kFp8 ? f32x4_t{0.f, 0.f, 0.f, 0.f} : cur[t][b];
      }
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        const int jj = WeightStep<WF>::a_piece(s4, g);
#pragma unroll
        for (int t = 0; t < TR; ++t) {
          const uint4 bw = ts[t].w[i].operand(s4, scl[t]);
#pragma unroll
          for (int b = 0; b < NB; ++b)
            part[t][b] = mfma_bf16(buf[jj * RB + 16 * b + (c ^ jj)], bw, part[t][b]);
        }
      }
#pragma unroll
      for (int t = 0; t < TR; ++t)
#pragma unroll
        for (int b = 0; b < NB; ++b)   // FP8: the K-step's partial sums times its block scale
          cur[t][b] = kFp8 ? WeightStep<WF>::scale_add(part[t][b], scl[t], cur[t][b]) : part[t][b];
      // the K-step's products are issued before its slot is reloaded, so that the slot's old
      // and new values never overlap and keep one register set across the loop's back edge
      // (where the compiler would otherwise copy the ring, waiting for every load in flight)
#pragma unroll
      for (int t = 0; t < TR; ++t)
#pragma unroll
        for (int b = 0; b < NB; ++b) asm volatile("" : "+v"(cur[t][b]) :: "memory");
#pragma unroll
      for (int t = 0; t < TR; ++t) ts[t].w[i].load(trow[t], min(q + P, ks - 1), lane);
      // parts of qper K-steps, or with kb >= 0 of qper up to K-step kb and qper2 after it
      if (PARTS && q < ks &&
          (++in_part == (kb < 0 || q < kb ? qper : qper2) || q + 1 == kb || q + 1 == ks)) {
#pragma unroll
        for (int t = 0; t < TR; ++t)
#pragma unroll
          for (int b = 0; b < NB; ++b) {
            tot[t][b] = first ? cur[t][b] : tot[t][b] + cur[t][b];
            cur[t][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
          }
        first = false;
        in_part = 0;
      }
      if (!PARTS && q + 1 == ks) {
#pragma unroll
        for (int t = 0; t < TR; ++t)
#pragma unroll
          for (int b = 0; b < NB; ++b) tot[t][b] = cur[t][b];
      }
      asm volatile("" ::: "memory");
      st.commit((i + 1) % PA, lds + ((q + 1) & 1) * rstride, src, min(q + 1, ks - 1));
      __syncthreads();
    }
  }
}

// One tile row per wavefront.
template <int WF, int P, int NB, int PA = P, bool PARTS = true>
__device__ __forceinline__ void tt_run(const TTRows& rows, const TTSrc& src, const uint8_t* trow,
                                       int ks, int qper, uint4* lds, f32x4_t (&tot)[NB],
                                       int kb = -1, int qper2 = 0) {
  const uint8_t* const tr1[1] = {trow};
  f32x4_t t1[1][NB];
  tt_run_tr<WF, P, NB, PA, PARTS, 1>(rows, src, tr1, ks, qper, lds, t1, kb, qper2);
#pragma unroll
  for (int b = 0; b < NB; ++b) tot[b] = t1[0][b];
}

// Dense IN matrix rows (W_down_latent and the shared gate/up) for a tile of up to 64
// tokens: tile rows [tr_first, tr_first + tr_count), 4 per workgroup.
struct InTTArgs {
  const uint8_t* w;
  int ks, qper, tr_r, tr_dn, tr_first, tr_count, n_grp, n_tiles;
  const uint16_t* x;
  int64_t T;
  int d;
  float* xc;
  uint16_t* xc_hl;   // [T][2][lp] hi/lo of x^c for the expert launch
  int l, lp;
  float* hs;
  uint16_t* hs_hl;   // [T][2][ms] hi/lo of h_s for the OUT launch
  int ms;
  int act;
  float bg, bl;
};

constexpr int kInTTBlocks = 4;    // 64 bf16 token rows
// Tile-row groups of the IN and OUT launches that take a token tile back to back on one XCD
// (xcd_gblock_item): 2 for OUT was 11% faster at 1024 tokens than 1 (3, 4 slower; the same at
// 64 tokens, one tile); IN measured best at 1.
constexpr int kInTTGroups = 1;
constexpr int kOutTTGroups = 2;

__global__ __launch_bounds__(kBlock) void k_in_tt(InTTArgs a) {
  extern __shared__ uint4 sm[];
  __shared__ TTRows rows;
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15, g = lane >> 4;
  int grp, tile;
  if (!xcd_gblock_item(blockIdx.x, a.n_grp, a.n_tiles, kInTTGroups, grp, tile)) return;
  const int64_t t0 = (int64_t)tile * kTTMaxSrc;
  const int nt = (int)min((int64_t)kTTMaxSrc, a.T - t0);
  if ((int)threadIdx.x < nt) rows.o0[threadIdx.x] = (uint32_t)((t0 + threadIdx.x) * a.d / 8);
  __syncthreads();
  const int tri = grp * kWavesPerBlock + wv;
  const bool live = tri < a.tr_count;
  const int tr = a.tr_first + (live ? tri : 0);
  f32x4_t tot[kInTTBlocks];
  // 4 weight K-steps and 2 activation K-steps in flight (measured against 2/2, 6/2, 8/4, 4/4)
  tt_run<0, 4, kInTTBlocks, 2>(rows, TTSrc{a.x, nullptr, nt, a.d, 0, 0},
                               a.w + (size_t)tr * a.ks * kBf16StepBytes, a.ks, a.qper, sm, tot);
  if (!live) return;
#pragma unroll
  for (int b = 0; b < kInTTBlocks; ++b) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int ti = 16 * b + 4 * g + v;
      if (tr < a.tr_r + a.tr_dn) {
        const int r = 16 * (tr - a.tr_r) + c;
        if (ti < nt && r < a.l) {
          a.xc[(t0 + ti) * a.l + r] = tot[b][v];
          store_hilo(a.xc_hl + (t0 + ti) * 2 * a.lp + r, a.lp, tot[b][v]);
        }
      } else {
        const int r = 8 * (tr - a.tr_r - a.tr_dn) + (c - 8);
        const float gate = from_gate_lane(tot[b][v]);
        if (c >= 8 && ti < nt && r < a.ms) {
          const float h = glu_act(gate, tot[b][v], a.act, a.bg, a.bl);
          a.hs[(t0 + ti) * a.ms + r] = h;
          store_hilo(a.hs_hl + (t0 + ti) * 2 * a.ms + r, a.ms, h);
        }
      }
    }
  }
}

// Router logits for a tile of up to 64 tokens: one workgroup per (4 TR router tile rows,
// logit sub-plane, token tile).  Plane p covers the K-steps [p qpp, (p+1) qpp) of the
// few-token router launch, its sub-plane q the run of qw K-steps that wavefront q of that
// launch's workgroup takes; the route adds sub-planes and planes in the same order for both
// launches, so a token's logits have the same bits in both.
struct RouterTTArgs {
  const uint8_t* w;
  int ks, qpp, tr_r, n_grp, zplanes, n_tiles;
  const uint16_t* x;
  int64_t T;
  int d, E;
  float* z;          // [zplanes][T][E]
};

// Tile rows per wavefront of the token-tiled router (TR): with 2 each A operand feeds both
// and a token tile is read by half as many workgroups (27% faster at 8192 tokens); below
// kRouterTTWideTokens tokens, 1 keeps twice the workgroups (faster at 64 tokens).
constexpr int kRouterTTWideTokens = 512;

template <int TR>
__global__ __launch_bounds__(kBlock) void k_router_tt(RouterTTArgs a) {
  extern __shared__ uint4 sm[];
  __shared__ TTRows rows;
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15, g = lane >> 4;
  int gp, tile;
  if (!xcd_item(blockIdx.x, a.n_grp * a.zplanes * kZSub, a.n_tiles, gp, tile)) return;
  const int np = a.zplanes * kZSub;
  const int grp = gp / np, sp = gp - grp * np;    // (tile-row group, sub-plane)
  // sub-plane sp = part sp % kZSub of plane sp / kZSub: the K-steps a wavefront of the
  // few-token router workgroup takes
  const int plane = sp / kZSub, part = sp - plane * kZSub;
  const int pr0 = min(a.ks, plane * a.qpp), pr1 = min(a.ks, pr0 + a.qpp);
  const int qw = cdiv(pr1 - pr0, kZSub);
  const int r0 = min(pr1, pr0 + part * qw), r1 = min(pr1, r0 + qw);
  const int64_t t0 = (int64_t)tile * kTTMaxSrc;
  const int nt = (int)min((int64_t)kTTMaxSrc, a.T - t0);
  float* zp = a.z + (int64_t)sp * a.T * a.E;
  if (r1 <= r0) {   // an empty part holds zeros, as in the few-token launch (uniform branch)
    constexpr int kGroupRows = 16 * kWavesPerBlock * TR;   // experts of a group
    for (int i = threadIdx.x; i < nt * kGroupRows; i += kBlock) {
      const int e = kGroupRows * grp + i % kGroupRows;
      if (e < a.E) zp[(t0 + i / kGroupRows) * a.E + e] = 0.f;
    }
    return;
  }
  // rows start at the plane's first column
  if ((int)threadIdx.x < nt) rows.o0[threadIdx.x] = (uint32_t)((t0 + threadIdx.x) * a.d / 8 + r0 * (kStepK / 8));
  __syncthreads();
  int tri[TR];
  const uint8_t* trow[TR];
#pragma unroll
  for (int t = 0; t < TR; ++t) {
    tri[t] = (grp * kWavesPerBlock + wv) * TR + t;
    trow[t] = a.w + ((size_t)(tri[t] < a.tr_r ? tri[t] : 0) * a.ks + r0) * kBf16StepBytes;
  }
  f32x4_t tot[TR][kInTTBlocks];
  tt_run_tr<0, 2, kInTTBlocks, 2, false, TR>(rows, TTSrc{a.x, nullptr, nt, a.d - r0 * kStepK, 0, 0},
                                             trow, r1 - r0, r1 - r0, sm, tot);
#pragma unroll
  for (int t = 0; t < TR; ++t) {
    const int e = 16 * tri[t] + c;
    if (tri[t] >= a.tr_r || e >= a.E) continue;
#pragma unroll
    for (int b = 0; b < kInTTBlocks; ++b)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int ti = 16 * b + 4 * g + v;
        if (ti < nt) zp[(t0 + ti) * a.E + e] = tot[t][b][v];
      }
  }
}

// OUT matrix for a tile of up to 32 tokens: [u_hat ; h_s] as hi/lo rows.
struct OutTTArgs {
  const uint8_t* w;
  int ks, ks_l, qper, n_tr, n_grp, n_tiles;
  int kb, qper2;           // parts of qper K-steps up to K-step kb, of qper2 after it
  const uint16_t* uh_hl;   // [T][2][l]
  const uint16_t* hs_hl;   // [T][2][ms]
  int d, l, ms, n0;        // n0: columns of the u_hat segment (0 without a latent)
  int64_t T;
  OutSink sink;
  const float* add_u;      // without a latent: Delta = u + the product
};

constexpr int kHiloTTBlocks = 4;  // 32 fp32 rows as 64 hi/lo rows
constexpr int kHiloTTRows = 32;

__global__ __launch_bounds__(kBlock) void k_out_tt(OutTTArgs a) {
  extern __shared__ uint4 sm[];
  __shared__ TTRows rows;
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15, g = lane >> 4;
  int grp, tile;
  if (!xcd_gblock_item(blockIdx.x, a.n_grp, a.n_tiles, kOutTTGroups, grp, tile)) return;
  const int64_t t0 = (int64_t)tile * kHiloTTRows;
  const int nt = (int)min((int64_t)kHiloTTRows, a.T - t0);
  if ((int)threadIdx.x < 2 * nt) {
    const int64_t row = 2 * t0 + threadIdx.x;    // hi/lo row of token t0 + threadIdx / 2
    rows.o0[threadIdx.x] = (uint32_t)(row * a.l / 8);
    rows.o1[threadIdx.x] = (uint32_t)(row * a.ms / 8);
  }
  __syncthreads();
  const int tr = grp * kWavesPerBlock + wv;
  const bool live = tr < a.n_tr;
  f32x4_t tot[kHiloTTBlocks];
  // 2 weight and 2 activation K-steps in flight: 7-8% faster than 4/4 (124 registers, 3 waves
  // per SIMD)
  tt_run<0, 2, kHiloTTBlocks, 2>(
      rows, TTSrc{a.uh_hl, a.hs_hl, 2 * nt, a.n0, a.ks_l * kStepK, a.ms},
      a.w + (size_t)(live ? tr : 0) * a.ks * kBf16StepBytes, a.ks, a.qper, sm, tot, a.kb,
      a.qper2);
  if (!live) return;
  const int r = 16 * tr + c;
  if (r >= a.d) return;
#pragma unroll
  for (int b = 0; b < kHiloTTBlocks; ++b) {
    const int i0 = 8 * b + 2 * g;
    const int64_t o0 = (t0 + i0) * a.d + r, o1 = o0 + a.d;
    const float y0 = tot[b][0] + tot[b][1], y1 = tot[b][2] + tot[b][3];
    if (i0 < nt) store_out(a.sink, o0, a.add_u ? a.add_u[o0] + y0 : y0);
    if (i0 + 1 < nt) store_out(a.sink, o1, a.add_u ? a.add_u[o1] + y1 : y1);
  }
}

// Work order of the token-tiled expert launches: 0 = xcd_item (every XCD walks one
// tile-row group through all units: measured faster on the decode batches than the
// chunks of chunk_item, which keep a chunk's activation rows in L2 but concentrate the
// XCD's weight reads on a few experts), > 0 = chunk_item with that many units per chunk.
constexpr int kExpChunk = 0;
// Work order of the long units (k_exp_tt), as kExpChunk or -1 = xcd_block_item: every XCD
// owns a block of tile-row groups and takes each unit through it, so that a unit's rows are
// fetched once per XCD instead of once per group (the group-major order fetched them again
// for every group; the expert down products took 8-12% less time in this order).
constexpr int kExpTTOrder = -1;

// Tile rows per wavefront of the long-unit launches: every A operand read from LDS feeds
// that many weight tiles, and one activation stage (and barrier) serves 4 x that many tile
// rows of the workgroup.  Two (MXFP4, FP8) take about 200 registers, 2 waves per SIMD:
// measured 5-9% faster than one at 3-4 waves on the FP8 long units, 1-2% on the MXFP4 ones.
template <int WF>
struct ExpTTRows {
  static constexpr int value = WF == 0 ? 1 : 2;
};

// The K-step loop for a unit of n positions (2n hi/lo rows in NB blocks), over the TR tile
// rows trow[t] of this wavefront.
template <int WF, bool GU, int NB, int TR>
__device__ __forceinline__ void exp_tt_unit(const ExpArgs& a, const TTRows& rows, uint4* sm,
                                            const uint8_t* const (&trow)[TR], const int (&tr)[TR],
                                            int p0, int n, int c, int g) {
  f32x4_t tot[TR][NB];
  // weights about 4 KiB per tile row ahead (4 MXFP4 K-steps, 2 FP8 or bf16 ones)
  tt_run_tr<WF, WF == 1 ? 4 : 2, NB, 2, false, TR>(
      rows, TTSrc{a.xin_hl, nullptr, 2 * n, a.kin, 0, 0}, trow, a.ks, a.ks, sm, tot);
#pragma unroll
  for (int t = 0; t < TR; ++t) {
    if (tr[t] >= a.n_tr) continue;
#pragma unroll
    for (int b = 0; b < NB; ++b)
      exp_store<GU>(a, p0, n, tr[t], c, 8 * b + 2 * g, tot[t][b][0] + tot[t][b][1],
                    tot[t][b][2] + tot[t][b][3]);
  }
}

// The same over one bf16 row per position (an input that is bf16 already, whose lo rows
// are zero): D row 16 b + 4 g + v is position 16 b + 4 g + v, with the same sum as hi + lo
// (hi + 0).
template <int WF, bool GU, int NB, int TR>
__device__ __forceinline__ void exp_tt_unit_single(const ExpArgs& a, const TTRows& rows,
                                                   uint4* sm, const uint8_t* const (&trow)[TR],
                                                   const int (&tr)[TR], int p0, int n, int c,
                                                   int g) {
  f32x4_t tot[TR][NB];
  tt_run_tr<WF, WF == 1 ? 4 : 2, NB, 2, false, TR>(
      rows, TTSrc{a.xin_hl, nullptr, n, a.kin, 0, 0}, trow, a.ks, a.ks, sm, tot);
#pragma unroll
  for (int t = 0; t < TR; ++t) {
    if (tr[t] >= a.n_tr) continue;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      exp_store<GU>(a, p0, n, tr[t], c, 16 * b + 4 * g, tot[t][b][0], tot[t][b][1]);
      exp_store<GU>(a, p0, n, tr[t], c, 16 * b + 4 * g + 2, tot[t][b][2], tot[t][b][3]);
    }
  }
}

// Work items per unit of the long-unit launch: 2 when its hi/lo input rows of a unit of up to
// 2 kHiloTTRows positions exceed one tile, else 1.
__host__ __device__ inline int exp_tt_halves(bool single, int nu) {
  return !single && nu > kHiloTTRows ? 2 : 1;
}

// Routed experts for the second list of the unit table: units [ctrl[1], ctrl[0]) (the first
// list, of short units, goes to k_exp).  A unit holds up to 32 positions, or up to 64 when
// the input is single bf16 rows (the token, without a latent); hi/lo inputs of such a unit go
// in parts of 32 positions, one work item each.  The hi/lo rows are written by their producer
// (x^c by the IN launch, h by the gate/up launches).  Wavefront wv of tile-row group wgi takes
// tile rows (4 wgi + wv) TR + t.  PART: 0 = every item, 1 = only the items whose rows fit one
// 16-row block (its registers those of that tile alone: 4 waves per SIMD instead of 2), 2 = the
// others.
template <int WF, bool GU, int PART>
__global__ __launch_bounds__(kBlock, PART == 1 ? 4 : ExpTTRows<WF>::value == 2 ? 2 : WF == 1 ? 4 : 3)
void k_exp_tt(ExpArgs a) {
  constexpr int TR = ExpTTRows<WF>::value;
  extern __shared__ uint4 sm[];
  __shared__ TTRows rows;
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15, g = lane >> 4;
  const bool single = GU && a.single;
  // hi/lo input rows with units longer than one tile: each unit in halves of kHiloTTRows
  const int halves = exp_tt_halves(single, a.nu);
  const int first = a.ctrl[1];
  const int n_items = min(a.ctrl[0] - first, a.max_units) * halves;
  int wgi, item;
  if (a.chunk < 0) {
    if (!xcd_block_item(blockIdx.x, a.wg_per_unit, n_items, wgi, item)) return;
  } else if (a.chunk > 0) {
    if (!chunk_item(blockIdx.x, n_items, a.wg_per_unit, a.chunk, wgi, item)) return;
  } else if (!xcd_item(blockIdx.x, a.wg_per_unit, a.max_units * halves, wgi, item) ||
             item >= n_items) {
    return;
  }
  const int u = item / halves, half = item - u * halves;
  const int4 un = *reinterpret_cast<const int4*>(a.units + 4 * (first + u));
  const int e = un.x;
  if (e < 0 || e >= a.E || un.z < 1 || un.z > a.nu || un.y < 0 || un.y + un.z > a.n_assign) return;
  const int p0 = un.y + half * kHiloTTRows;
  const int n = halves > 1 ? min(kHiloTTRows, un.z - half * kHiloTTRows) : un.z;
  if (n < 1 || n > (single ? kTTMaxSrc : kHiloTTRows)) return;
  const bool one_block = n <= (single ? 16 : 8);
  if (PART == 1 ? !one_block : PART == 2 && one_block) return;   // (uniform)
  int tr[TR];
  const uint8_t* trow[TR];
#pragma unroll
  for (int t = 0; t < TR; ++t) {
    tr[t] = (wgi * kWavesPerBlock + wv) * TR + t;
    trow[t] = a.experts + (size_t)e * a.expert_bytes + a.region_off +
              (size_t)(tr[t] < a.n_tr ? tr[t] : 0) * a.ks * WeightStep<WF>::SB;
  }
  if ((int)threadIdx.x < (single ? n : 2 * n)) {
    const int i = single ? threadIdx.x : threadIdx.x >> 1, hl = single ? 0 : threadIdx.x & 1;
    int64_t src = p0 + i;
    if (GU) {
      const int asg = a.perm[p0 + i];
      src = (asg >= 0 && asg < a.n_assign) ? asg / a.k : 0;
    }
    rows.o0[threadIdx.x] = (uint32_t)((src * 2 + hl) * a.kin_ld / 8);
  }
  __syncthreads();
  if constexpr (PART == 1) {
    if (single) exp_tt_unit_single<WF, GU, 1, TR>(a, rows, sm, trow, tr, p0, n, c, g);
    else exp_tt_unit<WF, GU, 1, TR>(a, rows, sm, trow, tr, p0, n, c, g);
  } else {
    if (single) {
      if (PART == 0 && n <= 16) exp_tt_unit_single<WF, GU, 1, TR>(a, rows, sm, trow, tr, p0, n, c, g);
      else if (n <= 32) exp_tt_unit_single<WF, GU, 2, TR>(a, rows, sm, trow, tr, p0, n, c, g);
      else exp_tt_unit_single<WF, GU, 4, TR>(a, rows, sm, trow, tr, p0, n, c, g);
      return;
    }
    if (PART == 0 && n <= 8) exp_tt_unit<WF, GU, 1, TR>(a, rows, sm, trow, tr, p0, n, c, g);
    else if (n <= 16) exp_tt_unit<WF, GU, 2, TR>(a, rows, sm, trow, tr, p0, n, c, g);
    else exp_tt_unit<WF, GU, 4, TR>(a, rows, sm, trow, tr, p0, n, c, g);
  }
}

// ------------------------------------------------------------------------------------
// Packing (once per layer).  bf16: one thread per (expert, tile row, K-step, sub-tile,
// lane) copies the lane's 8 columns of its row (zero for rows / columns past the
// matrix).  Row maps: plain (tile row t, lane row c -> 16t + c) or gated (c < 8: gate
// row 8t + c, c >= 8: up row H + 8t + c - 8 of a [gate ; up] matrix with H gate rows).
// MXFP4: the same tiles with 4-byte code words and the 16 rows' scale words.
// ------------------------------------------------------------------------------------
struct PackArgs {
  const uint8_t* src;     // canonical rows (bf16 elements or fp4 code bytes)
  const uint8_t* scales;  // MXFP4 scale bytes [n][rows][cols/32]
  int64_t src_stride, scale_stride;   // bytes between experts
  int rows, cols, gated;  // canonical rows (H = rows/2 when gated), columns
  int n_tr, ks_dst, q_off, ks_src;
  int n;                  // matrices (experts)
  uint8_t* dst;           // tile row 0 of the first matrix
  int64_t dst_stride;     // bytes between experts
};

__device__ __forceinline__ int packed_row(int t, int c, int rows, int gated) {
  if (!gated) {
    const int r = 16 * t + c;
    return r < rows ? r : -1;
  }
  const int H = rows / 2, r = 8 * t + (c & 7);
  if (r >= H) return -1;
  return c < 8 ? r : H + r;
}

__global__ __launch_bounds__(kBlock) void k_pack_bf16(PackArgs a) {
  const int64_t gid = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  const int64_t per_mat = (int64_t)a.n_tr * a.ks_src * 4 * kWave;
  if (gid >= per_mat * a.n) return;
  const int64_t ei = gid / per_mat;
  int64_t r = gid - ei * per_mat;
  const int lane = (int)(r % kWave); r /= kWave;
  const int s = (int)(r % 4); r /= 4;
  const int q = (int)(r % a.ks_src);
  const int t = (int)(r / a.ks_src);
  const int c = lane & 15, g = lane >> 4;
  const int row = packed_row(t, c, a.rows, a.gated);
  const int col = q * kStepK + 32 * s + 8 * g;
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (row >= 0 && col < a.cols)
    v = *reinterpret_cast<const uint4*>(a.src + ei * a.src_stride + ((int64_t)row * a.cols + col) * 2);
  uint8_t* dp = a.dst + ei * a.dst_stride + ((int64_t)t * a.ks_dst + a.q_off + q) * kBf16StepBytes +
                s * 1024 + lane * 16;
  *reinterpret_cast<uint4*>(dp) = v;
}

__global__ __launch_bounds__(kBlock) void k_pack_fp4(PackArgs a) {
  const int64_t gid = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  const int64_t per_mat = (int64_t)a.n_tr * a.ks_src * kWave;
  if (gid >= per_mat * a.n) return;
  const int64_t ei = gid / per_mat;
  int64_t r = gid - ei * per_mat;
  const int lane = (int)(r % kWave); r /= kWave;
  const int q = (int)(r % a.ks_src);
  const int t = (int)(r / a.ks_src);
  const int c = lane & 15, g = lane >> 4;
  const int row = packed_row(t, c, a.rows, a.gated);
  const int nb = a.cols / 32;
  // lane l: the MX block of row l % 16, columns 128 q + 32 (l / 16) .. +32 (16 bytes)
  uint32_t wd[4];
  const int col = q * kStepK + 32 * g;
#pragma unroll
  for (int s = 0; s < 4; ++s)
    wd[s] = (row >= 0 && col < a.cols)
                ? *reinterpret_cast<const uint32_t*>(a.src + ei * a.src_stride + (int64_t)row * (a.cols / 2) + col / 2 + 4 * s)
                : 0u;
  uint8_t* dp = a.dst + ei * a.dst_stride + ((int64_t)t * a.ks_dst + q) * kFp4StepBytes;
  *reinterpret_cast<uint4*>(dp + lane * 16) = make_uint4(wd[0], wd[1], wd[2], wd[3]);
  if (g == 0) {
    uint32_t sd = 0;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int blkc = 4 * q + s;
      const uint32_t sb = (row >= 0 && blkc < nb)
                              ? a.scales[ei * a.scale_stride + (int64_t)row * nb + blkc] : 127u;
      sd |= sb << (8 * s);
    }
    *reinterpret_cast<uint32_t*>(dp + 1024 + c * 4) = sd;
  }
}

// FP8 block-128: lane l's 32 bytes are the codes of row l % 16 at columns 128 q + 32 s +
// 8 (l / 16) .. +8 for s = 0..3; then the K-step's two fp32 block scales (the rows of
// lanes 0..7 and of lanes 8..15), padded to 16 bytes.
__global__ __launch_bounds__(kBlock) void k_pack_fp8(PackArgs a) {
  const int64_t gid = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  const int64_t per_mat = (int64_t)a.n_tr * a.ks_src * kWave;
  if (gid >= per_mat * a.n) return;
  const int64_t ei = gid / per_mat;
  int64_t r = gid - ei * per_mat;
  const int lane = (int)(r % kWave); r /= kWave;
  const int q = (int)(r % a.ks_src);
  const int t = (int)(r / a.ks_src);
  const int c = lane & 15, g = lane >> 4;
  const int row = packed_row(t, c, a.rows, a.gated);
  uint2 v[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int col = q * kStepK + 32 * s + 8 * g;
    v[s] = (row >= 0 && col < a.cols)
               ? *reinterpret_cast<const uint2*>(a.src + ei * a.src_stride + (int64_t)row * a.cols + col)
               : make_uint2(0u, 0u);
  }
  uint8_t* dp = a.dst + ei * a.dst_stride + ((int64_t)t * a.ks_dst + q) * kFp8StepBytes;
  *reinterpret_cast<uint4*>(dp + lane * 32) = make_uint4(v[0].x, v[0].y, v[1].x, v[1].y);
  *reinterpret_cast<uint4*>(dp + lane * 32 + 16) = make_uint4(v[2].x, v[2].y, v[3].x, v[3].y);
  if (lane < 2) {
    const int hrow = packed_row(t, 8 * lane, a.rows, a.gated);
    const int bc = (a.cols + 127) / 128;
    const float* sc = reinterpret_cast<const float*>(a.scales) + ei * a.scale_stride;
    *reinterpret_cast<float*>(dp + 2048 + 4 * lane) = hrow >= 0 ? sc[(hrow / 128) * bc + q] : 0.f;
  } else if (lane == 2) {
    *reinterpret_cast<uint2*>(dp + 2056) = make_uint2(0u, 0u);
  }
}

}  // namespace

// ------------------------------------------------------------------------------------
// Launches
// ------------------------------------------------------------------------------------
namespace {

RouteArgs route_args(const Shape& s, const float* bias, int64_t T, const Work& ws, int32_t* idx,
                     float* gw) {
  return RouteArgs{ws.z, route_planes(s), route_subplanes(s), T * s.E, bias, T, s.E, s.k, s.route_scale, idx, gw,
                   ws.counts, ws.offs, ws.perm, ws.inv, ws.units, ws.ctrl, unit_positions(s, T),
                   (int)even_units(s)};
}

}  // namespace

namespace {

InArgs in_args(const Shape& s, const uint8_t* dense, const uint16_t* x, int64_t T, const Work& ws,
               int tr_first, int tr_count) {
  InArgs a;
  a.w = dense;
  a.ks = s.ks_in;
  a.tr_r = s.tr_r; a.tr_dn = s.tr_dn; a.tr_sh = s.tr_sh;
  a.ntb = in_tokens_per_block(s);
  a.ksplit = choose_ksplit(s.tr_in, s.ks_in);
  a.router_wgs = 0;
  a.zplanes = s.zplanes;
  a.tr_first = tr_first;
  a.tr_count = tr_count;
  a.wg_per_blk = cdiv((int64_t)tr_count * a.ksplit, kWavesPerBlock);
  a.n_blk = cdiv(T, a.ntb);
  a.x = x; a.T = T; a.d = s.d;
  a.z = ws.z; a.E = s.E;
  a.xc = ws.xc; a.l = s.l;
  a.hs = ws.hs; a.ms = s.ms;
  a.act = s.act; a.bg = s.beta_gate; a.bl = s.beta_lin;
  a.route = 0;
  a.arrive = nullptr;
  a.n_arrive = 0;
  return a;
}

// Shared gate/up tile rows of the IN launch: all of them, the streaming that hides the
// route of a few tokens.
int in_launch_shared_rows(const Shape& s) { return s.tr_sh; }

}  // namespace

namespace {
// Without a latent the experts read the token itself: x (bf16) as the fp32 rows of the
// few-token launches and as the hi/lo rows (lo = 0) of the token-tiled ones.
__global__ __launch_bounds__(kBlock) void k_token_rows(const uint16_t* __restrict__ x, int64_t n,
                                                       float* __restrict__ xc, uint16_t* __restrict__ xc_hl,
                                                       int d) {
  const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (i >= n) return;
  const uint16_t v = x[i];
  xc[i] = __uint_as_float((uint32_t)v << 16);
  if (xc_hl) {
    const int64_t t = i / d, c = i - t * d;
    xc_hl[t * 2 * d + c] = v;
    xc_hl[t * 2 * d + d + c] = 0;
  }
}
}  // namespace

hipError_t launch_router(const Shape& s, const uint8_t* dense, const uint16_t* x, int64_t T,
                         bool router_only, const Work& ws, hipStream_t st) {
  if (!s.latent && !router_only) {
    const int64_t n = T * s.d;
    hipLaunchKernelGGL(k_token_rows, dim3((unsigned)cdiv(n, kBlock)), dim3(kBlock), 0, st, x, n,
                       ws.xc, token_tiled(s, T) ? ws.xc_hl : nullptr, s.d);
  }
  if (token_tiled(s, T)) {
    // larger batches: the router over tiles of 64 tokens (W_down_latent goes to the
    // token-tiled IN launch)
    RouterTTArgs a;
    a.w = dense;
    a.ks = s.ks_in;
    a.qpp = cdiv(s.ks_in, s.zplanes);
    a.tr_r = s.tr_r;
    const int tr = T >= kRouterTTWideTokens ? 2 : 1;
    a.n_grp = cdiv(s.tr_r, kWavesPerBlock * tr);
    a.zplanes = s.zplanes;
    a.n_tiles = cdiv(T, kTTMaxSrc);
    a.x = x; a.T = T; a.d = s.d; a.E = s.E;
    a.z = ws.z;
    const size_t lds = (size_t)2 * kInTTBlocks * 16 * 16 * 16;
    const dim3 grid((unsigned)xcd_grid((int64_t)a.n_grp * a.zplanes * kZSub, a.n_tiles));
    if (tr == 2) hipLaunchKernelGGL(k_router_tt<2>, grid, dim3(kBlock), lds, st, a);
    else hipLaunchKernelGGL(k_router_tt<1>, grid, dim3(kBlock), lds, st, a);
    return hipGetLastError();
  }
  if (!router_only && in_takes_router(s, T)) return hipSuccess;   // the IN launch takes them
  InArgs a = in_args(s, dense, x, T, ws, s.tr_r, router_only ? 0 : s.tr_dn);
  a.router_wgs = s.tr_r * s.zplanes;
  a.wg_per_blk += a.router_wgs;
  const size_t lds = (size_t)(T < a.ntb ? T : a.ntb) * s.ks_in * kStepK * 2;
  hipLaunchKernelGGL(k_router, dim3((unsigned)xcd_grid(a.wg_per_blk, a.n_blk)), dim3(kBlock), lds,
                     st, a);
  return hipGetLastError();
}

hipError_t launch_in(const Shape& s, const uint8_t* dense, const uint16_t* x, int64_t T,
                     const float* bias, int32_t* idx, float* gw, const Work& ws, hipStream_t st) {
  if (token_tiled(s, T)) {
    // W_down_latent and the shared gate/up over tiles of 64 tokens
    InTTArgs a;
    a.w = dense;
    a.ks = s.ks_in;
    a.qper = cdiv(s.ks_in, choose_ksplit(s.tr_in, s.ks_in));
    a.tr_r = s.tr_r; a.tr_dn = s.tr_dn;
    a.tr_first = s.tr_r; a.tr_count = s.tr_dn + s.tr_sh;
    a.n_grp = cdiv(a.tr_count, kWavesPerBlock);
    a.n_tiles = cdiv(T, kTTMaxSrc);
    a.x = x; a.T = T; a.d = s.d;
    a.xc = ws.xc; a.xc_hl = ws.xc_hl; a.l = s.l; a.lp = s.l;
    a.hs = ws.hs; a.hs_hl = ws.hs_hl; a.ms = s.ms;
    a.act = s.act; a.bg = s.beta_gate; a.bl = s.beta_lin;
    const size_t lds = (size_t)2 * kInTTBlocks * 16 * 16 * 16;
    hipLaunchKernelGGL(k_in_tt, dim3((unsigned)xcd_gblock_grid(a.n_grp, a.n_tiles, kInTTGroups)), dim3(kBlock), lds, st,
                       a);
    return hipGetLastError();
  }
  const bool all = in_takes_router(s, T);
  const int n_tr = all ? s.tr_dn + s.tr_sh : in_launch_shared_rows(s);
  InArgs a = in_args(s, dense, x, T, ws, s.tr_in - n_tr, n_tr);
  a.route = route_fused(s, T) ? 1 : 0;
  a.ra = route_args(s, bias, T, ws, idx, gw);
  if (all) {
    // the router rows first (the lowest workgroup numbers after the route's: dispatched
    // before the others, they wait for nothing), then W_down_latent and the shared gate/up
    a.router_wgs = s.tr_r * s.zplanes;
    a.wg_per_blk += a.router_wgs;
    a.arrive = ws.ctrl + kCtrlArrive;
    a.n_arrive = a.router_wgs * a.n_blk;
  }
  const int64_t grid = (a.wg_per_blk > 0 ? xcd_grid(a.wg_per_blk, a.n_blk) : 0) + a.route;
  if (grid == 0) return hipSuccess;   // no shared expert and a separate route
  const size_t lds = (size_t)(T < a.ntb ? T : a.ntb) * s.ks_in * kStepK * 2;
  hipLaunchKernelGGL(k_in, dim3((unsigned)grid), dim3(kBlock), lds, st, a);
  return hipGetLastError();
}

hipError_t launch_route(const Shape& s, const float* bias, int64_t T, const Work& ws,
                        int32_t* idx, float* gw, hipStream_t st) {
  RouteArgs a = route_args(s, bias, T, ws, idx, gw);
  hipLaunchKernelGGL(k_route, dim3((unsigned)T), dim3(kBlock), 0, st, a);
  return hipGetLastError();
}

constexpr int kQbLdsBins = 16384;

hipError_t launch_qb_hist(const Shape& s, const float* bias, int64_t T, int bins, int32_t* hist,
                          const Work& ws, hipStream_t st) {
  QbArgs a{};
  a.z = ws.z; a.zplanes = route_planes(s); a.zsub = route_subplanes(s); a.zplane = T * s.E;
  a.bias = bias; a.T = T; a.E = s.E; a.k = s.k; a.bins = bins;
  a.hist = hist;
  a.alpha = reinterpret_cast<float*>(ws.perm);   // T <= T k floats of the dispatch slot
  const unsigned grid = (unsigned)(T < 2048 ? T : 2048);
  hipLaunchKernelGGL(k_qb_alpha, dim3(grid), dim3(kBlock), 0, st, a);
  // counters of up to 16 Ki bins per workgroup (64 KiB of LDS), 512 tokens each
  a.eb = std::max(1, std::min(16, kQbLdsBins / bins));
  a.tc = 512;
  const int64_t n_eg = cdiv(s.E, a.eb), n_tb = cdiv(T, a.tc);
  hipLaunchKernelGGL(k_qb_count, dim3((unsigned)(n_eg * n_tb)), dim3(kBlock),
                     (size_t)a.eb * bins * 4, st, a);
  return hipGetLastError();
}

hipError_t launch_qb_readout(const Shape& s, const float* bias, int64_t T, int bins,
                             const int32_t* hist, float* new_bias, hipStream_t st) {
  QbArgs a{};
  a.bias = bias; a.T = T; a.E = s.E; a.k = s.k; a.bins = bins;
  a.chist = hist; a.new_bias = new_bias;
  hipLaunchKernelGGL(k_qb_readout, dim3((unsigned)s.E), dim3(kBlock), 0, st, a);
  hipLaunchKernelGGL(k_qb_centre, dim3(1), dim3(kBlock), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_dispatch(const Shape& s, const int32_t* idx, int64_t T, int32_t* counts,
                           int32_t* offs, int32_t* perm, int32_t* inv, int32_t* chunk_hist,
                           int32_t* units, int32_t* ctrl, hipStream_t st) {
  const int ct = dispatch_chunk_tokens(s.k);
  const int chunk = ct * s.k;
  const int64_t n = T * s.k;
  const int nch = cdiv(T, ct);
  hipLaunchKernelGGL(k_disp_count, dim3(nch), dim3(kBlock), 0, st, idx, n, s.E, chunk, chunk_hist);
  hipLaunchKernelGGL(k_disp_scan, dim3(1), dim3(1024), 0, st, nch, s.E, unit_positions(s, T),
                     small_unit_positions(s, T), (int)even_units(s), chunk_hist, counts, offs,
                     units, ctrl);
  hipLaunchKernelGGL(k_disp_scatter, dim3(nch), dim3(kBlock), 0, st, idx, n, s.E, chunk,
                     (const int32_t*)chunk_hist, (const int32_t*)offs, perm, inv);
  return hipGetLastError();
}

constexpr int kExpTTSplitTokens = 512;
template <int WF, bool GU>
void launch_exp_tt(bool split, unsigned grid, size_t lds1, size_t lds, hipStream_t st,
                   const ExpArgs& b) {
  if (split) {
    hipLaunchKernelGGL((k_exp_tt<WF, GU, 1>), dim3(grid), dim3(kBlock), lds1, st, b);
    hipLaunchKernelGGL((k_exp_tt<WF, GU, 2>), dim3(grid), dim3(kBlock), lds, st, b);
  } else {
    hipLaunchKernelGGL((k_exp_tt<WF, GU, 0>), dim3(grid), dim3(kBlock), lds, st, b);
  }
}

hipError_t launch_expert(const Shape& s, const uint8_t* experts, const uint8_t* dense, bool gu,
                         int64_t T, const Work& ws, hipStream_t st) {
  ExpArgs a{};
  a.experts = experts;
  a.expert_bytes = s.expert_bytes;
  a.region_off = gu ? 0 : s.gu_bytes;
  a.ks = gu ? s.ks_gu : s.ks_edn;
  a.n_tr = gu ? s.tr_gu : s.tr_edn;
  a.units = ws.units;
  a.ctrl = ws.ctrl;
  a.nu = unit_positions(s, T);
  a.max_units = (int)max_units(s, T);
  a.E = s.E; a.k = s.k;
  a.n_assign = T * s.k;
  a.perm = ws.perm;
  a.xin = gu ? ws.xc : ws.h;
  a.kin = gu ? s.l : s.m;
  a.out = gu ? ws.h : ws.eo;
  a.n_out = gu ? s.m : s.l;
  a.act = s.act; a.bg = s.beta_gate; a.bl = s.beta_lin;
  a.xin_hl = gu ? ws.xc_hl : ws.h_hl;
  a.kin_ld = gu ? s.l : s.m;
  a.out_hl = ws.h_hl;
  a.out_ld = s.m;
  a.single = gu && !s.latent ? 1 : 0;   // x itself: bf16, its lo rows zero
  // one wavefront per tile row and its whole K range (the per-item staging and the
  // cross-wavefront sum cost more than a K-split gains)
  a.ksplit = 1;
  a.wg_per_unit = cdiv(a.n_tr, kWavesPerBlock);
  a.chunk = 0;
  if (token_tiled(s, T)) {
    // the long units: K-step loop over tiles of their hi/lo rows
    ExpArgs b = a;
    b.max_units = (int)max_large_units(s, T);
    b.chunk = kExpTTOrder;
    const int halves = exp_tt_halves(b.single != 0, b.nu);
    const int ttr = s.wfmt == 1   ? ExpTTRows<1>::value
                    : s.wfmt == 2 ? ExpTTRows<2>::value
                                  : ExpTTRows<0>::value;
    b.wg_per_unit = cdiv(b.n_tr, kWavesPerBlock * ttr);
    if (b.max_units > 0) {
      const int64_t items = (int64_t)b.max_units * halves;
      const unsigned grid = (unsigned)(b.chunk > 0   ? chunk_grid(items, b.wg_per_unit, b.chunk)
                                       : b.chunk < 0 ? xcd_block_grid(b.wg_per_unit, items)
                                                     : xcd_grid(b.wg_per_unit, items));
      // From kExpTTSplitTokens tokens on, with at most 64 positions per expert on average (so
      // that many units are short), the items of one 16-row block in a launch of their own
      // first, then the others (each launch skips the rest): measured 1.7% faster on the
      // 1024-token Zipf(1.2) batch of 384 experts; 1% slower at 64 tokens, and no faster at
      // 8192 tokens over 896 experts (146 positions per expert), where the second launch
      // costs more than the first one's occupancy gains.
      const size_t lds1 = (size_t)2 * 1 * 16 * 16 * 16;
      const size_t lds = (size_t)2 * kHiloTTBlocks * 16 * 16 * 16;
      const bool split = T >= kExpTTSplitTokens && T * s.k <= (int64_t)64 * s.E;
      if (s.wfmt == 1) {
        if (gu) launch_exp_tt<1, true>(split, grid, lds1, lds, st, b);
        else launch_exp_tt<1, false>(split, grid, lds1, lds, st, b);
      } else if (s.wfmt == 2) {
        if (gu) launch_exp_tt<2, true>(split, grid, lds1, lds, st, b);
        else launch_exp_tt<2, false>(split, grid, lds1, lds, st, b);
      } else {
        if (gu) launch_exp_tt<0, true>(split, grid, lds1, lds, st, b);
        else launch_exp_tt<0, false>(split, grid, lds1, lds, st, b);
      }
      const hipError_t err = hipGetLastError();
      if (err != hipSuccess) return err;
    }
    // the short ones (the first list: its count is ctrl[1]) as for a few tokens
    a.ctrl = ws.ctrl + 1;
    a.nu = small_unit_positions(s, T);
    a.max_units = (int)max_small_units(s, T);
    a.chunk = kExpChunk;
  } else {
    a.out_hl = nullptr;
    const OutParts op = out_parts(s);
    if (!gu && op.nsd > 0) {
      if (!dense || T > kFewTokens) return hipErrorInvalidValue;
      a.sd_w = dense + s.in_bytes;
      a.sd_parts = op.nsd;
      a.sd_q0 = s.ks_l;
      a.sd_qper = op.qper2;
      a.sd_ks = s.ks_ms;
      a.sd_row = s.ks_out;
      a.sd_ntr = s.tr_out;
      a.sd_wgs = (int)(kXcds * cdiv((int64_t)cdiv(s.tr_out, kWavesPerBlock) * op.nsd, kXcds));
      a.sd_hs = ws.hs;
      a.sd_ms = s.ms;
      a.sd_T = (int)T;
      a.sd_d = s.d;
      a.sd_out = ws.ys;
    }
  }
  const unsigned grid = (unsigned)(a.sd_wgs + (a.chunk > 0 ? chunk_grid(a.max_units, a.wg_per_unit, a.chunk)
                                                           : xcd_grid(a.wg_per_unit, a.max_units)));
  size_t lds = (size_t)2 * a.nu * a.ks * kStepK * 2;
  const size_t sd_lds = (size_t)2 * T * a.sd_qper * kStepK * 2;
  if (a.sd_wgs > 0 && sd_lds > lds) lds = sd_lds;
  if (s.wfmt == 1) {
    if (gu) hipLaunchKernelGGL((k_exp<1, true>), dim3(grid), dim3(kBlock), lds, st, a);
    else hipLaunchKernelGGL((k_exp<1, false>), dim3(grid), dim3(kBlock), lds, st, a);
  } else if (s.wfmt == 2) {
    if (gu) hipLaunchKernelGGL((k_exp<2, true>), dim3(grid), dim3(kBlock), lds, st, a);
    else hipLaunchKernelGGL((k_exp<2, false>), dim3(grid), dim3(kBlock), lds, st, a);
  } else {
    if (gu) hipLaunchKernelGGL((k_exp<0, true>), dim3(grid), dim3(kBlock), lds, st, a);
    else hipLaunchKernelGGL((k_exp<0, false>), dim3(grid), dim3(kBlock), lds, st, a);
  }
  return hipGetLastError();
}

hipError_t launch_combine(const Shape& s, const uint8_t* dense, const float* gw, int64_t T,
                          const Work& ws, hipStream_t st) {
  const int bpt = cdiv(s.l, kBlock);
  hipLaunchKernelGGL(k_combine, dim3((unsigned)(T * bpt)), dim3(kBlock), 0, st, gw,
                     (const int32_t*)ws.inv, (const float*)ws.eo, T, s.k, s.l, bpt, ws.u);
  if (token_tiled(s, T) && !mx_profile(s) && s.latent)   // (the mx launches take their own norm)
    hipLaunchKernelGGL(k_norm, dim3((unsigned)T), dim3(kBlock), 0, st, (const float*)ws.u,
                       reinterpret_cast<const uint16_t*>(dense + s.gamma_off), s.l, s.use_norm,
                       s.eps, ws.uh, ws.uh_hl);
  return hipGetLastError();
}

hipError_t launch_out(const Shape& s, const uint8_t* dense, int64_t T, const Work& ws,
                      const OutSink& out, hipStream_t st, const Prefetch& pf) {
  if (token_tiled(s, T)) {
    // [u_hat ; h_s] hi/lo rows over tiles of 32 tokens
    OutTTArgs a;
    a.w = dense + s.in_bytes;
    a.ks = s.ks_out; a.ks_l = s.ks_l;
    const OutParts op = out_parts(s);   // the parts of the few-token launches
    a.qper = op.qper;
    a.kb = op.nsd > 0 ? op.ks_a : -1;
    a.qper2 = op.qper2;
    a.n_tr = s.tr_out;
    a.n_grp = cdiv(s.tr_out, kWavesPerBlock);
    a.n_tiles = cdiv(T, kHiloTTRows);
    a.uh_hl = ws.uh_hl; a.hs_hl = ws.hs_hl;
    a.d = s.d; a.l = s.l; a.ms = s.ms; a.n0 = s.latent ? s.l : 0;
    a.T = T; a.sink = out;
    a.add_u = s.latent ? nullptr : ws.u;
    const size_t lds = (size_t)2 * kHiloTTBlocks * 16 * 16 * 16;
    hipLaunchKernelGGL(k_out_tt, dim3((unsigned)xcd_gblock_grid(a.n_grp, a.n_tiles, kOutTTGroups)), dim3(kBlock), lds,
                       st, a);
    return hipGetLastError();
  }
  OutArgs a;
  const OutParts op = out_parts(s);
  a.w = dense + s.in_bytes;
  a.ks_row = s.ks_out; a.ks_l = s.ks_l;
  a.ks = op.ks_a;                    // with nsd > 0 the u_hat segment alone
  a.n_tr = s.tr_out;
  a.ntb = out_tokens_per_block(s);   // 2 * ntb hi/lo rows: at most one 16-row MFMA block
  a.n_blk = cdiv(T, a.ntb);
  a.ksplit = op.ksplit;
  a.wg_per_blk = cdiv((int64_t)a.n_tr * a.ksplit, kWavesPerBlock);
  a.u = ws.u; a.hs = ws.hs;
  a.gamma = reinterpret_cast<const uint16_t*>(dense + s.gamma_off);
  a.d = s.d; a.l = s.l; a.ms = s.ms; a.norm = s.use_norm; a.eps = s.eps;
  a.n0 = s.latent ? s.l : 0;
  a.n1 = op.nsd > 0 ? 0 : s.ms;
  a.ys = ws.ys;
  a.nsd = op.nsd;
  if (op.nsd > 0 && T > kFewTokens) return hipErrorInvalidValue;
  a.T = T; a.sink = out;
  a.add_u = s.latent ? nullptr : ws.u;
  a.prod_wgs = (int)xcd_grid(a.wg_per_blk, a.n_blk);
  a.pf = pf;
  a.pf_wgs = pf.p && pf.bytes >= 16 ? (int)((pf.bytes + kPrefetchWgBytes - 1) / kPrefetchWgBytes) : 0;
  const size_t lds = (size_t)2 * (T < a.ntb ? T : a.ntb) * a.ks * kStepK * 2;
  const dim3 grid((unsigned)(a.prod_wgs + a.pf_wgs));
  if (cdiv(a.ks, a.ksplit) <= kOutDeepRing)
    hipLaunchKernelGGL((k_out<kOutDeepRing>), grid, dim3(kBlock), lds, st, a);
  else
    hipLaunchKernelGGL((k_out<3>), grid, dim3(kBlock), lds, st, a);
  return hipGetLastError();
}

namespace {

hipError_t pack_bf16(const void* src, int64_t src_stride, int rows, int cols, int gated, int n_tr,
                     int ks_dst, int q_off, int n, uint8_t* dst, int64_t dst_stride,
                     hipStream_t st) {
  if (rows == 0 || cols == 0) return hipSuccess;
  PackArgs a{};
  a.src = static_cast<const uint8_t*>(src);
  a.src_stride = src_stride;
  a.rows = rows; a.cols = cols; a.gated = gated;
  a.n_tr = n_tr; a.ks_dst = ks_dst; a.q_off = q_off; a.ks_src = cdiv(cols, kStepK);
  a.n = n; a.dst = dst; a.dst_stride = dst_stride;
  const int64_t threads = (int64_t)n * n_tr * a.ks_src * 4 * kWave;
  hipLaunchKernelGGL(k_pack_bf16, dim3((unsigned)cdiv(threads, kBlock)), dim3(kBlock), 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pack_dense(const Shape& s, const DenseSrc& src, uint8_t* packed,
                             hipStream_t st) {
  hipError_t e;
  const int64_t row_in = (int64_t)s.ks_in * kBf16StepBytes;
  // IN: router, W_down_latent, shared gate/up (gated tiles)
  if ((e = pack_bf16(src.router, 0, s.E, s.d, 0, s.tr_r, s.ks_in, 0, 1, packed, 0, st)) != hipSuccess) return e;
  if (s.latent && (e = pack_bf16(src.wdn, 0, s.l, s.d, 0, s.tr_dn, s.ks_in, 0, 1,
                                 packed + s.tr_r * row_in, 0, st)) != hipSuccess)
    return e;
  if (s.ms > 0 && (e = pack_bf16(src.sgu, 0, 2 * s.ms, s.d, 1, s.tr_sh, s.ks_in, 0, 1,
                                 packed + (int64_t)(s.tr_r + s.tr_dn) * row_in, 0, st)) != hipSuccess)
    return e;
  // OUT: [W_up_latent | W_shared_down]
  uint8_t* out = packed + s.in_bytes;
  if (s.latent && (e = pack_bf16(src.wup, 0, s.d, s.l, 0, s.tr_out, s.ks_out, 0, 1, out, 0, st)) != hipSuccess)
    return e;
  if (s.ms > 0 && (e = pack_bf16(src.sdn, 0, s.d, s.ms, 0, s.tr_out, s.ks_out, s.ks_l, 1, out, 0,
                                 st)) != hipSuccess)
    return e;
  if (!s.latent) return hipSuccess;   // no latent: no norm gain
  return hipMemcpyAsync(packed + s.gamma_off, src.gamma, (size_t)s.l * 2, hipMemcpyDeviceToDevice, st);
}

hipError_t launch_pack_experts(const Shape& s, const void* gu, const void* gus, const void* dn,
                               const void* dns, int e0, int n, uint8_t* packed, hipStream_t st) {
  uint8_t* dst = packed + (size_t)e0 * s.expert_bytes;
  if (s.wfmt == 0) {
    hipError_t e = pack_bf16(gu, (int64_t)2 * s.m * s.l * 2, 2 * s.m, s.l, 1, s.tr_gu, s.ks_gu, 0, n,
                             dst, s.expert_bytes, st);
    if (e != hipSuccess) return e;
    return pack_bf16(dn, (int64_t)s.l * s.m * 2, s.l, s.m, 0, s.tr_edn, s.ks_edn, 0, n,
                     dst + s.gu_bytes, s.expert_bytes, st);
  }
  if (s.wfmt == 2) {
    PackArgs a{};
    const int64_t bgu = (int64_t)((2 * s.m + 127) / 128) * ((s.l + 127) / 128);
    const int64_t bdn = (int64_t)((s.l + 127) / 128) * ((s.m + 127) / 128);
    a.src = static_cast<const uint8_t*>(gu);
    a.scales = static_cast<const uint8_t*>(gus);
    a.src_stride = (int64_t)2 * s.m * s.l;
    a.scale_stride = bgu;
    a.rows = 2 * s.m; a.cols = s.l; a.gated = 1;
    a.n_tr = s.tr_gu; a.ks_dst = s.ks_gu; a.q_off = 0; a.ks_src = s.ks_gu;
    a.n = n; a.dst = dst; a.dst_stride = s.expert_bytes;
    int64_t threads = (int64_t)n * a.n_tr * a.ks_src * kWave;
    hipLaunchKernelGGL(k_pack_fp8, dim3((unsigned)cdiv(threads, kBlock)), dim3(kBlock), 0, st, a);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    a.src = static_cast<const uint8_t*>(dn);
    a.scales = static_cast<const uint8_t*>(dns);
    a.src_stride = (int64_t)s.l * s.m;
    a.scale_stride = bdn;
    a.rows = s.l; a.cols = s.m; a.gated = 0;
    a.n_tr = s.tr_edn; a.ks_dst = s.ks_edn; a.ks_src = s.ks_edn;
    a.dst = dst + s.gu_bytes;
    threads = (int64_t)n * a.n_tr * a.ks_src * kWave;
    hipLaunchKernelGGL(k_pack_fp8, dim3((unsigned)cdiv(threads, kBlock)), dim3(kBlock), 0, st, a);
    return hipGetLastError();
  }
  PackArgs a{};
  a.src = static_cast<const uint8_t*>(gu);
  a.scales = static_cast<const uint8_t*>(gus);
  a.src_stride = (int64_t)2 * s.m * (s.l / 2);
  a.scale_stride = (int64_t)2 * s.m * (s.l / 32);
  a.rows = 2 * s.m; a.cols = s.l; a.gated = 1;
  a.n_tr = s.tr_gu; a.ks_dst = s.ks_gu; a.q_off = 0; a.ks_src = s.ks_gu;
  a.n = n; a.dst = dst; a.dst_stride = s.expert_bytes;
  int64_t threads = (int64_t)n * a.n_tr * a.ks_src * kWave;
  hipLaunchKernelGGL(k_pack_fp4, dim3((unsigned)cdiv(threads, kBlock)), dim3(kBlock), 0, st, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  a.src = static_cast<const uint8_t*>(dn);
  a.scales = static_cast<const uint8_t*>(dns);
  a.src_stride = (int64_t)s.l * (s.m / 2);
  a.scale_stride = (int64_t)s.l * (s.m / 32);
  a.rows = s.l; a.cols = s.m; a.gated = 0;
  a.n_tr = s.tr_edn; a.ks_dst = s.ks_edn; a.ks_src = s.ks_edn;
  a.dst = dst + s.gu_bytes;
  threads = (int64_t)n * a.n_tr * a.ks_src * kWave;
  hipLaunchKernelGGL(k_pack_fp4, dim3((unsigned)cdiv(threads, kBlock)), dim3(kBlock), 0, st, a);
  return hipGetLastError();
}

}  // namespace moe
