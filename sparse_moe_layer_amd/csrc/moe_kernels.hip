// gfx950 kernels of the Stable LatentMoE FFN layer forward.
//
// Step order follows the Kimi K3 latent mixture-of-experts block card ("All 23 steps"
// and its KimiSparseMoeBlock.forward / moe_infer excerpt):
//   k_router       router logits z = x W_r
//   k_dense_x      x^c = x W_down_latent and the shared gate/up with its SiTU epilogue;
//                  for a few tokens its workgroup 0 meanwhile takes s = sigmoid(z), the
//                  top_k of s + b, G = s / sum(s) and sorts the assignments by expert
//   k_route        the same selection in its own launch for larger batches
//   k_disp_*       per-expert histogram -> scan -> stable permutation for larger batches
//                  (moe_infer's scatter_/argsort, kept on the device: no host round trip)
//   k_expert_*     routed gate/up (+ SiTU) and down, MXFP4 or bf16 weights
//   k_combine      u = sum_j G_j E_j in a fixed order (no atomics)
//   k_out          RMSNorm(u) W_up_latent + h_s W_shared_down -> Delta, one product over
//                  the concatenated row [W_up_latent[r] | W_shared_down[r]]
//
// The weight products are matrix-vector streams: every weight byte is read once per token
// through 16-byte non-temporal loads (64 lanes x 16 B = 1 KiB per load instruction), two
// rows (or row groups) in flight per wavefront, so decode is bound by HBM bandwidth.
// Activations stay fp32 end to end; the bf16 tokens meet bf16 weights in v_dot2_f32_bf16.
#include <climits>
#include <cmath>

#include "moe_device.hpp"
#include "moe_internal.hpp"

namespace moe {
namespace {

constexpr int kBlock = 256;  // 4 wavefronts per workgroup
constexpr int kWavesPerBlock = kBlock / kWave;

__device__ __forceinline__ int64_t global_wave() {
  return (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
}

// ------------------------------------------------------------------------------------
// Row products.  Lane l covers the 8-column chunks l, l+64, l+128, ... of a row; the
// per-lane sum runs in chunk order and the DPP reduction finishes it (fixed order).
// ------------------------------------------------------------------------------------

template <int NCH>
__device__ __forceinline__ void load_row(const uint16_t* row, int k8, int lane, uint4 (&w)[NCH]) {
  const uint4* r = reinterpret_cast<const uint4*>(row);
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int c = j * kWave + lane;
    w[j] = (c < k8) ? ld_stream(r + c) : make_uint4(0u, 0u, 0u, 0u);
  }
}

// bf16 weights x bf16 activations (packed pairs).
template <int NCH>
__device__ __forceinline__ float dot_bb(const uint4 (&w)[NCH], const uint4 (&x)[NCH]) {
  float acc = 0.f;
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    acc = dot2_bf16(w[j].x, x[j].x, acc);
    acc = dot2_bf16(w[j].y, x[j].y, acc);
    acc = dot2_bf16(w[j].z, x[j].z, acc);
    acc = dot2_bf16(w[j].w, x[j].w, acc);
  }
  return acc;
}

// bf16 weights x fp32 activations held in registers.
template <int NCH>
__device__ __forceinline__ float dot_bf(const uint4 (&w)[NCH], const float (&xs)[NCH][8]) {
  float acc = 0.f;
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const uint32_t q[4] = {w[j].x, w[j].y, w[j].z, w[j].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc = fmaf(bf16_lo(q[i]), xs[j][2 * i], acc);
      acc = fmaf(bf16_hi(q[i]), xs[j][2 * i + 1], acc);
    }
  }
  return acc;
}

template <int NCH>
__device__ __forceinline__ void load_x_f32(const float* xr, int k8, int lane, float (&xs)[NCH][8]) {
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int c = j * kWave + lane;
    if (c < k8) {
      const float4 a = reinterpret_cast<const float4*>(xr)[2 * c];
      const float4 b = reinterpret_cast<const float4*>(xr)[2 * c + 1];
      xs[j][0] = a.x; xs[j][1] = a.y; xs[j][2] = a.z; xs[j][3] = a.w;
      xs[j][4] = b.x; xs[j][5] = b.y; xs[j][6] = b.z; xs[j][7] = b.w;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) xs[j][i] = 0.f;
    }
  }
}

// An fp32 activation row staged in LDS as two planes: plane 0 holds columns 8c..8c+3 and
// plane 1 columns 8c+4..8c+7 of chunk c, so that a wavefront reading chunk j*64+lane
// reads 64 consecutive 16-byte words from each plane (no bank conflicts).
__device__ __forceinline__ void stage_x(const float* xr, int k8, int n_chunks, float4* p0, float4* p1) {
  const float4* x4 = reinterpret_cast<const float4*>(xr);
  for (int c = threadIdx.x; c < n_chunks; c += kBlock) {
    if (c < k8) {
      p0[c] = x4[2 * c];
      p1[c] = x4[2 * c + 1];
    } else {
      p0[c] = make_float4(0.f, 0.f, 0.f, 0.f);
      p1[c] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
}

// ------------------------------------------------------------------------------------
// Step ROUTE: one workgroup (4 wavefronts) per token.  Expert e = (4i + w)*64 + lane
// belongs to wavefront w, slot i.  Each wavefront finds the top-k of its share with k
// rounds of a DPP arg-max over a 64-bit key (order key of kappa = s + b in the high word,
// ~e in the low word: larger kappa first, then the lower index); the 4k candidates are
// then ranked in LDS.  G = route_scale * s / sum(s), the sum in selection order.
// For at most 4 tokens one workgroup handles all of them and then sorts the T*k
// assignments by expert (histogram, scan, stable rank) in LDS.
// ------------------------------------------------------------------------------------
struct RouteArgs {
  const float* z;
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
};

constexpr int kRouteSlots = 4;      // E <= 4 slots x 4 wavefronts x 64 lanes = 1024
constexpr int kMaxK = 64;

__device__ __forceinline__ void block_route_token(const RouteArgs& a, int64_t t, uint64_t* cand_key,
                                                  float* cand_s, int* sel_e, float* sel_s,
                                                  int* sidx) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x >> 6;
  uint64_t key[kRouteSlots];
  float sv[kRouteSlots];
  const float* zr = a.z + t * a.E;
#pragma unroll
  for (int i = 0; i < kRouteSlots; ++i) {
    const int e = (i * kWavesPerBlock + wv) * kWave + lane;
    if (e < a.E) {
      const float s = sigmoidf_(zr[e]);
      float kk = s + a.bias[e];
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

// The route of tokens t_begin..t_end-1 by one workgroup; with `dispatch`, also the
// counting sort of their (at most 256) assignments by expert.
__device__ void route_block(const RouteArgs& a, int64_t t_begin, int64_t t_end, bool dispatch) {
  __shared__ uint64_t cand_key[kWavesPerBlock * kMaxK];
  __shared__ float cand_s[kWavesPerBlock * kMaxK];
  __shared__ int sel_e[kMaxK];
  __shared__ float sel_s[kMaxK];
  __shared__ int sidx[kBlock];
  __shared__ int hist[1024];
  __shared__ int soff[1024];
  __shared__ int part[kBlock];
  for (int64_t t = t_begin; t < t_end; ++t)
    block_route_token(a, t, cand_key, cand_s, sel_e, sel_s, dispatch ? sidx : nullptr);
  if (!dispatch) return;
  // dispatch of the n = T*k <= 256 assignments
  const int n = (int)(a.T * a.k);
  const int tid = threadIdx.x;
  for (int e = tid; e < a.E; e += kBlock) hist[e] = 0;
  __syncthreads();
  if (tid < n) atomicAdd(&hist[sidx[tid]], 1);
  __syncthreads();
  // exclusive scan over experts: 4 consecutive experts per thread, then across threads
  int loc[4], ps = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = tid * 4 + i;
    loc[i] = (e < a.E) ? hist[e] : 0;
    ps += loc[i];
  }
  part[tid] = ps;
  __syncthreads();
  for (int o = 1; o < kBlock; o <<= 1) {
    const int v = (tid >= o) ? part[tid - o] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int run = part[tid] - ps;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = tid * 4 + i;
    if (e < a.E) {
      soff[e] = run;
      a.offs[e] = run;
      a.counts[e] = loc[i];
    }
    run += loc[i];
  }
  if (tid == 0) a.offs[a.E] = n;
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
// Step DENSE_X: router logits, latent down-projection, shared gate/up + activation.
// The token slice stays in registers; rows go two at a time.
// ------------------------------------------------------------------------------------
struct DenseXArgs {
  const uint16_t* x;
  int64_t T;
  int d;
  const uint16_t* wr;
  int E;
  float* z;
  const uint16_t* wdn;
  int l;
  float* xc;
  const uint16_t* sgu;
  int ms;
  float* hs;
  int act;
  float bg, bl;
  int rows_per_wave;     // router / latent rows per wavefront (even)
  int pairs_per_wave;    // shared gate/up row pairs per wavefront
  int waves_r, waves_dn, waves_sh;  // per token
  int route;             // 1: workgroup 0 routes and dispatches the (<= 4) tokens
  RouteArgs ra;
};

template <int NCH>
__device__ __forceinline__ void rows_x2(const uint16_t* w, int d, int r0, int r1,
                                        const uint4 (&xv)[NCH], int d8, int lane, float* out) {
  for (int r = r0; r < r1; r += 2) {
    const int rb = min(r + 1, r1 - 1);
    uint4 wa[NCH], wb[NCH];
    load_row<NCH>(w + (int64_t)r * d, d8, lane, wa);
    load_row<NCH>(w + (int64_t)rb * d, d8, lane, wb);
    const float a = wave_sum(dot_bb<NCH>(wa, xv));
    const float b = wave_sum(dot_bb<NCH>(wb, xv));
    if (lane == 0) {
      out[r] = a;
      if (rb != r) out[rb] = b;
    }
  }
}

template <int NCH>
__device__ __forceinline__ void dense_x_body(const DenseXArgs& a) {
  const int lane = threadIdx.x & (kWave - 1);
  if (a.route) {
    // the router logits come from the previous launch; this workgroup's selection runs
    // while the others stream the latent and shared weights
    if (blockIdx.x == 0) {
      route_block(a.ra, 0, a.T, true);
      return;
    }
  }
  const int64_t gw = global_wave() - (a.route ? kWavesPerBlock : 0);
  const int per_tok = a.waves_r + a.waves_dn + a.waves_sh;
  const int64_t t = gw / per_tok;
  if (t >= a.T) return;
  int w = (int)(gw - t * per_tok);
  const int d8 = a.d >> 3;
  const uint4* xr = reinterpret_cast<const uint4*>(a.x + t * (int64_t)a.d);
  uint4 xv[NCH];
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int c = j * kWave + lane;
    xv[j] = (c < d8) ? xr[c] : make_uint4(0u, 0u, 0u, 0u);
  }
  if (w < a.waves_r) {
    const int r0 = w * a.rows_per_wave, r1 = min(a.E, r0 + a.rows_per_wave);
    rows_x2<NCH>(a.wr, a.d, r0, r1, xv, d8, lane, a.z + t * a.E);
    return;
  }
  w -= a.waves_r;
  if (w < a.waves_dn) {
    const int r0 = w * a.rows_per_wave, r1 = min(a.l, r0 + a.rows_per_wave);
    rows_x2<NCH>(a.wdn, a.d, r0, r1, xv, d8, lane, a.xc + t * a.l);
    return;
  }
  w -= a.waves_dn;
  const int r0 = w * a.pairs_per_wave, r1 = min(a.ms, r0 + a.pairs_per_wave);
  for (int r = r0; r < r1; ++r) {
    uint4 wg[NCH], wu[NCH];
    load_row<NCH>(a.sgu + (int64_t)r * a.d, d8, lane, wg);
    load_row<NCH>(a.sgu + (int64_t)(a.ms + r) * a.d, d8, lane, wu);
    const float g = wave_sum(dot_bb<NCH>(wg, xv));
    const float u = wave_sum(dot_bb<NCH>(wu, xv));
    if (lane == 0) a.hs[t * a.ms + r] = glu_act(g, u, a.act, a.bg, a.bl);
  }
}

// Two entry points over the same body so that profilers tell the launches apart.
template <int NCH>
__global__ __launch_bounds__(kBlock) void k_router(DenseXArgs a) { dense_x_body<NCH>(a); }
template <int NCH>
__global__ __launch_bounds__(kBlock) void k_dense_x(DenseXArgs a) { dense_x_body<NCH>(a); }

// ------------------------------------------------------------------------------------
// Step DISPATCH for larger batches: deterministic counting sort by expert.
//   count:   per-chunk histograms (integer LDS atomics: exact counts)
//   scan:    per-expert prefix over chunks, then the exclusive scan over experts
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

__global__ __launch_bounds__(1024) void k_disp_scan(int n_chunks, int E, int32_t* chunk_hist,
                                                    int32_t* counts, int32_t* offs) {
  __shared__ int sc[1024];
  const int e = threadIdx.x;
  int tot = 0;
  if (e < E) {
    for (int c = 0; c < n_chunks; ++c) {
      const int v = chunk_hist[(int64_t)c * E + e];
      chunk_hist[(int64_t)c * E + e] = tot;
      tot += v;
    }
    counts[e] = tot;
  }
  sc[e] = (e < E) ? tot : 0;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int v = (e >= o) ? sc[e - o] : 0;
    __syncthreads();
    sc[e] += v;
    __syncthreads();
  }
  if (e < E) offs[e] = sc[e] - tot;
  if (e == 0) offs[E] = sc[1023];
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
// Routed experts.  A workgroup serves one dispatch position p and a run of row groups;
// its input row (x^c of the assignment's token for gate/up, h of position p for down)
// is staged once in LDS.
// ------------------------------------------------------------------------------------
struct ExpArgs {
  const uint8_t* experts;
  size_t expert_bytes, region_off;
  const int32_t* idx;
  const int32_t* perm;
  int64_t n_assign;
  int k;
  const float* xin;
  int kin;           // input row length
  int in_by_token;   // 1: input row = token of the assignment; 0: input row = position
  float* out;
  int n_out;         // output row length
  int n_units;       // row groups (MXFP4) or rows / row pairs (bf16)
  int units_per_wave;
  int wgs_per_pos;   // workgroups per position (MXFP4) / waves per position (bf16)
  int m;             // gate rows of the bf16 gate/up matrix
  int act;
  float bg, bl;
};

// MXFP4 row groups: 4 rows, J steps of (64 lanes x 16 code bytes + 16 x 4 scale bytes).
template <int J>
__device__ __forceinline__ void load_fp4_group(const uint8_t* gp, int lane, uint4 (&cw)[J],
                                               uint32_t (&sw)[J]) {
#pragma unroll
  for (int j = 0; j < J; ++j) {
    cw[j] = ld_stream(gp + j * kFp4StepBytes + lane * 16);
    sw[j] = ld_stream32(gp + j * kFp4StepBytes + 1024 + (lane >> 2) * 4);
  }
}

template <int J>
__device__ __forceinline__ void fma_fp4_step(uint4 cw, uint32_t sw, float4 xa, float4 xb,
                                             float (&acc)[4]) {
  const uint32_t cq[4] = {cw.x, cw.y, cw.z, cw.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float sc = e8m0_as_f32((sw >> (8 * q)) & 0xFFu);
    const float2_t v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cq[q], sc, 0);
    const float2_t v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cq[q], sc, 1);
    const float2_t v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cq[q], sc, 2);
    const float2_t v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cq[q], sc, 3);
    float s = acc[q];
    s = fmaf(v0.x, xa.x, s);
    s = fmaf(v0.y, xa.y, s);
    s = fmaf(v1.x, xa.z, s);
    s = fmaf(v1.y, xa.w, s);
    s = fmaf(v2.x, xb.x, s);
    s = fmaf(v2.y, xb.y, s);
    s = fmaf(v3.x, xb.z, s);
    s = fmaf(v3.y, xb.w, s);
    acc[q] = s;
  }
}

template <int J, bool GU>
__global__ __launch_bounds__(kBlock) void k_expert_fp4(ExpArgs a) {
  __shared__ float4 xp0[J * kWave], xp1[J * kWave];
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x >> 6;
  const int64_t pos = blockIdx.x / a.wgs_per_pos;
  if (pos >= a.n_assign) return;
  const int wg = (int)(blockIdx.x - pos * a.wgs_per_pos);
  const int asg = a.perm[pos];
  const int e = a.idx[asg];
  const int64_t xrow = a.in_by_token ? (int64_t)(asg / a.k) : pos;
  const uint8_t* base = a.experts + (size_t)e * a.expert_bytes + a.region_off;
  const int g0 = (wg * kWavesPerBlock + wv) * a.units_per_wave;
  const int g1 = min(a.n_units, g0 + a.units_per_wave);
  float* orow = a.out + pos * a.n_out;
  stage_x(a.xin + xrow * a.kin, a.kin >> 3, J * kWave, xp0, xp1);
  __syncthreads();
  for (int g = g0; g < g1; ++g) {
    // keep the LDS reads inside the loop (see k_out)
    asm volatile("" ::: "memory");
    uint4 cw[J];
    uint32_t sw[J];
    load_fp4_group<J>(base + (size_t)g * J * kFp4StepBytes, lane, cw, sw);
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < J; ++j)
      fma_fp4_step<J>(cw[j], sw[j], xp0[j * kWave + lane], xp1[j * kWave + lane], acc);
    float r[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) r[q] = wave_sum(acc[q]);
    if (lane == 0) {
      if (GU) {
        // row group g: gate rows 2g, 2g+1 and up rows 2g, 2g+1
        orow[2 * g] = glu_act(r[0], r[2], a.act, a.bg, a.bl);
        orow[2 * g + 1] = glu_act(r[1], r[3], a.act, a.bg, a.bl);
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) orow[4 * g + q] = r[q];
      }
    }
  }
}

// bf16 experts in canonical row order: gate/up [2m][kin] (unit = row pair i, m+i) and
// down [n_out][kin] (unit = row); the input row stays in registers.
template <int NCH, bool GU>
__global__ __launch_bounds__(kBlock) void k_expert_bf16(ExpArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t gw = global_wave();
  const int64_t pos = gw / a.wgs_per_pos;
  if (pos >= a.n_assign) return;
  const int chunk = (int)(gw - pos * a.wgs_per_pos);
  const int asg = a.perm[pos];
  const int e = a.idx[asg];
  const int64_t xrow = a.in_by_token ? (int64_t)(asg / a.k) : pos;
  const int k8 = a.kin >> 3;
  float xs[NCH][8];
  load_x_f32<NCH>(a.xin + xrow * a.kin, k8, lane, xs);
  const uint16_t* base =
      reinterpret_cast<const uint16_t*>(a.experts + (size_t)e * a.expert_bytes + a.region_off);
  const int u0 = chunk * a.units_per_wave, u1 = min(a.n_units, u0 + a.units_per_wave);
  float* orow = a.out + pos * a.n_out;
  for (int r = u0; r < u1; ++r) {
    if (GU) {
      uint4 wg[NCH], wu[NCH];
      load_row<NCH>(base + (int64_t)r * a.kin, k8, lane, wg);
      load_row<NCH>(base + (int64_t)(a.m + r) * a.kin, k8, lane, wu);
      const float g = wave_sum(dot_bf<NCH>(wg, xs));
      const float u = wave_sum(dot_bf<NCH>(wu, xs));
      if (lane == 0) orow[r] = glu_act(g, u, a.act, a.bg, a.bl);
    } else {
      uint4 wr[NCH];
      load_row<NCH>(base + (int64_t)r * a.kin, k8, lane, wr);
      const float v = wave_sum(dot_bf<NCH>(wr, xs));
      if (lane == 0) orow[r] = v;
    }
  }
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
// Step OUT: Delta[t, r] = [W_up_latent[r] | W_shared_down[r]] . [u_hat_t ; h_s,t], with
// u_hat = u / sqrt(mean(u^2) + eps) * gamma computed once per workgroup.  The activation
// row [u_hat ; h_s] (l + m_s fp32) sits in LDS in the two-plane layout.
// ------------------------------------------------------------------------------------
struct OutArgs {
  const uint16_t* wup;   // [d][l]
  const uint16_t* sdn;   // [d][ms] (ms may be 0)
  const uint16_t* gamma;
  int d, l, ms;
  int norm;
  float eps;
  const float* u;        // [T][l]
  const float* hs;       // [T][ms]
  int64_t T;
  float* delta;          // [T][d]
  int rows_per_wave;
  int wgs_per_tok;
};

// Row r of [W_up_latent | W_shared_down]: chunk c < l/8 from W_up_latent, then W_shared_down.
template <int NCH>
__device__ __forceinline__ void load_cat_row(const OutArgs& a, int r, int l8, int k8, int lane,
                                             uint4 (&w)[NCH]) {
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int c = j * kWave + lane;
    if (c < l8) w[j] = ld_stream(a.wup + (int64_t)r * a.l + 8 * c);
    else if (c < k8) w[j] = ld_stream(a.sdn + (int64_t)r * a.ms + 8 * (c - l8));
    else w[j] = make_uint4(0u, 0u, 0u, 0u);
  }
}

template <int NCH>
__global__ __launch_bounds__(kBlock) void k_out(OutArgs a) {
  __shared__ float4 xp0[NCH * kWave], xp1[NCH * kWave];
  __shared__ float red[kWavesPerBlock];
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x >> 6;
  const int64_t t = blockIdx.x / a.wgs_per_tok;
  if (t >= a.T) return;
  const int wg = (int)(blockIdx.x - t * a.wgs_per_tok);
  const int l8 = a.l >> 3, s8 = a.ms >> 3, k8 = l8 + s8;
  const int r0 = (wg * kWavesPerBlock + wv) * a.rows_per_wave;
  const int r1 = min(a.d, r0 + a.rows_per_wave);
  // stage u (then scale it) and h_s
  stage_x(a.u + t * a.l, l8, l8, xp0, xp1);
  if (s8 > 0) stage_x(a.hs + t * a.ms, s8, NCH * kWave - l8, xp0 + l8, xp1 + l8);
  else
    for (int c = l8 + threadIdx.x; c < NCH * kWave; c += kBlock) {
      xp0[c] = make_float4(0.f, 0.f, 0.f, 0.f);
      xp1[c] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
  __syncthreads();
  if (a.norm) {
    float ss = 0.f;
    for (int c = threadIdx.x; c < l8; c += kBlock) {
      const float4 p = xp0[c], q = xp1[c];
      ss = fmaf(p.x, p.x, ss); ss = fmaf(p.y, p.y, ss); ss = fmaf(p.z, p.z, ss); ss = fmaf(p.w, p.w, ss);
      ss = fmaf(q.x, q.x, ss); ss = fmaf(q.y, q.y, ss); ss = fmaf(q.z, q.z, ss); ss = fmaf(q.w, q.w, ss);
    }
    ss = wave_sum(ss);
    if (lane == 0) red[wv] = ss;
    __syncthreads();
    const float tot = (red[0] + red[1]) + (red[2] + red[3]);
    const float inv = 1.0f / sqrtf(tot / (float)a.l + a.eps);
    const uint4* g4 = reinterpret_cast<const uint4*>(a.gamma);
    for (int c = threadIdx.x; c < l8; c += kBlock) {
      const uint4 g = g4[c];
      float4 p = xp0[c], q = xp1[c];
      p.x = p.x * inv * bf16_lo(g.x); p.y = p.y * inv * bf16_hi(g.x);
      p.z = p.z * inv * bf16_lo(g.y); p.w = p.w * inv * bf16_hi(g.y);
      q.x = q.x * inv * bf16_lo(g.z); q.y = q.y * inv * bf16_hi(g.z);
      q.z = q.z * inv * bf16_lo(g.w); q.w = q.w * inv * bf16_hi(g.w);
      xp0[c] = p;
      xp1[c] = q;
    }
    __syncthreads();
  }
  for (int r = r0; r < r1; ++r) {
    // keep the LDS reads inside the loop: hoisting them would hold the whole row of
    // activations in registers and drop the occupancy to one wavefront per SIMD
    asm volatile("" ::: "memory");
    uint4 wa[NCH];
    load_cat_row<NCH>(a, r, l8, k8, lane, wa);
    float sa = 0.f;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const float4 p = xp0[j * kWave + lane], q = xp1[j * kWave + lane];
      const float xv[8] = {p.x, p.y, p.z, p.w, q.x, q.y, q.z, q.w};
      const uint32_t ua[4] = {wa[j].x, wa[j].y, wa[j].z, wa[j].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sa = fmaf(bf16_lo(ua[i]), xv[2 * i], sa);
        sa = fmaf(bf16_hi(ua[i]), xv[2 * i + 1], sa);
      }
    }
    sa = wave_sum(sa);
    if (lane == 0) a.delta[t * a.d + r] = sa;
  }
}

// ------------------------------------------------------------------------------------
// Expert packing (MXFP4): one thread per (expert, row group, step, lane) writes the
// lane's 16 code bytes (four rows' 8-column chunk) and, for lanes 0..15, the four rows'
// scale bytes of 32-column block step*16 + lane.
// ------------------------------------------------------------------------------------
struct PackArgs {
  const uint8_t* codes;   // [n][rows][cols/2]
  const uint8_t* scales;  // [n][rows][cols/32]
  int rows, cols, J, gu, m, n, n_rg;
  uint8_t* dst;           // first packed expert of the run
  size_t expert_bytes, region_off;
};

__global__ __launch_bounds__(kBlock) void k_pack_fp4(PackArgs a) {
  const int64_t gid = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  const int64_t total = (int64_t)a.n * a.n_rg * a.J * kWave;
  if (gid >= total) return;
  const int lane = (int)(gid % kWave);
  const int j = (int)((gid / kWave) % a.J);
  const int g = (int)((gid / ((int64_t)kWave * a.J)) % a.n_rg);
  const int64_t ei = gid / ((int64_t)kWave * a.J * a.n_rg);
  const int c = j * kWave + lane;
  const int c8 = a.cols >> 3, nb = a.cols >> 5;
  uint32_t wd[4], sd = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int R = a.gu ? (q < 2 ? 2 * g + q : a.m + 2 * g + (q - 2)) : 4 * g + q;
    const uint8_t* crow = a.codes + (ei * a.rows + R) * (int64_t)(a.cols / 2);
    wd[q] = (c < c8) ? *reinterpret_cast<const uint32_t*>(crow + 4 * c) : 0u;
    if (lane < 16) {
      const int blk = j * 16 + lane;
      const uint32_t sb = (blk < nb) ? a.scales[(ei * a.rows + R) * (int64_t)nb + blk] : 127u;
      sd |= sb << (8 * q);
    }
  }
  uint8_t* gp = a.dst + ei * (int64_t)a.expert_bytes + a.region_off +
                ((int64_t)g * a.J + j) * kFp4StepBytes;
  *reinterpret_cast<uint4*>(gp + lane * 16) = make_uint4(wd[0], wd[1], wd[2], wd[3]);
  if (lane < 16) *reinterpret_cast<uint32_t*>(gp + 1024 + lane * 4) = sd;
}

inline unsigned blocks_for_waves(int64_t waves) {
  return (unsigned)((waves + kWavesPerBlock - 1) / kWavesPerBlock);
}

inline int cdiv(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

}  // namespace

// Template dispatch over the chunks per lane (1..N): widths up to N * 512 columns.
#define MOE_SWITCH16(N, BODY)                                                            \
  do {                                                                                   \
    switch (N) {                                                                         \
      case 1: { constexpr int NC = 1; BODY; } break;                                     \
      case 2: { constexpr int NC = 2; BODY; } break;                                     \
      case 3: { constexpr int NC = 3; BODY; } break;                                     \
      case 4: { constexpr int NC = 4; BODY; } break;                                     \
      case 5: { constexpr int NC = 5; BODY; } break;                                     \
      case 6: { constexpr int NC = 6; BODY; } break;                                     \
      case 7: { constexpr int NC = 7; BODY; } break;                                     \
      case 8: { constexpr int NC = 8; BODY; } break;                                     \
      case 9: { constexpr int NC = 9; BODY; } break;                                     \
      case 10: { constexpr int NC = 10; BODY; } break;                                   \
      case 11: { constexpr int NC = 11; BODY; } break;                                   \
      case 12: { constexpr int NC = 12; BODY; } break;                                   \
      case 13: { constexpr int NC = 13; BODY; } break;                                   \
      case 14: { constexpr int NC = 14; BODY; } break;                                   \
      case 15: { constexpr int NC = 15; BODY; } break;                                   \
      case 16: { constexpr int NC = 16; BODY; } break;                                   \
      default: return hipErrorInvalidValue;                                              \
    }                                                                                    \
  } while (0)

#define MOE_SWITCH32(N, BODY)                                                          \
  do {                                                                                 \
    switch (N) {                                                                       \
      case 1: { constexpr int NC = 1; BODY; } break;                                   \
      case 2: { constexpr int NC = 2; BODY; } break;                                   \
      case 3: { constexpr int NC = 3; BODY; } break;                                   \
      case 4: { constexpr int NC = 4; BODY; } break;                                   \
      case 5: { constexpr int NC = 5; BODY; } break;                                   \
      case 6: { constexpr int NC = 6; BODY; } break;                                   \
      case 7: { constexpr int NC = 7; BODY; } break;                                   \
      case 8: { constexpr int NC = 8; BODY; } break;                                   \
      case 9: { constexpr int NC = 9; BODY; } break;                                   \
      case 10: { constexpr int NC = 10; BODY; } break;                                 \
      case 11: { constexpr int NC = 11; BODY; } break;                                 \
      case 12: { constexpr int NC = 12; BODY; } break;                                 \
      case 13: { constexpr int NC = 13; BODY; } break;                                 \
      case 14: { constexpr int NC = 14; BODY; } break;                                 \
      case 15: { constexpr int NC = 15; BODY; } break;                                 \
      case 16: { constexpr int NC = 16; BODY; } break;                                 \
      case 17: { constexpr int NC = 17; BODY; } break;                                 \
      case 18: { constexpr int NC = 18; BODY; } break;                                 \
      case 19: { constexpr int NC = 19; BODY; } break;                                 \
      case 20: { constexpr int NC = 20; BODY; } break;                                 \
      case 21: { constexpr int NC = 21; BODY; } break;                                 \
      case 22: { constexpr int NC = 22; BODY; } break;                                 \
      case 23: { constexpr int NC = 23; BODY; } break;                                 \
      case 24: { constexpr int NC = 24; BODY; } break;                                 \
      case 25: { constexpr int NC = 25; BODY; } break;                                 \
      case 26: { constexpr int NC = 26; BODY; } break;                                 \
      case 27: { constexpr int NC = 27; BODY; } break;                                 \
      case 28: { constexpr int NC = 28; BODY; } break;                                 \
      case 29: { constexpr int NC = 29; BODY; } break;                                 \
      case 30: { constexpr int NC = 30; BODY; } break;                                 \
      case 31: { constexpr int NC = 31; BODY; } break;                                 \
      case 32: { constexpr int NC = 32; BODY; } break;                                 \
      default: return hipErrorInvalidValue;                                            \
    }                                                                                  \
  } while (0)

static inline int chunks_per_lane(int k) { return cdiv(k / 8, kWave); }

bool route_fused(int64_t T, int k) { return T * k <= kBlock && T <= 4; }

namespace {

DenseXArgs dense_x_args(const Shape& s, const DenseW& w, const uint16_t* x, int64_t T,
                        const Work& ws) {
  DenseXArgs a;
  a.x = x; a.T = T; a.d = s.d;
  a.wr = w.router; a.E = s.E; a.z = ws.z;
  a.wdn = w.wdn; a.l = s.l; a.xc = ws.xc;
  a.sgu = w.sgu; a.ms = s.ms; a.hs = ws.hs;
  a.act = s.act; a.bg = s.beta_gate; a.bl = s.beta_lin;
  a.rows_per_wave = 4;
  a.pairs_per_wave = 2;
  a.waves_r = a.waves_dn = a.waves_sh = 0;
  a.route = 0;
  return a;
}

RouteArgs route_args(const Shape& s, const float* bias, int64_t T, const Work& ws, int32_t* idx,
                     float* gw) {
  return RouteArgs{ws.z, bias, T, s.E, s.k, s.route_scale, idx, gw, ws.counts, ws.offs,
                   ws.perm, ws.inv};
}

}  // namespace

hipError_t launch_router(const Shape& s, const DenseW& w, const uint16_t* x, int64_t T,
                         const Work& ws, hipStream_t st) {
  DenseXArgs a = dense_x_args(s, w, x, T, ws);
  a.rows_per_wave = 2;   // a small matrix: spread it over more wavefronts
  a.waves_r = cdiv(s.E, a.rows_per_wave);
  const int64_t waves = T * a.waves_r;
  MOE_SWITCH16(chunks_per_lane(s.d),
               hipLaunchKernelGGL(k_router<NC>, dim3(blocks_for_waves(waves)), dim3(kBlock), 0,
                                  st, a));
  return hipGetLastError();
}

hipError_t launch_dense_x(const Shape& s, const DenseW& w, const uint16_t* x, int64_t T,
                          const float* bias, int32_t* idx, float* gw, const Work& ws,
                          hipStream_t st) {
  DenseXArgs a = dense_x_args(s, w, x, T, ws);
  a.waves_dn = cdiv(s.l, a.rows_per_wave);
  a.waves_sh = (s.ms == 0) ? 0 : cdiv(s.ms, a.pairs_per_wave);
  a.route = route_fused(T, s.k) ? 1 : 0;
  a.ra = route_args(s, bias, T, ws, idx, gw);
  const int64_t waves = T * (a.waves_dn + a.waves_sh) + (a.route ? kWavesPerBlock : 0);
  MOE_SWITCH16(chunks_per_lane(s.d),
               hipLaunchKernelGGL(k_dense_x<NC>, dim3(blocks_for_waves(waves)), dim3(kBlock), 0,
                                  st, a));
  return hipGetLastError();
}

hipError_t launch_route(const Shape& s, const float* bias, int64_t T, const Work& ws,
                        int32_t* idx, float* gw, hipStream_t st) {
  RouteArgs a = route_args(s, bias, T, ws, idx, gw);
  hipLaunchKernelGGL(k_route, dim3((unsigned)T), dim3(kBlock), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_dispatch(const Shape& s, const int32_t* idx, int64_t T, int32_t* counts,
                           int32_t* offs, int32_t* perm, int32_t* inv, int32_t* chunk_hist,
                           hipStream_t st) {
  const int ct = dispatch_chunk_tokens(s.k);
  const int chunk = ct * s.k;
  const int64_t n = T * s.k;
  const int nch = cdiv(T, ct);
  hipLaunchKernelGGL(k_disp_count, dim3(nch), dim3(kBlock), 0, st, idx, n, s.E, chunk, chunk_hist);
  hipLaunchKernelGGL(k_disp_scan, dim3(1), dim3(1024), 0, st, nch, s.E, chunk_hist, counts, offs);
  hipLaunchKernelGGL(k_disp_scatter, dim3(nch), dim3(kBlock), 0, st, idx, n, s.E, chunk,
                     (const int32_t*)chunk_hist, (const int32_t*)offs, perm, inv);
  return hipGetLastError();
}

namespace {

ExpArgs expert_args(const Shape& s, const DenseW& w, const int32_t* idx, int64_t T,
                    const Work& ws) {
  ExpArgs a;
  a.experts = w.experts;
  a.expert_bytes = s.expert_bytes;
  a.idx = idx;
  a.perm = ws.perm;
  a.n_assign = T * s.k;
  a.k = s.k;
  a.m = s.m;
  a.act = s.act;
  a.bg = s.beta_gate;
  a.bl = s.beta_lin;
  return a;
}

hipError_t launch_fp4(ExpArgs a, int J, bool gu, hipStream_t st) {
  a.units_per_wave = 2;
  a.wgs_per_pos = cdiv(a.n_units, (int64_t)a.units_per_wave * kWavesPerBlock);
  const unsigned blocks = (unsigned)(a.n_assign * a.wgs_per_pos);
  if (gu) {
    MOE_SWITCH16(J, hipLaunchKernelGGL((k_expert_fp4<NC, true>), dim3(blocks), dim3(kBlock), 0, st, a));
  } else {
    MOE_SWITCH16(J, hipLaunchKernelGGL((k_expert_fp4<NC, false>), dim3(blocks), dim3(kBlock), 0, st, a));
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_expert_gu(const Shape& s, const DenseW& w, const int32_t* idx, int64_t T,
                            const Work& ws, hipStream_t st) {
  // x^c of the assignment's token -> h[p], p in dispatch order
  ExpArgs a = expert_args(s, w, idx, T, ws);
  a.region_off = 0;
  a.xin = ws.xc; a.kin = s.l; a.in_by_token = 1;
  a.out = ws.h; a.n_out = s.m;
  if (s.wfmt == 1) {
    a.n_units = s.m / 2;
    return launch_fp4(a, s.j_gu, true, st);
  }
  a.n_units = s.m;
  a.units_per_wave = 4;
  a.wgs_per_pos = cdiv(a.n_units, a.units_per_wave);
  const int64_t waves = a.n_assign * a.wgs_per_pos;
  MOE_SWITCH16(chunks_per_lane(s.l),
               hipLaunchKernelGGL((k_expert_bf16<NC, true>), dim3(blocks_for_waves(waves)),
                                  dim3(kBlock), 0, st, a));
  return hipGetLastError();
}

hipError_t launch_expert_down(const Shape& s, const DenseW& w, const int32_t* idx, int64_t T,
                              const Work& ws, hipStream_t st) {
  // h[p] -> E[p]
  ExpArgs a = expert_args(s, w, idx, T, ws);
  a.region_off = s.gu_bytes;
  a.xin = ws.h; a.kin = s.m; a.in_by_token = 0;
  a.out = ws.eo; a.n_out = s.l;
  if (s.wfmt == 1) {
    a.n_units = s.l / 4;
    return launch_fp4(a, s.j_dn, false, st);
  }
  a.n_units = s.l;
  a.units_per_wave = 8;
  a.wgs_per_pos = cdiv(a.n_units, a.units_per_wave);
  const int64_t waves = a.n_assign * a.wgs_per_pos;
  MOE_SWITCH16(chunks_per_lane(s.m),
               hipLaunchKernelGGL((k_expert_bf16<NC, false>), dim3(blocks_for_waves(waves)),
                                  dim3(kBlock), 0, st, a));
  return hipGetLastError();
}

hipError_t launch_combine(const Shape& s, const float* gw, int64_t T, const Work& ws,
                          hipStream_t st) {
  const int bpt = cdiv(s.l, kBlock);
  hipLaunchKernelGGL(k_combine, dim3((unsigned)(T * bpt)), dim3(kBlock), 0, st, gw,
                     (const int32_t*)ws.inv, (const float*)ws.eo, T, s.k, s.l, bpt, ws.u);
  return hipGetLastError();
}

hipError_t launch_out(const Shape& s, const DenseW& w, int64_t T, const Work& ws, float* delta,
                      hipStream_t st) {
  OutArgs a;
  a.wup = w.wup; a.sdn = w.sdn; a.gamma = w.gamma;
  a.d = s.d; a.l = s.l; a.ms = s.ms;
  a.norm = s.use_norm; a.eps = s.eps;
  a.u = ws.u; a.hs = ws.hs; a.T = T; a.delta = delta;
  a.rows_per_wave = 4;
  a.wgs_per_tok = cdiv(s.d, (int64_t)a.rows_per_wave * kWavesPerBlock);
  const unsigned blocks = (unsigned)(T * a.wgs_per_tok);
  MOE_SWITCH32(cdiv((s.l + s.ms) / 8, kWave),
               hipLaunchKernelGGL(k_out<NC>, dim3(blocks), dim3(kBlock), 0, st, a));
  return hipGetLastError();
}

hipError_t launch_pack(const Shape& s, const void* gu, const void* gus, const void* dn,
                       const void* dns, int e0, int n, uint8_t* packed, hipStream_t st) {
  uint8_t* dst = packed + (size_t)e0 * s.expert_bytes;
  if (s.wfmt == 0) {
    const size_t gub = (size_t)2 * s.m * s.l * 2, dnb = (size_t)s.l * s.m * 2;
    hipError_t err = hipMemcpy2DAsync(dst, s.expert_bytes, gu, gub, gub, n, hipMemcpyDeviceToDevice, st);
    if (err != hipSuccess) return err;
    return hipMemcpy2DAsync(dst + s.gu_bytes, s.expert_bytes, dn, dnb, dnb, n,
                            hipMemcpyDeviceToDevice, st);
  }
  PackArgs a;
  a.m = s.m; a.n = n; a.dst = dst; a.expert_bytes = s.expert_bytes;
  // gate/up: [2m][l], row groups of (gate 2g, 2g+1, up 2g, 2g+1)
  a.codes = static_cast<const uint8_t*>(gu); a.scales = static_cast<const uint8_t*>(gus);
  a.rows = 2 * s.m; a.cols = s.l; a.J = s.j_gu; a.gu = 1; a.n_rg = s.m / 2; a.region_off = 0;
  int64_t threads = (int64_t)n * a.n_rg * a.J * kWave;
  hipLaunchKernelGGL(k_pack_fp4, dim3((unsigned)cdiv(threads, kBlock)), dim3(kBlock), 0, st, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  // down: [l][m], row groups of 4 consecutive rows
  a.codes = static_cast<const uint8_t*>(dn); a.scales = static_cast<const uint8_t*>(dns);
  a.rows = s.l; a.cols = s.m; a.J = s.j_dn; a.gu = 0; a.n_rg = s.l / 4; a.region_off = s.gu_bytes;
  threads = (int64_t)n * a.n_rg * a.J * kWave;
  hipLaunchKernelGGL(k_pack_fp4, dim3((unsigned)cdiv(threads, kBlock)), dim3(kBlock), 0, st, a);
  return hipGetLastError();
}

}  // namespace moe
