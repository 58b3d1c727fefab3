// gfx950 kernels of the Stable LatentMoE FFN layer forward.
//
// Step order follows the Kimi K3 latent mixture-of-experts block card ("All 23 steps"
// and its KimiSparseMoeBlock.forward / moe_infer excerpt):
//   k_dense_x      router logits z = x W_r, x^c = x W_down_latent and the shared gate/up
//                  with its SiTU epilogue - every product that reads the bf16 tokens
//   k_topk         s = sigmoid(z), top_k of s + b, G = s / sum(s)  (one wavefront a token)
//   k_disp_*       per-expert histogram -> scan -> stable permutation (moe_infer's
//                  scatter_/argsort, kept on the device: no host round trip)
//   k_expert_*     routed gate/up (+ SiTU) and down, MXFP4 or bf16 weights
//   k_combine      u = sum_j G_j E_j in a fixed order (no atomics)
//   k_gemv_f32x    shared down, then RMSNorm + W_up_latent + y_shared  -> Delta
//
// All of these are weight-streaming matrix-vector products: each wavefront keeps one
// token's activation slice in registers and streams weight rows through 16-byte
// coalesced loads (64 lanes x 16 B = 1 KiB per load instruction), so the decode path is
// bound by HBM bandwidth.  Activations stay fp32 end to end.
#include <climits>
#include <cmath>

#include "moe_device.hpp"
#include "moe_internal.hpp"

namespace moe {
namespace {

constexpr int kBlock = 256;             // 4 wavefronts per workgroup
constexpr int kWavesPerBlock = kBlock / kWave;

__device__ __forceinline__ int64_t global_wave() {
  return (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
}

// ------------------------------------------------------------------------------------
// Dot products of one weight row with the register-resident activation slice.  Lane l
// covers 8-column chunks l, l+64, l+128, ...; the per-lane sum runs in chunk order and
// the wave_sum butterfly finishes it, so the order is fixed.
// ------------------------------------------------------------------------------------

// bf16 weights x bf16 activations (packed pairs), fp32 accumulation.
template <int NCH>
__device__ __forceinline__ float dot_bf16w_bf16x(const uint16_t* row, const uint4 (&xv)[NCH],
                                                 int k8, int lane) {
  const uint4* r = reinterpret_cast<const uint4*>(row);
  uint4 wv[NCH];
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int c = j * kWave + lane;
    wv[j] = (c < k8) ? r[c] : make_uint4(0u, 0u, 0u, 0u);
  }
  float acc = 0.f;
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    acc = dot2_bf16(wv[j].x, xv[j].x, acc);
    acc = dot2_bf16(wv[j].y, xv[j].y, acc);
    acc = dot2_bf16(wv[j].z, xv[j].z, acc);
    acc = dot2_bf16(wv[j].w, xv[j].w, acc);
  }
  return wave_sum(acc);
}

// bf16 weights x fp32 activations.
template <int NCH>
__device__ __forceinline__ float dot_bf16w_f32x(const uint16_t* row, const float (&xs)[NCH][8],
                                                int k8, int lane) {
  const uint4* r = reinterpret_cast<const uint4*>(row);
  uint4 wv[NCH];
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int c = j * kWave + lane;
    wv[j] = (c < k8) ? r[c] : make_uint4(0u, 0u, 0u, 0u);
  }
  float acc = 0.f;
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const uint32_t q[4] = {wv[j].x, wv[j].y, wv[j].z, wv[j].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc = fmaf(bf16_lo(q[i]), xs[j][2 * i], acc);
      acc = fmaf(bf16_hi(q[i]), xs[j][2 * i + 1], acc);
    }
  }
  return wave_sum(acc);
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

// ------------------------------------------------------------------------------------
// Phase A: router logits, latent down-projection, shared gate/up + activation.
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
  int rows_per_wave;     // router / latent rows per wavefront
  int pairs_per_wave;    // shared gate/up row pairs per wavefront
  int waves_r, waves_dn, waves_sh;  // per token
};

template <int NCH>
__global__ __launch_bounds__(kBlock) void k_dense_x(DenseXArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t gw = global_wave();
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
    for (int r = r0; r < r1; ++r) {
      const float v = dot_bf16w_bf16x<NCH>(a.wr + (int64_t)r * a.d, xv, d8, lane);
      if (lane == 0) a.z[t * a.E + r] = v;
    }
    return;
  }
  w -= a.waves_r;
  if (w < a.waves_dn) {
    const int r0 = w * a.rows_per_wave, r1 = min(a.l, r0 + a.rows_per_wave);
    for (int r = r0; r < r1; ++r) {
      const float v = dot_bf16w_bf16x<NCH>(a.wdn + (int64_t)r * a.d, xv, d8, lane);
      if (lane == 0) a.xc[t * a.l + r] = v;
    }
    return;
  }
  w -= a.waves_dn;
  const int r0 = w * a.pairs_per_wave, r1 = min(a.ms, r0 + a.pairs_per_wave);
  for (int r = r0; r < r1; ++r) {
    const float g = dot_bf16w_bf16x<NCH>(a.sgu + (int64_t)r * a.d, xv, d8, lane);
    const float u = dot_bf16w_bf16x<NCH>(a.sgu + (int64_t)(a.ms + r) * a.d, xv, d8, lane);
    if (lane == 0) a.hs[t * a.ms + r] = glu_act(g, u, a.act, a.bg, a.bl);
  }
}

// ------------------------------------------------------------------------------------
// Router selection: one wavefront per token.  kappa = sigmoid(z) + b in fp32; k rounds of
// a wavefront arg-max over (kappa desc, expert index asc); G = route_scale * s / sum(s)
// with the sum taken in selection order.
// ------------------------------------------------------------------------------------
struct TopkArgs {
  const float* z;
  const float* bias;
  int64_t T;
  int E, k;
  float route_scale;
  int32_t* idx;
  float* gw;
};

constexpr int kTopkSlots = 16;  // experts per lane: E <= 1024

__global__ __launch_bounds__(kBlock) void k_topk(TopkArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t t = global_wave();
  if (t >= a.T) return;
  float key[kTopkSlots], sv[kTopkSlots];
  uint32_t taken = 0;
  const float* zr = a.z + t * a.E;
#pragma unroll
  for (int i = 0; i < kTopkSlots; ++i) {
    const int e = i * kWave + lane;
    if (e < a.E) {
      const float s = sigmoidf_(zr[e]);
      const float kk = s + a.bias[e];
      sv[i] = s;
      key[i] = (kk != kk) ? -INFINITY : kk;
    } else {
      sv[i] = 0.f;
      key[i] = -INFINITY;
      taken |= 1u << i;
    }
  }
  float my_s = 0.f;
  for (int j = 0; j < a.k; ++j) {
    float bk = -INFINITY, bs = 0.f;
    int be = INT_MAX;
#pragma unroll
    for (int i = 0; i < kTopkSlots; ++i) {
      const int e = i * kWave + lane;
      const bool free_ = !((taken >> i) & 1u);
      if (free_ && (key[i] > bk || (key[i] == bk && e < be))) {
        bk = key[i];
        be = e;
        bs = sv[i];
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float ok = __shfl_xor(bk, o, kWave);
      const int oe = __shfl_xor(be, o, kWave);
      const float os = __shfl_xor(bs, o, kWave);
      if (ok > bk || (ok == bk && oe < be)) {
        bk = ok;
        be = oe;
        bs = os;
      }
    }
    if ((be & (kWave - 1)) == lane) taken |= 1u << (be >> 6);
    if (lane == j) my_s = bs;
    if (lane == 0) a.idx[t * a.k + j] = be;
  }
  float tot = 0.f;
  for (int j = 0; j < a.k; ++j) tot += __shfl(my_s, j, kWave);
  if (lane < a.k) a.gw[t * a.k + lane] = (my_s / tot) * a.route_scale;
}

// ------------------------------------------------------------------------------------
// Dispatch: deterministic counting sort of the T*k assignments by expert.
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
  for (int64_t a = a0 + threadIdx.x; a < a1; a += kBlock) atomicAdd(&hist[idx[a]], 1);
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
// Routed experts.  Work item = (dispatch position p, run of row groups).  The input row
// is x^c of the assignment's token (gate/up) or h of position p (down).
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
  int waves_per_pos;
  int m;             // gate rows of the bf16 gate/up matrix
  int act;
  float bg, bl;
};

// MXFP4, 4 rows per row group, J steps of 64 lanes x 8 columns.
template <int J, bool GU>
__global__ __launch_bounds__(kBlock) void k_expert_fp4(ExpArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t gw = global_wave();
  const int64_t pos = gw / a.waves_per_pos;
  if (pos >= a.n_assign) return;
  const int chunk = (int)(gw - pos * a.waves_per_pos);
  const int asg = a.perm[pos];
  const int e = a.idx[asg];
  const int64_t xrow = a.in_by_token ? (int64_t)(asg / a.k) : pos;
  float xs[J][8];
  load_x_f32<J>(a.xin + xrow * a.kin, a.kin >> 3, lane, xs);
  const uint8_t* base = a.experts + (size_t)e * a.expert_bytes + a.region_off;
  const int g0 = chunk * a.units_per_wave, g1 = min(a.n_units, g0 + a.units_per_wave);
  float* orow = a.out + pos * a.n_out;
  for (int g = g0; g < g1; ++g) {
    const uint8_t* gp = base + (size_t)g * J * kFp4StepBytes;
    uint4 cw[J];
    uint32_t sw[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
      cw[j] = *reinterpret_cast<const uint4*>(gp + j * kFp4StepBytes + lane * 16);
      sw[j] = *reinterpret_cast<const uint32_t*>(gp + j * kFp4StepBytes + 1024 + (lane >> 2) * 4);
    }
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const uint32_t cq[4] = {cw[j].x, cw[j].y, cw[j].z, cw[j].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float sc = e8m0_as_f32((sw[j] >> (8 * q)) & 0xFFu);
        const float2_t v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cq[q], sc, 0);
        const float2_t v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cq[q], sc, 1);
        const float2_t v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cq[q], sc, 2);
        const float2_t v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cq[q], sc, 3);
        float s = acc[q];
        s = fmaf(v0.x, xs[j][0], s);
        s = fmaf(v0.y, xs[j][1], s);
        s = fmaf(v1.x, xs[j][2], s);
        s = fmaf(v1.y, xs[j][3], s);
        s = fmaf(v2.x, xs[j][4], s);
        s = fmaf(v2.y, xs[j][5], s);
        s = fmaf(v3.x, xs[j][6], s);
        s = fmaf(v3.y, xs[j][7], s);
        acc[q] = s;
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[q] = wave_sum(acc[q]);
    if (lane == 0) {
      if (GU) {
        // row group g = gate rows 2g, 2g+1 and up rows 2g, 2g+1
        orow[2 * g] = glu_act(acc[0], acc[2], a.act, a.bg, a.bl);
        orow[2 * g + 1] = glu_act(acc[1], acc[3], a.act, a.bg, a.bl);
      } else {
        orow[4 * g + 0] = acc[0];
        orow[4 * g + 1] = acc[1];
        orow[4 * g + 2] = acc[2];
        orow[4 * g + 3] = acc[3];
      }
    }
  }
}

// bf16 experts in canonical row order: gate/up [2m][kin] (unit = row pair i, m+i) and
// down [n_out][kin] (unit = row).
template <int NCH, bool GU>
__global__ __launch_bounds__(kBlock) void k_expert_bf16(ExpArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t gw = global_wave();
  const int64_t pos = gw / a.waves_per_pos;
  if (pos >= a.n_assign) return;
  const int chunk = (int)(gw - pos * a.waves_per_pos);
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
      const float g = dot_bf16w_f32x<NCH>(base + (int64_t)r * a.kin, xs, k8, lane);
      const float u = dot_bf16w_f32x<NCH>(base + (int64_t)(a.m + r) * a.kin, xs, k8, lane);
      if (lane == 0) orow[r] = glu_act(g, u, a.act, a.bg, a.bl);
    } else {
      const float v = dot_bf16w_f32x<NCH>(base + (int64_t)r * a.kin, xs, k8, lane);
      if (lane == 0) orow[r] = v;
    }
  }
}

// ------------------------------------------------------------------------------------
// Gated combine in the latent: u[t] = sum_j G[t,j] E[inv[t,j]], j = 0..k-1 in order.
// ------------------------------------------------------------------------------------
__global__ __launch_bounds__(kBlock) void k_combine(const float* gw, const int32_t* inv,
                                                    const float* eo, int64_t T, int k, int l,
                                                    int blocks_per_tok, float* u) {
  const int64_t t = blockIdx.x / blocks_per_tok;
  const int r = (int)(blockIdx.x - t * blocks_per_tok) * kBlock + threadIdx.x;
  if (t >= T || r >= l) return;
  float acc = 0.f;
  for (int j = 0; j < k; ++j)
    acc = fmaf(gw[t * k + j], eo[(int64_t)inv[t * k + j] * l + r], acc);
  u[t * l + r] = acc;
}

// ------------------------------------------------------------------------------------
// out[t, r] = W[r] . xhat_t (+ add[t, r]), bf16 W [n_rows][kin], fp32 x; xhat is x or,
// with norm = 1, x / sqrt(mean(x^2) + eps) * gamma (the latent RMSNorm, computed by
// every wavefront from the whole row, identically).
// ------------------------------------------------------------------------------------
struct GemvArgs {
  const uint16_t* w;
  int n_rows;
  int kin;
  const float* xin;
  int64_t T;
  float* out;
  const float* add;
  const uint16_t* gamma;
  int norm;
  float eps;
  int rows_per_wave;
  int waves_per_tok;
};

template <int NCH>
__global__ __launch_bounds__(kBlock) void k_gemv_f32x(GemvArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t gw = global_wave();
  const int64_t t = gw / a.waves_per_tok;
  if (t >= a.T) return;
  const int w = (int)(gw - t * a.waves_per_tok);
  const int k8 = a.kin >> 3;
  float xs[NCH][8];
  load_x_f32<NCH>(a.xin + t * a.kin, k8, lane, xs);
  if (a.norm) {
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < NCH; ++j)
#pragma unroll
      for (int i = 0; i < 8; ++i) ss = fmaf(xs[j][i], xs[j][i], ss);
    ss = wave_sum(ss);
    const float inv = 1.0f / sqrtf(ss / (float)a.kin + a.eps);
    const uint4* gp = reinterpret_cast<const uint4*>(a.gamma);
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int c = j * kWave + lane;
      if (c < k8) {
        const uint4 g = gp[c];
        const uint32_t q[4] = {g.x, g.y, g.z, g.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          xs[j][2 * i] = xs[j][2 * i] * inv * bf16_lo(q[i]);
          xs[j][2 * i + 1] = xs[j][2 * i + 1] * inv * bf16_hi(q[i]);
        }
      }
    }
  }
  const int r0 = w * a.rows_per_wave, r1 = min(a.n_rows, r0 + a.rows_per_wave);
  for (int r = r0; r < r1; ++r) {
    float v = dot_bf16w_f32x<NCH>(a.w + (int64_t)r * a.kin, xs, k8, lane);
    if (lane == 0) {
      if (a.add) v += a.add[t * a.n_rows + r];
      a.out[t * a.n_rows + r] = v;
    }
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

// Chunk counts of 1..16 per lane cover widths up to 8192.
#define MOE_SWITCH16(N, BODY)                                                   \
  switch (N) {                                                                  \
    case 1: { constexpr int NC = 1; BODY; } break;                              \
    case 2: { constexpr int NC = 2; BODY; } break;                              \
    case 3: { constexpr int NC = 3; BODY; } break;                              \
    case 4: { constexpr int NC = 4; BODY; } break;                              \
    case 5: { constexpr int NC = 5; BODY; } break;                              \
    case 6: { constexpr int NC = 6; BODY; } break;                              \
    case 7: { constexpr int NC = 7; BODY; } break;                              \
    case 8: { constexpr int NC = 8; BODY; } break;                              \
    case 9: { constexpr int NC = 9; BODY; } break;                              \
    case 10: { constexpr int NC = 10; BODY; } break;                            \
    case 11: { constexpr int NC = 11; BODY; } break;                            \
    case 12: { constexpr int NC = 12; BODY; } break;                            \
    case 13: { constexpr int NC = 13; BODY; } break;                            \
    case 14: { constexpr int NC = 14; BODY; } break;                            \
    case 15: { constexpr int NC = 15; BODY; } break;                            \
    case 16: { constexpr int NC = 16; BODY; } break;                            \
    default: return hipErrorInvalidValue;                                       \
  }

static inline int chunks_per_lane(int k) { return cdiv(k / 8, kWave); }

hipError_t launch_dense_x(const Shape& s, const DenseW& w, const uint16_t* x, int64_t T,
                          bool router_only, const Work& ws, hipStream_t st) {
  DenseXArgs a;
  a.x = x; a.T = T; a.d = s.d;
  a.wr = w.router; a.E = s.E; a.z = ws.z;
  a.wdn = w.wdn; a.l = s.l; a.xc = ws.xc;
  a.sgu = w.sgu; a.ms = s.ms; a.hs = ws.hs;
  a.act = s.act; a.bg = s.beta_gate; a.bl = s.beta_lin;
  a.rows_per_wave = 8;
  a.pairs_per_wave = 4;
  a.waves_r = cdiv(s.E, a.rows_per_wave);
  a.waves_dn = router_only ? 0 : cdiv(s.l, a.rows_per_wave);
  a.waves_sh = (router_only || s.ms == 0) ? 0 : cdiv(s.ms, a.pairs_per_wave);
  const int64_t waves = T * (a.waves_r + a.waves_dn + a.waves_sh);
  MOE_SWITCH16(chunks_per_lane(s.d),
               hipLaunchKernelGGL(k_dense_x<NC>, dim3(blocks_for_waves(waves)), dim3(kBlock), 0,
                                  st, a));
  return hipGetLastError();
}

hipError_t launch_topk(const Shape& s, const float* bias, int64_t T, const Work& ws,
                       int32_t* idx, float* gw, hipStream_t st) {
  TopkArgs a{ws.z, bias, T, s.E, s.k, s.route_scale, idx, gw};
  hipLaunchKernelGGL(k_topk, dim3(blocks_for_waves(T)), dim3(kBlock), 0, st, a);
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
    a.units_per_wave = 8;
    a.waves_per_pos = cdiv(a.n_units, a.units_per_wave);
    const int64_t waves = a.n_assign * a.waves_per_pos;
    MOE_SWITCH16(s.j_gu, hipLaunchKernelGGL((k_expert_fp4<NC, true>),
                                            dim3(blocks_for_waves(waves)), dim3(kBlock), 0, st, a));
  } else {
    a.n_units = s.m;
    a.units_per_wave = 4;
    a.waves_per_pos = cdiv(a.n_units, a.units_per_wave);
    const int64_t waves = a.n_assign * a.waves_per_pos;
    MOE_SWITCH16(chunks_per_lane(s.l),
                 hipLaunchKernelGGL((k_expert_bf16<NC, true>), dim3(blocks_for_waves(waves)),
                                    dim3(kBlock), 0, st, a));
  }
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
    a.units_per_wave = 8;
    a.waves_per_pos = cdiv(a.n_units, a.units_per_wave);
    const int64_t waves = a.n_assign * a.waves_per_pos;
    MOE_SWITCH16(s.j_dn, hipLaunchKernelGGL((k_expert_fp4<NC, false>),
                                            dim3(blocks_for_waves(waves)), dim3(kBlock), 0, st, a));
  } else {
    a.n_units = s.l;
    a.units_per_wave = 8;
    a.waves_per_pos = cdiv(a.n_units, a.units_per_wave);
    const int64_t waves = a.n_assign * a.waves_per_pos;
    MOE_SWITCH16(chunks_per_lane(s.m),
                 hipLaunchKernelGGL((k_expert_bf16<NC, false>), dim3(blocks_for_waves(waves)),
                                    dim3(kBlock), 0, st, a));
  }
  return hipGetLastError();
}

hipError_t launch_combine(const Shape& s, const float* gw, int64_t T, const Work& ws,
                          hipStream_t st) {
  const int bpt = cdiv(s.l, kBlock);
  hipLaunchKernelGGL(k_combine, dim3((unsigned)(T * bpt)), dim3(kBlock), 0, st, gw,
                     (const int32_t*)ws.inv, (const float*)ws.eo, T, s.k, s.l, bpt, ws.u);
  return hipGetLastError();
}

hipError_t launch_shared_down(const Shape& s, const DenseW& w, int64_t T, const Work& ws,
                              float* delta, hipStream_t st) {
  // y_shared = W_sd h_s, written into delta (the up step adds y_routed in place)
  if (s.ms == 0) return hipSuccess;
  GemvArgs a;
  a.T = T;
  a.eps = s.eps;
  a.w = w.sdn; a.n_rows = s.d; a.kin = s.ms; a.xin = ws.hs; a.out = delta; a.add = nullptr;
  a.gamma = nullptr; a.norm = 0; a.rows_per_wave = 4;
  a.waves_per_tok = cdiv(s.d, a.rows_per_wave);
  MOE_SWITCH16(chunks_per_lane(s.ms),
               hipLaunchKernelGGL(k_gemv_f32x<NC>, dim3(blocks_for_waves(T * a.waves_per_tok)),
                                  dim3(kBlock), 0, st, a));
  return hipGetLastError();
}

hipError_t launch_up(const Shape& s, const DenseW& w, int64_t T, const Work& ws, float* delta,
                     hipStream_t st) {
  // delta = W_up RMSNorm(u) (+ y_shared already in delta)
  GemvArgs a;
  a.T = T;
  a.eps = s.eps;
  a.w = w.wup; a.n_rows = s.d; a.kin = s.l; a.xin = ws.u; a.out = delta;
  a.add = (s.ms > 0) ? delta : nullptr;
  a.gamma = w.gamma; a.norm = s.use_norm; a.rows_per_wave = 8;
  a.waves_per_tok = cdiv(s.d, a.rows_per_wave);
  MOE_SWITCH16(chunks_per_lane(s.l),
               hipLaunchKernelGGL(k_gemv_f32x<NC>, dim3(blocks_for_waves(T * a.waves_per_tok)),
                                  dim3(kBlock), 0, st, a));
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
