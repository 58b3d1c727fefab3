// gfx950 kernels of the compute-bound forward (the "mx8" precision profile).
//
// The same steps as the weight-streaming launches, in the order of the Kimi K3 latent
// mixture-of-experts block card, with the rounding points of the profile:
//   k_pf_in      z = x W_r, x^c = x W_down_latent, h_s = SiTU(x W_sg, x W_su) -> bf16,
//                one product over the packed IN matrix (bf16 MFMA)
//   k_pf_quant   x^c -> MXFP8-E4M3 (the experts' input)
//   (route and dispatch: the launches of the token-tiled path)
//   k_pf_exp     routed gate/up with SiTU and the MXFP8 conversion of h fused in its
//                epilogue, then routed down: FP8 activations x MXFP4 weights on the scaled
//                16x16x128 MFMA (v_mfma_scale_f32_16x16x128_f8f6f4), the E8M0 scales of both
//                operands applied by the matrix core
//   (combine and the RMSNorm, u_hat rounded to bf16)
//   k_pf_out     Delta = u_hat W_up_latent + h_s W_shared_down, one product over the packed
//                OUT matrix (bf16 MFMA)
//
// Tiling: a workgroup multiplies a tile of 16 NB activation rows (NB <= 4) with 4 x NT
// tile rows of weights (NT per wavefront).  K advances one K-step (128 columns) at a
// time: the activation rows of the next K-steps travel global -> registers -> LDS (two
// LDS buffers, one barrier per K-step) while every wavefront streams its own weight
// K-steps into registers, two K-steps ahead.  Each activation fragment read from LDS
// feeds NT MFMAs and each weight fragment NB MFMAs.
#include <climits>
#include <cmath>
#include <type_traits>

#include "moe_device.hpp"
#include "moe_internal.hpp"

namespace moe {
namespace {

typedef int i32x8_t __attribute__((ext_vector_type(8)));

constexpr int kPfRows = 64;      // activation rows per tile (NB = 4 blocks of 16)
constexpr int kPfNT = 4;         // weight tile rows per wavefront
constexpr int kPfWaves = kBlock / kWave;

// D += A B^T on one 16x16 block over 128 K: A = 16 rows of FP8-E4M3 (32 bytes per lane,
// lane l: row l % 16, K 16 (l/16) .. +16 in bytes 0..15 and K 64 + 16 (l/16) .. +16 in
// bytes 16..31), B = 16 rows of FP4-E2M1 (16 bytes per lane: row l % 16, K 32 (l/16) ..
// +32, low nibble first); sa / sb: the E8M0 scale of lane l's row over K block l / 16
// (K 32 (l/16) .. +32) of A and of B.
__device__ __forceinline__ f32x4_t mfma_fp8_fp4(uint4 alo, uint4 ahi, uint4 b, uint32_t sa,
                                                uint32_t sb, f32x4_t acc) {
  const i32x8_t av = {(int)alo.x, (int)alo.y, (int)alo.z, (int)alo.w,
                      (int)ahi.x, (int)ahi.y, (int)ahi.z, (int)ahi.w};
  const i32x8_t bv = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc, 0 /*A: E4M3*/, 4 /*B: E2M1*/,
                                                          0, (int)sa, 0, (int)sb);
}

// An fp32 value (already divided by its block scale, |y| < 512) to E4M3: the nearest value,
// ties to even, saturated at 448 (the conversion itself turns values past 464 into NaN).
__device__ __forceinline__ uint32_t to_e4m3(float y) {
  y = fminf(fmaxf(y, -448.f), 448.f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y, 0.f, 0, false) & 0xFFu;
}

// E8M0 byte of an MX block from its largest magnitude: 2^X with X = floor(log2 amax) - 8
// (8: the largest E4M3 exponent), the byte X + 127, clamped at 0 (amax of 0 or below 2^-119).
__device__ __forceinline__ uint32_t mx8_scale_byte(float amax) {
  const uint32_t ef = (__float_as_uint(amax) >> 23) & 0xFFu;
  return ef > 8u ? ef - 8u : 0u;
}
// 2^-X for the scale byte (X = byte - 127): an fp32 with exponent field 254 - byte.
__device__ __forceinline__ float mx8_inv_scale(uint32_t sbyte) { return __uint_as_float((254u - sbyte) << 23); }

// ------------------------------------------------------------------------------------
// The activation side of a tile.
//   AF 0: bf16 rows, 16 pieces of 16 bytes per K-step; columns [0, n0) from segment 0
//         (row r at word o0[r]), [c1, c1 + n1) from segment 1 (word o1[r]), zero elsewhere.
//   AF 1: MXFP8 rows padded to whole K-steps (128 code bytes and 4 scale bytes per
//         K-step): 8 pieces per K-step at word o0[r] + 8 q, the scale word at s0[r] + q.
// Rows r >= R are zero.  Thread piece i is idx = threadIdx + 256 i: row idx / PR, piece
// idx % PR, so that consecutive threads read consecutive bytes of a row.  Every load is
// issued (invalid pieces read word 0 of segment 0 and are zeroed when committed).  LDS
// word of (piece j, row r): j * RB + (r ^ j), conflict-free for the writes of a row's
// pieces and for the MFMA reads (16 lanes, one piece, 16 consecutive rows).
// ------------------------------------------------------------------------------------
struct PfRows {
  uint32_t o0[kPfRows];
  uint32_t o1[kPfRows];
  uint32_t s0[kPfRows];
};
struct PfSrc {
  const uint4* b0;
  const uint4* b1;
  const uint32_t* sc;    // AF 1: scale words
  int R, n0, c1, n1;
};

template <int AF, int NB>
struct PfStage {
  static constexpr int PR = AF ? 8 : 16;
  static constexpr int RB = 16 * NB;
  static constexpr int NP = (RB * PR + kBlock - 1) / kBlock;
  uint4 v[2][NP];
  uint32_t sv[2];
  uint32_t o0[NP], o1[NP];
  bool rv[NP];
  uint32_t so;
  bool srv;
  __device__ __forceinline__ int row_of(int i) const { return (threadIdx.x + i * kBlock) / PR; }
  __device__ __forceinline__ int piece_of(int i) const { return (threadIdx.x + i * kBlock) % PR; }
  __device__ __forceinline__ void init(const PfRows& rows, const PfSrc& src) {
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int r = row_of(i);
      rv[i] = r < RB && r < src.R;
      o0[i] = rv[i] ? rows.o0[r] : 0u;
      o1[i] = rv[i] && !AF && src.n1 > 0 ? rows.o1[r] : 0u;
    }
    srv = AF && (int)threadIdx.x < src.R && (int)threadIdx.x < RB;
    so = srv ? rows.s0[threadIdx.x] : 0u;
  }
  __device__ __forceinline__ bool in0(int i, const PfSrc& src, int q) const {
    return rv[i] && (AF || q * kStepK + 8 * piece_of(i) < src.n0);
  }
  __device__ __forceinline__ bool in1(int i, const PfSrc& src, int q) const {
    const int col = q * kStepK + 8 * piece_of(i);
    return !AF && rv[i] && col >= src.c1 && col < src.c1 + src.n1;
  }
  template <int SLOT>
  __device__ __forceinline__ void load(const PfSrc& src, int q) {
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      uint32_t w = 0u;
      const uint4* base = src.b0;
      if (AF) {
        w = rv[i] ? o0[i] + 8u * q + piece_of(i) : 0u;
      } else {
        const int col = q * kStepK + 8 * piece_of(i);
        const bool a0 = in0(i, src, q), a1 = in1(i, src, q);
        w = a0 ? o0[i] + (col >> 3) : a1 ? o1[i] + ((col - src.c1) >> 3) : 0u;
        base = a1 ? src.b1 : src.b0;
      }
      v[SLOT][i] = base[w];
    }
    if (AF) sv[SLOT] = src.sc[srv ? so + q : 0u];
  }
  template <int SLOT>
  __device__ __forceinline__ void commit(uint4* buf, uint32_t* sbuf, const PfSrc& src, int q) const {
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int idx = threadIdx.x + i * kBlock;
      if (idx < RB * PR) {
        const int r = idx / PR, j = idx % PR;
        const bool z = !(in0(i, src, q) || in1(i, src, q));
        const uint4 x = v[SLOT][i];
        buf[j * RB + (r ^ j)] = make_uint4(z ? 0u : x.x, z ? 0u : x.y, z ? 0u : x.z, z ? 0u : x.w);
      }
    }
    if (AF && (int)threadIdx.x < RB) sbuf[threadIdx.x] = srv ? sv[SLOT] : 0u;
  }
};

// The K loop of a tile: acc[t][b] = D of activation block b x the wavefront's tile row t
// (trow[t]; waves or tile rows without work pass tile row 0 of the same matrix and drop
// the result).  AF 0 pairs with bf16 weights (WF 0), AF 1 with MXFP4 weights (WF 1).
template <int AF, int NB, int NT>
__device__ __forceinline__ void pf_run(const PfRows& rows, const PfSrc& src,
                                       const uint8_t* const (&trow)[NT], int ks, uint4* lds,
                                       uint32_t* slds, f32x4_t (&acc)[NT][NB]) {
  constexpr int WF = AF;
  constexpr int RB = 16 * NB;
  constexpr int PR = PfStage<AF, NB>::PR;
  const int lane = threadIdx.x & (kWave - 1);
  const int c = lane & 15, g = lane >> 4;
  WeightStep<WF> w[2][NT];
  PfStage<AF, NB> st;
  st.init(rows, src);
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    w[0][t].load(trow[t], 0, lane);
    w[1][t].load(trow[t], min(1, ks - 1), lane);
  }
  st.template load<0>(src, 0);
  st.template load<1>(src, min(1, ks - 1));
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[t][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  asm volatile("" ::: "memory");
  st.template commit<0>(lds, slds, src, 0);
  __syncthreads();
  // one K-step with the weights of slot SLOT and LDS buffer q & 1
  auto step = [&](auto slot_c, int q) {
    constexpr int SLOT = decltype(slot_c)::value;
    st.template load<SLOT>(src, min(q + 2, ks - 1));
    const uint4* buf = lds + (q & 1) * RB * PR;
    if (AF) {
      const uint32_t* sb = slds + (q & 1) * RB;
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int r = 16 * b + c;
        const uint4 alo = buf[g * RB + (r ^ g)];
        const uint4 ahi = buf[(4 + g) * RB + (r ^ (4 + g))];
        const uint32_t sa = (sb[r] >> (8 * g)) & 0xFFu;
#pragma unroll
        for (int t = 0; t < NT; ++t)
          acc[t][b] = mfma_fp8_fp4(alo, ahi, w[SLOT][t].w[0], sa, (w[SLOT][t].sc >> (8 * g)) & 0xFFu,
                                   acc[t][b]);
      }
    } else {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int j = 4 * s + g;
        uint4 af[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) af[b] = buf[j * RB + ((16 * b + c) ^ j)];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const uint4 bw = w[SLOT][t].operand(s, 0.f);
#pragma unroll
          for (int b = 0; b < NB; ++b) acc[t][b] = mfma_bf16(af[b], bw, acc[t][b]);
        }
      }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) w[SLOT][t].load(trow[t], min(q + 2, ks - 1), lane);
    asm volatile("" ::: "memory");
    st.template commit<SLOT ^ 1>(lds + ((q + 1) & 1) * RB * PR, slds + ((q + 1) & 1) * RB, src,
                                 min(q + 1, ks - 1));
    __syncthreads();
  };
  for (int q = 0; q < ks; q += 2) {
    step(std::integral_constant<int, 0>{}, q);
    if (q + 1 < ks) step(std::integral_constant<int, 1>{}, q + 1);
  }
}

// ------------------------------------------------------------------------------------
// Dense products for a tile of up to 64 tokens: k_pf_in over the IN matrix (router
// logits -> z, W_down_latent -> x^c fp32, shared gate/up -> SiTU -> h_s bf16), k_pf_out
// over the OUT matrix (-> Delta).  Work item (tile-row group, token tile); the tiles of
// one group run back to back on one XCD so that the group's weights come from its L2.
// ------------------------------------------------------------------------------------
struct PfDenseArgs {
  const uint8_t* w;
  int ks, tr_count, n_grp, n_tiles;
  const uint16_t* a0;    // segment 0 rows (x, or u_hat bf16)
  int lda0, n0;
  const uint16_t* a1;    // segment 1 rows (h_s bf16) from column c1
  int lda1, c1, n1;
  int64_t T;
  // IN epilogue
  int tr_r, tr_dn;
  float* z;
  int E;
  float* xc;
  int l;
  uint16_t* hs;
  int ms, act;
  float bg, bl;
  // OUT epilogue
  float* delta;
  int d;
};

template <bool IN>
__global__ __launch_bounds__(kBlock) void k_pf_dense(PfDenseArgs a) {
  extern __shared__ uint4 sm[];
  __shared__ PfRows rows;
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15, g = lane >> 4;
  int grp, tile;
  if (!xcd_item(blockIdx.x, a.n_grp, a.n_tiles, grp, tile)) return;
  const int64_t t0 = (int64_t)tile * kPfRows;
  const int nt = (int)min((int64_t)kPfRows, a.T - t0);
  if ((int)threadIdx.x < nt) {
    rows.o0[threadIdx.x] = (uint32_t)((t0 + threadIdx.x) * a.lda0 / 8);
    rows.o1[threadIdx.x] = (uint32_t)((t0 + threadIdx.x) * a.lda1 / 8);
  }
  __syncthreads();
  const uint8_t* trow[kPfNT];
  int tr[kPfNT];
#pragma unroll
  for (int t = 0; t < kPfNT; ++t) {
    tr[t] = (grp * kPfWaves + wv) * kPfNT + t;
    trow[t] = a.w + (size_t)(tr[t] < a.tr_count ? tr[t] : 0) * a.ks * kBf16StepBytes;
  }
  f32x4_t acc[kPfNT][4];
  pf_run<0, 4, kPfNT>(rows, PfSrc{reinterpret_cast<const uint4*>(a.a0), reinterpret_cast<const uint4*>(a.a1),
                                  nullptr, nt, a.n0, a.c1, a.n1},
                      trow, a.ks, sm, nullptr, acc);
#pragma unroll
  for (int t = 0; t < kPfNT; ++t) {
    if (tr[t] >= a.tr_count) continue;
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int ti = 16 * b + 4 * g + v;
        const int64_t tok = t0 + ti;
        const float y = acc[t][b][v];
        if (!IN) {
          const int r = 16 * tr[t] + c;
          if (ti < nt && r < a.d) a.delta[tok * a.d + r] = y;
        } else if (tr[t] < a.tr_r) {
          const int e = 16 * tr[t] + c;
          if (ti < nt && e < a.E) a.z[tok * a.E + e] = y;
        } else if (tr[t] < a.tr_r + a.tr_dn) {
          const int r = 16 * (tr[t] - a.tr_r) + c;
          if (ti < nt && r < a.l) a.xc[tok * a.l + r] = y;
        } else {
          const int r = 8 * (tr[t] - a.tr_r - a.tr_dn) + (c - 8);
          const float gate = from_gate_lane(y);
          if (c >= 8 && ti < nt && r < a.ms) {
            const float h = glu_act(gate, y, a.act, a.bg, a.bl);
            a.hs[tok * a.ms + r] = (uint16_t)(pack_bf16x2(h, 0.f) & 0xFFFFu);
          }
        }
      }
  }
}

// x^c fp32 [T][l] -> MXFP8 rows of ks K-steps: codes [T][128 ks], scales [T][4 ks] (blocks
// past l are zero).  One thread per (token, block of 32).
__global__ __launch_bounds__(kBlock) void k_pf_quant(const float* __restrict__ xc, int64_t T, int l,
                                                     int ks, uint8_t* __restrict__ codes,
                                                     uint8_t* __restrict__ scales) {
  const int64_t gid = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  const int nbk = 4 * ks;
  if (gid >= T * nbk) return;
  const int64_t t = gid / nbk;
  const int blk = (int)(gid - t * nbk);
  uint4* dst = reinterpret_cast<uint4*>(codes + t * 128 * ks + 32 * blk);
  if (32 * blk >= l) {
    dst[0] = make_uint4(0u, 0u, 0u, 0u);
    dst[1] = make_uint4(0u, 0u, 0u, 0u);
    scales[t * nbk + blk] = 0;
    return;
  }
  const float4* src = reinterpret_cast<const float4*>(xc + t * l + 32 * blk);
  float v[32];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float4 p = src[i];
    v[4 * i] = p.x; v[4 * i + 1] = p.y; v[4 * i + 2] = p.z; v[4 * i + 3] = p.w;
  }
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const uint32_t sb = mx8_scale_byte(amax);
  const float inv = mx8_inv_scale(sb);
  uint32_t wd[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    wd[i] = to_e4m3(v[4 * i] * inv) | (to_e4m3(v[4 * i + 1] * inv) << 8) |
            (to_e4m3(v[4 * i + 2] * inv) << 16) | (to_e4m3(v[4 * i + 3] * inv) << 24);
  dst[0] = make_uint4(wd[0], wd[1], wd[2], wd[3]);
  dst[1] = make_uint4(wd[4], wd[5], wd[6], wd[7]);
  scales[t * nbk + blk] = (uint8_t)sb;
}

// ------------------------------------------------------------------------------------
// Routed experts, FP8 x MXFP4.  Work item (tile-row group, unit); a unit is a run of at
// most 64 dispatch positions of one expert.  Gate/up: input rows x^c_q of the positions'
// tokens; each wavefront's 4 tile rows (8 gate + 8 up rows each) give one MX block of 32
// columns of h = SiTU(gate, up), converted to MXFP8 in the epilogue.  Down: input rows
// h_q of the positions, output E fp32.
// ------------------------------------------------------------------------------------
struct PfExpArgs {
  const uint8_t* experts;
  size_t expert_bytes, region_off;
  int ks, n_tr, n_grp;
  const int32_t* units;
  const int32_t* ctrl;
  int max_units, nu, E, k;
  int64_t n_assign;
  const int32_t* perm;
  const uint8_t* xq;        // input codes, rows of 128 ks bytes
  const uint8_t* xs;        // input scales, rows of 4 ks bytes
  // gate/up output: h as MXFP8 rows of ks_out K-steps
  uint8_t* hq;
  uint8_t* hsc;
  int ks_out, m, act;
  float bg, bl;
  // down output
  float* out;
  int n_out;
};

template <bool GU, int NB>
__device__ __forceinline__ void pf_exp_unit(const PfExpArgs& a, const PfRows& rows, uint4* sm,
                                            uint32_t* ssm, const uint8_t* const (&trow)[kPfNT],
                                            const int (&tr)[kPfNT], int wblk, int p0, int n) {
  const int lane = threadIdx.x & (kWave - 1);
  const int c = lane & 15, g = lane >> 4;
  f32x4_t acc[kPfNT][NB];
  pf_run<1, NB, kPfNT>(rows, PfSrc{reinterpret_cast<const uint4*>(a.xq), nullptr,
                                   reinterpret_cast<const uint32_t*>(a.xs), n, 0, 0, 0},
                       trow, a.ks, sm, ssm, acc);
  if (!GU) {
#pragma unroll
    for (int t = 0; t < kPfNT; ++t) {
      const int r = 16 * tr[t] + c;
      if (tr[t] >= a.n_tr || r >= a.n_out) continue;
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int i = 16 * b + 4 * g + v;
          if (i < n) a.out[(int64_t)(p0 + i) * a.n_out + r] = acc[t][b][v];
        }
    }
    return;
  }
  // h block wblk (columns 32 wblk .. +32) of each position: lanes c >= 8 hold column
  // 32 wblk + 8 t + (c - 8) of tile row t
  const bool blk_live = 32 * wblk < a.m;
  const int nbk = 4 * a.ks_out;
  if (32 * wblk >= 128 * a.ks_out) return;
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int i = 16 * b + 4 * g + v;
      float h[kPfNT];
      float amax = 0.f;
#pragma unroll
      for (int t = 0; t < kPfNT; ++t) {
        const float y = acc[t][b][v];
        const float gate = from_gate_lane(y);
        const int col = 8 * tr[t] + (c - 8);
        h[t] = (blk_live && col < a.m) ? glu_act(gate, y, a.act, a.bg, a.bl) : 0.f;
        if (c < 8) h[t] = 0.f;
        amax = fmaxf(amax, fabsf(h[t]));
      }
      // the block's largest magnitude: lanes 8..15 of the 16-lane row (lanes 0..7 hold 0)
      amax = fmaxf(amax, __shfl_xor(amax, 1, kWave));
      amax = fmaxf(amax, __shfl_xor(amax, 2, kWave));
      amax = fmaxf(amax, __shfl_xor(amax, 4, kWave));
      amax = fmaxf(amax, __shfl_xor(amax, 8, kWave));
      const uint32_t sb = mx8_scale_byte(amax);
      const float inv = mx8_inv_scale(sb);
      if (i < n) {
        const int64_t p = p0 + i;
        if (c >= 8) {
#pragma unroll
          for (int t = 0; t < kPfNT; ++t)
            a.hq[p * 128 * a.ks_out + 32 * wblk + 8 * t + (c - 8)] = (uint8_t)to_e4m3(h[t] * inv);
        }
        if (c == 8) a.hsc[p * nbk + wblk] = (uint8_t)sb;
      }
    }
}

template <bool GU>
__global__ __launch_bounds__(kBlock) void k_pf_exp(PfExpArgs a) {
  extern __shared__ uint4 sm[];
  __shared__ PfRows rows;
  __shared__ uint32_t ssm[2 * kPfRows];
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n_units = min(a.ctrl[0], a.max_units);
  int grp, u;
  if (!xcd_item(blockIdx.x, a.n_grp, a.max_units, grp, u) || u >= n_units) return;
  const int4 un = *reinterpret_cast<const int4*>(a.units + 4 * u);
  const int e = un.x, p0 = un.y, n = un.z;
  if (e < 0 || e >= a.E || n < 1 || n > a.nu || n > kPfRows || p0 < 0 || p0 + n > a.n_assign) return;
  if ((int)threadIdx.x < n) {
    const int p = p0 + threadIdx.x;
    int64_t src = p;
    if (GU) {
      const int asg = a.perm[p];
      src = (asg >= 0 && asg < a.n_assign) ? asg / a.k : 0;
    }
    rows.o0[threadIdx.x] = (uint32_t)(src * 8 * a.ks);     // 16-byte words (128 ks bytes per row)
    rows.s0[threadIdx.x] = (uint32_t)(src * a.ks);         // scale words (4 ks bytes per row)
  }
  __syncthreads();
  const int wblk = grp * kPfWaves + wv;    // this wavefront's tile rows 4 wblk .. 4 wblk + 3
  const uint8_t* base = a.experts + (size_t)e * a.expert_bytes + a.region_off;
  const uint8_t* trow[kPfNT];
  int tr[kPfNT];
#pragma unroll
  for (int t = 0; t < kPfNT; ++t) {
    tr[t] = wblk * kPfNT + t;
    trow[t] = base + (size_t)(tr[t] < a.n_tr ? tr[t] : 0) * a.ks * kFp4StepBytes;
  }
  if (n <= 16) pf_exp_unit<GU, 1>(a, rows, sm, ssm, trow, tr, wblk, p0, n);
  else if (n <= 32) pf_exp_unit<GU, 2>(a, rows, sm, ssm, trow, tr, wblk, p0, n);
  else if (n <= 48) pf_exp_unit<GU, 3>(a, rows, sm, ssm, trow, tr, wblk, p0, n);
  else pf_exp_unit<GU, 4>(a, rows, sm, ssm, trow, tr, wblk, p0, n);
}

// u_hat = RMSNorm(u) * gamma rounded to bf16 (the OUT product's input), one workgroup per
// token, in the fixed reduction order of the other paths.
__global__ __launch_bounds__(kBlock) void k_pf_norm(const float* __restrict__ u,
                                                    const uint16_t* __restrict__ gamma, int l,
                                                    int norm, float eps, uint16_t* __restrict__ uh) {
  __shared__ float red[kPfWaves];
  const int64_t t = blockIdx.x;
  const float* ur = u + t * l;
  float inv = 1.f;
  if (norm) {
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
    inv = 1.0f / sqrtf(tot / (float)l + eps);
  }
  for (int col = threadIdx.x; col < l; col += kBlock) {
    const float gm = norm ? __uint_as_float((uint32_t)gamma[col] << 16) : 1.f;
    const float v = norm ? ur[col] * inv * gm : ur[col];
    uh[t * l + col] = (uint16_t)(pack_bf16x2(v, 0.f) & 0xFFFFu);
  }
}

constexpr size_t kPfDenseLds = (size_t)2 * kPfRows * 16 * 16;   // two K-steps of 64 bf16 rows
constexpr size_t kPfExpLds = (size_t)2 * kPfRows * 8 * 16;      // two K-steps of 64 FP8 rows

}  // namespace

hipError_t launch_pf_in(const Shape& s, const uint8_t* dense, const uint16_t* x, int64_t T,
                        const PfWork& pw, float* z, float* xc, hipStream_t st) {
  PfDenseArgs a{};
  a.w = dense;
  a.ks = s.ks_in;
  a.tr_count = s.tr_in;
  a.n_grp = cdiv(s.tr_in, kPfWaves * kPfNT);
  a.n_tiles = cdiv(T, kPfRows);
  a.a0 = x; a.lda0 = s.d; a.n0 = s.d;
  a.a1 = x; a.lda1 = 0; a.c1 = 0; a.n1 = 0;
  a.T = T;
  a.tr_r = s.tr_r; a.tr_dn = s.tr_dn;
  a.z = z; a.E = s.E;
  a.xc = xc; a.l = s.l;
  a.hs = pw.hs; a.ms = s.ms; a.act = s.act; a.bg = s.beta_gate; a.bl = s.beta_lin;
  hipLaunchKernelGGL(k_pf_dense<true>, dim3((unsigned)xcd_grid(a.n_grp, a.n_tiles)), dim3(kBlock),
                     kPfDenseLds, st, a);
  return hipGetLastError();
}

hipError_t launch_pf_quant(const Shape& s, const float* xc, int64_t T, const PfWork& pw,
                           hipStream_t st) {
  const int64_t n = T * 4 * s.ks_gu;
  hipLaunchKernelGGL(k_pf_quant, dim3((unsigned)cdiv(n, kBlock)), dim3(kBlock), 0, st, xc, T, s.l,
                     s.ks_gu, pw.xq, pw.xs);
  return hipGetLastError();
}

hipError_t launch_pf_expert(const Shape& s, const uint8_t* experts, bool gu, int64_t T,
                            const Work& ws, const PfWork& pw, hipStream_t st) {
  PfExpArgs a{};
  a.experts = experts;
  a.expert_bytes = s.expert_bytes;
  a.region_off = gu ? 0 : s.gu_bytes;
  a.ks = gu ? s.ks_gu : s.ks_edn;
  a.n_tr = gu ? s.tr_gu : s.tr_edn;
  a.n_grp = cdiv(a.n_tr, kPfWaves * kPfNT);
  a.units = ws.units;
  a.ctrl = ws.ctrl;
  a.nu = unit_positions(s, T);
  a.max_units = (int)max_units(s, T);
  a.E = s.E; a.k = s.k;
  a.n_assign = T * s.k;
  a.perm = ws.perm;
  a.xq = gu ? pw.xq : pw.hq;
  a.xs = gu ? pw.xs : pw.hsc;
  a.hq = pw.hq; a.hsc = pw.hsc;
  a.ks_out = s.ks_edn;
  a.m = s.m; a.act = s.act; a.bg = s.beta_gate; a.bl = s.beta_lin;
  a.out = ws.eo;
  a.n_out = s.l;
  const unsigned grid = (unsigned)xcd_grid(a.n_grp, a.max_units);
  if (gu) hipLaunchKernelGGL(k_pf_exp<true>, dim3(grid), dim3(kBlock), kPfExpLds, st, a);
  else hipLaunchKernelGGL(k_pf_exp<false>, dim3(grid), dim3(kBlock), kPfExpLds, st, a);
  return hipGetLastError();
}

hipError_t launch_pf_norm(const Shape& s, const uint8_t* dense, int64_t T, const Work& ws,
                          const PfWork& pw, hipStream_t st) {
  hipLaunchKernelGGL(k_pf_norm, dim3((unsigned)T), dim3(kBlock), 0, st, (const float*)ws.u,
                     reinterpret_cast<const uint16_t*>(dense + s.gamma_off), s.l, s.use_norm, s.eps,
                     pw.uh);
  return hipGetLastError();
}

hipError_t launch_pf_out(const Shape& s, const uint8_t* dense, int64_t T, const PfWork& pw,
                         float* delta, hipStream_t st) {
  PfDenseArgs a{};
  a.w = dense + s.in_bytes;
  a.ks = s.ks_out;
  a.tr_count = s.tr_out;
  a.n_grp = cdiv(s.tr_out, kPfWaves * kPfNT);
  a.n_tiles = cdiv(T, kPfRows);
  a.a0 = pw.uh; a.lda0 = s.l; a.n0 = s.l;
  a.a1 = s.ms > 0 ? pw.hs : pw.uh; a.lda1 = s.ms; a.c1 = s.ks_l * kStepK; a.n1 = s.ms;
  a.T = T;
  a.delta = delta; a.d = s.d;
  hipLaunchKernelGGL(k_pf_dense<false>, dim3((unsigned)xcd_grid(a.n_grp, a.n_tiles)), dim3(kBlock),
                     kPfDenseLds, st, a);
  return hipGetLastError();
}

}  // namespace moe
