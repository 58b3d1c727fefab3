// gfx950 kernels of the compute-bound forward (the "mx8" and "mx4" precision profiles).
//
// The same steps as the weight-streaming launches, in the order of the Kimi K3 latent
// mixture-of-experts block card, with the rounding points of the profile:
//   k_pf_in      z = x W_r, x^c = x W_down_latent, h_s = SiTU(x W_sg, x W_su) -> bf16,
//                one product over the packed IN matrix (bf16 MFMA)
//   k_pf_quant   x^c -> MXFP8-E4M3 (mx8) or MXFP4-E2M1 (mx4), the experts' input
//   (route and dispatch: the launches of the token-tiled path)
//   k_pf_exp     routed gate/up with SiTU and the MX conversion of h fused in its
//                epilogue, then routed down: MX activations x MXFP4 weights on the scaled
//                16x16x128 MFMA (v_mfma_scale_f32_16x16x128_f8f6f4; FP8 x FP4 in mx8, FP4 x
//                FP4 in mx4), the E8M0 scales of both operands applied by the matrix core
//   (combine and the RMSNorm, u_hat rounded to bf16)
//   k_pf_out     Delta = u_hat W_up_latent + h_s W_shared_down, one product over the packed
//                OUT matrix (bf16 MFMA)
//
// Tiling: a workgroup multiplies a tile of 16 NB activation rows (NB <= 10) with 4 x NT
// tile rows of weights (NT per wavefront: kPfNT for the experts, kPfDenseNT for the dense
// products).  K advances one K-step (128 columns) at a
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

constexpr int kPfDenseNB = 6;    // dense products: tiles of 96 tokens
constexpr int kPfExpNB = 4;      // routed experts: units of up to 64 positions
static_assert(16 * kPfExpNB == kPfUnitPositions, "dispatch units fill one expert tile");
// the most activation rows of a tile (the row tables hold this many)
constexpr int kPfRows = 16 * (kPfDenseNB > kPfExpNB ? kPfDenseNB : kPfExpNB);
static_assert(kPfRows <= kBlock, "one thread per activation row sets the row tables");
constexpr int kPfNT = 4;         // weight tile rows per wavefront: routed experts
constexpr int kPfDenseNT = 2;    // dense products (2 workgroups per CU fit 256 registers)
constexpr int kPfWaves = kBlock / kWave;
constexpr int kPfDenseDepth = 2;   // K-steps in flight: bf16 weights (4 KiB per tile row)
constexpr int kPfExpDepth = 2;     // MXFP4 weights (1 KiB per tile row)

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

// The same over one 16x16 block with both operands FP4-E2M1: A laid out as B (16 bytes per
// lane: row l % 16, K 32 (l/16) .. +32, low nibble first).
__device__ __forceinline__ f32x4_t mfma_fp4_fp4(uint4 a, uint4 b, uint32_t sa, uint32_t sb,
                                                f32x4_t acc) {
  const i32x8_t av = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
  const i32x8_t bv = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc, 4 /*A: E2M1*/, 4 /*B: E2M1*/,
                                                          0, (int)sa, 0, (int)sb);
}

// An fp32 value (already divided by its block scale, |y| < 512) to E4M3: the nearest value,
// ties to even, saturated at 448 (the conversion itself turns values past 464 into NaN).
__device__ __forceinline__ uint32_t to_e4m3(float y) {
  y = fminf(fmaxf(y, -448.f), 448.f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y, 0.f, 0, false) & 0xFFu;
}

// E8M0 byte of an MX block from its largest magnitude: 2^X with X = floor(log2 amax) - EMAX
// (the element format's largest exponent: 8 for E4M3, 2 for E2M1), the byte X + 127, clamped
// at 0 (amax of 0 or below 2^(EMAX - 127)).
template <uint32_t EMAX>
__device__ __forceinline__ uint32_t mx_scale_byte(float amax) {
  const uint32_t ef = (__float_as_uint(amax) >> 23) & 0xFFu;
  return ef > EMAX ? ef - EMAX : 0u;
}
// 2^-X for the scale byte (X = byte - 127): an fp32 with exponent field 254 - byte.
__device__ __forceinline__ float mx_inv_scale(uint32_t sbyte) { return __uint_as_float((254u - sbyte) << 23); }

// An fp32 value (already divided by its block scale, |y| < 8) to its E2M1 code: the nearest
// of 0, 0.5, 1, 1.5, 2, 3, 4, 6 with halfway cases to the even code (0.25 -> 0, 0.75 -> 1,
// 1.25 -> 1, 1.75 -> 2, 2.5 -> 2, 3.5 -> 4, 5 -> 4), saturated at 6, as the count of
// thresholds below |y|; the sign bit only on a non-zero magnitude.
__device__ __forceinline__ uint32_t e2m1_code(float y) {
  const float a = fabsf(y);
  const uint32_t m = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                     (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
                     (uint32_t)(a > 5.f);
  return m | (y < 0.f && m != 0u ? 8u : 0u);
}
// Eight fp32 values times inv as E2M1 codes, the first in the low nibble.
__device__ __forceinline__ uint32_t pack8_e2m1(float4 x0, float4 x1, float inv) {
  return e2m1_code(x0.x * inv) | (e2m1_code(x0.y * inv) << 4) | (e2m1_code(x0.z * inv) << 8) |
         (e2m1_code(x0.w * inv) << 12) | (e2m1_code(x1.x * inv) << 16) |
         (e2m1_code(x1.y * inv) << 20) | (e2m1_code(x1.z * inv) << 24) | (e2m1_code(x1.w * inv) << 28);
}

// tanh of the compute-bound epilogues: the odd series x (1 - x^2/3 + 2 x^4/15) below
// |x| = 1/16 (relative error < 1e-8 there), else (1 - e^-2|x|) / (1 + e^-2|x|) with the
// hardware exponential (relative error below 1e-6), sign restored.
__device__ __forceinline__ float tanh_fast(float x) {
  const float ax = fabsf(x), x2 = x * x;
  const float series = x * (1.f + x2 * (-1.f / 3.f + x2 * (2.f / 15.f)));
  const float e = __expf(-2.f * ax);
  const float r = __fdividef(1.f - e, 1.f + e);
  return ax < 0.0625f ? series : copysignf(r, x);
}
__device__ __forceinline__ float sigmoid_fast(float g) { return __fdividef(1.f, 1.f + __expf(-g)); }

// SiTU-GLU (act 0) or SwiGLU (act 1) with the fast tanh and sigmoid; rbg, rbl = 1 / beta.
__device__ __forceinline__ float glu_act_fast(float g, float u, int act, float rbg, float bg,
                                              float rbl, float bl) {
  if (act == 0) return (bg * tanh_fast(g * rbg) * sigmoid_fast(g)) * (bl * tanh_fast(u * rbl));
  return g * sigmoid_fast(g) * u;
}

// Four fp32 values (already divided by their block scale) as E4M3 bytes, the first in the
// low byte.
__device__ __forceinline__ uint32_t pack4_e4m3(float a, float b, float c, float d) {
  a = fminf(fmaxf(a, -448.f), 448.f); b = fminf(fmaxf(b, -448.f), 448.f);
  c = fminf(fmaxf(c, -448.f), 448.f); d = fminf(fmaxf(d, -448.f), 448.f);
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

// A value of another lane of the same quad (DPP quad permutation CTRL).
template <int CTRL>
__device__ __forceinline__ float quad_perm_f32(float v) {
  return __uint_as_float((uint32_t)__builtin_amdgcn_mov_dpp((int)__float_as_uint(v), CTRL, 0xF, 0xF, false));
}

// The value of lane c ^ 8 within each 16-lane row (DPP row rotate by 8).
__device__ __forceinline__ float swap_half_rows(float v) {
  return __uint_as_float((uint32_t)__builtin_amdgcn_update_dpp(0, (int)__float_as_uint(v), 0x128, 0xF, 0xF, false));
}

// ------------------------------------------------------------------------------------
// The activation side of a tile.
//   AF 0: bf16 rows, 16 pieces of 16 bytes per K-step; columns [0, n0) from segment 0
//         (row r at word o0[r]), [c1, c1 + n1) from segment 1 (word o1[r]), zero elsewhere.
//   AF 1: MXFP8 rows padded to whole K-steps (128 code bytes and 4 scale bytes per
//         K-step): 8 pieces per K-step at word o0[r] + 8 q, the scale word at s0[r] + q.
//   AF 2: MXFP4 rows, likewise with 64 code bytes per K-step: 4 pieces at word o0[r] + 4 q.
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

template <int AF, int NB, int P>
struct PfStage {
  static constexpr int PR = AF == 2 ? 4 : AF == 1 ? 8 : 16;
  static constexpr int RB = 16 * NB;
  static constexpr int NP = (RB * PR + kBlock - 1) / kBlock;
  uint4 v[P][NP];
  uint32_t sv[P];
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
  // K-step q into register slot `slot` (a constant once the caller's loop is unrolled)
  __device__ __forceinline__ void load(int slot, const PfSrc& src, int q) {
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      uint32_t w = 0u;
      const uint4* base = src.b0;
      if (AF) {
        w = rv[i] ? o0[i] + (uint32_t)PR * q + piece_of(i) : 0u;
      } else {
        const int col = q * kStepK + 8 * piece_of(i);
        const bool a0 = in0(i, src, q), a1 = in1(i, src, q);
        w = a0 ? o0[i] + (col >> 3) : a1 ? o1[i] + ((col - src.c1) >> 3) : 0u;
        base = a1 ? src.b1 : src.b0;
      }
      const uint4 x = base[w];
#pragma unroll
      for (int sl = 0; sl < P; ++sl)
        if (sl == slot) v[sl][i] = x;
    }
    if (AF) {
      const uint32_t x = src.sc[srv ? so + q : 0u];
#pragma unroll
      for (int sl = 0; sl < P; ++sl)
        if (sl == slot) sv[sl] = x;
    }
  }
  // Register slot `slot`, holding K-step q, into an LDS buffer (invalid pieces as zeros).
  __device__ __forceinline__ void commit(int slot, uint4* buf, uint32_t* sbuf, const PfSrc& src,
                                         int q) const {
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int idx = threadIdx.x + i * kBlock;
      if (idx < RB * PR) {
        const int r = idx / PR, j = idx % PR;
        const bool z = !(in0(i, src, q) || in1(i, src, q));
        uint4 x = v[0][i];
#pragma unroll
        for (int sl = 1; sl < P; ++sl)
          if (sl == slot) x = v[sl][i];
        buf[j * RB + (r ^ j)] = make_uint4(z ? 0u : x.x, z ? 0u : x.y, z ? 0u : x.z, z ? 0u : x.w);
      }
    }
    if (AF && (int)threadIdx.x < RB) {
      uint32_t x = sv[0];
#pragma unroll
      for (int sl = 1; sl < P; ++sl)
        if (sl == slot) x = sv[sl];
      sbuf[threadIdx.x] = srv ? x : 0u;
    }
  }
};

// The K loop of a tile: acc[t][b] = D of activation block b x the wavefront's tile row t
// (trow[t]; waves or tile rows without work pass tile row 0 of the same matrix and drop
// the result).  AF 0 pairs with bf16 weights (WF 0), AF 1 and 2 with MXFP4 weights (WF 1).  P
// K-steps of weights and of activation rows are in flight (register rings, slot q % P
// holds K-step q); the rows of K-step q + 1 go to LDS at the end of step q.
template <int AF, int NB, int NT, int P>
__device__ __forceinline__ void pf_run(const PfRows& rows, const PfSrc& src,
                                       const uint8_t* const (&trow)[NT], int ks, uint4* lds,
                                       uint32_t* slds, f32x4_t (&acc)[NT][NB]) {
  constexpr int WF = AF ? 1 : 0;
  constexpr int RB = 16 * NB;
  constexpr int PR = PfStage<AF, NB, P>::PR;
  const int lane = threadIdx.x & (kWave - 1);
  const int c = lane & 15, g = lane >> 4;
  WeightStep<WF> w[P][NT];
  PfStage<AF, NB, P> st;
  st.init(rows, src);
#pragma unroll
  for (int i = 0; i < P; ++i) {
#pragma unroll
    for (int t = 0; t < NT; ++t) w[i][t].template load<true>(trow[t], min(i, ks - 1), lane);
    st.load(i, src, min(i, ks - 1));
  }
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[t][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  asm volatile("" ::: "memory");
  st.commit(0, lds, slds, src, 0);
  __syncthreads();
  for (int q0 = 0; q0 < ks; q0 += P) {
#pragma unroll
    for (int sl = 0; sl < P; ++sl) {
      const int q = q0 + sl;
      if (q >= ks) break;
      // slot sl held K-step q (already in LDS buffer q & 1): refill it with q + P
      st.load(sl, src, min(q + P, ks - 1));
      const uint4* buf = lds + (q & 1) * RB * PR;
      if (AF == 2) {
        const uint32_t* sb = slds + (q & 1) * RB;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const int r = 16 * b + c;
          const uint4 af = buf[g * RB + (r ^ g)];
          const uint32_t sa = (sb[r] >> (8 * g)) & 0xFFu;
#pragma unroll
          for (int t = 0; t < NT; ++t)
            acc[t][b] = mfma_fp4_fp4(af, w[sl][t].w[0], sa, (w[sl][t].sc >> (8 * g)) & 0xFFu, acc[t][b]);
        }
      } else if (AF) {
        const uint32_t* sb = slds + (q & 1) * RB;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const int r = 16 * b + c;
          const uint4 alo = buf[g * RB + (r ^ g)];
          const uint4 ahi = buf[(4 + g) * RB + (r ^ (4 + g))];
          const uint32_t sa = (sb[r] >> (8 * g)) & 0xFFu;
#pragma unroll
          for (int t = 0; t < NT; ++t)
            acc[t][b] = mfma_fp8_fp4(alo, ahi, w[sl][t].w[0], sa, (w[sl][t].sc >> (8 * g)) & 0xFFu,
                                     acc[t][b]);
        }
      } else {
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
          const int j = 4 * s4 + g;
          uint4 af[NB];
#pragma unroll
          for (int b = 0; b < NB; ++b) af[b] = buf[j * RB + ((16 * b + c) ^ j)];
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            const uint4 bw = w[sl][t].operand(s4, 0.f);
#pragma unroll
            for (int b = 0; b < NB; ++b) acc[t][b] = mfma_bf16(af[b], bw, acc[t][b]);
          }
        }
      }
      // the K-step's products are issued before its slot is reloaded, so that the slot's old
      // and new values never overlap and keep one register set across the loop's back edge
      // (where the compiler would otherwise copy the rings, waiting for every load in flight)
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int b = 0; b < NB; ++b) asm volatile("" : "+v"(acc[t][b]) :: "memory");
#pragma unroll
      for (int t = 0; t < NT; ++t) w[sl][t].template load<true>(trow[t], min(q + P, ks - 1), lane);
      asm volatile("" ::: "memory");
      st.commit((sl + 1) % P, lds + ((q + 1) & 1) * RB * PR, slds + ((q + 1) & 1) * RB, src,
                min(q + 1, ks - 1));
      __syncthreads();
    }
  }
}

// ------------------------------------------------------------------------------------
// Dense products for a tile of up to 16 kPfDenseNB tokens: k_pf_in over the IN matrix (router
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
  float bg, bl, rbg, rbl;
  // OUT epilogue
  OutSink sink;
  int d;
};

template <bool IN>
__global__ __launch_bounds__(kBlock, 2) void k_pf_dense(PfDenseArgs a) {
  extern __shared__ uint4 sm[];
  __shared__ PfRows rows;
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15, g = lane >> 4;
  int grp, tile;
  if (!xcd_item(blockIdx.x, a.n_grp, a.n_tiles, grp, tile)) return;
  const int64_t t0 = (int64_t)tile * 16 * kPfDenseNB;
  const int nt = (int)min((int64_t)16 * kPfDenseNB, a.T - t0);
  if ((int)threadIdx.x < nt) {
    rows.o0[threadIdx.x] = (uint32_t)((t0 + threadIdx.x) * a.lda0 / 8);
    rows.o1[threadIdx.x] = (uint32_t)((t0 + threadIdx.x) * a.lda1 / 8);
  }
  __syncthreads();
  const uint8_t* trow[kPfDenseNT];
  int tr[kPfDenseNT];
#pragma unroll
  for (int t = 0; t < kPfDenseNT; ++t) {
    tr[t] = (grp * kPfWaves + wv) * kPfDenseNT + t;
    trow[t] = a.w + (size_t)(tr[t] < a.tr_count ? tr[t] : 0) * a.ks * kBf16StepBytes;
  }
  f32x4_t acc[kPfDenseNT][kPfDenseNB];
  pf_run<0, kPfDenseNB, kPfDenseNT, kPfDenseDepth>(rows, PfSrc{reinterpret_cast<const uint4*>(a.a0), reinterpret_cast<const uint4*>(a.a1),
                                  nullptr, nt, a.n0, a.c1, a.n1},
                      trow, a.ks, sm, nullptr, acc);
  const bool lo = c < 8;
#pragma unroll
  for (int t = 0; t < kPfDenseNT; ++t) {
#pragma unroll
    for (int b = 0; b < kPfDenseNB; ++b)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int ti = 16 * b + 4 * g + v;
        const int64_t tok = t0 + ti;
        const float y = acc[t][b][v];
        if (tr[t] >= a.tr_count) continue;
        if (!IN) {
          const int r = 16 * tr[t] + c;
          if (ti < nt && r < a.d) store_out(a.sink, tok * a.d + r, y);
        } else if (tr[t] < a.tr_r) {
          const int e = 16 * tr[t] + c;
          if (ti < nt && e < a.E) a.z[tok * a.E + e] = y;
        } else if (tr[t] < a.tr_r + a.tr_dn) {
          const int r = 16 * (tr[t] - a.tr_r) + c;
          if (ti < nt && r < a.l) a.xc[tok * a.l + r] = y;
        }
      }
  }
  if (!IN) return;
  // shared gate/up rows: tile rows t, t + 1 form a pair; lane c < 8 evaluates the h_s of
  // tile row t (its gate, the up value of lane c + 8), lane c >= 8 that of tile row t + 1
  const int sh0 = a.tr_r + a.tr_dn;
#pragma unroll
  for (int t = 0; t < kPfDenseNT; t += 2)
#pragma unroll
    for (int b = 0; b < kPfDenseNB; ++b)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float send = lo ? acc[t + 1][b][v] : acc[t][b][v];
        const float recv = swap_half_rows(send);
        const float gate = lo ? acc[t][b][v] : recv;
        const float up = lo ? recv : acc[t + 1][b][v];
        const int trm = tr[lo ? t : t + 1];
        const int ti = 16 * b + 4 * g + v;
        const int r = 8 * (trm - sh0) + (c & 7);
        if (trm >= sh0 && trm < a.tr_count && ti < nt && r < a.ms) {
          const float h = glu_act_fast(gate, up, a.act, a.rbg, a.bg, a.rbl, a.bl);
          a.hs[(t0 + ti) * a.ms + r] = (uint16_t)(pack_bf16x2(h, 0.f) & 0xFFFFu);
        }
      }
}

// x^c fp32 [T][l] -> MX rows of ks K-steps: codes [T][128 ks] E4M3 bytes (FP4 false) or
// [T][64 ks] bytes of E2M1 pairs (FP4 true), scales [T][4 ks] (blocks past l are zero).
// One thread per (token, block of 32).
template <bool FP4>
__global__ __launch_bounds__(kBlock) void k_pf_quant(const float* __restrict__ xc, int64_t T, int l,
                                                     int ks, uint8_t* __restrict__ codes,
                                                     uint8_t* __restrict__ scales) {
  const int64_t gid = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  const int nbk = 4 * ks;
  if (gid >= T * nbk) return;
  const int64_t t = gid / nbk;
  const int blk = (int)(gid - t * nbk);
  constexpr int kBlkBytes = FP4 ? 16 : 32;
  uint4* dst = reinterpret_cast<uint4*>(codes + t * 4 * kBlkBytes * ks + kBlkBytes * blk);
  if (32 * blk >= l) {
    dst[0] = make_uint4(0u, 0u, 0u, 0u);
    if (!FP4) dst[1] = make_uint4(0u, 0u, 0u, 0u);
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
  if (FP4) {
    const uint32_t sb = mx_scale_byte<2>(amax);
    const float inv = mx_inv_scale(sb);
    uint32_t wd[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      wd[i] = pack8_e2m1(make_float4(v[8 * i], v[8 * i + 1], v[8 * i + 2], v[8 * i + 3]),
                         make_float4(v[8 * i + 4], v[8 * i + 5], v[8 * i + 6], v[8 * i + 7]), inv);
    dst[0] = make_uint4(wd[0], wd[1], wd[2], wd[3]);
    scales[t * nbk + blk] = (uint8_t)sb;
    return;
  }
  const uint32_t sb = mx_scale_byte<8>(amax);
  const float inv = mx_inv_scale(sb);
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
// Routed experts, MX activations (AF 1: MXFP8, AF 2: MXFP4) x MXFP4 weights.  Work item
// (tile-row group, unit); a unit is a run of at most 16 kPfExpNB dispatch positions of one
// expert.  Gate/up: input rows x^c_q of the positions' tokens; each wavefront's 4 tile rows
// (8 gate + 8 up rows each) give one MX block of 32 columns of h = SiTU(gate, up), converted
// to the same MX format in the epilogue.  Down: input rows h_q of the positions, output E
// fp32.
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
  const uint8_t* xq;        // input codes, rows of 128 ks (AF 1) or 64 ks (AF 2) bytes
  const uint8_t* xs;        // input scales, rows of 4 ks bytes
  // gate/up output: h as MX rows of ks_out K-steps
  uint8_t* hq;
  uint8_t* hsc;
  int ks_out, m, act;
  float bg, bl, rbg, rbl;
  // down output
  float* out;
  int n_out;
};

template <bool GU, int NB, int AF>
__device__ __forceinline__ void pf_exp_unit(const PfExpArgs& a, const PfRows& rows, uint4* sm,
                                            uint32_t* ssm, const uint8_t* const (&trow)[kPfNT],
                                            const int (&tr)[kPfNT], int wblk, int p0, int n) {
  const int lane = threadIdx.x & (kWave - 1);
  const int c = lane & 15, g = lane >> 4;
  f32x4_t acc[kPfNT][NB];
  pf_run<AF, NB, kPfNT, kPfExpDepth>(rows, PfSrc{reinterpret_cast<const uint4*>(a.xq), nullptr,
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
  // h block wblk (columns 32 wblk .. +32) of each position, 16 positions (one activation
  // block) at a time through a wavefront-private LDS tile (fp32, rows of 36 words).  Tile
  // row t holds the gate of column 8 t + (c % 8) in lane c < 8 and its up value in lane
  // c + 8; the pair swaps halves so that lane c < 8 evaluates tile rows 0, 1 and lane
  // c >= 8 tile rows 2, 3.  Then lane l converts row l / 4, columns 8 (l % 4) .. +8: the
  // block's largest magnitude over the quad of lanes, the E8M0 byte, 8 codes, one 8-byte
  // (E4M3) or 4-byte (E2M1) store.
  const int nbk = 4 * a.ks_out;
  if (32 * wblk >= 128 * a.ks_out) return;
  const bool lo = c < 8;
  float* tile = reinterpret_cast<float*>(sm) + (threadIdx.x >> 6) * 16 * 36;
  const int rr = lane >> 2, qq = lane & 3;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // the previous block's reads are done
#pragma unroll
    for (int v = 0; v < 4; ++v)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        // lane c < 8 sends its gate of tile row 2 + tt, lane c + 8 its up of tile row tt
        const float send = lo ? acc[2 + tt][b][v] : acc[tt][b][v];
        const float recv = swap_half_rows(send);
        const float gate = lo ? acc[tt][b][v] : recv;
        const float up = lo ? recv : acc[2 + tt][b][v];
        const int t = lo ? tt : 2 + tt;
        const int col = 8 * tr[t] + (c & 7);
        const float h = col < a.m ? glu_act_fast(gate, up, a.act, a.rbg, a.bg, a.rbl, a.bl) : 0.f;
        tile[(4 * g + v) * 36 + 8 * t + (c & 7)] = h;
      }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // the tile is written
    const float4 x0 = *reinterpret_cast<const float4*>(tile + rr * 36 + 8 * qq);
    const float4 x1 = *reinterpret_cast<const float4*>(tile + rr * 36 + 8 * qq + 4);
    float amax = fmaxf(fmaxf(fmaxf(fabsf(x0.x), fabsf(x0.y)), fmaxf(fabsf(x0.z), fabsf(x0.w))),
                       fmaxf(fmaxf(fabsf(x1.x), fabsf(x1.y)), fmaxf(fabsf(x1.z), fabsf(x1.w))));
    amax = fmaxf(amax, quad_perm_f32<0xB1>(amax));   // lanes 1, 0, 3, 2 of the quad
    amax = fmaxf(amax, quad_perm_f32<0x4E>(amax));   // lanes 2, 3, 0, 1
    const uint32_t sb = AF == 2 ? mx_scale_byte<2>(amax) : mx_scale_byte<8>(amax);
    const float inv = mx_inv_scale(sb);
    const int i = 16 * b + rr;
    if (AF == 2 && i < n) {
      const int64_t p = p0 + i;
      *reinterpret_cast<uint32_t*>(a.hq + p * 64 * a.ks_out + 16 * wblk + 4 * qq) = pack8_e2m1(x0, x1, inv);
      if (qq == 0) a.hsc[p * nbk + wblk] = (uint8_t)sb;
    } else if (i < n) {
      const int64_t p = p0 + i;
      const uint2 w2 = make_uint2(pack4_e4m3(x0.x * inv, x0.y * inv, x0.z * inv, x0.w * inv),
                                  pack4_e4m3(x1.x * inv, x1.y * inv, x1.z * inv, x1.w * inv));
      *reinterpret_cast<uint2*>(a.hq + p * 128 * a.ks_out + 32 * wblk + 8 * qq) = w2;
      if (qq == 0) a.hsc[p * nbk + wblk] = (uint8_t)sb;
    }
  }
}

// Work order of the expert launches: chunks of 8 units through every tile-row group
// (chunk_item; measured against 2, 4, 16 and 32: the units of one expert share its weight
// slices in L2 best at 8 when an expert has many units).
constexpr int kPfChunk = 8;

// Two workgroups per compute unit (a register budget of 256 per lane): while one waits at
// its barrier or for its loads the other issues MFMAs.
template <bool GU, int AF>
__global__ __launch_bounds__(kBlock, 2) void k_pf_exp(PfExpArgs a) {
  extern __shared__ uint4 sm[];
  __shared__ PfRows rows;
  __shared__ uint32_t ssm[2 * kPfRows];
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n_units = min(a.ctrl[0], a.max_units);
  int grp, u;
  if (!chunk_item(blockIdx.x, n_units, a.n_grp, kPfChunk, grp, u)) return;
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
    rows.o0[threadIdx.x] = (uint32_t)(src * (AF == 2 ? 4 : 8) * a.ks);   // 16-byte words of the row
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
  // blocks of 16 positions: the unit's count rounded up to one of the built tile heights
  const int nb = (n + 15) / 16;
  if (nb <= 1) pf_exp_unit<GU, 1, AF>(a, rows, sm, ssm, trow, tr, wblk, p0, n);
  else if (nb <= 2) pf_exp_unit<GU, 2, AF>(a, rows, sm, ssm, trow, tr, wblk, p0, n);
  else pf_exp_unit<GU, kPfExpNB, AF>(a, rows, sm, ssm, trow, tr, wblk, p0, n);
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

// The combine and the norm in one pass, one workgroup per token, for the mx launches (whose
// only use of u is u_hat): u_t = sum_j G[t,j] E[inv[t,j]] stays in registers, with the same
// fmaf chain per element as k_combine, and the sum of squares and u_hat follow k_pf_norm's
// order (thread i takes the column groups 4 i + 1024 c), so the bits are those of the two
// kernels.  l <= 4 * kBlock * kPfCnChunks.
constexpr int kPfCnChunks = 8;
__global__ __launch_bounds__(kBlock) void k_pf_combine_norm(
    const float* __restrict__ gw, const int32_t* __restrict__ inv, const float* __restrict__ eo,
    int k, int l, const uint16_t* __restrict__ gamma, int norm, float eps,
    uint16_t* __restrict__ uh) {
  __shared__ float sg[kMaxK];
  __shared__ int si[kMaxK];
  __shared__ float red[kPfWaves];
  const int64_t t = blockIdx.x;
  if ((int)threadIdx.x < k) {
    sg[threadIdx.x] = gw[t * k + threadIdx.x];
    si[threadIdx.x] = inv[t * k + threadIdx.x];
  }
  __syncthreads();
  const int l4 = l / 4;
  const float4* e4 = reinterpret_cast<const float4*>(eo);
  float4 u[kPfCnChunks];
#pragma unroll
  for (int ch = 0; ch < kPfCnChunks; ++ch) {
    const int c4 = threadIdx.x + kBlock * ch;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    if (c4 < l4) {
      for (int j0 = 0; j0 < k; j0 += 16) {
        float4 v[16];
#pragma unroll
        for (int i = 0; i < 16; ++i)
          v[i] = (j0 + i < k) ? e4[(int64_t)si[j0 + i] * l4 + c4] : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (j0 + i < k) {
            const float g = sg[j0 + i];
            acc.x = fmaf(g, v[i].x, acc.x);
            acc.y = fmaf(g, v[i].y, acc.y);
            acc.z = fmaf(g, v[i].z, acc.z);
            acc.w = fmaf(g, v[i].w, acc.w);
          }
      }
    }
    u[ch] = acc;
  }
  float rs = 1.f;
  if (norm) {
    const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x >> 6;
    float ss = 0.f;
#pragma unroll
    for (int ch = 0; ch < kPfCnChunks; ++ch)
      if ((int)threadIdx.x + kBlock * ch < l4) {
        ss = fmaf(u[ch].x, u[ch].x, ss); ss = fmaf(u[ch].y, u[ch].y, ss);
        ss = fmaf(u[ch].z, u[ch].z, ss); ss = fmaf(u[ch].w, u[ch].w, ss);
      }
    ss = wave_sum(ss);
    if (lane == 0) red[wv] = ss;
    __syncthreads();
    const float tot = (red[0] + red[1]) + (red[2] + red[3]);
    rs = 1.0f / sqrtf(tot / (float)l + eps);
  }
#pragma unroll
  for (int ch = 0; ch < kPfCnChunks; ++ch) {
    const int c4 = threadIdx.x + kBlock * ch;
    if (c4 >= l4) continue;
    const float uv[4] = {u[ch].x, u[ch].y, u[ch].z, u[ch].w};
    uint32_t w[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float o[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int col = 4 * c4 + 2 * h + q;
        const float gm = norm ? __uint_as_float((uint32_t)gamma[col] << 16) : 1.f;
        o[q] = norm ? uv[2 * h + q] * rs * gm : uv[2 * h + q];
      }
      w[h] = pack_bf16x2(o[0], o[1]);
    }
    *reinterpret_cast<uint2*>(uh + t * l + 4 * c4) = make_uint2(w[0], w[1]);
  }
}

constexpr size_t kPfDenseLds = (size_t)2 * 16 * kPfDenseNB * 16 * 16;   // two K-steps of the bf16 rows
// two K-steps of the FP8 rows, and room for the gate/up epilogue's wavefront-private tiles
constexpr size_t kPfExpEpiLds = (size_t)kPfWaves * 16 * 36 * 4;
constexpr size_t kPfExpLds = (size_t)2 * 16 * kPfExpNB * 8 * 16 > kPfExpEpiLds
                                 ? (size_t)2 * 16 * kPfExpNB * 8 * 16 : kPfExpEpiLds;

}  // namespace

hipError_t launch_pf_in(const Shape& s, const uint8_t* dense, const uint16_t* x, int64_t T,
                        const PfWork& pw, float* z, float* xc, hipStream_t st) {
  PfDenseArgs a{};
  a.w = dense;
  a.ks = s.ks_in;
  a.tr_count = s.tr_in;
  a.n_grp = cdiv(s.tr_in, kPfWaves * kPfDenseNT);
  a.n_tiles = cdiv(T, 16 * kPfDenseNB);
  a.a0 = x; a.lda0 = s.d; a.n0 = s.d;
  a.a1 = x; a.lda1 = 0; a.c1 = 0; a.n1 = 0;
  a.T = T;
  a.tr_r = s.tr_r; a.tr_dn = s.tr_dn;
  a.z = z; a.E = s.E;
  a.xc = xc; a.l = s.l;
  a.hs = pw.hs; a.ms = s.ms; a.act = s.act; a.bg = s.beta_gate; a.bl = s.beta_lin;
  a.rbg = 1.f / s.beta_gate; a.rbl = 1.f / s.beta_lin;
  hipLaunchKernelGGL(k_pf_dense<true>, dim3((unsigned)xcd_grid(a.n_grp, a.n_tiles)), dim3(kBlock),
                     kPfDenseLds, st, a);
  return hipGetLastError();
}

hipError_t launch_pf_quant(const Shape& s, const float* xc, int64_t T, const PfWork& pw,
                           hipStream_t st) {
  const int64_t n = T * 4 * s.ks_gu;
  if (s.prec == 2)
    hipLaunchKernelGGL(k_pf_quant<true>, dim3((unsigned)cdiv(n, kBlock)), dim3(kBlock), 0, st, xc, T,
                       s.l, s.ks_gu, pw.xq, pw.xs);
  else
    hipLaunchKernelGGL(k_pf_quant<false>, dim3((unsigned)cdiv(n, kBlock)), dim3(kBlock), 0, st, xc, T,
                       s.l, s.ks_gu, pw.xq, pw.xs);
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
  a.rbg = 1.f / s.beta_gate; a.rbl = 1.f / s.beta_lin;
  a.out = ws.eo;
  a.n_out = s.l;
  const unsigned grid = (unsigned)chunk_grid(a.max_units, a.n_grp, kPfChunk);
  if (s.prec == 2) {
    if (gu) hipLaunchKernelGGL((k_pf_exp<true, 2>), dim3(grid), dim3(kBlock), kPfExpLds, st, a);
    else hipLaunchKernelGGL((k_pf_exp<false, 2>), dim3(grid), dim3(kBlock), kPfExpLds, st, a);
  } else {
    if (gu) hipLaunchKernelGGL((k_pf_exp<true, 1>), dim3(grid), dim3(kBlock), kPfExpLds, st, a);
    else hipLaunchKernelGGL((k_pf_exp<false, 1>), dim3(grid), dim3(kBlock), kPfExpLds, st, a);
  }
  return hipGetLastError();
}

hipError_t launch_pf_combine_norm(const Shape& s, const uint8_t* dense, const float* gw, int64_t T,
                                  const Work& ws, const PfWork& pw, hipStream_t st) {
  if (s.l > 4 * kBlock * kPfCnChunks || s.k > kMaxK) {
    const hipError_t e = launch_combine(s, dense, gw, T, ws, st);
    return e != hipSuccess ? e : launch_pf_norm(s, dense, T, ws, pw, st);
  }
  hipLaunchKernelGGL(k_pf_combine_norm, dim3((unsigned)T), dim3(kBlock), 0, st, gw,
                     (const int32_t*)ws.inv, (const float*)ws.eo, s.k, s.l,
                     reinterpret_cast<const uint16_t*>(dense + s.gamma_off), s.use_norm, s.eps,
                     pw.uh);
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
                         const OutSink& out, hipStream_t st) {
  PfDenseArgs a{};
  a.w = dense + s.in_bytes;
  a.ks = s.ks_out;
  a.tr_count = s.tr_out;
  a.n_grp = cdiv(s.tr_out, kPfWaves * kPfDenseNT);
  a.n_tiles = cdiv(T, 16 * kPfDenseNB);
  a.a0 = pw.uh; a.lda0 = s.l; a.n0 = s.l;
  a.a1 = s.ms > 0 ? pw.hs : pw.uh; a.lda1 = s.ms; a.c1 = s.ks_l * kStepK; a.n1 = s.ms;
  a.T = T;
  a.sink = out; a.d = s.d;
  hipLaunchKernelGGL(k_pf_dense<false>, dim3((unsigned)xcd_grid(a.n_grp, a.n_tiles)), dim3(kBlock),
                     kPfDenseLds, st, a);
  return hipGetLastError();
}

}  // namespace moe
