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
// The dense products (k_pf_gemm) take tiles of 256 x 256, the experts (k_pf_exp) tiles of
// one unit's rows (up to 160) x 256 weight rows; both copy their operands global -> LDS
// directly into a ring of K stages, one workgroup per compute unit.
#include <climits>
#include <cmath>
#include <type_traits>

#include "moe_device.hpp"
#include "moe_internal.hpp"

namespace moe {
namespace {

typedef int i32x8_t __attribute__((ext_vector_type(8)));

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
// hardware exponential and reciprocal (v_exp_f32, v_rcp_f32: about 1 ulp each; relative
// error below 1e-6), sign restored.  (A plain division compiles to the IEEE sequence of
// about ten instructions.)
constexpr float kLog2e = 1.4426950408889634f;
__device__ __forceinline__ float tanh_fast(float x) {
  const float ax = fabsf(x), x2 = x * x;
  const float series = x * (1.f + x2 * (-1.f / 3.f + x2 * (2.f / 15.f)));
  const float e = __builtin_amdgcn_exp2f(-2.f * kLog2e * ax);
  const float r = (1.f - e) * __builtin_amdgcn_rcpf(1.f + e);
  return ax < 0.0625f ? series : copysignf(r, x);
}
// (e^-g past the fp32 range: the reciprocal of infinity is 0)
__device__ __forceinline__ float sigmoid_fast(float g) {
  return __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-kLog2e * g));
}

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
// Dense products (bf16 MFMA 32x32x16): k_pf_gemm<true> over the IN matrix (router logits ->
// z, W_down_latent -> x^c fp32, shared gate/up -> SiTU -> h_s bf16), k_pf_gemm<false> over
// the OUT matrix (-> Delta).
//
// Both operands are packed rows: tiles of 16 rows, each a run of K-steps of 4 KiB in the
// layout of the packed weights (sub-tile s of 32 columns: lane chunk 16 g + j holds row j,
// columns 32 s + 8 g .. +8).  A 32-row MFMA operand of a 16-column slice then reads 4 runs
// of 256 contiguous bytes (lanes 0-15 and 32-47 from one tile, 16-31 and 48-63 from the
// next): no LDS bank conflicts, and the LDS copy of a tile's K-range is a straight copy of
// its global bytes.
//
// A workgroup computes 256 rows x 256 weight rows (4 wavefronts of 128 x 128 in a 2 x 2
// grid, 16 accumulator blocks of 32 x 32 each in the AGPRs, one wavefront per SIMD), K in
// stages of 32 columns: the stage's 32 KiB (both operands) is copied global -> LDS directly
// three stages ahead (a ring of five buffers, one barrier per stage; no staging registers),
// and its operands are read into registers while the previous stage is multiplied.
// Each wavefront reads 16 KiB of operands per stage for 32 products: 64 KiB of LDS reads
// and 32 KiB of copies per CU against 1024 cycles of the matrix core, within LDS bandwidth
// while the reads overlap the products.  XCD x runs groups of 4 row tiles x 8 weight tiles
// together, so that its 32 workgroups in flight read each row tile 8 times and each weight
// tile 4 times from its L2 at about the same K.
// ------------------------------------------------------------------------------------
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kGemmTile = 256;                 // rows and weight rows of a workgroup
constexpr int kGemmTiles16 = kGemmTile / 16;   // 16-row tiles per operand
constexpr int kGemmStageK = 32;                // columns per stage (one sub-tile)
constexpr int kGemmStageWords = 2 * kGemmTiles16 * 64;   // 16-byte words of a stage: 32 KiB
constexpr int kGemmThreads = 256;              // 4 wavefronts, one per SIMD
static_assert(kGemmStageWords == 8 * kGemmThreads, "8 copies per thread and stage");
constexpr int kGemmRing = 5;                   // stage buffers (160 KiB of LDS)
static_assert(32 * 132 * 4 <= kGemmStageWords * 16, "an epilogue slab fits a stage buffer");
constexpr int kGemmGroupM = 4, kGemmGroupN = 8;

// Byte offset of (row r, column c) in packed rows of ks K-steps.
__host__ __device__ __forceinline__ size_t packed_off(int64_t r, int c, int ks) {
  return ((size_t)(r >> 4) * ks + (c >> 7)) * 4096 + (size_t)((c >> 5) & 3) * 1024 +
         (size_t)((((c >> 3) & 3) << 4) + (int)(r & 15)) * 16 + (size_t)(c & 7) * 2;
}
// Rows of a packed activation buffer: the rows rounded up to whole workgroup tiles.
__host__ __device__ inline int64_t packed_rows(int64_t T) { return (T + kGemmTile - 1) / kGemmTile * kGemmTile; }

// x bf16 [T][d] -> packed rows of ks K-steps (rows T .. packed_rows(T) and columns past d
// zero).  One thread per 16-byte piece of the packed buffer, in its order: the writes are
// contiguous, and the 64 lanes of a wavefront read 64 contiguous bytes of each of 16 rows.
__global__ __launch_bounds__(kBlock) void k_pf_pack_x(const uint16_t* __restrict__ x, int64_t T, int d,
                                                      int ks, int64_t rows, uint8_t* __restrict__ out) {
  const int64_t gid = (int64_t)blockIdx.x * kBlock + threadIdx.x;   // piece of the packed buffer
  if (gid >= rows * ks * 16) return;
  const int64_t tq = gid >> 8;                   // (16-row tile, K-step)
  const int p = (int)(gid & 255);                // lane chunk of the K-step: 64 s + 16 g + j
  const int64_t t = tq / ks;
  const int q = (int)(tq - t * ks);
  const int64_t r = 16 * t + (p & 15);
  const int c = 128 * q + 32 * (p >> 6) + 8 * ((p >> 4) & 3);
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (r < T && c < d) v = *reinterpret_cast<const uint4*>(x + r * d + c);
  reinterpret_cast<uint4*>(out)[gid] = v;
}

// Work item of workgroup `bid`: (row tile mt, weight tile nt).  Groups of 4 x 8 tiles go
// round-robin to the XCDs (bid % 8), the 32 workgroups of a group back to back on one XCD.
__device__ __forceinline__ bool gemm_item(int bid, int n_m, int n_n, int& mt, int& nt) {
  constexpr int per = kGemmGroupM * kGemmGroupN;
  const int x = bid % kXcds, j = bid / kXcds;
  const int g = (j / per) * kXcds + x, r = j % per;
  const int gm = (n_m + kGemmGroupM - 1) / kGemmGroupM, gn = (n_n + kGemmGroupN - 1) / kGemmGroupN;
  if (g >= gm * gn) return false;
  mt = (g % gm) * kGemmGroupM + r % kGemmGroupM;
  nt = (g / gm) * kGemmGroupN + r / kGemmGroupM;
  return mt < n_m && nt < n_n;
}
__host__ inline int64_t gemm_grid(int64_t n_m, int64_t n_n) {
  const int64_t per = kGemmGroupM * kGemmGroupN;
  const int64_t groups = ((n_m + kGemmGroupM - 1) / kGemmGroupM) * ((n_n + kGemmGroupN - 1) / kGemmGroupN);
  return ((groups + kXcds - 1) / kXcds) * kXcds * per;
}

struct PfGemmArgs {
  const uint8_t* w;      // packed weights: tr_count tile rows of ks K-steps
  const uint8_t* a;      // packed activation rows of ks K-steps (packed_rows(T) of them)
  int ks, tr_count, n_m, n_n;
  int64_t T;
  // IN epilogue
  int tr_r, tr_dn;
  float* z;
  int E;
  float* xc;
  int l;
  uint8_t* ao;           // the OUT launch's packed rows: h_s from column hs_col0
  int ks_out, hs_col0, ms, act;
  float bg, bl, rbg, rbl;
  // OUT epilogue
  OutSink sink;
  int d;
};

// One direct global -> LDS copy of 16 bytes per lane: lane l's bytes at `src` land at LDS
// address lds + 16 l (lds wavefront-uniform).  Written as inline assembly so that the
// compiler does not see an LDS write in flight and make every later LDS read wait for all
// copies (the ring below waits for exactly the stage it reads); the instruction writes no
// register.
__device__ __forceinline__ void copy_to_lds(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds) : "memory");
}

// The LDS read that follows product i of a stage's 32 (-1: none): reads 0-11 after every
// second product of the first 24, reads 12-15 after products 24-27, none after the last 4.
__host__ __device__ constexpr int gemm_read_after(int i) {
  return i < 24 ? ((i & 1) ? i >> 1 : -1) : (i < 28 ? i - 12 : -1);
}

template <bool IN>
__global__ __launch_bounds__(kGemmThreads, 1) void k_pf_gemm(PfGemmArgs a) {
  // the ring of stage buffers (16 row tiles, then 16 weight tiles, 1 KiB each): 160 KiB
  __shared__ uint4 lds[kGemmRing * kGemmStageWords];
  int mt, nt;
  if (!gemm_item(blockIdx.x, a.n_m, a.n_n, mt, nt)) return;
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wv & 1, wn = wv >> 1;     // the wave's 128 rows and 128 weight rows
  // Thread chunk i (0..7) of a stage: LDS word i * 256 + tid: operand i / 4 (row tiles, then
  // weight tiles), tile 4 (i % 4) + wave, 16-byte piece lane of the tile's 1 KiB (one sub-tile
  // of 32 columns).
  const size_t tile_bytes = (size_t)a.ks * 4096;
  const uint8_t* src_a = a.a + (size_t)(mt * kGemmTiles16 + wv) * tile_bytes + lane * 16;
  const uint8_t* src_w = a.w + lane * 16;
  const int tr0 = nt * kGemmTiles16 + wv;   // weight tile of chunk 4 + i: tr0 + 4 i (tile row 0 past the end)
  const int nk = a.ks * (kStepK / kGemmStageK);
  auto dma_stage = [&](const uint4* dst, int k) {
    const uint32_t base = (uint32_t)(uintptr_t)dst + 1024u * wv;   // (low 32 bits: the LDS address)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      copy_to_lds(src_a + (size_t)(4 * i) * tile_bytes + (size_t)k * 1024,
                  __builtin_amdgcn_readfirstlane(base + 4096u * i));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tr = tr0 + 4 * i;
      copy_to_lds(src_w + (size_t)(tr < a.tr_count ? tr : 0) * tile_bytes + (size_t)k * 1024,
                  __builtin_amdgcn_readfirstlane(base + 4096u * (4 + i)));
    }
  };
  auto dma_clamped = [&](const uint4* dst, int k) { dma_stage(dst, k < nk ? k : nk - 1); };
  f32x16_t acc[4][4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = f32x16_t{};
  // Operands: lane l takes row l % 32 of a 32-row block, columns 8 (l / 32) .. +8 of a
  // 16-column slice h of the stage (lane chunk 16 (2 h + l / 32) + row of the sub-tile); row
  // block mb = tiles 8 wm + 2 mb, +1; weight block nb = tiles 8 wn + 2 nb, +1.
  const int lrow = lane & 31, lk = lane >> 5;
  const int a_word = (8 * wm + (lrow >> 4)) * 64 + lk * 16 + (lrow & 15);
  const int w_word = kGemmTiles16 * 64 + (8 * wn + (lrow >> 4)) * 64 + lk * 16 + (lrow & 15);
  // Operands of one stage (both 16-column slices: 8 row pieces, 8 weight pieces) from LDS
  // into registers, and the stage's 32 products from registers.
  auto read_stage = [&](const uint4* L, uint4 (&af)[2][4], uint4 (&bw)[2][4]) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int b = 0; b < 4; ++b) af[h][b] = L[a_word + 2 * b * 64 + 32 * h];
#pragma unroll
      for (int b = 0; b < 4; ++b) bw[h][b] = L[w_word + 2 * b * 64 + 32 * h];
    }
  };
  // The 32 products of a stage held in (af, bw), with the 16 reads of the next stage's
  // operands (from L into naf, nbw) spread among them (read_after: the read, if any, that
  // follows product i), in the order the next stage's products take them (per slice: row
  // piece 0, the four weight pieces, row pieces 1-3), and the 8 copies of stage kd into
  // buffer D, one before every fourth product (issued together they hold the wavefront at
  // the memory unit, behind the other wavefronts' copies, while its matrix core waits).  Issued in bursts, the reads of four
  // wavefronts that leave a barrier together queue at the LDS for hundreds of cycles, and
  // each matrix core stands idle until its wavefront has issued all 16; spread out, the LDS
  // serves them while the products run.  The last products follow the last read, so that
  // the wait for all reads that the compiler puts at the loop's head finds them done.
  auto mma_read = [&](const uint4 (&af)[2][4], const uint4 (&bw)[2][4], const uint4* L,
                      uint4 (&naf)[2][4], uint4 (&nbw)[2][4], const uint4* D, int kd) {
    const int kc = kd < nk ? kd : nk - 1;
    const uint32_t dbase = (uint32_t)(uintptr_t)D + 1024u * wv;
#pragma unroll
    for (int s8 = 0; s8 < 8; ++s8) {
      __builtin_amdgcn_sched_barrier(0);
      if (s8 < 4) copy_to_lds(src_a + (size_t)(4 * s8) * tile_bytes + (size_t)kc * 1024,
                              __builtin_amdgcn_readfirstlane(dbase + 4096u * s8));
      else {
        const int tr = tr0 + 4 * (s8 - 4);
        copy_to_lds(src_w + (size_t)(tr < a.tr_count ? tr : 0) * tile_bytes + (size_t)kc * 1024,
                    __builtin_amdgcn_readfirstlane(dbase + 4096u * s8));
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 4 * s8; i < 4 * s8 + 4; ++i) {
        const int h = i >> 4, mb = (i >> 2) & 3, nb = i & 3;
        acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, af[h][mb]),
                                                             __builtin_bit_cast(bf16x8_t, bw[h][nb]),
                                                             acc[mb][nb], 0, 0, 0);
        const int r = gemm_read_after(i);
        if (r >= 0) {
          const int rh = r >> 3, j = r & 7;
          if (j == 0) naf[rh][0] = L[a_word + 32 * rh];
          else if (j <= 4) nbw[rh][j - 1] = L[w_word + 2 * (j - 1) * 64 + 32 * rh];
          else naf[rh][j - 4] = L[a_word + 2 * (j - 4) * 64 + 32 * rh];
        }
      }
#pragma unroll
      for (int i = 4 * s8; i < 4 * s8 + 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);     // a product
        if (gemm_read_after(i) >= 0) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // an LDS read
      }
    }
  };
  // Stage k lives in buffer k % 5.  Its copies are issued three stages ahead, its operands
  // read into registers one stage ahead (while stage k - 1 is multiplied), so the matrix
  // core never waits for LDS.  Iteration k: wait until this thread's copies of stage k + 1
  // have landed (those of k + 2 and k + 3 may still fly: 16 instructions) and its reads of
  // stage k - 1 are done (those of stage k, the last 16 LDS operations, may still fly but for
  // the first: the wait counter holds 15 at most),
  // barrier (the same for everyone), issue stage k + 4 into the buffer of stage k - 1, read
  // stage k + 1 while multiplying stage k.  Past the last stage the copies and reads repeat
  // it, unused.  (A bare s_barrier: __syncthreads() would also wait for every LDS read in
  // flight.)
  auto buf = [&](int k) -> const uint4* { return lds + (k % kGemmRing) * kGemmStageWords; };
  auto wait_stage = [&]() {
    asm volatile("s_waitcnt vmcnt(16) lgkmcnt(15)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  uint4 o0a[2][4], o0b[2][4], o1a[2][4], o1b[2][4];   // two register sets of operands
  dma_stage(buf(0), 0);
  dma_clamped(buf(1), 1);
  dma_clamped(buf(2), 2);
  dma_clamped(buf(3), 3);
  asm volatile("s_waitcnt vmcnt(24)" ::: "memory");   // stage 0 has landed
  __syncthreads();
  read_stage(buf(0), o0a, o0b);
  for (int k = 0; k < nk; k += 2) {
    wait_stage();
    mma_read(o0a, o0b, buf(k + 1), o1a, o1b, buf(k + 4), k + 4);
    __builtin_amdgcn_sched_barrier(0);
    wait_stage();
    mma_read(o1a, o1b, buf(k + 2), o0a, o0b, buf(k + 5), k + 5);
    __builtin_amdgcn_sched_barrier(0);
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // the repeated reads
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the repeated copies, before LDS is reused
  // Epilogue through LDS, 32 rows of the wavefront's 128 x 128 at a time: the accumulators
  // (accumulator i of block (mb, nb): row 32 mb + 8 (i / 4) + 4 (l / 32) + i % 4, column
  // 32 nb + l % 32 of the wave's tile) go to a wavefront-private fp32 slab of 32 rows x 128
  // columns (row stride 132 words), then each lane takes 4 consecutive columns of a row
  // (16-byte stores), or in the shared expert's tile rows 2 gate columns and their up
  // values 8 columns further on.
  __syncthreads();   // every wavefront is done with the last stage's operands
  float* slab = reinterpret_cast<float*>(lds + wv * kGemmStageWords);
  const int64_t rbase = (int64_t)mt * kGemmTile + 128 * wm;
  const int nbase = nt * kGemmTile + 128 * wn;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        slab[(8 * (i >> 2) + 4 * lk + (i & 3)) * 132 + 32 * nb + lrow] = acc[mb][nb][i];
    // (one wavefront writes and reads its own slab: its LDS operations complete in order)
#pragma unroll 4
    for (int it = 0; it < 16; ++it) {
      const int r = 2 * it + lk, c4 = 4 * lrow;        // row of the slab, first column
      const int64_t row = rbase + 32 * mb + r;
      const int n = nbase + c4;                        // first weight row of the four
      const float4 y = *reinterpret_cast<const float4*>(slab + r * 132 + c4);
      if (row >= a.T) continue;
      if (!IN) {
        if (n < a.d) store_out4(a.sink, row * a.d + n, y);   // (d is a multiple of 8)
        continue;
      }
      const int tr = n >> 4, cc = n & 15;              // tile row and its columns cc .. cc + 3
      if (tr >= a.tr_count) continue;
      if (tr < a.tr_r) {
        const int e = 16 * tr + cc;
        float* z = a.z + row * a.E + e;
        if (e + 3 < a.E && (a.E & 3) == 0) *reinterpret_cast<float4*>(z) = y;
        else {
          if (e < a.E) z[0] = y.x;
          if (e + 1 < a.E) z[1] = y.y;
          if (e + 2 < a.E) z[2] = y.z;
          if (e + 3 < a.E) z[3] = y.w;
        }
      } else if (tr < a.tr_r + a.tr_dn) {
        const int r2 = 16 * (tr - a.tr_r) + cc;       // l is a multiple of 8
        if (r2 < a.l) *reinterpret_cast<float4*>(a.xc + row * a.l + r2) = y;
      } else {
        // the lane's tile row holds 8 gate and 8 up columns: the lane takes gate columns
        // 2 (lane % 4), +1 and their up values 8 further on (every lane evaluates two SiTU
        // values): h_s columns hc, hc + 1
        const int g0 = 16 * (lrow >> 2) + 2 * (lrow & 3);
        const float2 gv = *reinterpret_cast<const float2*>(slab + r * 132 + g0);
        const float2 uv = *reinterpret_cast<const float2*>(slab + r * 132 + g0 + 8);
        const int hc = 8 * (tr - a.tr_r - a.tr_dn) + 2 * (lrow & 3);
        if (hc < a.ms) {   // ms is a multiple of 8: both columns
          const float h0 = glu_act_fast(gv.x, uv.x, a.act, a.rbg, a.bg, a.rbl, a.bl);
          const float h1 = glu_act_fast(gv.y, uv.y, a.act, a.rbg, a.bg, a.rbl, a.bl);
          *reinterpret_cast<uint32_t*>(a.ao + packed_off(row, a.hs_col0 + hc, a.ks_out)) = pack_bf16x2(h0, h1);
        }
      }
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
// (tile-row group, unit); a unit is a run of at most kPfUnitPositions dispatch positions
// of one expert (an expert's positions split into near-equal runs).  Gate/up: input rows
// x^c_q of the positions' tokens; each wavefront's 4 tile rows (8 gate + 8 up rows each)
// give one MX block of 32 columns of h = SiTU(gate, up), converted to the same MX format in
// the epilogue.  Down: input rows h_q of the positions, output E fp32.
//
// Two workgroups per compute unit (78 KiB of LDS and 256 registers each, so that one's
// epilogue and prologue run beside the other's products), of 4 wavefronts, each
// multiplying the unit's 16 NB rows (NB <= 10) with its own 4 tile rows (64 weight rows):
// a tile row's weights are read once per unit, and an expert's once per step when it has
// at most 160 positions.
// Both operands of a K-step (the unit's activation rows with their scale words, the
// workgroup's 16 weight tile rows with theirs) are copied global -> LDS directly, into two
// rings of K-step stages; every wavefront issues the same number of copies per stage, so
// one counted wait and one barrier per K-step order both rings.  The activation rows are
// gathered: each lane of a copy names its own row.
// ------------------------------------------------------------------------------------
struct PfExpArgs {
  const uint8_t* experts;
  size_t expert_bytes, region_off;
  int ks, n_tr, n_grp, chunk;
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

constexpr int kPxNT = 4;                       // weight tile rows per wavefront
constexpr int kPxWaves = kBlock / kWave;       // 4
constexpr int kPxTR = kPxWaves * kPxNT;        // weight tile rows per workgroup
constexpr int kPxMaxNB = kPfUnitPositions / 16;
static_assert(16 * kPxMaxNB == kPfUnitPositions && kPfUnitPositions <= kBlock,
              "a unit fills at most kPxMaxNB blocks; one thread per row sets the row table");
constexpr int kPxRingBytes = 79872;            // 78 KiB of LDS for the rings (two workgroups per CU)
// Ring depths: 2 weight stages of 17 KiB, as many activation stages as fit (2 for 160-row
// tiles), at most 6.
constexpr int kPxWDepth = 2;
constexpr int kPxMaxADepth = 6;

// Direct global -> LDS copies from a wavefront-uniform base and a 32-bit lane offset: 16
// bytes (lane l's at lds + 16 l) or 4 bytes (at lds + 4 l) per lane.
__device__ __forceinline__ void copy_to_lds_at(uint32_t off, const void* base, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "s"(lds) : "memory");
}
__device__ __forceinline__ void copy4_to_lds_at(uint32_t off, const void* base, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1" ::"v"(off), "s"(base), "s"(lds) : "memory");
}
// s_waitcnt immediate that waits for vector memory operations alone (at most n in flight)
__host__ __device__ constexpr int vm_wait_imm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }

// Two rings of K-step stages.  Activation stage: codes (row-major, piece j of row r at
// 16-byte word PR r + (j ^ swz(r)); padded to whole copies of every wavefront), then the
// scale words (256 rows: one copy of 64 per wavefront).  Row-major, a copy of 64 lanes takes
// 8 (AF 1) or 16 (AF 2) whole rows, 8 or 16 cache lines; the swizzle makes the 16 rows of an
// MFMA operand's piece land in 16 different bank groups.  Weight stage: codes (tile row t at
// words 64 t .. +64, in the order of the packed weights), then the scale words (tile row t,
// row c at word 16 t + c).  The weights come from HBM once per unit and their ring runs
// DW - 1 K-steps ahead, the activation rows (read by all of the unit's tile-row groups)
// DA - 1 K-steps ahead.
template <int AF, int NB>
struct PxLayout {
  static constexpr int RB = 16 * NB;
  static constexpr int PR = AF == 2 ? 4 : 8;                    // 16-byte pieces per K-step row
  __device__ static int swz(int r) { return AF == 2 ? (r >> 2) & 3 : (r >> 1) & 7; }
  __device__ static int word(int r, int j) { return PR * r + (j ^ swz(r)); }
  static constexpr int A_WORDS = RB * PR;
  static constexpr int A_COPIES = (A_WORDS + 4 * kWave - 1) / (4 * kWave);   // per wavefront
  static constexpr int AS_OFF = A_COPIES * 4 * kWave * 16;
  static constexpr int A_BYTES = AS_OFF + 4 * kWave * 4;
  static constexpr int WS_OFF = kPxTR * 1024;
  static constexpr int W_BYTES = WS_OFF + kPxTR * 64;
  static constexpr int DW = kPxWDepth;
  static constexpr int A_RING = DW * W_BYTES;                    // the activation ring's offset
  static constexpr int DA_FIT = (kPxRingBytes - A_RING) / A_BYTES;
  static constexpr int DA = DA_FIT < kPxMaxADepth ? DA_FIT : kPxMaxADepth;
  static constexpr int AC = A_COPIES + 1, WC = kPxNT + 1;        // copies per wavefront and stage
  // Copies in flight after the later of K-step k's two stages: turn j issues weight stage
  // j + DW - 1, then activation stage j + DA - 1, so with DA <= DW activation stage k comes
  // last (turn k - DA + 1, DA - 2 turns after it), else weight stage k (turn k - DW + 1,
  // its activation stage and DW - 2 turns after it).
  static constexpr int WAIT = DA <= DW ? (DA - 2) * (AC + WC) : AC + (DW - 2) * (AC + WC);
  static_assert(DA >= 2 && DW >= 2, "a K-step in flight in each ring");
  static_assert(WAIT <= 63, "the wait counter holds the copies in flight");
  static_assert(kPxWaves * kWave >= RB, "the scale copies cover the rows");
  static_assert(NB % 2 == 0, "block 0 of a K-step takes register set 0");
};

template <bool GU, int AF, int NB>
__device__ __forceinline__ void px_unit(const PfExpArgs& a, uint8_t* ring, const int32_t* srcrow,
                                        const uint8_t* ebase, const uint8_t* const (&trow)[kPxNT],
                                        const int (&tr)[kPxNT], int wblk, int p0, int n) {
  using Lay = PxLayout<AF, NB>;
  constexpr int PR = Lay::PR, DA = Lay::DA, DW = Lay::DW;
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15, g = lane >> 4;
  const uint32_t ring_lds = (uint32_t)(uintptr_t)ring;   // (low 32 bits: the LDS address)
  // This lane's sources: a wavefront-uniform base (per K-step) and a 32-bit lane offset.
  // The input rows are the unit's own (down: rows p0 .. of h; srcrow relative to p0) or
  // gathered tokens (gate/up: the launch checks that the T rows span less than 4 GiB).
  // Activation copy i of the wavefront fills words (4 i + wv) 64 .. +64 of the stage: word
  // wd holds row wd / PR, piece (wd % PR) ^ swz (rows past the unit, and the padding, read
  // the unit's first row: in bounds, never used).
  const uint32_t row_bytes = 16u * PR * (uint32_t)a.ks;
  const uint8_t* xq = a.xq + (GU ? 0 : (size_t)p0 * row_bytes);
  const uint8_t* xs = a.xs + (GU ? 0 : (size_t)p0 * 4 * a.ks);
  uint32_t aoff[Lay::A_COPIES];
#pragma unroll
  for (int i = 0; i < Lay::A_COPIES; ++i) {
    const int wd = (4 * i + wv) * kWave + lane;
    const int r = wd < Lay::A_WORDS ? wd / PR : 0;
    const int j = wd < Lay::A_WORDS ? (wd % PR) ^ Lay::swz(r) : 0;
    aoff[i] = (uint32_t)srcrow[r < n ? r : 0] * row_bytes + 16u * j;
  }
  const int sr = kWave * wv + lane;
  const uint32_t soff = (uint32_t)srcrow[sr < n ? sr : 0] * 4u * (uint32_t)a.ks;
  const int tl = lane >> 4;
  const uint32_t wsoff =
      (uint32_t)((tl == 0 ? trow[0] : tl == 1 ? trow[1] : tl == 2 ? trow[2] : trow[3]) - ebase) + 1024u + 4u * c;
  // activation stage j (K-step min(j, ks - 1)) into its ring slot j % DA; weight stage j likewise
  auto issue_a = [&](int j) {
    const int q = j < a.ks ? j : a.ks - 1;
    const uint32_t base = ring_lds + (uint32_t)(Lay::A_RING + (j % DA) * Lay::A_BYTES);
    const uint8_t* src = xq + (size_t)q * 16 * PR;
#pragma unroll
    for (int i = 0; i < Lay::A_COPIES; ++i)
      copy_to_lds_at(aoff[i], src, __builtin_amdgcn_readfirstlane(base + (4 * i + wv) * 1024));
    copy4_to_lds_at(soff, xs + 4 * q, __builtin_amdgcn_readfirstlane(base + Lay::AS_OFF + 256 * wv));
  };
  auto issue_w = [&](int j) {
    const int q = j < a.ks ? j : a.ks - 1;
    const uint32_t base = ring_lds + (uint32_t)((j % DW) * Lay::W_BYTES);
#pragma unroll
    for (int t = 0; t < kPxNT; ++t)
      copy_to_lds_at(16u * lane, trow[t] + (size_t)q * kFp4StepBytes,
                     __builtin_amdgcn_readfirstlane(base + (kPxNT * wv + t) * 1024));
    copy4_to_lds_at(wsoff, ebase + (size_t)q * kFp4StepBytes,
                    __builtin_amdgcn_readfirstlane(base + Lay::WS_OFF + 256 * wv));
  };
  auto a_stage = [&](int q) { return ring + Lay::A_RING + (q % DA) * Lay::A_BYTES; };
  auto w_stage = [&](int q) { return ring + (q % DW) * Lay::W_BYTES; };
  f32x4_t acc[kPxNT][NB];
#pragma unroll
  for (int t = 0; t < kPxNT; ++t)
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[t][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int ks = a.ks;
  // Operands in registers: the weight fragments of a K-step and the activation fragments of
  // a 16-row block (two sets: block b in set b % 2; NB is even, so block 0 of the next K-step
  // takes set 0).
  uint4 bw[kPxNT], al[2], ah[2];
  uint32_t bs[kPxNT], sa[2];
  auto read_w = [&](const uint8_t* st) {
    const uint4* W = reinterpret_cast<const uint4*>(st);
    const uint8_t* WS = st + Lay::WS_OFF;
#pragma unroll
    for (int t = 0; t < kPxNT; ++t) {
      bw[t] = W[(kPxNT * wv + t) * kWave + lane];
      bs[t] = WS[((kPxNT * wv + t) * 16 + c) * 4 + g];   // byte g of row c's scale word
    }
  };
  auto read_a = [&](const uint8_t* st, int b, int set) {
    const uint4* A = reinterpret_cast<const uint4*>(st);
    const int r = 16 * b + c;
    al[set] = A[Lay::word(r, g)];
    if (AF != 2) ah[set] = A[Lay::word(r, 4 + g)];
    sa[set] = st[Lay::AS_OFF + 4 * r + g];   // byte g of row r's scale word (no shift after the read)
  };
  auto mma_block = [&](int b, int set) {
#pragma unroll
    for (int t = 0; t < kPxNT; ++t)
      acc[t][b] = AF == 2 ? mfma_fp4_fp4(al[set], bw[t], sa[set], bs[t], acc[t][b])
                          : mfma_fp8_fp4(al[set], ah[set], bw[t], sa[set], bs[t], acc[t][b]);
  };
  // Turn k (before K-step k's products): this wavefront's copies of both stages of K-step k
  // have landed (the copies complete in order: WAIT counts those issued after the later
  // one) and its LDS reads are done; after the barrier everyone's have, and the slots just
  // read take weight stage k + DW - 1 and activation stage k + DA - 1.  (Past the last
  // K-step the copies repeat it, unused.)
  auto turn = [&](int k) {
    __builtin_amdgcn_s_waitcnt(vm_wait_imm(Lay::WAIT) & ~(15 << 8));
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    issue_w(k + DW - 1);
    issue_a(k + DA - 1);
  };
  // K-step q.  Each block's 4 products run while the next block's fragments are read (a
  // product, a read, ...); the barrier comes before the last block, whose products cover the
  // read of the next K-step's first block; the next K-step's weight fragments are read once
  // the last products are issued (the other workgroup on the compute unit fills the wait).
  auto kstep = [&](int q) {
    const uint8_t* st = a_stage(q);
#pragma unroll
    for (int b = 0; b + 1 < NB; ++b) {
      __builtin_amdgcn_sched_barrier(0);
      read_a(st, b + 1, (b + 1) & 1);
      mma_block(b, b & 1);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, AF == 2 ? 0 : 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    turn(q + 1);
    read_a(a_stage(q + 1), 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    mma_block(NB - 1, 1);
    __builtin_amdgcn_sched_barrier(0);
    read_w(w_stage(q + 1));
    __builtin_amdgcn_sched_barrier(0);
  };
  // The prologue issues what turns -1, -2, ... would have (in the same order), so that the
  // same count of copies follows every stage.
  constexpr int D = DA > DW ? DA : DW;
#pragma unroll
  for (int j = 1 - D; j < 0; ++j) {
    if (j + DW - 1 >= 0) issue_w(j + DW - 1);
    if (j + DA - 1 >= 0) issue_a(j + DA - 1);
  }
  turn(0);
  read_w(w_stage(0));
  read_a(a_stage(0), 0, 0);
  for (int q = 0; q < ks; ++q) kstep(q);
  // the repeated copies land before the ring is reused
  __builtin_amdgcn_s_waitcnt(vm_wait_imm(0));
  __syncthreads();
  if (!GU) {
#pragma unroll
    for (int t = 0; t < kPxNT; ++t) {
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
  float* tile = reinterpret_cast<float*>(ring) + wv * 16 * 36;
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

template <bool GU, int AF>
__global__ __launch_bounds__(kBlock, 2) void k_pf_exp(PfExpArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t ring[kPxRingBytes];
  __shared__ int32_t srcrow[kPfUnitPositions];
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n_units = min(a.ctrl[0], a.max_units);
  int grp, u;
  if (!chunk_item(blockIdx.x, n_units, a.n_grp, a.chunk, grp, u)) return;
  const int4 un = *reinterpret_cast<const int4*>(a.units + 4 * u);
  const int e = un.x, p0 = un.y, n = un.z;
  if (e < 0 || e >= a.E || n < 1 || n > a.nu || n > kPfUnitPositions || p0 < 0 || p0 + n > a.n_assign)
    return;
  // the input row of each position: the token's x^c_q row (gate/up) or the position's h_q
  // row, counted from the unit's first (down)
  if ((int)threadIdx.x < n) {
    int src = threadIdx.x;
    if (GU) {
      const int asg = a.perm[p0 + threadIdx.x];
      src = (asg >= 0 && asg < a.n_assign) ? asg / a.k : 0;
    }
    srcrow[threadIdx.x] = src;
  }
  __syncthreads();
  const int wblk = grp * kPxWaves + wv;    // this wavefront's tile rows 4 wblk .. 4 wblk + 3
  const uint8_t* base = a.experts + (size_t)e * a.expert_bytes + a.region_off;
  const uint8_t* trow[kPxNT];
  int tr[kPxNT];
#pragma unroll
  for (int t = 0; t < kPxNT; ++t) {
    tr[t] = wblk * kPxNT + t;
    trow[t] = base + (size_t)(tr[t] < a.n_tr ? tr[t] : 0) * a.ks * kFp4StepBytes;
  }
  // blocks of 16 positions: the unit's count rounded up to one of the built tile heights
  const int nb = (n + 15) / 16;
  if (nb <= 2) px_unit<GU, AF, 2>(a, ring, srcrow, base, trow, tr, wblk, p0, n);
  else if (nb <= 4) px_unit<GU, AF, 4>(a, ring, srcrow, base, trow, tr, wblk, p0, n);
  else if (nb <= 6) px_unit<GU, AF, 6>(a, ring, srcrow, base, trow, tr, wblk, p0, n);
  else if (nb <= 8) px_unit<GU, AF, 8>(a, ring, srcrow, base, trow, tr, wblk, p0, n);
  else px_unit<GU, AF, kPxMaxNB>(a, ring, srcrow, base, trow, tr, wblk, p0, n);
}

// Zero the padding columns of a token's packed OUT row: u_hat columns l .. 128 ks_l and
// h_s columns ms .. 128 ks_ms (the padded weights there are zero, but 0 x a stale NaN is not).
__device__ __forceinline__ void zero_out_pads(uint8_t* ao, int64_t t, int l, int ks_l, int ms,
                                              int ks_ms, int ks_out) {
  for (int c = l + (int)threadIdx.x; c < 128 * ks_l; c += kBlock)
    *reinterpret_cast<uint16_t*>(ao + packed_off(t, c, ks_out)) = 0;
  for (int c = ms + (int)threadIdx.x; c < 128 * ks_ms; c += kBlock)
    *reinterpret_cast<uint16_t*>(ao + packed_off(t, 128 * ks_l + c, ks_out)) = 0;
}

// u_hat = RMSNorm(u) * gamma rounded to bf16 into the OUT product's packed rows, one
// workgroup per token, in the fixed reduction order of the other paths.
__global__ __launch_bounds__(kBlock) void k_pf_norm(const float* __restrict__ u,
                                                    const uint16_t* __restrict__ gamma, int l,
                                                    int norm, float eps, uint8_t* __restrict__ ao,
                                                    int ks_l, int ms, int ks_ms, int ks_out) {
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
    *reinterpret_cast<uint16_t*>(ao + packed_off(t, col, ks_out)) = (uint16_t)(pack_bf16x2(v, 0.f) & 0xFFFFu);
  }
  zero_out_pads(ao, t, l, ks_l, ms, ks_ms, ks_out);
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
    uint8_t* __restrict__ ao, int ks_l, int ms, int ks_ms, int ks_out) {
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
    // columns 4 c4 .. +4 lie in one 8-column piece of the packed row
    *reinterpret_cast<uint2*>(ao + packed_off(t, 4 * c4, ks_out)) = make_uint2(w[0], w[1]);
  }
  zero_out_pads(ao, t, l, ks_l, ms, ks_ms, ks_out);
}

}  // namespace

hipError_t launch_pf_in(const Shape& s, const uint8_t* dense, const uint16_t* x, int64_t T,
                        const PfWork& pw, float* z, float* xc, hipStream_t st) {
  const int64_t rows = packed_rows(T);
  hipLaunchKernelGGL(k_pf_pack_x, dim3((unsigned)cdiv(rows * s.ks_in * 16, kBlock)), dim3(kBlock), 0, st,
                     x, T, s.d, s.ks_in, rows, pw.ax);
  PfGemmArgs a{};
  a.w = dense;
  a.a = pw.ax;
  a.ks = s.ks_in;
  a.tr_count = s.tr_in;
  a.n_m = cdiv(T, kGemmTile);
  a.n_n = cdiv(s.tr_in, kGemmTiles16);
  a.T = T;
  a.tr_r = s.tr_r; a.tr_dn = s.tr_dn;
  a.z = z; a.E = s.E;
  a.xc = xc; a.l = s.l;
  a.ao = pw.ao; a.ks_out = s.ks_out; a.hs_col0 = s.ks_l * kStepK;
  a.ms = s.ms; a.act = s.act; a.bg = s.beta_gate; a.bl = s.beta_lin;
  a.rbg = 1.f / s.beta_gate; a.rbl = 1.f / s.beta_lin;
  hipLaunchKernelGGL(k_pf_gemm<true>, dim3((unsigned)gemm_grid(a.n_m, a.n_n)), dim3(kGemmThreads), 0, st, a);
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
  a.n_grp = cdiv(a.n_tr, kPxTR);
  // the gathered gate/up input is addressed by 32-bit offsets from its start
  if (gu && T * (int64_t)(s.prec == 2 ? 64 : 128) * a.ks > (int64_t)UINT32_MAX) return hipErrorInvalidValue;
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
  // Work order: XCD x walks its share of the unit table in chunks of `chunk` units, each
  // chunk through every tile-row group (chunk_item).  With about one unit per expert (chunk
  // 1) a unit's groups run back to back and its activation rows stay in the XCD's L2; with
  // many units per expert the chunk spans them, so that the units of one expert read each
  // weight slice at about the same time.
  a.chunk = clampi((int)cdiv(a.n_assign, (int64_t)s.E * a.nu), 1, 8);
  const unsigned grid = (unsigned)chunk_grid(a.max_units, a.n_grp, a.chunk);
  if (s.prec == 2) {
    if (gu) hipLaunchKernelGGL((k_pf_exp<true, 2>), dim3(grid), dim3(kBlock), 0, st, a);
    else hipLaunchKernelGGL((k_pf_exp<false, 2>), dim3(grid), dim3(kBlock), 0, st, a);
  } else {
    if (gu) hipLaunchKernelGGL((k_pf_exp<true, 1>), dim3(grid), dim3(kBlock), 0, st, a);
    else hipLaunchKernelGGL((k_pf_exp<false, 1>), dim3(grid), dim3(kBlock), 0, st, a);
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
                     pw.ao, s.ks_l, s.ms, s.ks_ms, s.ks_out);
  return hipGetLastError();
}

hipError_t launch_pf_norm(const Shape& s, const uint8_t* dense, int64_t T, const Work& ws,
                          const PfWork& pw, hipStream_t st) {
  hipLaunchKernelGGL(k_pf_norm, dim3((unsigned)T), dim3(kBlock), 0, st, (const float*)ws.u,
                     reinterpret_cast<const uint16_t*>(dense + s.gamma_off), s.l, s.use_norm, s.eps,
                     pw.ao, s.ks_l, s.ms, s.ks_ms, s.ks_out);
  return hipGetLastError();
}

hipError_t launch_pf_out(const Shape& s, const uint8_t* dense, int64_t T, const PfWork& pw,
                         const OutSink& out, hipStream_t st) {
  PfGemmArgs a{};
  a.w = dense + s.in_bytes;
  a.a = pw.ao;
  a.ks = s.ks_out;
  a.tr_count = s.tr_out;
  a.n_m = cdiv(T, kGemmTile);
  a.n_n = cdiv(s.tr_out, kGemmTiles16);
  a.T = T;
  a.sink = out; a.d = s.d;
  hipLaunchKernelGGL(k_pf_gemm<false>, dim3((unsigned)gemm_grid(a.n_m, a.n_n)), dim3(kGemmThreads), 0, st, a);
  return hipGetLastError();
}

size_t pf_packed_bytes(const Shape& s, int64_t T, bool out) {
  return (size_t)packed_rows(T) * (out ? s.ks_out : s.ks_in) * kStepK * 2;
}

}  // namespace moe
