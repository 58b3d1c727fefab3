// Device helpers shared by the gfx950 kernels of the LatentMoE layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_internal.hpp"

namespace moe {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t w) {
  return __builtin_bit_cast(bf16x2_t, w);
}

// a.lo*b.lo + a.hi*b.hi + c with bf16 pairs, fp32 accumulate (exact bf16 products).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(a), as_bf16x2(b), c, false);
}

// Two floats rounded to bf16 (round to nearest even) in one 32-bit word, a in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2_t v;
  v.x = (__bf16)a;
  v.y = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

// Delta of element i to where the OUT step puts it (OutSink, moe_internal.hpp).
__device__ __forceinline__ void store_out(const OutSink& o, int64_t i, float v) {
  if (o.delta) o.delta[i] = v;
  if (o.res) {
    const float r = o.res[i] + v;
    o.res[i] = r;
    if (o.xn) o.xn[i] = (uint16_t)(pack_bf16x2(r, 0.f) & 0xFFFFu);
  }
}
// The same for four consecutive columns i .. i + 3 (i a multiple of 4: 16-byte stores).
__device__ __forceinline__ void store_out4(const OutSink& o, int64_t i, float4 v) {
  if (o.delta) *reinterpret_cast<float4*>(o.delta + i) = v;
  if (o.res) {
    float4 r = *reinterpret_cast<const float4*>(o.res + i);
    r.x += v.x; r.y += v.y; r.z += v.z; r.w += v.w;
    *reinterpret_cast<float4*>(o.res + i) = r;
    if (o.xn) *reinterpret_cast<uint2*>(o.xn + i) = make_uint2(pack_bf16x2(r.x, r.y), pack_bf16x2(r.z, r.w));
  }
}

// D += A B for one 16x16x32 bf16 block (fp32 accumulation); A rows and B columns are
// held as 8 consecutive K values per lane (lane l: row / column l % 16, K 8 (l / 16)..).
__device__ __forceinline__ f32x4_t mfma_bf16(uint4 a, uint4 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Eight E2M1 codes (one 32-bit word, low nibble first) times the E8M0 scale, as bf16.
// E2M1 x 2^(e-127) is exact in bf16 for every code and every scale byte 1..254 whose
// product stays below the bf16 maximum.
__device__ __forceinline__ uint4 fp4x8_to_bf16(uint32_t codes, float scale) {
  const bf16x2_t b0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 0);
  const bf16x2_t b1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 1);
  const bf16x2_t b2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 2);
  const bf16x2_t b3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 3);
  return make_uint4(__builtin_bit_cast(uint32_t, b0), __builtin_bit_cast(uint32_t, b1),
                    __builtin_bit_cast(uint32_t, b2), __builtin_bit_cast(uint32_t, b3));
}

// Eight E4M3 codes (two 32-bit words, lowest byte first) as bf16, exactly (every E4M3
// value has at most 4 significant bits and an exponent within the bf16 range).
__device__ __forceinline__ uint4 fp8x8_to_bf16(uint32_t lo, uint32_t hi) {
  const bf16x2_t b0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  const bf16x2_t b1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  const bf16x2_t b2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  const bf16x2_t b3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  return make_uint4(__builtin_bit_cast(uint32_t, b0), __builtin_bit_cast(uint32_t, b1),
                    __builtin_bit_cast(uint32_t, b2), __builtin_bit_cast(uint32_t, b3));
}

// Streaming (non-temporal) loads for weights that are read once per call.
__device__ __forceinline__ uint4 ld_stream(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint32_t ld_stream32(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
}

// ---- wavefront reductions through DPP row shifts and row broadcasts -----------------
// The partial results travel lane i-1 -> i inside each 16-lane row, then row 0 -> 1,
// row 2 -> 3 and rows 0+1 -> 2, 3; lane 63 ends with the total.  The order of the
// additions is fixed, so the result is deterministic.
template <int CTRL, int ROW_MASK, bool BOUND>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t old, uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, CTRL, ROW_MASK, 0xF, BOUND);
}
template <int CTRL, int ROW_MASK, bool BOUND>
__device__ __forceinline__ float dpp_f32(float v) {
  return __uint_as_float(dpp_u32<CTRL, ROW_MASK, BOUND>(0u, __float_as_uint(v)));
}

constexpr int kDppRowShr1 = 0x111, kDppRowShr2 = 0x112, kDppRowShr4 = 0x114,
              kDppRowShr8 = 0x118, kDppRowBcast15 = 0x142, kDppRowBcast31 = 0x143;

__device__ __forceinline__ float wave_sum_to_lane63(float v) {
  v += dpp_f32<kDppRowShr1, 0xF, true>(v);
  v += dpp_f32<kDppRowShr2, 0xF, true>(v);
  v += dpp_f32<kDppRowShr4, 0xF, true>(v);
  v += dpp_f32<kDppRowShr8, 0xF, true>(v);
  v += dpp_f32<kDppRowBcast15, 0xA, false>(v);
  v += dpp_f32<kDppRowBcast31, 0xC, false>(v);
  return v;
}

// Sum over the 64 lanes, returned to every lane (wavefront-uniform).
__device__ __forceinline__ float wave_sum(float v) {
  return __uint_as_float(
      (uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(wave_sum_to_lane63(v)), 63));
}

template <int CTRL, int ROW_MASK, bool BOUND>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  const uint32_t lo = dpp_u32<CTRL, ROW_MASK, BOUND>(0u, (uint32_t)v);
  const uint32_t hi = dpp_u32<CTRL, ROW_MASK, BOUND>(0u, (uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// Maximum of an unsigned 64-bit key over the 64 lanes (0 is the identity).
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  v = max_u64(v, dpp_u64<kDppRowShr1, 0xF, true>(v));
  v = max_u64(v, dpp_u64<kDppRowShr2, 0xF, true>(v));
  v = max_u64(v, dpp_u64<kDppRowShr4, 0xF, true>(v));
  v = max_u64(v, dpp_u64<kDppRowShr8, 0xF, true>(v));
  v = max_u64(v, dpp_u64<kDppRowBcast15, 0xA, false>(v));
  v = max_u64(v, dpp_u64<kDppRowBcast31, 0xC, false>(v));
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 63);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 63);
  return ((uint64_t)hi << 32) | lo;
}

// Unsigned key with the order of the float (after -0 -> +0).
__device__ __forceinline__ uint32_t float_order_key(float f) {
  const uint32_t u = __float_as_uint(f + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// E8M0 byte -> the fp32 whose exponent field is that byte (2^(e-127) for e in 1..254).
__device__ __forceinline__ float e8m0_as_f32(uint32_t e) { return __uint_as_float(e << 23); }

__device__ __forceinline__ float sigmoidf_(float g) { return 1.0f / (1.0f + expf(-g)); }

// SiTU-GLU (act 0) or SwiGLU (act 1) of one gate/up pair.
__device__ __forceinline__ float glu_act(float g, float u, int act, float bg, float bl) {
  if (act == 0) {
    const float a = bg * tanhf(g / bg) * sigmoidf_(g);
    return a * (bl * tanhf(u / bl));
  }
  return g * sigmoidf_(g) * u;
}

// The weight operand of one K-step of one tile row.  WF: 0 bf16, 1 MXFP4, 2 FP8 E4M3 with
// 128 x 128 block scales.
//   bf16: four 16x16x32 MFMAs, sub-tile s (1 KiB) with lane l holding row l % 16, columns
//     32s + 8 (l / 16) .. +8.
//   MXFP4: lane l holds one whole MX block, the 32 codes of row l % 16, columns 32 (l / 16)
//     .. +32, and its scale (byte l / 16 of the row's scale word); the four MFMAs take codes
//     8s .. 8s+7 of every lane, i.e. columns 32 (l / 16) + 8s .. +8, so the activation
//     operand is read with the roles of s and l / 16 swapped (a_piece).  The same bytes are
//     the B operand of the scaled 16x16x128 FP4 MFMA, which takes the whole block at once.
//   FP8: lane l holds 32 codes, 8 per sub-tile in the bf16 order (columns 32s + 8 (l / 16)
//     .. +8), converted exactly to bf16; a K-step lies in one 128 x 128 block of the rows of
//     each half of the tile row (gate rows in lanes l % 16 < 8, up rows in the others, or one
//     block for plain tile rows), so the K-step's partial sum is scaled by its block's fp32
//     scale and added to the running sum.
template <int WF>
struct WeightStep {
  static constexpr bool kFp4 = WF == 1, kFp8 = WF == 2;
  static constexpr int SB = kFp4 ? kFp4StepBytes : kFp8 ? kFp8StepBytes : kBf16StepBytes;
  static constexpr int NW = kFp4 ? 1 : kFp8 ? 2 : 4;
  uint4 w[NW];
  uint32_t sc;
  // K-step q of the tile row.  Streaming (non-temporal) loads where every weight is read
  // once per call; cached loads where several workgroups read the same weights in a short
  // window (the compute-bound launches).
  template <bool CACHED = false>
  __device__ __forceinline__ void load(const uint8_t* trow, int q, int lane) {
    const uint8_t* p = trow + (size_t)q * SB;
    if (kFp4) {
      w[0] = CACHED ? *reinterpret_cast<const uint4*>(p + lane * 16) : ld_stream(p + lane * 16);
      sc = CACHED ? *reinterpret_cast<const uint32_t*>(p + 1024 + (lane & 15) * 4)
                  : ld_stream32(p + 1024 + (lane & 15) * 4);
    } else if (kFp8) {
      w[0] = ld_stream(p + lane * 32);
      w[1] = ld_stream(p + lane * 32 + 16);
      sc = ld_stream32(p + 2048 + ((lane & 15) >= 8 ? 4 : 0));
    } else {
#pragma unroll
      for (int s = 0; s < NW; ++s)
        w[s] = CACHED ? *reinterpret_cast<const uint4*>(p + s * 1024 + lane * 16)
                      : ld_stream(p + s * 1024 + lane * 16);
    }
  }
  // the lane's E8M0 scale as an fp32 power of two (MXFP4), or its fp32 block scale (FP8)
  __device__ __forceinline__ float scale(int g) const {
    return kFp8 ? __uint_as_float(sc) : e8m0_as_f32((sc >> (8 * g)) & 0xFFu);
  }
  // the B operand of MFMA s
  __device__ __forceinline__ uint4 operand(int s, float scl) const {
    if (kFp4) {
      const uint32_t cd = s == 0 ? w[0].x : s == 1 ? w[0].y : s == 2 ? w[0].z : w[0].w;
      return fp4x8_to_bf16(cd, scl);
    }
    if (kFp8) {
      const uint4 v = w[s >> 1];
      return fp8x8_to_bf16((s & 1) ? v.z : v.x, (s & 1) ? v.w : v.y);
    }
    return w[s];
  }
  // The 8-column piece (0..15) of the K-step that lane group g feeds to MFMA s.
  static __device__ __forceinline__ int a_piece(int s, int g) { return kFp4 ? 4 * g + s : 4 * s + g; }
  // acc + A W^T over the K-step: ap points at piece 0 of the lane's staged row, pieces
  // `stride` words apart.
  __device__ __forceinline__ f32x4_t mma(const uint4* ap, int stride, int g, f32x4_t acc) const {
    const float scl = kFp4 ? scale(g) : 0.f;
    f32x4_t part = kFp8 ? f32x4_t{0.f, 0.f, 0.f, 0.f} : acc;
#pragma unroll
    for (int s = 0; s < 4; ++s) part = mfma_bf16(ap[a_piece(s, g) * stride], operand(s, scl), part);
    if (kFp8) return scale_add(part, scale(g), acc);
    return part;
  }
  // acc + scale * part (the FP8 block scale applied to a K-step's partial sums)
  static __device__ __forceinline__ f32x4_t scale_add(f32x4_t part, float scl, f32x4_t acc) {
    return f32x4_t{fmaf(scl, part[0], acc[0]), fmaf(scl, part[1], acc[1]),
                   fmaf(scl, part[2], acc[2]), fmaf(scl, part[3], acc[3])};
  }
};

// Lanes c >= 8 receive the value of lane c - 8 of their 16-lane row (gate -> up lane).
__device__ __forceinline__ float from_gate_lane(float v) {
  return __uint_as_float(dpp_u32<kDppRowShr8, 0xF, true>(0u, __float_as_uint(v)));
}

// Workgroups go round-robin to the 8 XCDs (each with its own L2).  A launch over
// n_groups x n_blk items (tile-row groups x token blocks) maps workgroup bid to the item
// so that all token blocks of one group run on one XCD, back to back: the group's
// weights come from HBM once and from that XCD's L2 for the other blocks.  The launch has
// 8 * ceil(n_groups / 8) * n_blk workgroups; the padding ones return false.
constexpr int kXcds = 8;
__device__ __forceinline__ bool xcd_item(int bid, int n_groups, int n_blk, int& grp, int& blk) {
  const int x = bid % kXcds, j = bid / kXcds;
  const int gi = j / n_blk;
  blk = j - gi * n_blk;
  grp = x + kXcds * gi;
  return grp < n_groups;
}
__host__ inline int64_t xcd_grid(int64_t n_groups, int64_t n_blk) {
  return kXcds * ((n_groups + kXcds - 1) / kXcds) * n_blk;
}
// The same with groups taken G at a time: XCD x walks blocks x, x + 8, ... of G consecutive
// groups, each block tile by tile, the G groups of a tile back to back, so that workgroups
// in flight on the XCD share each activation tile G ways while the block's weights stay in
// its L2.  G = 1 is xcd_item.
__device__ __forceinline__ bool xcd_gblock_item(int bid, int n_groups, int n_blk, int G, int& grp,
                                                int& blk) {
  const int x = bid % kXcds, j = bid / kXcds;
  const int bi = j / (G * n_blk), r = j - bi * G * n_blk;
  blk = r / G;
  grp = (x + kXcds * bi) * G + (r - blk * G);
  return grp < n_groups;
}
__host__ inline int64_t xcd_gblock_grid(int64_t n_groups, int64_t n_blk, int64_t G) {
  const int64_t nb = (n_groups + G - 1) / G;
  return kXcds * ((nb + kXcds - 1) / kXcds) * G * n_blk;
}

// Work order over (unit, tile-row group) items when the number of units is known only on
// the device: XCD x takes a contiguous range of the units (so of the experts, the unit
// table being sorted by expert) and walks it in chunks of `chunk` units, each chunk
// through every tile-row group: a chunk's activation rows stay in that XCD's L2 across
// the groups, and the units of one expert in a chunk read each weight slice close
// together in time.  Items past a range return false (they come last on each XCD).
__device__ __forceinline__ bool chunk_item(int bid, int n_units, int n_grp, int chunk, int& grp,
                                           int& u) {
  const int x = bid % kXcds, j = bid / kXcds;
  const int per_xcd = (n_units + kXcds - 1) / kXcds;
  const int c = j / (chunk * n_grp), r = j - c * chunk * n_grp;
  grp = r / chunk;
  const int ui = c * chunk + (r - grp * chunk);
  u = x * per_xcd + ui;
  return ui < per_xcd && u < n_units;
}
// Work order where XCD x owns a contiguous block of the tile-row groups and walks the units
// in table order, each unit through its block of groups back to back: a unit's activation
// rows are fetched once per XCD, and the XCD's slice of an expert's weights stays in its L2
// while the expert's units pass.  Items past the groups or the units return false.
__device__ __forceinline__ bool xcd_block_item(int bid, int n_grp, int n_units, int& grp, int& u) {
  const int x = bid % kXcds, j = bid / kXcds;
  const int gx = (n_grp + kXcds - 1) / kXcds;
  u = j / gx;
  grp = x * gx + (j - u * gx);
  return grp < n_grp && u < n_units;
}
__host__ inline int64_t xcd_block_grid(int64_t n_grp, int64_t max_units) {
  return kXcds * ((n_grp + kXcds - 1) / kXcds) * max_units;
}
__host__ inline int64_t chunk_grid(int64_t max_units, int64_t n_grp, int64_t chunk) {
  const int64_t per_xcd = (max_units + kXcds - 1) / kXcds;
  return kXcds * ((per_xcd + chunk - 1) / chunk) * chunk * n_grp;
}

}  // namespace moe
