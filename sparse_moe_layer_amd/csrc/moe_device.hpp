// Device helpers shared by the gfx950 kernels of the LatentMoE layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_internal.hpp"

namespace moe {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t w) {
  return __builtin_bit_cast(bf16x2_t, w);
}

// a.lo*b.lo + a.hi*b.hi + c with bf16 pairs, fp32 accumulate (exact bf16 products).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(a), as_bf16x2(b), c, false);
}

// Butterfly sum over the 64 lanes; every lane receives the same, order-fixed result.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// E8M0 byte -> the fp32 whose exponent field is that byte (2^(e-127) for e in 1..254).
__device__ __forceinline__ float e8m0_as_f32(uint32_t e) { return __uint_as_float(e << 23); }

__device__ __forceinline__ float sigmoidf_(float g) { return 1.0f / (1.0f + expf(-g)); }

// SiTU-GLU (act 0) or SwiGLU (act 1) of one gate/up pair.
__device__ __forceinline__ float glu_act(float g, float u, int act, float bg, float bl) {
  if (act == 0) {
    float a = bg * tanhf(g / bg) * sigmoidf_(g);
    return a * (bl * tanhf(u / bl));
  }
  return g * sigmoidf_(g) * u;
}

}  // namespace moe
