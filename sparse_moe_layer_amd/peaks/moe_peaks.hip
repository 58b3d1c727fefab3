// Peak-rate probes of one MI355X (declarations and contract in include/moe_peaks.h): an HBM
// read stream and loops of matrix-core instructions, the instruments that put the layer's
// achieved rates beside what this GPU reaches at all.
#include <hip/hip_runtime.h>

#include "moe_peaks.h"

#define MOE_PEAKS_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));

constexpr int kBlock = 256;
constexpr int kChains = 8;   // independent accumulators per wavefront (cover the MFMA latency)

__device__ __forceinline__ uint32_t xor4(u32x4_t v) { return v.x ^ v.y ^ v.z ^ v.w; }
// every element of an accumulator is used, so that each stays one register block in the loop
__device__ __forceinline__ float sum4(f32x4_t v) { return (v[0] + v[1]) + (v[2] + v[3]); }
__device__ __forceinline__ float sum16(f32x16_t v) {
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += v[i];
  return s;
}

// Grid-stride read of n16 16-byte words, kReadDepth loads in flight per lane.
constexpr int kReadDepth = 8;
__global__ __launch_bounds__(kBlock) void k_peak_read(const u32x4_t* __restrict__ src, int64_t n16,
                                                      uint32_t* __restrict__ out) {
  const int64_t tid = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * kBlock;
  uint32_t acc = 0;
  int64_t i = tid;
  for (; i + (kReadDepth - 1) * stride < n16; i += kReadDepth * stride) {
    u32x4_t v[kReadDepth];
#pragma unroll
    for (int j = 0; j < kReadDepth; ++j) v[j] = __builtin_nontemporal_load(src + i + j * stride);
#pragma unroll
    for (int j = 0; j < kReadDepth; ++j) acc ^= xor4(v[j]);
  }
  for (; i < n16; i += stride) acc ^= xor4(__builtin_nontemporal_load(src + i));
  out[tid] = acc;
}

// Operand words that depend on the lane (so nothing is a compile-time constant); every
// byte pattern is a finite value in each format used (E4M3 0x38 = 1.0, E2M1 0x2 = 1.0,
// bf16 0x3F80 = 1.0), so the sums stay finite.
template <int KIND>
__global__ __launch_bounds__(kBlock) void k_peak_mfma(int iters, float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int64_t tid = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  float s = 0.f;
  if constexpr (KIND == MOE_PEAK_BF16_16X16X32 || KIND == MOE_PEAK_BF16_32X32X16) {
    const uint32_t w = 0x3F803F80u ^ (uint32_t)(lane & 1), w2 = w ^ 2u;
    const bf16x8_t a = __builtin_bit_cast(bf16x8_t, make_uint4(w, w, w, w));
    const bf16x8_t b = __builtin_bit_cast(bf16x8_t, make_uint4(w2, w2, w2, w2));
    if constexpr (KIND == MOE_PEAK_BF16_16X16X32) {
      f32x4_t acc[kChains] = {};
      for (int it = 0; it < iters; ++it)
#pragma unroll
        for (int c = 0; c < kChains; ++c)   // (the accumulator tied in place: with the
          // builtin the register allocator rotates the blocks through copies in this loop)
          asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc[c]) : "v"(a), "v"(b));
#pragma unroll
      for (int c = 0; c < kChains; ++c) s += sum4(acc[c]);
    } else {
      f32x16_t acc[kChains] = {};
      for (int it = 0; it < iters; ++it)
#pragma unroll
        for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
#pragma unroll
      for (int c = 0; c < kChains; ++c) s += sum16(acc[c]);
    }
  } else {
    // A and B formats of the scaled instruction: 0 = E4M3, 4 = E2M1 (FP4 operands use the
    // first four words of the eight)
    constexpr int FA = (KIND == MOE_PEAK_FP4_FP4_16X16X128 || KIND == MOE_PEAK_FP4_FP4_32X32X64) ? 4 : 0;
    constexpr int FB = (KIND == MOE_PEAK_FP8_FP8_16X16X128 || KIND == MOE_PEAK_FP8_FP8_32X32X64) ? 0 : 4;
    const int w8 = 0x38383838 ^ (lane & 1), w4 = 0x22222222 ^ (lane & 1);
    const int v8 = w8 ^ 2, v4 = w4 ^ 2;   // B differs from A (distinct registers)
    const i32x8_t a = FA == 0 ? i32x8_t{w8, w8, w8, w8, w8, w8, w8, w8} : i32x8_t{w4, w4, w4, w4, 0, 0, 0, 0};
    const i32x8_t b = FB == 0 ? i32x8_t{v8, v8, v8, v8, v8, v8, v8, v8} : i32x8_t{v4, v4, v4, v4, 0, 0, 0, 0};
    if constexpr (KIND == MOE_PEAK_FP8_FP8_32X32X64 || KIND == MOE_PEAK_FP4_FP4_32X32X64) {
      f32x16_t acc[kChains] = {};
      for (int it = 0; it < iters; ++it)
#pragma unroll
        for (int c = 0; c < kChains; ++c)
          acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[c], FA, FB, 0, 127, 0, 127);
#pragma unroll
      for (int c = 0; c < kChains; ++c) s += sum16(acc[c]);
    } else {
      f32x4_t acc[kChains] = {};
      if constexpr (KIND == MOE_PEAK_FP4_FP4_16X16X128) {
        // both operands four registers: the accumulator tied in place as for bf16 above
        const u32x4_t a4 = {(uint32_t)a[0], (uint32_t)a[1], (uint32_t)a[2], (uint32_t)a[3]};
        const u32x4_t b4 = {(uint32_t)b[0], (uint32_t)b[1], (uint32_t)b[2], (uint32_t)b[3]};
        const int one = 127;   // E8M0 1.0
        for (int it = 0; it < iters; ++it)
#pragma unroll
          for (int c = 0; c < kChains; ++c)
            asm volatile("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %3 op_sel_hi:[0,0,0] cbsz:4 blgp:4"
                         : "+a"(acc[c]) : "v"(a4), "v"(b4), "v"(one));
      } else {
        for (int it = 0; it < iters; ++it)
#pragma unroll
          for (int c = 0; c < kChains; ++c) {
            acc[c] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc[c], FA, FB, 0, 127, 0, 127);
            asm volatile("" : "+a"(acc[c]));
          }
      }
#pragma unroll
      for (int c = 0; c < kChains; ++c) s += sum4(acc[c]);
    }
  }
  out[tid] = s;
}

// Multiply-adds of one instruction of each kind (M x N x K).
constexpr double kMacs[MOE_PEAK_NUM_KINDS] = {16.0 * 16 * 32, 32.0 * 32 * 16, 16.0 * 16 * 128,
                                              16.0 * 16 * 128, 16.0 * 16 * 128, 32.0 * 32 * 64,
                                              32.0 * 32 * 64};

}  // namespace

MOE_PEAKS_EXPORT int moe_peak_read(const void* src, size_t bytes, uint32_t* out, size_t out_words,
                                   int32_t grid, moe_peaks_stream_t stream) {
  if (!src || !out || bytes % 16 || ((uintptr_t)src % 16) || grid < 1 ||
      out_words < (size_t)grid * kBlock)
    return 1;
  hipLaunchKernelGGL(k_peak_read, dim3((unsigned)grid), dim3(kBlock), 0, (hipStream_t)stream,
                     static_cast<const u32x4_t*>(src), (int64_t)(bytes / 16), out);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

MOE_PEAKS_EXPORT int moe_peak_mfma(int32_t kind, int32_t grid, int32_t iters, float* out,
                                   size_t out_words, double* flops, moe_peaks_stream_t stream) {
  if (kind < 0 || kind >= MOE_PEAK_NUM_KINDS || grid < 1 || iters < 1 || !out || !flops ||
      out_words < (size_t)grid * kBlock)
    return 1;
  const dim3 g((unsigned)grid), b(kBlock);
  hipStream_t st = (hipStream_t)stream;
  switch (kind) {
    case 0: hipLaunchKernelGGL(k_peak_mfma<0>, g, b, 0, st, iters, out); break;
    case 1: hipLaunchKernelGGL(k_peak_mfma<1>, g, b, 0, st, iters, out); break;
    case 2: hipLaunchKernelGGL(k_peak_mfma<2>, g, b, 0, st, iters, out); break;
    case 3: hipLaunchKernelGGL(k_peak_mfma<3>, g, b, 0, st, iters, out); break;
    case 4: hipLaunchKernelGGL(k_peak_mfma<4>, g, b, 0, st, iters, out); break;
    case 5: hipLaunchKernelGGL(k_peak_mfma<5>, g, b, 0, st, iters, out); break;
    default: hipLaunchKernelGGL(k_peak_mfma<6>, g, b, 0, st, iters, out); break;
  }
  *flops = 2.0 * kMacs[kind] * kChains * (double)iters * (double)grid * (kBlock / 64);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}
