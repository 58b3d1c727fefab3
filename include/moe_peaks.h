/*
 * moe_peaks.h - C ABI of libmoe_peaks.so: peak-rate probes of one MI355X (gfx950).
 *
 * These are the measuring instruments of the benchmark, not part of the layer: a plain
 * HBM read stream and loops of matrix-core instructions with no memory traffic.  Their
 * rates are the "measured peaks" that the layer's roofline fractions are quoted against
 * next to the published figures (8 TB/s HBM; dense matrix cores 2.5 PFLOP/s bf16, 5.0 fp8,
 * 10.1 fp4).
 *
 * Conventions: device pointers, asynchronous on `stream` (a hipStream_t), no host
 * synchronisation, nothing allocated.  Return 0 on success, 1 for an invalid argument
 * (nothing launched), 4 when the launch fails.
 */
#ifndef MOE_PEAKS_H_
#define MOE_PEAKS_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* moe_peaks_stream_t; /* the same type as hipStream_t */

/* Matrix-core instruction of a probe loop (dense, no sparsity). */
typedef enum moe_peak_kind {
  MOE_PEAK_BF16_16X16X32 = 0,      /* v_mfma_f32_16x16x32_bf16 */
  MOE_PEAK_BF16_32X32X16 = 1,      /* v_mfma_f32_32x32x16_bf16 */
  MOE_PEAK_FP8_FP8_16X16X128 = 2,  /* scaled 16x16x128, both operands E4M3 */
  MOE_PEAK_FP8_FP4_16X16X128 = 3,  /* scaled 16x16x128, A E4M3, B E2M1 (the layer's mx8 experts) */
  MOE_PEAK_FP4_FP4_16X16X128 = 4,  /* scaled 16x16x128, both operands E2M1 */
  MOE_PEAK_FP8_FP8_32X32X64 = 5,   /* scaled 32x32x64, both operands E4M3 */
  MOE_PEAK_FP4_FP4_32X32X64 = 6,   /* scaled 32x32x64, both operands E2M1 */
  MOE_PEAK_NUM_KINDS = 7
} moe_peak_kind;

/* Read `bytes` (a multiple of 16, 16-byte aligned) from src with non-temporal 16-byte loads,
 * `grid` workgroups of 256 lanes walking the buffer with a grid stride; each lane writes the
 * XOR of what it read to out[lane id] (out: at least grid * 256 words), so that no load can
 * be dropped.  Errors: 1 for a null or misaligned pointer, grid < 1 or out_words too small. */
int moe_peak_read(const void* src, size_t bytes, uint32_t* out, size_t out_words, int32_t grid,
                  moe_peaks_stream_t stream);

/* `grid` workgroups of 4 wavefronts; every wavefront issues `iters` rounds of 8 independent
 * instructions of `kind` on register operands, then writes one float per lane to out[lane id]
 * (out: at least grid * 256 floats).  *flops receives the floating-point operations of the
 * launch (2 per multiply-add).  Errors: 1 for an unknown kind, grid < 1, iters < 1, a null
 * pointer or out_words too small. */
int moe_peak_mfma(int32_t kind, int32_t grid, int32_t iters, float* out, size_t out_words,
                  double* flops, moe_peaks_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_PEAKS_H_ */
