// Internal interface between the C ABI (moe_api.hip) and the kernels (moe_kernels.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;

// One MXFP4 "row group" step: 64 lanes x 16 bytes of codes (four rows' 8-column chunks
// per lane) followed by 16 x 4 bytes of E8M0 scales (four rows' scale of the 32-column
// block that each quad of lanes covers).
constexpr int kFp4StepBytes = 1024 + 64;

// Shape of one layer plus everything derived from it that the launches need.
struct Shape {
  int d, l, E, k, m, ms;
  int use_norm;
  float eps, route_scale, beta_gate, beta_lin;
  int act;    // 0 SiTU, 1 SwiGLU
  int wfmt;   // 0 bf16, 1 MXFP4
  // MXFP4 packing: steps (of 64 lanes x 8 columns) per row group of the two matrices
  int j_gu, j_dn;
  size_t gu_bytes;      // packed gate/up bytes of one expert
  size_t expert_bytes;  // packed bytes of one expert (256-byte multiple)
};

// Row-major views of the workspace of one forward call.
struct Work {
  float* xc;       // [T][l]
  float* hs;       // [T][ms]
  float* h;        // [T*k][m]   dispatch order
  float* eo;       // [T*k][l]   dispatch order
  float* u;        // [T][l]
  int32_t* perm;   // [T*k]
  int32_t* inv;    // [T*k]
  int32_t* counts; // [E]
  int32_t* offs;   // [E+1]
  float* z;        // [T][E]
  int32_t* chunk_hist;  // [n_chunks][E]
};

struct DenseW {
  const uint16_t* router;
  const uint16_t* wdn;
  const uint16_t* wup;
  const uint16_t* gamma;
  const uint16_t* sgu;
  const uint16_t* sdn;
  const uint8_t* experts;
};

// Tokens per dispatch chunk (so that a chunk holds at most 256 assignments).
inline int dispatch_chunk_tokens(int k) { return k >= 256 ? 1 : 256 / k; }

hipError_t launch_router(const Shape& s, const DenseW& w, const uint16_t* x, int64_t T,
                         const Work& ws, hipStream_t st);
// latent down + shared gate/up; for route_fused batches also the route and the dispatch
hipError_t launch_dense_x(const Shape& s, const DenseW& w, const uint16_t* x, int64_t T,
                          const float* bias, int32_t* idx, float* gw, const Work& ws,
                          hipStream_t st);
// The route step in its own launch (no dispatch).
bool route_fused(int64_t T, int k);
hipError_t launch_route(const Shape& s, const float* bias, int64_t T, const Work& ws,
                        int32_t* idx, float* gw, hipStream_t st);
hipError_t launch_dispatch(const Shape& s, const int32_t* idx, int64_t T, int32_t* counts,
                           int32_t* offs, int32_t* perm, int32_t* inv, int32_t* chunk_hist,
                           hipStream_t st);
hipError_t launch_expert_gu(const Shape& s, const DenseW& w, const int32_t* idx, int64_t T,
                            const Work& ws, hipStream_t st);
hipError_t launch_expert_down(const Shape& s, const DenseW& w, const int32_t* idx, int64_t T,
                              const Work& ws, hipStream_t st);
hipError_t launch_combine(const Shape& s, const float* gw, int64_t T, const Work& ws,
                          hipStream_t st);
hipError_t launch_out(const Shape& s, const DenseW& w, int64_t T, const Work& ws, float* delta,
                      hipStream_t st);
hipError_t launch_pack(const Shape& s, const void* gu, const void* gus, const void* dn,
                       const void* dns, int e0, int n, uint8_t* packed, hipStream_t st);

}  // namespace moe
