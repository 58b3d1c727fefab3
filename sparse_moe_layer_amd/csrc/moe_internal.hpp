// Internal interface between the C ABI (moe_api.hip) and the kernels (moe_kernels.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;
constexpr int kBlock = 256;             // 4 wavefronts per workgroup
constexpr int kTileRows = 16;           // weight rows per packed tile (MFMA 16x16x32)
constexpr int kStepK = 128;             // input columns per K-step
constexpr int kBf16StepBytes = 4096;    // bf16 K-step: 4 sub-tiles of 16 rows x 32 columns
constexpr int kFp4StepBytes = 1024 + 64;  // MXFP4 K-step: 16 rows x 128 codes + 16 x 4 scales
constexpr int kFp8StepBytes = 2048 + 16;  // FP8 block-128 K-step: 16 rows x 128 codes + the
                                          // gate-half and up-half block scales (fp32), padded
constexpr int kCtrlWords = 64;          // control words at the head of the workspace
// Control word kCtrlArrive (its own 128-byte line): the router workgroups of the IN launch of
// a few tokens that have stored their logits; zero between calls (the route zeroes it once
// all have arrived; a workspace starts with its control words zero).  The next word counts
// waits that ended at the spin limit.
constexpr int kCtrlArrive = 32;
constexpr int kMaxK = 64;               // experts per token the kernels are built for

__host__ __device__ inline int cdiv(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

// Shape of one layer plus everything derived from it that the launches need.
struct Shape {
  int d, l, E, k, m, ms;   // l: the experts' input / output width (d when not latent)
  int latent;              // 1: W_down_latent / norm / W_up_latent around the experts
  int use_norm;
  float eps, route_scale, beta_gate, beta_lin;
  int act;    // 0 SiTU, 1 SwiGLU
  int wfmt;   // 0 bf16, 1 MXFP4, 2 FP8 E4M3 with 128 x 128 block scales (routed experts)
  int prec;   // 0 fp32 activations; the mx profiles (bf16 u_hat / h_s, MX expert inputs):
              // 1 mx8 (MXFP8-E4M3), 2 mx4 (MXFP4-E2M1)
  // packed dense weights: IN = [router ; W_down_latent ; shared gate/up] over K = d,
  // OUT = [W_up_latent | W_shared_down] over K = l (padded) + m_s
  int ks_in, tr_r, tr_dn, tr_sh, tr_in;
  int zplanes;   // router K-ranges computed apart (partial logit planes summed by the route),
                 // each held as kZSub sub-planes (its K-range split in kZSub parts)
  int ks_l, ks_ms, ks_out, tr_out;
  size_t in_bytes, out_bytes, gamma_off, dense_bytes;
  // packed experts: gate/up tiles (8 gate + 8 up rows) over K = l, then down tiles over K = m
  int ks_gu, tr_gu, ks_edn, tr_edn;
  int step_bytes;       // bytes of one expert K-step (MXFP4 or bf16)
  size_t gu_bytes;      // packed gate/up bytes of one expert
  size_t expert_bytes;  // packed bytes of one expert (256-byte multiple)
};

// Operands of the mx launches (in the hi/lo slot of the workspace).  Code rows hold 128
// E4M3 bytes (mx8) or 64 bytes of two E2M1 codes (mx4, low nibble first) per K-step.
struct PfWork {
  uint8_t* xq;     // [T][128 ks_gu]    x^c codes (K-steps padded with zeros)
  uint8_t* xs;     // [T][4 ks_gu]      its E8M0 block scales
  uint8_t* hq;     // [T*k][128 ks_edn] h codes, dispatch order
  uint8_t* hsc;    // [T*k][4 ks_edn]
  uint8_t* ao;     // the OUT product's input [u_hat | h_s] in bf16, packed rows of ks_out
                   // K-steps (tiles of 16 rows, the packed weights' layout)
  uint8_t* ax;     // the tokens x, packed rows of ks_in K-steps
};
// Bytes of the packed rows of T tokens (rounded up to whole 256-row tiles) for the OUT
// product (out) or the IN product.
size_t pf_packed_bytes(const Shape& s, int64_t T, bool out);

// Row-major views of the workspace of one forward call.
struct Work {
  int32_t* ctrl;   // [kCtrlWords]: [0] unit count, [1] units in the first (short) list
  float* xc;       // [T][l]
  float* hs;       // [T][ms]
  float* h;        // [T*k][m]   dispatch order
  float* eo;       // [T*k][l]   dispatch order
  float* u;        // [T][l]
  float* uh;       // [T][l]     RMSNorm(u) * gamma (token-tiled launches)
  // token-tiled launches: fp32 activations as bf16 hi/lo row pairs [rows][2][width]
  uint16_t* xc_hl; // [T][2][l]
  uint16_t* hs_hl; // [T][2][ms]
  uint16_t* h_hl;  // [T*k][2][m]
  uint16_t* uh_hl; // [T][2][l]
  int32_t* perm;   // [T*k]
  int32_t* inv;    // [T*k]
  int32_t* counts; // [E]
  int32_t* offs;   // [E+1]
  float* z;        // [zplanes * kZSub][T][E] partial logits; plane 0 holds the logits after
                   // the route
  int32_t* chunk_hist;  // [n_chunks][E]
  int32_t* units;  // [max_units][4]: expert, first position, positions, 0
  PfWork pf;       // the mx8 operands (same memory as the hi/lo rows)
  float2* ys;      // few tokens: W_sd h_s partial sums [parts][T][d] (hi/lo rows' memory)
};

// Tokens per dispatch chunk (so that a chunk holds at most 256 assignments).
inline int dispatch_chunk_tokens(int k) { return k >= 256 ? 1 : 256 / k; }

inline int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }
// Tokens per workgroup of the IN launches (bf16 rows of d columns in LDS, next to the
// route's own LDS).
inline int in_tokens_per_block(const Shape& s) { return clampi(45056 / (s.ks_in * kStepK * 2), 1, 16); }
// With this few tokens the route and the dispatch run inside the IN launch, and every
// product stages all its activation rows at once (the decode launches); larger batches
// take the token-tiled launches.
// The mx profiles always take their own launches (moe_prefill.hip).
inline bool mx_profile(const Shape& s) { return s.prec != 0; }
inline bool route_fused(const Shape& s, int64_t T) {
  return s.prec == 0 && T <= 4 && T * s.k <= kBlock && T <= in_tokens_per_block(s);
}
inline bool token_tiled(const Shape& s, int64_t T) { return !route_fused(s, T); }
// Largest batch of the few-token launches.
constexpr int kFewTokens = 4;
// With few tokens of a latent layer (FP32 profile) the IN launch also takes the router rows
// and W_down_latent: its route workgroup waits for the router workgroups' arrivals.
inline bool in_takes_router(const Shape& s, int64_t T) {
  return s.prec == 0 && s.latent && route_fused(s, T);
}

// Wavefronts per tile row: split K until a single token's launch has enough wavefronts
// to keep every compute unit streaming (about 16 per CU), keeping at least 8 K-steps per
// wavefront.  The split depends on the matrix alone, never on the batch, so a token's
// result has the same bits in every batch (the summation order is fixed per matrix).
inline int choose_ksplit(int64_t tile_rows, int ks) {
  int ksplit = 1;
  while (ksplit < 4 && tile_rows * ksplit < 4096 && ks / (2 * ksplit) >= 8) ksplit *= 2;
  return ksplit;
}
// The OUT product's partial sums, added in order.  Without a latent or a shared expert: ks_a
// = all K-steps in parts of qper.  A latent layer with a shared expert (FP32 profile): the
// u_hat segment's ks_a = ks_l K-steps in parts of qper (its K-split), then the h_s segment in
// nsd parts of qper2; with few tokens the expert down launch forms those (h_s is ready after
// the IN launch) and the OUT launch adds them, the token-tiled OUT launch forms the same.
constexpr int kSdParts = 4;
struct OutParts {
  int ks_a, ksplit, qper, nsd, qper2;   // qper = cdiv(ks_a, ksplit)
};
inline OutParts out_parts(const Shape& s) {
  OutParts o;
  if (s.latent && s.ms > 0 && s.prec == 0) {
    // the u_hat segment alone is short: split while each part keeps 4 K-steps
    o.ks_a = s.ks_l;
    o.ksplit = 1;
    while (o.ksplit < 4 && s.tr_out * o.ksplit < 4096 && s.ks_l / (2 * o.ksplit) >= 4) o.ksplit *= 2;
    o.qper = cdiv(s.ks_l, o.ksplit);
    o.qper2 = cdiv(s.ks_ms, s.ks_ms < kSdParts ? s.ks_ms : kSdParts);
    o.nsd = cdiv(s.ks_ms, o.qper2);
  } else {
    o.ks_a = s.ks_out;
    o.ksplit = choose_ksplit(s.tr_out, s.ks_out);
    o.qper = cdiv(s.ks_out, o.ksplit);
    o.nsd = 0;
    o.qper2 = 0;
  }
  return o;
}
// Tokens per workgroup of the OUT launch of a few tokens (hi/lo rows of the K-steps it stages).
inline int out_tokens_per_block(const Shape& s) {
  return clampi(57344 / (out_parts(s).ks_a * kStepK * 4), 1, 8);
}
// Bytes of Work::ys for a call of T tokens (kept monotonic in T).
inline size_t sd_partial_bytes(const Shape& s, int64_t T) {
  const int64_t t = T < kFewTokens ? T : kFewTokens;
  return (size_t)out_parts(s).nsd * t * s.d * 8;
}
constexpr int kTiledUnitPositions = 32;
// Without a latent the gate/up input is the token (one bf16 row per position), so a unit of
// the token-tiled launches holds up to 64 positions: an expert's weights are read once per 64
// of its positions.  The launches whose input is hi/lo rows take such a unit in two halves.
constexpr int kTiledUnitPositionsSingle = 64;
// Positions per unit of the mx launches (at most 10 blocks of 16 rows in the expert tile);
// an expert's positions split into near-equal runs (even_units).  With more than two such
// units per expert on average the units hold at most 128 (8 blocks): an expert's weights
// are then read several times either way, and the shorter units measured faster there
// (1.3% on a share of 112 experts at 8192 tokens, where an expert averages 1170 positions).
constexpr int kPfUnitPositions = 160;
constexpr int kPfUnitPositionsMany = 128;
// Positions of one expert per unit of the expert launches (2 hi/lo rows each; one FP8
// row each in the mx launches).
inline int unit_positions(const Shape& s, int64_t T) {
  if (mx_profile(s))
    return T * s.k > (int64_t)2 * kPfUnitPositions * s.E ? kPfUnitPositionsMany : kPfUnitPositions;
  if (token_tiled(s, T)) return s.latent ? kTiledUnitPositions : kTiledUnitPositionsSingle;
  // few tokens: all rows of a unit staged at once (2 hi/lo rows of the widest expert
  // input per position, within 56 KiB of LDS)
  const int ks = s.ks_gu > s.ks_edn ? s.ks_gu : s.ks_edn;
  const int fit = clampi(57344 / (ks * kStepK * 4), 1, 4);
  const int t = T < 1 ? 1 : (int)T;
  return t < fit ? t : fit;
}
// Whether an expert's positions split into near-equal units (the mx launches, whose tile
// height follows the unit) or into full units and a tail.
inline bool even_units(const Shape& s) { return mx_profile(s); }
inline int64_t max_units(const Shape& s, int64_t T) {
  const int64_t n = T * s.k, nu = unit_positions(s, T);
  const int64_t b = n / nu + (n < s.E ? n : s.E);
  return b < n ? b : n;
}
// Units of at most this many positions form the first list of the unit table and take
// the expert kernel for few positions (all rows staged at once, no barrier in the K loop);
// in the token-tiled launches that is within 32 KiB of LDS, so that five workgroups share
// a compute unit.  The larger units take the token-tiled expert kernel.
inline int small_unit_positions(const Shape& s, int64_t T) {
  const int nu = unit_positions(s, T);
  if (mx_profile(s) || !token_tiled(s, T)) return nu;
  const int ks = s.ks_gu > s.ks_edn ? s.ks_gu : s.ks_edn;
  const int w = clampi(32768 / (ks * kStepK * 4), 1, 4);
  return w < nu ? w : nu;
}
// Bounds of the two lists: every expert has at most one unit shorter than nu positions,
// and a large unit holds more than small_unit_positions of them.
inline int64_t max_small_units(const Shape& s, int64_t T) {
  const int64_t n = T * s.k, w = small_unit_positions(s, T);
  if (w >= unit_positions(s, T)) return max_units(s, T);
  const int64_t b = n < s.E ? n : s.E;
  return b < max_units(s, T) ? b : max_units(s, T);
}
inline int64_t max_large_units(const Shape& s, int64_t T) {
  const int64_t n = T * s.k, w = small_unit_positions(s, T);
  if (w >= unit_positions(s, T)) return 0;
  const int64_t b = n / (w + 1);
  return b < max_units(s, T) ? b : max_units(s, T);
}

// Where the OUT step puts Delta: delta[i] (when not null) and, with a residual stream,
// res[i] += Delta and xn[i] = the new res[i] rounded to bf16 (the next layer's input;
// when not null).
struct OutSink {
  float* delta;
  float* res;
  uint16_t* xn;
};

// Bytes that the OUT launch of a few tokens also reads, in workgroups after those of its
// product, so that they sit in the caches when the next call starts (the next layer's router
// and W_down_latent rows); `flag` is always 0 (the value read is kept, never stored).
struct Prefetch {
  const uint8_t* p;
  size_t bytes;
  uint32_t* sink;
  int flag;
};

// router_only: the router rows alone (otherwise W_down_latent rides in the same launch)
hipError_t launch_router(const Shape& s, const uint8_t* dense, const uint16_t* x, int64_t T,
                         bool router_only, const Work& ws, hipStream_t st);
hipError_t launch_in(const Shape& s, const uint8_t* dense, const uint16_t* x, int64_t T,
                     const float* bias, int32_t* idx, float* gw, const Work& ws, hipStream_t st);
// Quantile Balancing statistics: counts of r = alpha - s into hist [E][bins] (added to
// what it holds), and the centred biases read from such counts over T tokens.
hipError_t launch_qb_hist(const Shape& s, const float* bias, int64_t T, int bins, int32_t* hist,
                          const Work& ws, hipStream_t st);
hipError_t launch_qb_readout(const Shape& s, const float* bias, int64_t T, int bins,
                             const int32_t* hist, float* new_bias, hipStream_t st);
hipError_t launch_route(const Shape& s, const float* bias, int64_t T, const Work& ws,
                        int32_t* idx, float* gw, hipStream_t st);
// The logit planes the route sums: the router launch's K-split, or 1 (mx profiles: plain
// logits).
inline int route_planes(const Shape& s) { return mx_profile(s) ? 1 : s.zplanes; }
// Sub-planes per logit plane: a plane's K-range in kZSub parts, stored apart and added in
// order by the route, ((z0 + z1) + z2) + z3 (the order in which the four wavefronts of a
// few-token router workgroup would add them), so that the token-tiled router can take each
// part in a workgroup of its own.
constexpr int kZSub = 4;
inline int route_subplanes(const Shape& s) { return mx_profile(s) ? 1 : kZSub; }
hipError_t launch_dispatch(const Shape& s, const int32_t* idx, int64_t T, int32_t* counts,
                           int32_t* offs, int32_t* perm, int32_t* inv, int32_t* chunk_hist,
                           int32_t* units, int32_t* ctrl, hipStream_t st);
// dense: the packed dense weights (the down launch of a few tokens also takes W_sd h_s)
hipError_t launch_expert(const Shape& s, const uint8_t* experts, const uint8_t* dense, bool gu,
                         int64_t T, const Work& ws, hipStream_t st);
// the combine, and for the token-tiled launches of the FP32 profile the norm
hipError_t launch_combine(const Shape& s, const uint8_t* dense, const float* gw, int64_t T,
                          const Work& ws, hipStream_t st);
hipError_t launch_out(const Shape& s, const uint8_t* dense, int64_t T, const Work& ws,
                      const OutSink& out, hipStream_t st, const Prefetch& pf = Prefetch{});
// Bytes of the packed dense weights that the first launch of a few-token forward reads (the
// router and W_down_latent tile rows at the start of the IN matrix).
inline size_t first_launch_dense_bytes(const Shape& s) {
  return (size_t)(s.tr_r + s.tr_dn) * s.ks_in * kBf16StepBytes;
}

// The mx launches (moe_prefill.hip).
hipError_t launch_pf_in(const Shape& s, const uint8_t* dense, const uint16_t* x, int64_t T,
                        const PfWork& pw, float* z, float* xc, hipStream_t st);
hipError_t launch_pf_quant(const Shape& s, const float* xc, int64_t T, const PfWork& pw,
                           hipStream_t st);
hipError_t launch_pf_expert(const Shape& s, const uint8_t* experts, bool gu, int64_t T,
                            const Work& ws, const PfWork& pw, hipStream_t st);
hipError_t launch_pf_norm(const Shape& s, const uint8_t* dense, int64_t T, const Work& ws,
                          const PfWork& pw, hipStream_t st);
// the combine and the norm of the mx launches in one pass (u itself is not stored)
hipError_t launch_pf_combine_norm(const Shape& s, const uint8_t* dense, const float* gw, int64_t T,
                                  const Work& ws, const PfWork& pw, hipStream_t st);
hipError_t launch_pf_out(const Shape& s, const uint8_t* dense, int64_t T, const PfWork& pw,
                         const OutSink& out, hipStream_t st);

// Packing.  Dense: canonical bf16 [rows][K] into the tiles of the IN or OUT matrix.
struct DenseSrc {
  const uint16_t* router;
  const uint16_t* wdn;
  const uint16_t* wup;
  const uint16_t* gamma;
  const uint16_t* sgu;
  const uint16_t* sdn;
};
hipError_t launch_pack_dense(const Shape& s, const DenseSrc& src, uint8_t* packed,
                             hipStream_t st);
hipError_t launch_pack_experts(const Shape& s, const void* gu, const void* gus, const void* dn,
                               const void* dns, int e0, int n, uint8_t* packed, hipStream_t st);

}  // namespace moe
