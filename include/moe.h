/*
 * moe.h - C ABI of the MI355X (gfx950) Stable LatentMoE FFN layer library (libmoe.so).
 *
 * The library computes the inference forward pass of one Kimi K3 Stable LatentMoE FFN
 * layer, as the Kimi K3 latent mixture-of-experts block card defines it (its "All 23
 * steps" equations and the code excerpt of KimiSparseMoeBlock.forward / moe_infer):
 *
 *   s = sigmoid(x W_r);  I = top_k(s + b);  G = s_I / sum(s_I)        (router)
 *   x^c = x W_down_latent                                           (latent down, d -> l)
 *   h_j = 4 tanh(g/4) sigmoid(g) * 25 tanh(u/25), g|u = x^c W_gate|up (routed SiTU-GLU)
 *   E_j = h_j W_down;   u = sum_j G_j E_j                            (latent combine)
 *   y_routed = RMSNorm(u) W_up_latent                                (norm, then l -> d)
 *   y_shared = SiTU-GLU(x) at full width (two shared experts merged into one)
 *   Delta = y_routed + y_shared
 *
 * Conventions shared by every entry point
 *   - All pointers are device pointers unless stated otherwise.  The caller allocates
 *     and owns every buffer; the library never allocates, frees or retains memory and
 *     keeps no state between calls outside the workspace the caller passes.
 *   - Matrices are row-major [out, in] as nn.Linear stores them.  bf16 is passed as its
 *     16-bit pattern.  Weight, token and output buffers must be 16-byte aligned.
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL is the null stream)
 *     and performs no host synchronisation.  Outputs are valid once the stream reaches
 *     them.  Calls on one stream are ordered; concurrent calls on different streams
 *     must use distinct workspaces and outputs.
 *   - Arguments are validated before anything is launched; on any error nothing is
 *     written and the status says why.  MOE_ERR_HIP reports a failed launch
 *     (hipGetLastError after the launches).  NaN or Inf inside the data are not
 *     checked: they propagate.
 *   - Results are deterministic: the same inputs give bit-identical outputs (no
 *     floating-point atomics; every sum has a fixed order).
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 7

typedef struct ihipStream_t* moe_stream_t; /* the same type as hipStream_t */

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1, /* null or misaligned pointer, negative size, k > E, ... */
  MOE_ERR_UNSUPPORTED = 2, /* a shape, format or precision combination not built */
  MOE_ERR_WORKSPACE = 3,   /* workspace or packed buffer smaller than required */
  MOE_ERR_HIP = 4          /* a HIP launch or runtime call failed */
} moe_status;

typedef enum moe_act {
  MOE_ACT_SITU = 0,  /* beta_gate tanh(g/beta_gate) sigmoid(g) * beta_lin tanh(u/beta_lin) */
  MOE_ACT_SWIGLU = 1 /* g sigmoid(g) u  (the K2 block card's expert activation) */
} moe_act;

typedef enum moe_wfmt {
  MOE_WFMT_BF16 = 0,  /* bf16 expert weights */
  MOE_WFMT_MXFP4 = 1, /* E2M1 codes, two per byte (low nibble = even column), plus one
                         E8M0 scale byte per 32 consecutive input columns of a row */
  MOE_WFMT_FP8_B128 = 2 /* FP8 E4M3 codes, one per byte, plus one fp32 scale per block of
                           128 x 128 weights (the K2 block card's expert format); the
                           scale multiplies the fp32 partial sums of its block */
} moe_wfmt;

typedef enum moe_precision {
  MOE_PREC_FP32 = 0, /* activations kept in fp32 between all steps; Delta in fp32 */
  MOE_PREC_MX8 = 1,  /* the compute-bound profile: the experts' input x^c and hidden h are
                        converted to MXFP8-E4M3 (blocks of 32 along K; OCP MX conversion:
                        scale 2^(floor(log2 amax) - 8), elements rounded to nearest even,
                        saturated at 448) and multiplied with the MXFP4 weights on the
                        scaled FP8 x FP4 matrix cores; u_hat and h_s are rounded to bf16
                        before W_up_latent and W_shared_down; everything else as FP32.
                        The walkthrough's deployment recipe: MXFP4 weights, MXFP8
                        activations.  Needs MXFP4 experts. */
  MOE_PREC_MX4 = 2   /* MX8 with MXFP4-E2M1 in place of MXFP8-E4M3 for x^c and h (the same
                        OCP MX rule with the E2M1 element: scale 2^(floor(log2 amax) - 2),
                        elements rounded to nearest even, saturated at 6), multiplied with
                        the MXFP4 weights on the scaled FP4 x FP4 matrix cores: both
                        operands in the walkthrough's weight format.  A reported variant,
                        not a default: its error against FP32 is about ten times MX8's.
                        Needs MXFP4 experts. */
} moe_precision;

/* Layer shape and options.  K3: d_model 7168, d_latent 3584, n_experts 896, top_k 16,
 * d_expert 3072, d_shared 6144 (two merged 3072-wide shared experts), SiTU with
 * beta_gate 4 and beta_lin 25, route_scale 1, use_latent_norm 1 (block card: parameter
 * table and config fields; walkthrough: SituAndMul and the activation_situ_* fields).
 * A non-latent block (d_latent 0; the K2 block card: 384 SwiGLU experts top-8, gate
 * scale 2.827, one shared expert) routes the token itself: the experts read x and write
 * d-wide rows, and Delta = sum_j G_j E_j + the shared path (no W_down_latent, norm or
 * W_up_latent; it needs a shared expert). */
typedef struct moe_config {
  int32_t d_model;         /* d: token width; multiple of 8 */
  int32_t d_latent;        /* l: latent width of the routed experts; multiple of 8; 0 for a
                              non-latent block (the experts then take the d-wide token) */
  int32_t n_experts;       /* E: routed experts, 1..1024 */
  int32_t top_k;           /* k: experts per token, 1..min(E, 64) */
  int32_t d_expert;        /* m: routed expert hidden width; multiple of 8 */
  int32_t d_shared;        /* m_s: shared hidden width (0 = no shared path); multiple of 8 */
  int32_t use_latent_norm; /* 1: RMSNorm between the latent sum and W_up_latent */
  float rms_eps;           /* RMSNorm epsilon */
  float route_scale;       /* multiplies the renormalised gate weights (1 for K3) */
  float beta_gate;         /* SiTU gate cap (4) */
  float beta_lin;          /* SiTU up-branch cap (25) */
  int32_t act;             /* moe_act */
  int32_t expert_wfmt;     /* moe_wfmt; MXFP4 needs the expert widths divisible by 32 */
  int32_t precision;       /* moe_precision */
} moe_config;

/* Canonical dense weights, bf16 [out, in] (as moe_pack_dense reads them).  Without a
 * latent (d_latent 0) w_down_latent, w_up_latent and norm_gamma are not read (may be
 * null). */
typedef struct moe_dense_src {
  const void* router;        /* W_r           [E, d]       bf16 */
  const void* w_down_latent; /* W_down_latent [l, d]       bf16 */
  const void* w_up_latent;   /* W_up_latent   [d, l]       bf16 */
  const void* norm_gamma;    /* RMSNorm gain  [l]          bf16 (copied even without norm) */
  const void* shared_gu;     /* shared gate rows then up rows [2 m_s, d] bf16 (m_s > 0) */
  const void* shared_down;   /* shared down   [d, m_s]     bf16 (m_s > 0) */
} moe_dense_src;

/* The weights of a forward call: both buffers in the packed layouts written by
 * moe_pack_dense and moe_pack_experts, 256-byte aligned. */
typedef struct moe_weights {
  const void* dense;
  const void* experts;
} moe_weights;

/* Canonical routed-expert storage for a run of consecutive experts, each pointer at
 * the first expert of the run.  Gate/up of an expert are stacked: rows 0..m-1 gate,
 * rows m..2m-1 up, each row l wide; down is [l, m].
 *   BF16:  gu = [n][2m][l] bf16, down = [n][l][m] bf16, scale pointers unused.
 *   MXFP4: gu = [n][2m][l/2] code bytes, gu_scale = [n][2m][l/32] E8M0 bytes,
 *          down = [n][l][m/2], down_scale = [n][l][m/32].
 *   FP8_B128: gu = [n][2m][l] E4M3 bytes, gu_scale = [n][ceil(2m/128)][ceil(l/128)] fp32,
 *          down = [n][l][m], down_scale = [n][ceil(l/128)][ceil(m/128)] fp32.
 * For a non-latent block l is d_model. */
typedef struct moe_expert_src {
  const void* gu;
  const void* gu_scale;
  const void* down;
  const void* down_scale;
} moe_expert_src;

/* ABI version of the library (MOE_ABI_VERSION it was built with). */
int moe_abi_version(void);

/* Static string naming a status code. */
const char* moe_status_str(moe_status s);

/* Bytes of the packed dense-weight buffer (host call, no launch).
 * Errors: MOE_ERR_INVALID_ARG (null pointer or invalid config), MOE_ERR_UNSUPPORTED. */
moe_status moe_packed_dense_size(const moe_config* cfg, size_t* bytes);

/* Rewrite the canonical dense weights into the tiled order the kernels stream (a
 * one-time copy per layer).  The packed buffer holds two matrices of 16-row tiles:
 *   IN  = [W_r ; W_down_latent ; shared gate/up] over the d input columns, and
 *   OUT = [W_up_latent | W_shared_down] over l (padded to 128) + m_s input columns,
 * plus a copy of the norm gain.  In a tile, every 16 rows x 32 columns form 1 KiB in
 * the operand order of the 16x16x32 bf16 matrix instruction; shared gate/up tiles carry
 * 8 gate rows and the matching 8 up rows.  Rows and columns past the matrices are zero.
 * packed: moe_packed_dense_size bytes, 256-byte aligned; sources 16-byte aligned.
 * Errors: MOE_ERR_INVALID_ARG (null or misaligned pointer), MOE_ERR_WORKSPACE
 * (packed_bytes too small), MOE_ERR_HIP. */
moe_status moe_pack_dense(const moe_config* cfg, const moe_dense_src* src, void* packed,
                          size_t packed_bytes, moe_stream_t stream);

/* Bytes of the packed routed-expert buffer for the whole layer (host call, no launch).
 * Errors: MOE_ERR_INVALID_ARG (null pointer or invalid config), MOE_ERR_UNSUPPORTED. */
moe_status moe_packed_experts_size(const moe_config* cfg, size_t* bytes);

/* Rewrite canonical experts e0..e0+n-1 into the kernel-native order inside `packed`
 * (a buffer of moe_packed_experts_size bytes for the whole layer, 256-byte aligned).
 * The run may be any sub-range, so a layer can be packed in pieces.  Each expert holds
 * gate/up tiles (8 gate rows + the matching 8 up rows over l columns) and then down
 * tiles (16 rows over m columns), in K-steps of 128 columns; MXFP4 K-steps are 1 KiB of
 * codes in the operand order of the matrix instruction plus the 16 rows' four scale
 * bytes, so one wavefront load brings both.  The code and scale bytes are moved, not
 * changed.  Errors: MOE_ERR_INVALID_ARG (null or misaligned pointer, range outside
 * 0..E), MOE_ERR_WORKSPACE (packed_bytes too small), MOE_ERR_HIP. */
moe_status moe_pack_experts(const moe_config* cfg, const moe_expert_src* src, int32_t e0,
                            int32_t n, void* packed, size_t packed_bytes, moe_stream_t stream);

/* Bytes of workspace that moe_layer_forward needs for up to max_tokens tokens.  A workspace
 * starts with its first 256 bytes (the control words, slot [0]) zero, e.g. cleared once after
 * it is allocated; every call leaves them that way.  (With at most 4 tokens of a latent layer
 * in MOE_PREC_FP32, one word counts the router workgroups that have stored their logits, and
 * the route waits for all of them.) */
moe_status moe_workspace_size(const moe_config* cfg, int64_t max_tokens, size_t* bytes);

/* Offsets (bytes) of the intermediates inside the workspace of a call with n_tokens,
 * for inspection after moe_layer_forward (host call).  Layouts, all row-major:
 *   [0] control words (internal: [0] = number of units of the expert launches, [1] = how
 *       many of them, first in the unit table, are short enough for the few-token kernel)
 *   [1] x^c    [T][l]   fp32     latent down-projection
 *   [2] h_s    [T][m_s] fp32     shared SiTU-GLU hidden
 *   [3] h      [T*k][m] fp32     routed expert hidden, rows in dispatch order
 *   [4] E      [T*k][l] fp32     routed expert outputs, rows in dispatch order
 *   [5] u      [T][l]   fp32     gated latent sum before the norm
 *   [6] u_hat  [T][l]   fp32     RMSNorm(u) * gamma (written for batches that take the
 *                                token-tiled launches, see moe_step)
 *   [7] FP32: bf16 row pairs (hi = bf16(v), lo = bf16(v - hi)) of x^c [T][2][l], h_s
 *                                [T][2][m_s], h [T*k][2][m] and u_hat [T][2][l], each part
 *                                256-aligned (token-tiled launches; internal)
 *       MX8:  x^c as E4M3 codes [T][128 ceil(l/128)] and E8M0 scales [T][4 ceil(l/128)],
 *             h as codes [T*k][128 ceil(m/128)] and scales [T*k][4 ceil(m/128)] (dispatch
 *             order; K-steps past l or m zero), u_hat bf16 [T][l], h_s bf16 [T][m_s],
 *             each part 256-aligned (internal); the slots [2] h_s and [3] h stay unused
 *       MX4:  as MX8 with rows of 64 bytes of E2M1 code pairs (low nibble first) per
 *             K-step of 128 in place of 128 E4M3 bytes, in the same parts
 *       FP32 with at most 4 tokens of a latent layer: partial sums of h_s W_shared_down
 *             over 4 ranges of m_s, float pairs (hi-row, lo-row sums) [4][T][d] (internal)
 *   [8] perm   [T*k]    int32    dispatch order -> assignment t*k+j
 *   [9] inv    [T*k]    int32    assignment -> dispatch order
 *  [10] counts [E]      int32    assignments per expert
 *  [11] offsets[E+1]    int32    exclusive scan of counts
 *  [12] z      [P][T][E] fp32   router logits as P partial planes over ranges of d (their
 *                                sum, added four at a time and then in order; P = 8 at
 *                                d = 7168); after the route, plane 0 holds the logits
 *  [13] per-chunk expert histograms of the dispatch (internal)
 *  [14] unit table of the expert launches (internal) */
#define MOE_WS_NUM_SLOTS 15
moe_status moe_workspace_layout(const moe_config* cfg, int64_t n_tokens,
                                size_t offsets[MOE_WS_NUM_SLOTS]);

/* The layer forward (block card: KimiSparseMoeBlock.forward), for n_tokens tokens.
 *   x         [T, d] bf16 tokens (batch and positions flattened, as the card's code does)
 *   bias      [E] fp32 selection bias (e_score_correction_bias; frozen at inference)
 *   delta     [T, d] fp32 output Delta_ffn = y_routed + y_shared
 *   topk_idx  [T, k] int32 selected experts, in descending s + b, ties to the lower index
 *   topk_w    [T, k] fp32 gate weights route_scale * s / sum(s) in the same order
 *   workspace at least moe_workspace_size(cfg, n_tokens) bytes, 256-byte aligned
 * n_tokens == 0 returns MOE_OK after checking cfg, launches nothing and touches no pointer.  Errors: MOE_ERR_INVALID_ARG,
 * MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP. */
moe_status moe_layer_forward(const moe_config* cfg, const moe_weights* w, const float* bias,
                             const void* x, int64_t n_tokens, float* delta, int32_t* topk_idx,
                             float* topk_w, void* workspace, size_t workspace_bytes,
                             moe_stream_t stream);

/* moe_layer_forward for callers that cannot allocate device memory (code under HIP graph
 * capture, serving loops or harnesses that forbid allocation): the same launches and the
 * same results as moe_layer_forward, with the intermediates in a buffer inside the library
 * instead of a caller's workspace.  Each GPU the library runs on holds one such buffer of
 * MOE_STATIC_WORKSPACE_BYTES (zero at load, kept until the process ends); the call
 * allocates nothing and frees nothing.
 *   - The buffer's device address is looked up once per device, on the first call with
 *     that device current; `stream` must belong to the current device.
 *   - Every call on one GPU shares its buffer and leaves the last call's intermediates in
 *     it.  Nothing in it has to start at zero (each step writes what a later step reads),
 *     but calls that overlap on one GPU (other streams, other threads) race on it and give
 *     undefined results: serialise them.
 *   - MOE_ERR_WORKSPACE when moe_workspace_size(cfg, n_tokens) exceeds
 *     MOE_STATIC_WORKSPACE_BYTES (K3 shape: up to 64 tokens fit), before anything runs.
 * Arguments, layouts and the other errors as moe_layer_forward. */
#define MOE_STATIC_WORKSPACE_BYTES ((size_t)64 << 20)
moe_status moe_layer_forward_noalloc(const moe_config* cfg, const moe_weights* w, const float* bias,
                                     const void* x, int64_t n_tokens, float* delta,
                                     int32_t* topk_idx, float* topk_w, moe_stream_t stream);

/* moe_layer_forward_residual that also starts streaming the next layer's weights during this
 * layer's tail (the chain of decoder blocks of the K3 model, the port notes' "Measured" and
 * "Not measured (and why)": decode streams every layer's weights in turn).  With few tokens
 * (the decode launches) the last launch of this call also reads the bytes of `next` that the
 * next call's first launch will read (its router and W_down_latent rows, about 64 MB at the K3
 * shape), in workgroups after those of its own product, so that the read fills that launch's
 * drain and leaves them in the GPU's caches.  `next`: the next layer's weights (same config),
 * or null for none; results are those of moe_layer_forward_residual, bit for bit.  Larger
 * batches ignore `next`.  Errors as moe_layer_forward_residual, MOE_ERR_INVALID_ARG for a
 * null or misaligned buffer in `next`. */
moe_status moe_layer_forward_residual_prefetch(const moe_config* cfg, const moe_weights* w,
                                               const float* bias, const void* x, int64_t n_tokens,
                                               float* residual, void* x_next, float* delta,
                                               int32_t* topk_idx, float* topk_w, void* workspace,
                                               size_t workspace_bytes, const moe_weights* next,
                                               moe_stream_t stream);

/* Steps of the forward, in launch order.  With few tokens (at most 4, fewer for very
 * wide d) each product stages all its activation rows at once; larger batches take
 * token-tiled launches (tiles of up to 64 tokens or 32 assignments of one expert, the
 * weights read once per tile) whose sums follow the same order, so a token's results
 * have the same bits in both.  Where the two differ it is said below.  MOE_PREC_MX8
 * maps the steps onto its own launches: ROUTER computes all products with the token
 * (router logits, x^c, h_s), IN converts x^c to MXFP8, EXPERT_GU converts h to MXFP8 in
 * its epilogue, COMBINE also normalises and rounds u_hat to bf16. */
typedef enum moe_step {
  MOE_STEP_ROUTER = 0,      /* router logits z = x W_r (partial planes), and in the same
                               launch x^c = x W_down_latent (larger batches: in IN; at most
                               4 tokens of a latent layer in MOE_PREC_FP32: nothing, IN
                               takes both) */
  MOE_STEP_IN = 1,          /* shared gate/up + SiTU; with few tokens one workgroup of the
                               same launch also takes the top-k, the gate weights and the
                               dispatch */
  MOE_STEP_ROUTE = 2,       /* sigmoid, top_k(s + b), gate weights (larger batches; launches
                               nothing otherwise) */
  MOE_STEP_DISPATCH = 3,    /* histogram, scan, stable permutation by expert (larger
                               batches; launches nothing otherwise) */
  MOE_STEP_EXPERT_GU = 4,   /* routed gate/up + SiTU */
  MOE_STEP_EXPERT_DOWN = 5, /* routed down; with few tokens of a latent layer (FP32) also the
                               partial sums of h_s W_shared_down, which OUT adds */
  MOE_STEP_COMBINE = 6,     /* u = sum_j G_j E_j (larger batches: and u_hat) */
  MOE_STEP_OUT = 7,         /* Delta = RMSNorm(u) W_up_latent + h_s W_shared_down */
  MOE_NUM_STEPS = 8
} moe_step;

/* moe_layer_forward with per-step timing: identical work and results, and additionally
 * records step_events[s] on `stream` just before step s is launched (s = 0..7) and
 * step_events[MOE_NUM_STEPS] after the last one.  step_events holds MOE_NUM_STEPS + 1
 * hipEvent_t handles created by the caller (with timing enabled), or NULL entries for
 * boundaries that need no event; they are only recorded, never synchronised on.  For
 * profilers and benchmarks; errors as moe_layer_forward. */
moe_status moe_layer_forward_timed(const moe_config* cfg, const moe_weights* w,
                                   const float* bias, const void* x, int64_t n_tokens,
                                   float* delta, int32_t* topk_idx, float* topk_w,
                                   void* workspace, size_t workspace_bytes,
                                   void* const* step_events, moe_stream_t stream);

/* moe_layer_forward with the residual add after the block fused into its last step: the
 * K3 block card's block output is Δ_ffn, which the decoder layer adds to its residual
 * stream (h <- h + Δ).  residual: device fp32 [T][d], read and written, residual += Δ
 * (one fp32 add per element).  x_next: device bf16 [T][d] or null: the updated residual
 * rounded to bf16 (nearest, ties to even), the next layer's input; it may be x itself
 * (x is read only before the last step).  delta: fp32 [T][d] or null (Δ then not
 * stored).  Layer after layer on one stream this chains a decoder's MoE blocks with no
 * extra pass over the activations.  Alignment 16 bytes for residual and x_next;
 * MOE_ERR_INVALID_ARG for a null residual (T > 0); otherwise as moe_layer_forward. */
moe_status moe_layer_forward_residual(const moe_config* cfg, const moe_weights* w,
                                      const float* bias, const void* x, int64_t n_tokens,
                                      float* residual, void* x_next, float* delta,
                                      int32_t* topk_idx, float* topk_w, void* workspace,
                                      size_t workspace_bytes, moe_stream_t stream);

/* Steps step_begin..step_end-1 of moe_layer_forward alone (0 <= begin <= end <= 8).
 * Each step reads what the earlier steps left in `workspace`, topk_idx and topk_w, so a
 * range that starts after step 0 is only meaningful on the buffers of an earlier call
 * with the same config, weights, tokens and n_tokens.  Running [0, MOE_NUM_STEPS) is
 * moe_layer_forward.  For profilers, benchmarks and callers that interleave the steps
 * of several layers; errors as moe_layer_forward, plus MOE_ERR_INVALID_ARG for a bad
 * range. */
moe_status moe_layer_forward_steps(const moe_config* cfg, const moe_weights* w,
                                   const float* bias, const void* x, int64_t n_tokens,
                                   float* delta, int32_t* topk_idx, float* topk_w,
                                   void* workspace, size_t workspace_bytes, int32_t step_begin,
                                   int32_t step_end, moe_stream_t stream);

/* The router step alone (block card: z = x W_r, s = sigmoid(z), top_k(s + b), and G;
 * toy chapter: the bias selects, the raw score weights).  Same arguments and output
 * layout as the corresponding ones of moe_layer_forward; the logits are left in the
 * workspace slot [12].  The router runs as in MOE_PREC_FP32 whatever cfg->precision
 * says (the profiles differ after the route). */
moe_status moe_route(const moe_config* cfg, const moe_weights* w, const float* bias,
                     const void* x, int64_t n_tokens, int32_t* topk_idx, float* topk_w,
                     void* workspace, size_t workspace_bytes, moe_stream_t stream);

/* The dispatch step alone (block card's moe_infer: per-expert histogram, then the
 * assignments ordered by expert).  From topk_idx [T, k] it writes counts [E], offsets
 * [E+1] (exclusive scan, offsets[E] = T*k), perm [T*k] (dispatch order -> assignment
 * t*k+j; within an expert, assignments in increasing t*k+j) and inv [T*k] (the inverse).
 * workspace: at least moe_workspace_size(cfg, n_tokens) bytes (its unit table and unit
 * count are rewritten too).  Every index in topk_idx must lie in 0..E-1; this is not
 * checked. */
moe_status moe_dispatch(const moe_config* cfg, const int32_t* topk_idx, int64_t n_tokens,
                        int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv,
                        void* workspace, size_t workspace_bytes, moe_stream_t stream);

/* Quantile Balancing statistics of the router (toy chapter "Quantile Balancing: giving
 * every expert a fair shot"; walkthrough "Stable 之三：Quantile Balancing" and its histogram
 * estimate).  The training-side step next to S1: it reads the router and the current
 * biases and leaves the forward untouched.
 *
 * moe_qb_histogram: the router of n_tokens tokens x (as in moe_route; workspace slot [12]
 * then holds the scores s = sigmoid(z), [T][E] fp32 in its first plane), then per token the cutoff alpha = the (k+1)-th largest
 * s + b (float32) and, for every expert e, r = alpha - s_e (float32: the bias expert e
 * needs to make the token's top k) counted into hist[e * n_bins + bin], with n_bins
 * uniform bins over [lo, hi] = [min(bias) - 1, max(bias) + 1] (float32) and bin =
 * floor((r - lo) * (n_bins / (hi - lo))) clamped to 0 .. n_bins - 1.  hist: device int32
 * [E][n_bins], ADDED to (the caller zeroes it; calls over several micro-batches with the
 * same biases accumulate, integer atomics, so the counts do not depend on the order).
 * Needs top_k < n_experts and top_k <= 63; 1 <= n_bins <= MOE_QB_MAX_BINS.  workspace:
 * at least moe_workspace_size(cfg, n_tokens) bytes.  n_tokens = 0 does nothing.
 *
 * moe_qb_readout: from such counts over n_tokens tokens in all, the new biases
 * new_bias[E] (device float32): per expert the first bin where the cumulative count
 * reaches ceil(n_tokens * k / E), at lo + w (t + (ceil(q) - C) / c_t) (w the bin width,
 * C the count below bin t, c_t the bin's), then the mean over the experts subtracted.
 * The estimate is within one bin width of the exact order statistic.  bias must be the
 * biases the counts were taken with (they fix lo and hi).  Asynchronous. */
#define MOE_QB_MAX_BINS 16384
moe_status moe_qb_histogram(const moe_config* cfg, const moe_weights* w, const float* bias,
                            const void* x, int64_t n_tokens, int32_t n_bins, int32_t* hist,
                            void* workspace, size_t workspace_bytes, moe_stream_t stream);
moe_status moe_qb_readout(const moe_config* cfg, const float* bias, int32_t n_bins,
                          const int32_t* hist, int64_t n_tokens, float* new_bias,
                          moe_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */
