/*
 * moe_layer_route.h -- C ABI of the MI355X (gfx950) gpt-oss MoE block forward.
 *
 * The operation is the MoE block of gpt-oss as the xserv page "Phase 19:
 * gpt-oss-20b MoE support" describes it:
 *   - section 1, architecture table, "MoE" row: a plain Linear router with
 *     bias, E experts, top-k (gpt-oss: 32 or 128 experts, k = 4), expert
 *     intermediate size I (2880), hidden size H (2880, not a multiple of 128);
 *   - section 1, architecture table, activation row: the clamped interleaved
 *     GLU  gate = gu[0::2], up = gu[1::2], gate <= 7, up in [-7, 7],
 *     h = (up + 1) * gate * sigmoid(1.702 * gate);
 *   - section 2, forward pipeline: router -> top-k softmax -> per-expert
 *     gate_up GEMM -> bias -> GLU -> per-expert down GEMM -> bias -> weighted
 *     sum over the k selected experts only (unselected experts are skipped,
 *     never multiplied by 0); the expert ids stay on the device and the host
 *     never synchronises.
 *
 * Conventions for every call below:
 *   - All tensor pointers are DEVICE pointers owned by the caller; the
 *     library never allocates, frees, copies to the host or synchronises the
 *     host.  Inputs are never modified.
 *   - bf16 means IEEE bfloat16 (stored as 16-bit words); all tensors are
 *     row-major and densely packed.
 *   - Every pointer that is read or written with 16-byte vector accesses
 *     (x, Wr, Wgu, Wd, h, o, y and the workspace) must be 16-byte aligned;
 *     bias, id, weight and index arrays must be 4-byte aligned.
 *   - All work is enqueued on `stream` (a hipStream_t; NULL = the default
 *     stream) and the call returns at once.  Results are valid once the
 *     stream reaches the call.  Nothing depends on host-side state between
 *     calls, so the calls can be captured in a HIP graph.
 *   - Arguments are validated on the host before anything is enqueued; an
 *     invalid call returns a non-zero status and enqueues nothing.  A failed
 *     launch returns MOE_ERR_HIP.  moe_last_error() gives a message for the
 *     last failing call on the calling thread.  No exception crosses the ABI.
 *   - T = 0 is a valid call that enqueues nothing.
 *   - Limits: 1 <= E <= 256, 1 <= k <= min(E, 8), 8 <= H, I <= 16384 with
 *     H % 8 == 0 and I % 8 == 0, 0 <= T and T * k < 2^31.
 *   - Results are bitwise reproducible: no floating-point atomics are used.
 *   - Calls that share a workspace must not overlap in time.
 */
#ifndef MOE_LAYER_ROUTE_H
#define MOE_LAYER_ROUTE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Every entry point is exported from the shared library. */
#if defined(__GNUC__) || defined(__clang__)
#define MOE_API __attribute__((visibility("default")))
#else
#define MOE_API
#endif

#define MOE_ABI_VERSION 1
#define MOE_MAX_E 256
#define MOE_MAX_K 8
#define MOE_MAX_DIM 16384

/* Status codes returned by every call that can fail. */
#define MOE_OK 0
#define MOE_ERR_INVALID_ARG 1   /* null/misaligned pointer, bad size or k */
#define MOE_ERR_UNSUPPORTED 2   /* valid request the library does not implement */
#define MOE_ERR_WORKSPACE 3     /* workspace missing or smaller than moe_workspace_bytes() */
#define MOE_ERR_HIP 4           /* a HIP launch or runtime call failed */

/* Execution path of the expert GEMMs (moe_forward_ex, moe_gate_up, moe_down). */
#define MOE_PATH_AUTO 0   /* chosen on the host from T*k/E only */
#define MOE_PATH_GEMV 1   /* weight streaming: each weight byte read once per pass of <=32 rows */
#define MOE_PATH_GEMM 2   /* LDS-tiled MFMA grouped GEMM */

/* Version of this ABI (MOE_ABI_VERSION). */
MOE_API int moe_abi_version(void);

/* Static text for a status code. */
MOE_API const char* moe_status_str(int status);

/* Message describing the last failing call made on this thread ("" if none). */
MOE_API const char* moe_last_error(void);

/*
 * Bytes of device workspace that moe_forward / moe_forward_ex need for these
 * sizes (0 when T == 0).  The caller allocates it (any 256-byte aligned
 * device buffer, contents irrelevant) and may reuse it across calls.
 * Returns 0 and sets moe_last_error() for sizes outside the limits.
 */
MOE_API size_t moe_workspace_bytes(int64_t T, int32_t H, int32_t E, int32_t k, int32_t I);

/* The expert path (MOE_PATH_GEMV or MOE_PATH_GEMM) that MOE_PATH_AUTO takes
 * for these sizes; it depends on T, E and k only (mean rows per expert). */
MOE_API int moe_expert_path(int64_t T, int32_t E, int32_t k);

/*
 * moe_route -- router logits, top-k and softmax weights
 * (architecture table "MoE" row; forward pipeline, first two steps).
 *
 *   x   bf16 [T][H]     token activations
 *   Wr  bf16 [E][H]     router weight (Linear form: one row per expert)
 *   br  bf16 [E]        router bias
 *   topk_ids  int32 [T][k]  out: the k experts with the largest logits
 *                           l[t][e] = sum_h x[t][h] * Wr[e][h] + br[e], ordered
 *                           by (logit descending, expert index ascending); equal
 *                           logits go to the lower index.  The decision is made
 *                           on the logits rounded to float32 from a float64
 *                           accumulation.
 *   topk_w    float [T][k]  out: softmax over the k selected logits
 *                           (w_j = exp(l_j - l_0) / sum_i exp(l_i - l_0)); each
 *                           row sums to 1.
 */
MOE_API int moe_route(const void* x, const void* Wr, const void* br,
              int64_t T, int32_t H, int32_t E, int32_t k,
              int32_t* topk_ids, float* topk_w, void* stream);

/* Router methods of moe_route_ex. */
#define MOE_ROUTE_AUTO 0    /* exact below 64K logits (T*E), MFMA + refinement above */
#define MOE_ROUTE_EXACT 1   /* every logit as an exact-product float64 sum */
#define MOE_ROUTE_MFMA 2    /* bf16 MFMA logits with error bounds; ties near the top k
                               recomputed exactly; same decision as MOE_ROUTE_EXACT */

/* moe_route with the router method forced (MOE_ROUTE_*); both methods give
 * the same topk_ids (and topk_w within 1e-6), so the choice only affects speed.
 * moe_route is moe_route_ex(..., MOE_ROUTE_AUTO, stream). */
MOE_API int moe_route_ex(const void* x, const void* Wr, const void* br,
                         int64_t T, int32_t H, int32_t E, int32_t k,
                         int32_t* topk_ids, float* topk_w, int32_t method, void* stream);

/*
 * moe_forward -- the whole MoE block forward (forward pipeline, all steps).
 *
 *   x, Wr, br       as in moe_route
 *   Wgu  bf16 [E][H][2I]   gate_up weight in x.W form; output columns are
 *                          interleaved gate0, up0, gate1, up1, ...
 *   bgu  bf16 [E][2I]      gate_up bias, interleaved the same way
 *   Wd   bf16 [E][I][H]    down weight in x.W form
 *   bd   bf16 [E][H]       down bias
 *   y    bf16 [T][H]       out: y[t] = sum_j w[t][j] * (h_j . Wd[e_j] + bd[e_j]),
 *                          h_j = GLU(x[t] . Wgu[e_j] + bgu[e_j]); products in
 *                          bf16 x bf16, accumulation in float32, h rounded to
 *                          bf16 before the down GEMM, y rounded once to bf16.
 *   topk_ids_out, topk_w_out   optional outputs (NULL to skip) of the routing
 *                          decision, same meaning as in moe_route.
 *   workspace, workspace_bytes  scratch of at least moe_workspace_bytes(...).
 */
MOE_API int moe_forward(const void* x, const void* Wr, const void* br,
                const void* Wgu, const void* bgu, const void* Wd, const void* bd,
                int64_t T, int32_t H, int32_t E, int32_t k, int32_t I,
                void* y, int32_t* topk_ids_out, float* topk_w_out,
                void* workspace, size_t workspace_bytes, void* stream);

/* moe_forward with the expert path forced (MOE_PATH_*); used to test both
 * paths at every shape.  moe_forward is moe_forward_ex(..., MOE_PATH_AUTO). */
MOE_API int moe_forward_ex(const void* x, const void* Wr, const void* br,
                   const void* Wgu, const void* bgu, const void* Wd, const void* bd,
                   int64_t T, int32_t H, int32_t E, int32_t k, int32_t I,
                   void* y, int32_t* topk_ids_out, float* topk_w_out,
                   void* workspace, size_t workspace_bytes, int32_t path, void* stream);

/*
 * moe_forward_noalloc -- moe_forward without a workspace argument, for callers
 * that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation.  Same arguments, meaning
 * and result bits as moe_forward (same kernels, path chosen as MOE_PATH_AUTO);
 * the caller still owns x, the weights, y and the optional id/weight outputs.
 * The intermediates live in a 64 MiB array of the library's own, one per GPU,
 * held until the process ends: about T*k*(2I + 4H + 16) bytes are needed
 * (T*k <= 3880 at H = I = 2880, i.e. T <= 970 at k = 4), and larger sizes
 * return MOE_ERR_INVALID_ARG without enqueuing anything.  Nothing is
 * allocated and nothing needs to start at zero.  Every call on a GPU shares
 * that GPU's array and finds the last call's contents in it: calls that
 * overlap on one GPU (different streams, or host threads) race and must be
 * serialised by the caller.  The first call on a device looks the array's
 * address up on that device (the device current on the calling thread).
 */
MOE_API int moe_forward_noalloc(const void* x, const void* Wr, const void* br,
                                const void* Wgu, const void* bgu, const void* Wd, const void* bd,
                                int64_t T, int32_t H, int32_t E, int32_t k, int32_t I,
                                void* y, int32_t* topk_ids_out, float* topk_w_out, void* stream);

/*
 * moe_forward_ep -- one expert-parallel rank's share of the layer: experts
 * are split across ranks by contiguous ranges, every rank routes all T tokens
 * over all E experts, keeps only the (token, slot) pairs whose expert it holds
 * (the others are skipped, never multiplied by 0) and returns its part of y.
 * Summing y_partial over the ranks gives y (xserv "Phase 19: gpt-oss-20b MoE
 * support", section 2: expert parallelism filters by expert range and the
 * partial outputs are summed by one all-reduce).
 *
 *   x, Wr, br            as in moe_forward (the whole router: [E][H], [E])
 *   e_begin, n_local     this rank holds experts [e_begin, e_begin + n_local)
 *   Wgu_local bf16 [n_local][H][2I], bgu_local bf16 [n_local][2I],
 *   Wd_local bf16 [n_local][I][H], bd_local bf16 [n_local][H]: those experts
 *   y_partial float [T][H] out: sum over this rank's experts of
 *                        topk_w[t][j] * (h_j . Wd[e_j] + bd[e_j]), in float32
 *                        (0 for a token none of whose experts is here)
 *   topk_ids_out, topk_w_out, workspace, workspace_bytes, path: as in
 *                        moe_forward_ex; the workspace size is
 *                        moe_workspace_bytes(T, H, E, k, I) with the full E.
 * Errors: the range must satisfy 0 <= e_begin, 1 <= n_local,
 * e_begin + n_local <= E (MOE_ERR_INVALID_ARG otherwise); other checks as in
 * moe_forward.
 */
MOE_API int moe_forward_ep(const void* x, const void* Wr, const void* br,
                   const void* Wgu_local, const void* bgu_local, const void* Wd_local, const void* bd_local,
                   int64_t T, int32_t H, int32_t E, int32_t k, int32_t I, int32_t e_begin, int32_t n_local,
                   float* y_partial, int32_t* topk_ids_out, float* topk_w_out,
                   void* workspace, size_t workspace_bytes, int32_t path, void* stream);

/*
 * moe_permute -- expert-contiguous order of the T*k (token, slot) pairs: the
 * device-side bookkeeping that replaces copying every token to every expert
 * (forward pipeline; ids never leave the device).
 *
 *   topk_ids int32 [T][k]  in
 *   cnt  int32 [E]    out: number of slots routed to each expert
 *   off  int32 [E+1]  out: exclusive prefix sum of cnt (off[E] = T*k)
 *   rows int32 [T*k]  out: rows[off[e] + r] = the r-th slot s = t*k + j with
 *                     topk_ids[t][j] == e, in increasing s (stable)
 *   pos  int32 [T*k]  out: inverse of rows (rows[pos[s]] == s)
 * A slot whose id lies outside [0, E) is skipped: it appears in no segment of
 * rows, pos[s] = -1, and off[E] counts only the others.
 */
MOE_API int moe_permute(const int32_t* topk_ids, int64_t T, int32_t E, int32_t k,
                int32_t* cnt, int32_t* off, int32_t* rows, int32_t* pos, void* stream);

/*
 * moe_gate_up -- per-expert gate_up GEMM + bias + clamped GLU for all experts
 * in one launch (architecture table activation row; forward pipeline).
 *
 *   x bf16 [T][H], Wgu bf16 [E][H][2I], bgu bf16 [E][2I]
 *   cnt, off, rows    as produced by moe_permute
 *   h  bf16 [T*k][I]  out, in permuted order: h[off[e] + r] belongs to slot
 *                     rows[off[e] + r] (token rows[...] / k) and expert e.
 *   path              MOE_PATH_* (AUTO picks from T*k/E)
 */
MOE_API int moe_gate_up(const void* x, const void* Wgu, const void* bgu,
                const int32_t* cnt, const int32_t* off, const int32_t* rows,
                int64_t T, int32_t H, int32_t E, int32_t k, int32_t I,
                void* h, int32_t path, void* stream);

/*
 * moe_down -- per-expert down GEMM + bias for all experts in one launch.
 *
 *   h  bf16 [T*k][I] in permuted order (moe_gate_up), Wd bf16 [E][I][H],
 *   bd bf16 [E][H], cnt/off as produced by moe_permute
 *   o  float [T*k][H] out, permuted order: o[off[e]+r] = h[off[e]+r] . Wd[e] + bd[e]
 */
MOE_API int moe_down(const void* h, const void* Wd, const void* bd,
             const int32_t* cnt, const int32_t* off,
             int64_t T, int32_t H, int32_t E, int32_t k, int32_t I,
             float* o, int32_t path, void* stream);

/*
 * moe_combine -- routing-weighted sum over each token's k expert outputs,
 * summed in float32 in the fixed order j = 0..k-1 and rounded once to bf16.
 * Only the selected slots are read.
 *
 *   o float [T*k][H] (moe_down), pos int32 [T*k] (moe_permute),
 *   topk_w float [T][k] (moe_route)
 *   y bf16 [T][H] out: y[t] = sum_j topk_w[t][j] * o[pos[t*k + j]], over the
 *                     slots with pos >= 0 (skipped slots add nothing)
 */
MOE_API int moe_combine(const float* o, const int32_t* pos, const float* topk_w,
                int64_t T, int32_t H, int32_t k, void* y, void* stream);

/*
 * moe_forward_padded -- moe_forward for a statically sized batch whose tail
 * is padding, with the per-expert loads exported.  The verify-graph page
 * (static buffers, pad tails zeroed for determinism) and the Phase 19 page's
 * per-layer expert-load recorder are the callers this serves.
 *   n_valid            device int32 (nullable: every row valid), read on the
 *                      device when the call runs, clamped to [0, T]: rows
 *                      t >= n_valid are padding.  A padding row is routed to no
 *                      expert (topk_ids -1, topk_w 0), costs no expert work,
 *                      and its y row is 0.  Grids are sized from T alone, so a
 *                      captured graph replays with any n_valid.
 *   expert_counts_out  device int32 [E] (nullable): cnt[e], the number of
 *                      (valid token, slot) pairs routed to expert e.
 * Every other argument is as in moe_forward_ex (workspace: moe_workspace_bytes).
 */
MOE_API int moe_forward_padded(const void* x, const void* Wr, const void* br,
                               const void* Wgu, const void* bgu, const void* Wd, const void* bd,
                               int64_t T, int32_t H, int32_t E, int32_t k, int32_t I,
                               const int32_t* n_valid, void* y, int32_t* topk_ids_out, float* topk_w_out,
                               int32_t* expert_counts_out, void* workspace, size_t workspace_bytes,
                               int32_t path, void* stream);

/* moe_forward_padded_mxfp4, moe_forward_padded_fp8 -- moe_forward_padded with
 * MXFP4 or FP8 expert weights: the weight arguments, their formats and the
 * workspace (moe_workspace_bytes, moe_workspace_bytes_fp8) are those of
 * moe_forward_mxfp4_ex and moe_forward_fp8_ex; n_valid, expert_counts_out,
 * the padding rows' outputs and every other argument are as in
 * moe_forward_padded. */
MOE_API int moe_forward_padded_mxfp4(const void* x, const void* Wr, const void* br,
                                     const void* Wgu_q, const void* Wgu_s, const void* bgu,
                                     const void* Wd_q, const void* Wd_s, const void* bd,
                                     int64_t T, int32_t H, int32_t E, int32_t k, int32_t I,
                                     const int32_t* n_valid, void* y, int32_t* topk_ids_out, float* topk_w_out,
                                     int32_t* expert_counts_out, void* workspace, size_t workspace_bytes,
                                     int32_t path, void* stream);
MOE_API int moe_forward_padded_fp8(const void* x, const void* Wr, const void* br,
                                   const void* Wgu_q, const float* Wgu_s, const void* bgu,
                                   const void* Wd_q, const float* Wd_s, const void* bd,
                                   int64_t T, int32_t H, int32_t E, int32_t k, int32_t I,
                                   const int32_t* n_valid, void* y, int32_t* topk_ids_out, float* topk_w_out,
                                   int32_t* expert_counts_out, void* workspace, size_t workspace_bytes,
                                   int32_t path, void* stream);

/* moe_forward_ep_mxfp4, moe_forward_ep_fp8 -- moe_forward_ep with MXFP4 or FP8
 * expert weights: the rank's own experts [e_begin, e_begin + n_local) in the
 * formats of moe_forward_mxfp4_ex and moe_forward_fp8_ex, indexed from 0
 * (codes and scales of n_local experts; bgu_local, bd_local as in
 * moe_forward_ep); workspace as moe_workspace_bytes or moe_workspace_bytes_fp8
 * for the whole E.  y_partial (float32 [T][H]) and every other argument are as
 * in moe_forward_ep: only local slots are computed, the others are skipped,
 * and tokens with no local expert get 0. */
MOE_API int moe_forward_ep_mxfp4(const void* x, const void* Wr, const void* br,
                                 const void* Wgu_q_local, const void* Wgu_s_local, const void* bgu_local,
                                 const void* Wd_q_local, const void* Wd_s_local, const void* bd_local,
                                 int64_t T, int32_t H, int32_t E, int32_t k, int32_t I,
                                 int32_t e_begin, int32_t n_local, float* y_partial,
                                 int32_t* topk_ids_out, float* topk_w_out,
                                 void* workspace, size_t workspace_bytes, int32_t path, void* stream);
MOE_API int moe_forward_ep_fp8(const void* x, const void* Wr, const void* br,
                               const void* Wgu_q_local, const float* Wgu_s_local, const void* bgu_local,
                               const void* Wd_q_local, const float* Wd_s_local, const void* bd_local,
                               int64_t T, int32_t H, int32_t E, int32_t k, int32_t I,
                               int32_t e_begin, int32_t n_local, float* y_partial,
                               int32_t* topk_ids_out, float* topk_w_out,
                               void* workspace, size_t workspace_bytes, int32_t path, void* stream);

/*
 * MXFP4 expert weights (W4A16) -- xserv "Phase 19: gpt-oss-20b MoE support",
 * section 5: the expert weights are 4-bit E2M1 values with one UE8M0
 * (power-of-two) scale per 32 values; activations, biases, the router and
 * every output stay as in moe_forward.
 *
 * Format, for a weight with contraction dimension K and N output columns
 * (gate_up: K = H, N = 2I; down: K = I, N = H), stored K-contiguous:
 *   codes  uint8 [E][N][K/2]   row n holds the K values of output column n,
 *                              two per byte: k = 2i in bits 0-3, k = 2i+1 in
 *                              bits 4-7.  E2M1 code: bit 3 sign, bits 2-1
 *                              exponent (bias 1), bit 0 mantissa; magnitudes
 *                              0, 0.5, 1, 1.5, 2, 3, 4, 6.
 *   scales uint8 [E][K/32][N]  the 32 values k = 32b .. 32b+31 of column n are
 *                              multiplied by 2^(scales[e][b][n] - 127); 255 is
 *                              NaN (block-major: the scales of one block of
 *                              all columns are contiguous).
 * The weight value is E2M1(code) * 2^(scale - 127), exactly.  Requires
 * H % 32 == 0 and I % 32 == 0; codes and scales 16-byte aligned.
 */

/*
 * moe_quantize_mxfp4 -- converts bf16 weights W [E][K][N] (x.W form, as in
 * moe_forward) to the MXFP4 format above, one 32-value block at a time: the
 * shared exponent is floor(log2(max |v|)) - 2 clamped to [-127, 127] (-127
 * for an all-zero block), and each v / 2^exponent is rounded to the nearest
 * E2M1 value, ties to the even code, magnitudes above 6 saturated to 6; the
 * sign bit of a code is the sign bit of v.  (The microscaling formats'
 * reference conversion.)  K % 32 == 0, N % 8 == 0.
 *   W       bf16 [E][K][N]   in
 *   codes   uint8 [E][N][K/2]   out
 *   scales  uint8 [E][K/32][N]  out
 */
MOE_API int moe_quantize_mxfp4(const void* W, int32_t E, int32_t K, int32_t N, void* codes, void* scales,
                               void* stream);

/*
 * moe_forward_mxfp4 -- moe_forward with MXFP4 expert weights:
 *   Wgu_q uint8 [E][2I][H/2], Wgu_s uint8 [E][H/32][2I]   gate_up (columns
 *                          interleaved gate0, up0, gate1, ... as in moe_forward)
 *   Wd_q  uint8 [E][H][I/2],  Wd_s  uint8 [E][I/32][H]    down
 * Every other argument, the workspace size (moe_workspace_bytes) and the
 * result's definition are those of moe_forward with the weights replaced by
 * their exact dequantised values; the dequantised weights are bf16 operands
 * of the same float32-accumulating products.  Expert paths as in moe_forward:
 * MOE_PATH_GEMV streams the 4-bit weights (one pass over each live expert's
 * weights per 32 rows), MOE_PATH_GEMM is the LDS-tiled MFMA grouped GEMM;
 * AUTO picks from T*k/E as moe_expert_path does.
 */
MOE_API int moe_forward_mxfp4(const void* x, const void* Wr, const void* br,
                              const void* Wgu_q, const void* Wgu_s, const void* bgu,
                              const void* Wd_q, const void* Wd_s, const void* bd,
                              int64_t T, int32_t H, int32_t E, int32_t k, int32_t I,
                              void* y, int32_t* topk_ids_out, float* topk_w_out,
                              void* workspace, size_t workspace_bytes, void* stream);

/* moe_forward_mxfp4 with the expert path forced (MOE_PATH_*); both paths give
 * the same result within rounding.  moe_forward_mxfp4 is this with MOE_PATH_AUTO. */
MOE_API int moe_forward_mxfp4_ex(const void* x, const void* Wr, const void* br,
                                 const void* Wgu_q, const void* Wgu_s, const void* bgu,
                                 const void* Wd_q, const void* Wd_s, const void* bd,
                                 int64_t T, int32_t H, int32_t E, int32_t k, int32_t I,
                                 void* y, int32_t* topk_ids_out, float* topk_w_out,
                                 void* workspace, size_t workspace_bytes, int32_t path, void* stream);

/* Stage calls of moe_forward_mxfp4: moe_gate_up and moe_down with MXFP4
 * weights (same inputs, outputs, layouts and path argument otherwise). */
MOE_API int moe_gate_up_mxfp4(const void* x, const void* Wgu_q, const void* Wgu_s, const void* bgu,
                              const int32_t* cnt, const int32_t* off, const int32_t* rows,
                              int64_t T, int32_t H, int32_t E, int32_t k, int32_t I, void* h,
                              int32_t path, void* stream);
MOE_API int moe_down_mxfp4(const void* h, const void* Wd_q, const void* Wd_s, const void* bd,
                           const int32_t* cnt, const int32_t* off,
                           int64_t T, int32_t H, int32_t E, int32_t k, int32_t I, float* o,
                           int32_t path, void* stream);

/*
 * FP8 W8A8 experts -- xserv "Phase 19: gpt-oss-20b MoE support", section 5:
 * 8-bit weights with one scalar scale per expert, stored transposed
 * ([E][N][K], the contraction dimension contiguous), and 8-bit activations;
 * the scales are applied after the product.  Router, biases and outputs stay
 * as in moe_forward.
 *
 * Format: OCP FP8 E4M3 -- bit 7 sign, bits 6-3 exponent (bias 7), bits 2-0
 * mantissa; exponent 0 is subnormal (m * 2^-9); largest finite 448; 0x7F and
 * 0xFF are NaN; no infinities.  A tensor slice with maximum |a| = amax has
 * the float32 scale s = amax / 448 and the codes E4M3(a * (448 / amax)),
 * each operation rounded in float32, E4M3 rounding to nearest with ties to
 * the even code and saturating at 448 (NaN -> 0x7F); amax = 0 gives s = 1.
 * The value of a code is E4M3(code) * s.
 *   Weights:     one scale per expert and matrix.
 *   Activations: one scale per row: a token's row of x for gate_up, a (token,
 *                slot) row of h for down, where h is first rounded to bf16.
 * gate_up = (codes_x . codes_W) * s_x[t] * s_W[e] + bias (the float32 sum of
 * exact code products), then the clamped GLU as in moe_forward; down likewise
 * with the h codes.  Requires H % 16 == 0 and I % 16 == 0; code arrays
 * 16-byte aligned, scale arrays 4-byte aligned.
 */

/*
 * moe_quantize_fp8 -- bf16 weights W [E][K][N] (x.W form, as in moe_forward)
 * to codes [E][N][K] and one scale per expert.  K % 16 == 0, N % 8 == 0.
 *   W       bf16 [E][K][N]     in
 *   codes   uint8 [E][N][K]    out
 *   scales  float32 [E]        out (also used as scratch during the call)
 */
MOE_API int moe_quantize_fp8(const void* W, int32_t E, int32_t K, int32_t N, void* codes, float* scales,
                             void* stream);

/*
 * moe_quantize_rows_fp8 -- bf16 rows a [R][K] to codes [R][K] and one scale
 * per row (the activation quantisation moe_forward_fp8 applies to x and h).
 * K % 16 == 0; R = 0 is a no-op.
 */
MOE_API int moe_quantize_rows_fp8(const void* a, int64_t R, int32_t K, void* codes, float* scales, void* stream);

/* Bytes of workspace moe_forward_fp8 needs: moe_workspace_bytes plus the x
 * and h codes and their row scales (T*H + T*k*I bytes and 4*(T + T*k)). */
MOE_API size_t moe_workspace_bytes_fp8(int64_t T, int32_t H, int32_t E, int32_t k, int32_t I);

/*
 * moe_forward_fp8 -- moe_forward with FP8 W8A8 experts:
 *   Wgu_q uint8 [E][2I][H], Wgu_s float32 [E]   gate_up (columns interleaved
 *                          gate0, up0, gate1, ... as in moe_forward)
 *   Wd_q  uint8 [E][H][I],  Wd_s  float32 [E]   down
 * x is quantised per token and h per (token, slot) row on the device, inside
 * the call.  Every other argument and output is as in moe_forward; the
 * workspace must hold moe_workspace_bytes_fp8(...) bytes.  Expert paths, both
 * on the FP8 matrix cores: MOE_PATH_GEMV streams the 8-bit weights (one pass
 * over each live expert's weights per 32 rows), MOE_PATH_GEMM is the
 * LDS-tiled grouped GEMM; AUTO picks from T*k/E as moe_expert_path does.
 */
MOE_API int moe_forward_fp8(const void* x, const void* Wr, const void* br,
                            const void* Wgu_q, const float* Wgu_s, const void* bgu,
                            const void* Wd_q, const float* Wd_s, const void* bd,
                            int64_t T, int32_t H, int32_t E, int32_t k, int32_t I,
                            void* y, int32_t* topk_ids_out, float* topk_w_out,
                            void* workspace, size_t workspace_bytes, void* stream);

/* moe_forward_fp8 with the expert path forced (MOE_PATH_*). */
MOE_API int moe_forward_fp8_ex(const void* x, const void* Wr, const void* br,
                               const void* Wgu_q, const float* Wgu_s, const void* bgu,
                               const void* Wd_q, const float* Wd_s, const void* bd,
                               int64_t T, int32_t H, int32_t E, int32_t k, int32_t I,
                               void* y, int32_t* topk_ids_out, float* topk_w_out,
                               void* workspace, size_t workspace_bytes, int32_t path, void* stream);

/* Stage calls of moe_forward_fp8.  gate_up takes the x codes and row scales
 * (moe_quantize_rows_fp8 of x: xq [T][H], sx [T]) and writes bf16 h as
 * moe_gate_up does; down takes the h codes and row scales (hq [T*k][I], sh
 * [T*k], in the permuted row order of h) and writes o as moe_down does. */
MOE_API int moe_gate_up_fp8(const void* xq, const float* sx, const void* Wgu_q, const float* Wgu_s,
                            const void* bgu, const int32_t* cnt, const int32_t* off, const int32_t* rows,
                            int64_t T, int32_t H, int32_t E, int32_t k, int32_t I, void* h,
                            int32_t path, void* stream);
MOE_API int moe_down_fp8(const void* hq, const float* sh, const void* Wd_q, const float* Wd_s,
                         const void* bd, const int32_t* cnt, const int32_t* off,
                         int64_t T, int32_t H, int32_t E, int32_t k, int32_t I, float* o,
                         int32_t path, void* stream);

/* ---------------------------------------------------------------------------
 * Measurement probes.  They are not part of the block: they measure what a
 * plain hand-written kernel gets from the matrix cores and from HBM on this
 * GPU, the "achievable" context printed next to the roofline fractions (which
 * use the published peaks).  Both are asynchronous on stream; time them with
 * events around the call.
 * ------------------------------------------------------------------------- */

/* moe_probe_mfma_bf16 -- workgroups x 4 waves, each wave iters rounds of
 * eight independent 32x32x16 bf16 MFMAs on all-ones operands:
 * workgroups * 4 * iters * 8 * 32768 flops.
 *   out float [workgroups * 4] (device, caller-owned): one value per wave,
 *       exactly 2048 * iters when iters <= 8191 (a check of the result).
 * iters in [1, 2^20), workgroups in [1, 65535]. */
MOE_API int moe_probe_mfma_bf16(int32_t iters, int32_t workgroups, float* out, void* stream);

/* moe_probe_read -- read buf (device, 16-byte aligned, bytes a multiple of
 * 16) once with 16-byte loads, consecutive lanes on consecutive bytes, each
 * workgroup one contiguous chunk of about bytes / workgroups.
 *   out uint32 [workgroups * 4] (device, caller-owned): one XOR-fold per
 *       wave; the XOR of all of them equals the XOR of buf's 32-bit words.
 * workgroups in [1, 65535]; bytes = 0 writes zeros. */
MOE_API int moe_probe_read(const void* buf, size_t bytes, int32_t workgroups, uint32_t* out, void* stream);

/* moe_probe_mfma_dot_bf16 -- out[m][n] = sum_k A[m][k] * B[n][k] formed as
 * the MFMA router forms its logits (Phase 19 page, section 1 "MoE" row: the
 * router is a Linear over the hidden state): v_mfma_f32_16x16x32_bf16 over K
 * in steps of 32, in increasing K, into one float32 accumulator that starts
 * at 0.  It exposes the instruction's own accumulation error, which the
 * router's error bound has to cover.
 *   A bf16 [M][K], B bf16 [16][K] (device, 16-byte aligned, row-major)
 *   out float [M][16] (device, caller-owned)
 * M a positive multiple of 16 (at most 16 * 65535), K a positive multiple of
 * 32 (at most 2^20), A below 2 GiB; otherwise MOE_ERR_INVALID_ARG. */
MOE_API int moe_probe_mfma_dot_bf16(const void* A, const void* B, int32_t M, int32_t K, float* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_LAYER_ROUTE_H */
