/*
 * moe_mi355x.h -- C ABI of the routed-expert Mixture-of-Experts forward path on
 * one AMD Instinct MI355X (gfx950).
 *
 * The layer, for T tokens of hidden size H, E experts, top-k routing and expert
 * intermediate size I, runs as five calls on one HIP stream:
 *
 *   moe_route_topk         router logits -> top-k expert ids and weights
 *   moe_permute            atomic-free counting sort + gather into a padded,
 *                          expert-grouped row layout
 *   moe_grouped_glu_gemm   one grouped GEMM for every expert's gate and up
 *                          projections, SwiGLU fused into its epilogue
 *   moe_grouped_glu_gemm_gather  the same GEMM reading token rows of x through
 *                          row_token (the permute's gather folded into its loads)
 *   moe_grouped_down_gemm  one grouped GEMM for every expert's down projection
 *   moe_combine            fp32 score-weighted gather-sum back to token order
 *
 * FP8 expert weights (the same GEMMs reading OCP E4M3 weights, half the bytes):
 *   moe_quantize_fp8       block-scaled E4M3 codes of bf16 expert weights
 *   moe_grouped_glu_gemm_fp8w, moe_grouped_glu_gemm_gather_fp8w,
 *   moe_grouped_down_gemm_fp8w
 *
 * The clamped-SwiGLU variant of the gate/up GEMM:
 *   moe_grouped_glu_gemm_clamped
 *
 * The router projection fused with top-k (logits need not reach memory):
 *   moe_router_prepare, moe_router_topk
 *
 * Training (the forward with its gate/up output kept, and the backward):
 *   moe_grouped_gemm       plain grouped GEMM C[p] = A[p] W[e]^T (gate/up output
 *                          gu = x_perm W_gu^T; input gradients on transposed weights)
 *   moe_grouped_gemm_swiglu_backward  dh = dy W_down and the SwiGLU backward in one
 *                          GEMM (dh never reaches memory)
 *   moe_swiglu, moe_swiglu_backward, moe_transpose_experts, moe_combine_backward,
 *   moe_route_backward, moe_permute_backward, moe_grouped_wgrad
 *   on row-pair tiled operands: moe_grouped_gemm_tiled, moe_swiglu_tiled,
 *   moe_swiglu_backward_tiled, moe_grouped_wgrad_tiled
 *
 * The forward on row-pair tiled operands (this library's faster memory order for
 * x_perm, h and the expert weights; every result bit for bit the row-major
 * call's):
 *   moe_tile_rows, moe_untile_rows, moe_permute_tiled, moe_grouped_glu_gemm_tiled,
 *   moe_grouped_glu_gemm_gather_tiled, moe_grouped_down_gemm_tiled,
 *   moe_tile_fp8_rows, moe_untile_fp8_rows, moe_grouped_glu_gemm_fp8w_tiled,
 *   moe_grouped_down_gemm_fp8w_tiled
 *
 * Routing that also counts the permute's histogram:
 *   moe_route_hist_workspace_size, moe_route_topk_hist, moe_permute_from_hist
 * The layer after routing as one persistent kernel:
 *   moe_fused_layer_workspace_size, moe_fused_layer, moe_fused_layer_status
 * The permute without a workspace, for callers that cannot allocate:
 *   moe_permute_noalloc, moe_permute_noalloc_max_workspace
 * The debug build's queries: moe_debug_build, moe_debug_status, moe_debug_reset
 * Measurement probes: moe_probe_copy, moe_probe_read, moe_probe_mfma_bf16
 *
 * Sources (page title, section):
 *   [Halo]      Halo, "Performance": Levers that help (grouped GEMM instead of a
 *               per-expert loop; the atomic-free expert permute; fused GLU);
 *               Levers that do not help here (small-M experts are bound by
 *               weight bandwidth; fp8 halves the expert-weight bytes)
 *   [PocketLLM] "Qwen4-Exp Heterogeneous TP4 Performance": Runtime architecture
 *               (top-10 of 512 routed experts); Confirmed architecture decisions
 *               (only active experts move weight bytes)
 *   [prime-rl]  prime-rl pull request 3885: Changes (single-pass local layout: one
 *               gather into the padded expert-grouped layout and one fp32
 *               score-weighted gather-sum back; 32-bit row offsets must not
 *               overflow silently; FP8 expert weights quantized once per
 *               optimizer step, blockwise FP8 grouped GEMMs; the layout's gathers
 *               in backward too; forward, dgrad and wgrad grouped GEMMs; weight
 *               gradients in fp32; the forward keeps its gate/up output)
 *
 * Conventions
 *   - Every tensor pointer is a DEVICE pointer, row-major, 16-byte aligned.
 *     bf16 tensors are raw 16-bit values (moe_bf16). When T == 0, pointers to
 *     buffers whose size is proportional to T may be NULL.
 *   - The caller owns every buffer. The library never allocates, frees or keeps
 *     a pointer after a call returns; buffers must stay alive until the stream
 *     work that uses them completes.
 *   - Every call validates its arguments on the host first. On an error it
 *     returns a nonzero moe_status, enqueues nothing and leaves outputs untouched;
 *     moe_last_error_message() then describes the error (thread-local text).
 *   - On success the work is only enqueued on `stream` (NULL = the default
 *     stream). No call synchronises, copies device->host or needs expert counts
 *     on the host: the GEMMs read counts and offsets on the device, and the
 *     layout buffers are sized by P_max, the largest row count any routing can
 *     need. Device faults surface at the caller's next synchronisation.
 *   - Results are deterministic: no atomics anywhere, fixed reduction orders,
 *     so the same inputs give bitwise-identical outputs.
 *   - Row indices are int32 (P_max < 2^31); element offsets are 64-bit.
 *   - Calls are thread-safe; concurrent calls on different streams do not
 *     interact except through buffers the caller shares.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t moe_bf16;   /* raw bf16 bits */
typedef void *moe_stream_t;  /* a hipStream_t; NULL = default stream */

typedef enum moe_status {
    MOE_OK = 0,
    MOE_ERR_NULL_POINTER = 1,       /* a required pointer is NULL */
    MOE_ERR_INVALID_SHAPE = 2,      /* a size is out of range (see each call) */
    MOE_ERR_INVALID_ALIGN = 3,      /* align is not a power of two in [1, 256] */
    MOE_ERR_SIZE_OVERFLOW = 4,      /* P_max too small, or rows would reach 2^31 */
    MOE_ERR_MISALIGNED_POINTER = 5, /* a tensor pointer is not 16-byte aligned */
    MOE_ERR_WORKSPACE_TOO_SMALL = 6,
    MOE_ERR_HIP = 7,                /* a HIP call failed; see moe_last_error_message */
    MOE_ERR_INVALID_VALUE = 8,      /* a scalar argument is out of range (see each call) */
    MOE_ERR_PRECONDITION = 9        /* debug build only: a precondition on device data failed
                                       (moe_debug_status) */
} moe_status;

#define MOE_MAX_K 32    /* largest top-k */
#define MOE_MAX_E 1024  /* most experts */
#define MOE_MAX_ALIGN 256

/* Static text for a status code. */
const char *moe_status_string(int status);

/* Text of the last error returned on this thread ("" if none). */
const char *moe_last_error_message(void);

/* Rows the padded layout can need: T*k + E*(align-1) (each expert's segment is
 * rounded up to a multiple of align). -1 if an argument is out of range. */
int64_t moe_padded_rows_max(int64_t T, int32_t k, int32_t E, int32_t align);

/* Device workspace bytes moe_permute needs for T tokens, top-k, E experts. */
moe_status moe_permute_workspace_size(int64_t T, int32_t k, int32_t E, size_t *bytes);

/*
 * Top-k routing [PocketLLM, Runtime architecture: top-10 routing over 512
 * experts; prime-rl, Changes: the top-k scores weight the gather-sum].
 *   logits    [T, E] fp32, finite (unchecked; non-finite input gives
 *             unspecified ids)
 *   topk_idx  [T, k] int32 out: per token the k experts with the largest logits,
 *             larger logit first; an exact tie (float ==, so -0 == +0) goes to the
 *             lower expert id
 *   topk_w    [T, k] fp32 out: softmax over the k selected logits,
 *             w_j = exp(l_j - l_0) / sum_i exp(l_i - l_0)
 * Shapes: 1 <= E <= MOE_MAX_E, 1 <= k <= min(E, MOE_MAX_K), T >= 0.
 */
moe_status moe_route_topk(const float *logits, int64_t T, int32_t E, int32_t k,
                          int32_t *topk_idx, float *topk_w, moe_stream_t stream);

/*
 * Padded expert-grouped layout and token gather, without atomics [Halo, Levers
 * that help: the atomic-free expert permute; prime-rl, Changes: one gather into
 * the padded expert-grouped layout].  Over the flat routes r = t*k + j:
 *   expert_counts   [E] int32 out: routes per expert
 *   expert_offsets  [E+1] int32 out: offsets[0] = 0, offsets[e+1] = offsets[e]
 *                   + counts[e] rounded up to a multiple of align
 *   route_row       [T*k] int32 out: the layout row of route r; the routes of
 *                   expert e fill rows offsets[e], offsets[e]+1, ... in ascending r
 *   row_token       [P_max] int32 out: the token of each row, -1 on pad rows and
 *                   on every row at or past offsets[E]
 *   x_perm          [P_max, H] bf16 out: x_perm[p] = x[row_token[p]] bit for bit
 *                   on routed rows, zero on pad rows inside a segment; rows at or
 *                   past offsets[E] are not written. NULL skips the gather (the
 *                   layout only, for moe_grouped_glu_gemm_gather); x may then be
 *                   NULL too
 *   x               [T, H] bf16;  topk_idx [T, k] int32, each in [0, E) and
 *                   distinct per token (unchecked)
 *   workspace       device scratch of moe_permute_workspace_size() bytes
 * Shapes: H % 64 == 0, align a power of two <= MOE_MAX_ALIGN,
 *         moe_padded_rows_max(T,k,E,align) <= P_max < 2^31.
 */
moe_status moe_permute(const moe_bf16 *x, const int32_t *topk_idx, int64_t T, int32_t H,
                       int32_t E, int32_t k, int32_t align, int64_t P_max,
                       int32_t *expert_counts, int32_t *expert_offsets, int32_t *route_row,
                       int32_t *row_token, moe_bf16 *x_perm, void *workspace,
                       size_t workspace_bytes, moe_stream_t stream);

/*
 * Routing and the permute's counting in one kernel [prime-rl, Changes: a
 * single-pass local layout; PocketLLM, Remaining prefill attribution: the router
 * is a phase of its own]. moe_route_topk_hist computes exactly what
 * moe_route_topk computes and, in the same kernel, the number of routes to each
 * expert among each workgroup's tokens, into `workspace` (an opaque histogram of
 * moe_route_hist_workspace_size(T, k, E) bytes). moe_permute_from_hist then
 * builds the same layout and x_perm as moe_permute (bit for bit; arguments as
 * there) from that histogram instead of counting topk_idx again. Pass both calls
 * the same T, E, k, topk_idx and workspace, in stream order; the workspace is
 * overwritten by moe_permute_from_hist.
 */
moe_status moe_route_hist_workspace_size(int64_t T, int32_t k, int32_t E, size_t *bytes);
moe_status moe_route_topk_hist(const float *logits, int64_t T, int32_t E, int32_t k, int32_t *topk_idx,
                               float *topk_w, void *workspace, size_t workspace_bytes, moe_stream_t stream);
moe_status moe_permute_from_hist(const moe_bf16 *x, const int32_t *topk_idx, int64_t T, int32_t H,
                                 int32_t E, int32_t k, int32_t align, int64_t P_max,
                                 int32_t *expert_counts, int32_t *expert_offsets, int32_t *route_row,
                                 int32_t *row_token, moe_bf16 *x_perm, void *workspace,
                                 size_t workspace_bytes, moe_stream_t stream);

/*
 * The layer after routing as one persistent kernel [prime-rl, Changes: the fused
 * "Mega MoE" op -- dispatch, experts and combine in one kernel; the page measured
 * it slower than the split path on one node]. One cooperative launch (one
 * workgroup per compute unit, all resident) runs, with a grid-wide barrier
 * between phases: the permute's counting sort, scan and scatter; the gate/up GEMM
 * reading token rows of x in place through row_token (no x_perm); the down GEMM;
 * the combine. Outputs equal, bit for bit, those of moe_permute with x_perm NULL,
 * moe_grouped_glu_gemm_gather, moe_grouped_down_gemm and moe_combine on the same
 * inputs:
 *   x [T, H] bf16, topk_idx / topk_w [T, k] from moe_route_topk,
 *   w_gate_up [E, 2I, H], w_down [E, H, I] bf16
 *   expert_counts [E], expert_offsets [E+1], route_row [T*k], row_token [P_max]
 *   int32 out (as moe_permute); h [P_max, I], y [P_max, H] bf16 out (as the
 *   GEMMs); out [T, H] bf16 out (as moe_combine)
 *   workspace: moe_fused_layer_workspace_size(T, k, E) bytes (barrier words and
 *   the histogram; reset by the call itself)
 * Shapes and errors as for those calls (T >= 1, T * H * 2 < 2^32); a device
 * without cooperative launch gives MOE_ERR_HIP. Every wait at a barrier is
 * bounded: if a workgroup never arrives, the others stop after about a second and
 * moe_fused_layer_status (which synchronises `stream`) returns MOE_ERR_HIP;
 * MOE_OK otherwise. Calls that overlap on one workspace race.
 */
moe_status moe_fused_layer_workspace_size(int64_t T, int32_t k, int32_t E, size_t *bytes);
moe_status moe_fused_layer(const moe_bf16 *x, const int32_t *topk_idx, const float *topk_w,
                           const moe_bf16 *w_gate_up, const moe_bf16 *w_down, int64_t T, int32_t H, int32_t E,
                           int32_t k, int32_t I, int32_t align, int64_t P_max, int32_t *expert_counts,
                           int32_t *expert_offsets, int32_t *route_row, int32_t *row_token, moe_bf16 *h,
                           moe_bf16 *y, moe_bf16 *out, void *workspace, size_t workspace_bytes,
                           moe_stream_t stream);
moe_status moe_fused_layer_status(const void *workspace, moe_stream_t stream);

/*
 * moe_permute without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the per-chunk histogram goes to a fixed device array inside
 * the library (4 MiB per device that runs it, held until the process ends) instead
 * of `workspace`. Arguments, outputs and errors otherwise as for moe_permute. It
 * needs moe_permute_workspace_size(T, k, E) <= moe_permute_noalloc_max_workspace()
 * bytes (about ceil(T*k/256) * E * 4), else MOE_ERR_WORKSPACE_TOO_SMALL and nothing
 * is enqueued. Calls that overlap on one device (two streams or threads at once)
 * share that array and race; serialise them. Nothing is allocated, freed or
 * cleared: every call rewrites the whole histogram before reading it.
 */
moe_status moe_permute_noalloc(const moe_bf16 *x, const int32_t *topk_idx, int64_t T, int32_t H,
                               int32_t E, int32_t k, int32_t align, int64_t P_max,
                               int32_t *expert_counts, int32_t *expert_offsets, int32_t *route_row,
                               int32_t *row_token, moe_bf16 *x_perm, moe_stream_t stream);
size_t moe_permute_noalloc_max_workspace(void);

/*
 * Grouped gate/up GEMM with SwiGLU [Halo, Levers that help: one grouped expert
 * matmul instead of a per-expert loop, fused GLU; prime-rl, Changes: gate and up
 * run as one GEMM ahead of a SwiGLU].  For every expert e and every row p of its
 * padded segment [offsets[e], offsets[e+1]):
 *   g = x_perm[p] . w_gate_up[e, i, :],  u = x_perm[p] . w_gate_up[e, I+i, :]
 *   h[p, i] = bf16_rne(silu(g) * u)      (fp32 accumulation and epilogue)
 *   w_gate_up       [E, 2I, H] bf16: rows [0, I) gate, rows [I, 2I) up
 *   expert_counts, expert_offsets as produced by moe_permute (device)
 *   h               [P_max, I] bf16 out; rows at or past offsets[E] not written
 * An expert with no rows reads none of its weights.
 * Kernel choice: 256-row MFMA tiles, except for the FP8-weight GEMMs when
 * P_max <= 64*E -- few rows per expert, where the weights' bytes bound the GEMM
 * [Halo, Levers that do not help here] -- which use a weight-streaming kernel
 * that reads each active expert's weights once per 32 rows of its segment. Both
 * compute the same values up to fp32 summation order.
 * Shapes: H % 64 == 0, I % 64 == 0, 1 <= E <= MOE_MAX_E, 0 < P_max < 2^31, 4*H*I < 2^32
 * (one expert's weights addressed with 32-bit byte offsets).
 */
moe_status moe_grouped_glu_gemm(const moe_bf16 *x_perm, const moe_bf16 *w_gate_up,
                                const int32_t *expert_counts, const int32_t *expert_offsets,
                                int32_t E, int32_t H, int32_t I, int64_t P_max, moe_bf16 *h,
                                moe_stream_t stream);

/*
 * moe_grouped_glu_gemm with the permute's gather folded into the A loads
 * [prime-rl, Changes: one gather into the padded expert-grouped layout -- here
 * the layout rows are read in place from x].  For every routed row p:
 *   h[p] = the h row moe_grouped_glu_gemm computes from x_perm[p] = x[row_token[p]]
 *   x          [T, H] bf16, the tokens (not permuted)
 *   row_token  [P_max] int32 from moe_permute (values in [0, T) or -1; unchecked)
 * Rows of h that are pad rows of a segment hold unspecified values (their token
 * is taken as 0); rows at or past offsets[E] are not written.
 * Shapes as for moe_grouped_glu_gemm, plus T >= 1 and T * H * 2 < 2^32 (32-bit
 * byte offsets into x), else MOE_ERR_SIZE_OVERFLOW.
 */
moe_status moe_grouped_glu_gemm_gather(const moe_bf16 *x, const int32_t *row_token,
                                       const moe_bf16 *w_gate_up, const int32_t *expert_counts,
                                       const int32_t *expert_offsets, int64_t T, int32_t E,
                                       int32_t H, int32_t I, int64_t P_max, moe_bf16 *h,
                                       moe_stream_t stream);

/*
 * Grouped down GEMM [Halo, Levers that help: grouped GEMM].  For every expert e
 * and every row p of its padded segment:
 *   y[p, c] = bf16_rne(h[p] . w_down[e, c, :])   (fp32 accumulation)
 *   w_down  [E, H, I] bf16;  y [P_max, H] bf16 out (rows past offsets[E] not written)
 * Shapes as for moe_grouped_glu_gemm.
 */
moe_status moe_grouped_down_gemm(const moe_bf16 *h, const moe_bf16 *w_down,
                                 const int32_t *expert_counts, const int32_t *expert_offsets,
                                 int32_t E, int32_t H, int32_t I, int64_t P_max, moe_bf16 *y,
                                 moe_stream_t stream);

/*
 * Row-pair tiled operands.  The same three GEMM steps (and the permute's gather)
 * with bf16 matrices stored in a tiled order this library defines for gfx950 --
 * not a layout the pages use: a matrix [R, C] (R even, C % 32 == 0) is kept as
 * 2 x 32 blocks of 128 bytes, element (r, c) at
 *     ((r / 2) * (C / 32) + c / 32) * 64 + (r % 2) * 32 + c % 32.
 * The GEMMs stream operands through LDS 32 columns at a time; in this order one
 * such piece of two neighbouring rows is one whole 128-byte line, which lifts the
 * per-CU operand stream that bounds them.  The computation is the one documented
 * for the row-major calls, with the same fp32 summation order, so every output
 * is bit-identical to theirs once un-tiled.
 *
 * moe_tile_rows / moe_untile_rows: row-major [rows, cols] <-> tiled, bf16,
 *   rows even and >= 0, cols a positive multiple of 32, src and dst distinct
 *   device buffers of rows * cols elements; enqueued on `stream`.
 *   Expert weights are tiled once per weight update: w_gate_up [E, 2I, H] as
 *   rows = E * 2I, cols = H; w_down [E, H, I] as rows = E * H, cols = I (each
 *   expert's rows are an even count, so no block spans two experts).
 * moe_permute_tiled: moe_permute with x_perm [P_max, H] written tiled. Every row
 *   pair below offsets[E] is written whole, pad rows as zeros (when offsets[E]
 *   is odd, row offsets[E] is written as zeros too); pairs past it are not
 *   written.
 * moe_grouped_glu_gemm_tiled: x_perm and w_gate_up tiled; h [P_max, I] written tiled.
 * moe_grouped_glu_gemm_gather_tiled: x [T, H] row-major (read through row_token),
 *   w_gate_up tiled, h written tiled.
 * moe_grouped_down_gemm_tiled: h and w_down tiled; y [P_max, H] row-major, so
 *   moe_combine reads it unchanged.
 * Arguments, shapes and errors as for the row-major calls, plus P_max even
 * (MOE_ERR_INVALID_SHAPE otherwise): the tiled buffers hold whole row pairs.
 */
moe_status moe_tile_rows(const moe_bf16 *src, int64_t rows, int32_t cols, moe_bf16 *dst, moe_stream_t stream);
moe_status moe_untile_rows(const moe_bf16 *src, int64_t rows, int32_t cols, moe_bf16 *dst, moe_stream_t stream);
moe_status moe_permute_tiled(const moe_bf16 *x, const int32_t *topk_idx, int64_t T, int32_t H,
                             int32_t E, int32_t k, int32_t align, int64_t P_max,
                             int32_t *expert_counts, int32_t *expert_offsets, int32_t *route_row,
                             int32_t *row_token, moe_bf16 *x_perm, void *workspace,
                             size_t workspace_bytes, moe_stream_t stream);
moe_status moe_grouped_glu_gemm_tiled(const moe_bf16 *x_perm, const moe_bf16 *w_gate_up,
                                      const int32_t *expert_counts, const int32_t *expert_offsets,
                                      int32_t E, int32_t H, int32_t I, int64_t P_max, moe_bf16 *h,
                                      moe_stream_t stream);
moe_status moe_grouped_glu_gemm_gather_tiled(const moe_bf16 *x, const int32_t *row_token,
                                             const moe_bf16 *w_gate_up, const int32_t *expert_counts,
                                             const int32_t *expert_offsets, int64_t T, int32_t E,
                                             int32_t H, int32_t I, int64_t P_max, moe_bf16 *h,
                                             moe_stream_t stream);
moe_status moe_grouped_down_gemm_tiled(const moe_bf16 *h, const moe_bf16 *w_down,
                                       const int32_t *expert_counts, const int32_t *expert_offsets,
                                       int32_t E, int32_t H, int32_t I, int64_t P_max, moe_bf16 *y,
                                       moe_stream_t stream);

/*
 * FP8 expert weights (moe_quantize_fp8's codes) in tiled order: a code matrix
 * [R, K] (R % 4 == 0, K % 32 == 0) kept as 4 x 32-byte blocks, code (r, c) at
 *     ((r / 4) * (K / 32) + c / 32) * 128 + (r % 4) * 32 + c % 32,
 * so one 32-code k stage of four neighbouring rows is one 128-byte line. The
 * scales are unchanged (one per 64 rows, row-major). moe_tile_fp8_rows /
 * moe_untile_fp8_rows convert [rows, cols] codes (w8_gate_up as rows = E * 2I,
 * cols = H; w8_down as E * H, I), once per weight update; rows a multiple of 4.
 * The two GEMMs take those codes with x_perm / h as for the bf16 tiled calls
 * and compute what the *_fp8w calls compute, always on the 256-row MFMA tiles
 * (never the weight-streaming kernel), so they equal the *_fp8w calls bit for
 * bit wherever those use the MFMA tiles (P_max > 64 E). (No gathering variant:
 * with tiled FP8 weights that kernel does not fit its scalar registers.)
 */
moe_status moe_tile_fp8_rows(const uint8_t *src, int64_t rows, int32_t cols, uint8_t *dst, moe_stream_t stream);
moe_status moe_untile_fp8_rows(const uint8_t *src, int64_t rows, int32_t cols, uint8_t *dst, moe_stream_t stream);
moe_status moe_grouped_glu_gemm_fp8w_tiled(const moe_bf16 *x_perm, const uint8_t *w8_gate_up,
                                           const float *scale_gate_up, const int32_t *expert_counts,
                                           const int32_t *expert_offsets, int32_t E, int32_t H, int32_t I,
                                           int64_t P_max, moe_bf16 *h, moe_stream_t stream);
moe_status moe_grouped_down_gemm_fp8w_tiled(const moe_bf16 *h, const uint8_t *w8_down, const float *scale_down,
                                            const int32_t *expert_counts, const int32_t *expert_offsets,
                                            int32_t E, int32_t H, int32_t I, int64_t P_max, moe_bf16 *y,
                                            moe_stream_t stream);

/*
 * Score-weighted gather-sum [prime-rl, Changes: one fp32 score-weighted
 * gather-sum back].  Per token t, a gather (no scatter-add):
 *   out[t, c] = bf16_rne( sum_{j=0..k-1} topk_w[t, j] * y[route_row[t*k+j], c] )
 * summed in fp32 in ascending j.
 *   y [P_max, H] bf16;  route_row [T*k] int32 in [0, P_max) (unchecked);
 *   topk_w [T, k] fp32;  out [T, H] bf16 out
 * Shapes: H % 64 == 0, 1 <= k <= MOE_MAX_K.
 */
moe_status moe_combine(const moe_bf16 *y, const int32_t *route_row, const float *topk_w,
                       int64_t T, int32_t H, int32_t k, int64_t P_max, moe_bf16 *out,
                       moe_stream_t stream);

/*
 * Block-scaled FP8 expert weights [prime-rl, Changes: FP8 expert weights
 * quantized once per optimizer step; Halo, Levers that do not help here: fp8
 * halves the expert-weight bytes].  Format: OCP E4M3 (e4m3fn: bias 7, no
 * infinity, S.1111.111 is NaN, largest finite 448).  w [E, R, K] is cut into
 * blocks of 64 consecutive rows of one expert over all of K:
 *   scale[e, b]  = max|w[e, 64b .. 64b+63, :]| / 448   (fp32; 1.0 if all zero)
 *   w8[e, r, c]  = E4M3 code nearest to clamp(w[e, r, c] / scale[e, r/64], +-448),
 *                  ties to the even code (fp32 division)
 * so w[e, r, c] ~= scale[e, r/64] * value(w8[e, r, c]).
 *   w      [E, R, K] bf16 (finite values; unchecked)
 *   w8     [E, R, K] uint8 out;  scale [E, R/64] fp32 out
 * Quantize w_gate_up as [E, 2I, H] (gate and up rows fall in separate blocks)
 * and w_down as [E, H, I].
 * Shapes: R % 64 == 0, K % 64 == 0, 1 <= E, E * R / 64 < 2^31.
 */
moe_status moe_quantize_fp8(const moe_bf16 *w, int64_t E, int32_t R, int32_t K, uint8_t *w8,
                            float *scale, moe_stream_t stream);

/*
 * moe_grouped_glu_gemm with FP8 weights from moe_quantize_fp8 [prime-rl,
 * Changes: blockwise FP8 grouped GEMMs].  For every routed row p of expert e:
 *   g = scale_gu[e, i/64]     * (x_perm[p] . value(w8_gate_up[e, i, :]))
 *   u = scale_gu[e, (I+i)/64] * (x_perm[p] . value(w8_gate_up[e, I+i, :]))
 *   h[p, i] = bf16_rne(silu(g) * u)
 * The codes are widened to bf16 exactly; products and sums in fp32, the scale
 * applied to the fp32 sum.
 *   w8_gate_up [E, 2I, H] uint8;  scale_gate_up [E, 2I/64] fp32
 * Other arguments, outputs and shapes as for moe_grouped_glu_gemm.
 */
moe_status moe_grouped_glu_gemm_fp8w(const moe_bf16 *x_perm, const uint8_t *w8_gate_up,
                                     const float *scale_gate_up, const int32_t *expert_counts,
                                     const int32_t *expert_offsets, int32_t E, int32_t H, int32_t I,
                                     int64_t P_max, moe_bf16 *h, moe_stream_t stream);

/* moe_grouped_glu_gemm_gather with FP8 weights (as moe_grouped_glu_gemm_fp8w). */
moe_status moe_grouped_glu_gemm_gather_fp8w(const moe_bf16 *x, const int32_t *row_token,
                                            const uint8_t *w8_gate_up, const float *scale_gate_up,
                                            const int32_t *expert_counts,
                                            const int32_t *expert_offsets, int64_t T, int32_t E,
                                            int32_t H, int32_t I, int64_t P_max, moe_bf16 *h,
                                            moe_stream_t stream);

/*
 * moe_grouped_down_gemm with FP8 weights:
 *   y[p, c] = bf16_rne(scale_down[e, c/64] * (h[p] . value(w8_down[e, c, :])))
 *   w8_down [E, H, I] uint8;  scale_down [E, H/64] fp32
 */
moe_status moe_grouped_down_gemm_fp8w(const moe_bf16 *h, const uint8_t *w8_down,
                                      const float *scale_down, const int32_t *expert_counts,
                                      const int32_t *expert_offsets, int32_t E, int32_t H, int32_t I,
                                      int64_t P_max, moe_bf16 *y, moe_stream_t stream);

/*
 * Router projection fused with top-k routing [PocketLLM, Remaining prefill
 * attribution: the router is a phase of its own].  The fp32 router weight
 * w_router [H, E] is prepared once per weight update into two bf16 matrices
 * stored expert-major, w_hi = bf16_rne(w_router^T) and w_lo = bf16_rne(w_router^T
 * - w_hi) ([E, H] each).  moe_router_topk then computes, per token,
 *   logits[t, e] = sum_h x[t, h] (w_hi[e, h] + w_lo[e, h])   (fp32 accumulation;
 *                  within about 2^-16 relative of the fp32 projection per term)
 * and routes on them exactly as moe_route_topk does on its input logits (same
 * order, ties and softmax).  logits [T, E] fp32 is written only if non-NULL.
 *   x [T, H] bf16;  topk_idx [T, k] int32, topk_w [T, k] fp32 out.
 * Shapes: H % 64 == 0, 1 <= k <= min(E, MOE_MAX_K), 1 <= E <= MOE_MAX_E.
 */
moe_status moe_router_prepare(const float *w_router, int32_t H, int32_t E, moe_bf16 *w_hi, moe_bf16 *w_lo,
                              moe_stream_t stream);
moe_status moe_router_topk(const moe_bf16 *x, const moe_bf16 *w_hi, const moe_bf16 *w_lo, int64_t T, int32_t H,
                           int32_t E, int32_t k, float *logits, int32_t *topk_idx, float *topk_w,
                           moe_stream_t stream);

/*
 * The gate/up GEMM with a clamped SwiGLU [prime-rl PR 3885, Changes: the V4.1
 * recipes run a clamped SwiGLU]; the pages give neither its form nor its constant,
 * so the limit is an argument and the form is the plainest reading -- the gate
 * pre-activation capped at +limit, the up projection clipped to [-limit, limit]:
 *   h[p, i] = bf16_rne( silu(min(g, limit)) * min(max(u, -limit), limit) )
 * with g, u the fp32 sums of moe_grouped_glu_gemm.  limit = +inf is exactly
 * moe_grouped_glu_gemm.  Arguments and shapes as moe_grouped_glu_gemm; limit
 * must be >= 0 (a NaN or negative limit: MOE_ERR_INVALID_VALUE).
 */
moe_status moe_grouped_glu_gemm_clamped(const moe_bf16 *x_perm, const moe_bf16 *w_gate_up,
                                        const int32_t *expert_counts, const int32_t *expert_offsets, int32_t E,
                                        int32_t H, int32_t I, int64_t P_max, float limit, moe_bf16 *h,
                                        moe_stream_t stream);

/*
 * ---- training: forward with saved gate/up output, and the backward ----
 *
 * Backward recipe for one layer (gradients of a loss with dL/dout = dout):
 *   forward:  moe_route_topk, moe_permute, gu = moe_grouped_gemm(x_perm, w_gate_up)
 *             [P_max, 2I], h = moe_swiglu(gu), y = moe_grouped_down_gemm(h, w_down),
 *             out = moe_combine(y)
 *   backward: dy, dw = moe_combine_backward(dout, y); dlogits = moe_route_backward(dw);
 *             dgu = moe_grouped_gemm_swiglu_backward(dy, w_down^T, gu)  (or, in two
 *             steps, dh = moe_grouped_gemm(dy, w_down^T); dgu = moe_swiglu_backward(dh, gu));
 *             dx_perm = moe_grouped_gemm(dgu, w_gate_up^T); dx = moe_permute_backward;
 *             dW_down = moe_grouped_wgrad(dy, h); dW_gate_up = moe_grouped_wgrad(dgu, x_perm)
 *   where w^T comes from moe_transpose_experts once per weight update.
 * Pad rows: moe_combine_backward zeroes dy's pad rows, so every later step may run
 * over whole padded segments and the weight gradients get nothing from them.
 */

/*
 * Plain grouped GEMM: for every row p of expert e's padded segment,
 *   c[p, n] = bf16_rne( sum_k a[p, k] w[e, n, k] )     (fp32 accumulation)
 *   a [P_max, K] bf16;  w [E, N, K] bf16;  c [P_max, N] bf16 out (rows past offsets[E]
 *   not written).  The gate/up output: a = x_perm, w = w_gate_up, N = 2I, K = H.
 *   The input gradients: a = dy, w = w_down^T [E, I, H] (N = I, K = H) for dh, and
 *   a = dgu, w = w_gate_up^T [E, H, 2I] (N = H, K = 2I) for dx_perm.
 * Shapes: K % 64 == 0, N % 64 == 0, 4*N*K < 2^32, 1 <= E <= MOE_MAX_E, 0 < P_max < 2^31.
 */
moe_status moe_grouped_gemm(const moe_bf16 *a, const moe_bf16 *w, const int32_t *expert_counts,
                            const int32_t *expert_offsets, int32_t E, int32_t K, int32_t N, int64_t P_max,
                            moe_bf16 *c, moe_stream_t stream);

/*
 * The input-gradient GEMM of the down projection with the SwiGLU backward in its
 * epilogue [prime-rl PR 3885, Changes: grouped dgrad GEMMs of the expert path; the
 * SwiGLU backward folded into the GEMM that produces dh]: for every row p of
 * expert e's padded segment and 0 <= i < I,
 *   dh[p, i]      = bf16_rne( sum_c dy[p, c] w_down_t[e, i, c] )   (fp32 accumulation)
 *   dgu[p, i]     = bf16_rne( dh[p, i] u silu'(g) ),  dgu[p, I + i] = bf16_rne( dh[p, i] silu(g) )
 * with g = gu[p, i], u = gu[p, I + i] and the fp32 arithmetic of moe_swiglu_backward,
 * so dgu equals moe_swiglu_backward(moe_grouped_gemm(dy, w_down_t), gu) bit for bit;
 * dh itself is never written.
 *   dy [P_max, H] bf16;  w_down_t [E, I, H] bf16 (moe_transpose_experts of w_down);
 *   gu [P_max, 2I] bf16 (the forward's saved gate/up output);  dgu [P_max, 2I] bf16 out
 *   (rows past offsets[E] not written).
 * Shapes: H % 64 == 0, I % 64 == 0, 4*H*I < 2^32, 1 <= E <= MOE_MAX_E, 0 < P_max < 2^31;
 * every pointer 16-byte aligned.
 */
moe_status moe_grouped_gemm_swiglu_backward(const moe_bf16 *dy, const moe_bf16 *w_down_t, const moe_bf16 *gu,
                                            const int32_t *expert_counts, const int32_t *expert_offsets,
                                            int32_t E, int32_t H, int32_t I, int64_t P_max, moe_bf16 *dgu,
                                            moe_stream_t stream);

/*
 * SwiGLU on saved gate/up rows, gu = [g | u] ([P_max, 2I], g the first I columns):
 *   moe_swiglu:           h[p, i] = bf16_rne(silu(g) u)
 *   moe_swiglu_backward:  dgu[p, i] = bf16_rne(dh u silu'(g)),  dgu[p, I+i] = bf16_rne(dh silu(g)),
 *                         silu'(g) = s (1 + g (1 - s)),  s = sigmoid(g)
 * over the rows p < offsets[E] (fp32 arithmetic); h, dh [P_max, I].  I % 64 == 0.
 */
moe_status moe_swiglu(const moe_bf16 *gu, const int32_t *expert_offsets, int32_t E, int32_t I,
                      int64_t P_max, moe_bf16 *h, moe_stream_t stream);
moe_status moe_swiglu_backward(const moe_bf16 *dh, const moe_bf16 *gu, const int32_t *expert_offsets,
                               int32_t E, int32_t I, int64_t P_max, moe_bf16 *dgu, moe_stream_t stream);

/*
 * Expert weight transpose, once per weight update: wt[e, c, r] = w[e, r, c].
 *   w [E, R, C] bf16;  wt [E, C, R] bf16 out.  R % 64 == 0, C % 64 == 0.
 */
moe_status moe_transpose_experts(const moe_bf16 *w, int64_t E, int32_t R, int32_t C, moe_bf16 *wt,
                                 moe_stream_t stream);

/*
 * Backward of the combine [prime-rl, Changes: gathers in backward too]:
 *   dw[t, j] = sum_c dout[t, c] y[route_row[t*k+j], c]          (fp32; fixed order)
 *   dy[route_row[t*k+j], c] = bf16_rne(topk_w[t, j] dout[t, c])
 *   dy[p, :] = 0 for every pad row p < offsets[E] (row_token[p] == -1)
 *   dout [T, H] bf16;  y [P_max, H] bf16;  dy [P_max, H] bf16 out;  dw [T, k] fp32 out
 *   route_row, topk_w, row_token, expert_offsets as from the forward.
 * Shapes: H % 64 == 0, 1 <= k <= min(E, MOE_MAX_K), 0 < P_max < 2^31.
 */
moe_status moe_combine_backward(const moe_bf16 *dout, const moe_bf16 *y, const int32_t *route_row,
                                const float *topk_w, const int32_t *row_token,
                                const int32_t *expert_offsets, int64_t T, int32_t H, int32_t E, int32_t k,
                                int64_t P_max, moe_bf16 *dy, float *dw, moe_stream_t stream);

/*
 * Backward of the routing softmax (over the k selected logits):
 *   dlogits[t, topk_idx[t, j]] = topk_w[t, j] (dw[t, j] - sum_i topk_w[t, i] dw[t, i]),
 *   dlogits[t, e] = 0 for every expert not selected.   dlogits [T, E] fp32 out.
 */
moe_status moe_route_backward(const int32_t *topk_idx, const float *topk_w, const float *dw, int64_t T,
                              int32_t E, int32_t k, float *dlogits, moe_stream_t stream);

/*
 * Backward of the permute: dx[t, c] = bf16_rne( sum_j dx_perm[route_row[t*k+j], c] ),
 * summed in fp32 in ascending j (the combine's gather with unit weights).
 *   dx_perm [P_max, H] bf16;  dx [T, H] bf16 out.  Shapes as for moe_combine.
 */
moe_status moe_permute_backward(const moe_bf16 *dx_perm, const int32_t *route_row, int64_t T, int32_t H,
                                int32_t k, int64_t P_max, moe_bf16 *dx, moe_stream_t stream);

/*
 * Expert weight gradients, K-grouped over each expert's padded segment [prime-rl,
 * Changes: one K-grouped GEMM per weight; weight gradients into fp32]:
 *   dw[e, m, n] = sum over rows p of e's segment of a[p, m] b[p, n]   (fp32 out)
 *   a [P_max, M] bf16 (pad rows must be zero: dy and dgu from this recipe are);
 *   b [P_max, N] bf16, or with row_token non-NULL the token matrix x [T, N] read as
 *   b[p] = x[row_token[p]] (a zero row where row_token[p] == -1);
 *   dw [E, M, N] fp32 out; an expert with no rows gets zeros.
 *   dW_down: a = dy, b = h (M = H, N = I).  dW_gate_up: a = dgu, b = x_perm (M = 2I, N = H).
 * Shapes: M % 64 == 0, N % 64 == 0, 1 <= E <= MOE_MAX_E, 0 < P_max < 2^31.
 * dw must be 16-byte aligned (MOE_ERR_MISALIGNED_POINTER otherwise).
 */
moe_status moe_grouped_wgrad(const moe_bf16 *a, const moe_bf16 *b, const int32_t *row_token,
                             const int32_t *expert_counts, const int32_t *expert_offsets, int32_t E,
                             int32_t M, int32_t N, int64_t P_max, float *dw, moe_stream_t stream);

/*
 * The training steps on row-pair tiled operands (the order moe_tile_rows writes,
 * see "Row-pair tiled operands" above). Each call computes exactly what its
 * row-major counterpart computes -- the same MFMAs, the same fp32 order, the same
 * roundings -- so its outputs are those of that call bit for bit once un-tiled;
 * only where operands are read from and written to changes. Recipe (the weights
 * tiled once per update: w_gate_up and w_down as for the tiled forward, and
 * w_gate_up^T [E, H, 2I] from moe_transpose_experts, then moe_tile_rows):
 *   forward:  moe_route_topk, moe_permute_tiled (x_perm tiled),
 *             gu = moe_grouped_gemm_tiled(x_perm, w_gate_up) (gu row-major),
 *             h = moe_swiglu_tiled(gu) (h tiled), y = moe_grouped_down_gemm_tiled(h, w_down),
 *             out = moe_combine(y)
 *   backward: dy, dw = moe_combine_backward(dout, y) (row-major), moe_route_backward,
 *             dh = moe_grouped_gemm(dy, w_down^T) (row-major operands),
 *             dgu = moe_swiglu_backward_tiled(dh, gu) (dgu tiled),
 *             dx_perm = moe_grouped_gemm_tiled(dgu, w_gate_up^T tiled) (dx_perm row-major),
 *             moe_permute_backward,
 *             dW_down = moe_grouped_wgrad_tiled(dy, 0, h, 1),
 *             dW_gate_up = moe_grouped_wgrad_tiled(dgu, 1, x_perm, 1).
 *
 * moe_grouped_gemm_tiled: moe_grouped_gemm with a [P_max, K] and w [E, N, K] tiled;
 *   c [P_max, N] row-major out.
 * moe_swiglu_tiled: moe_swiglu with h [P_max, I] written tiled; a row of the last
 *   pair at or past offsets[E] is written as zeros.
 * moe_swiglu_backward_tiled: moe_swiglu_backward (dh and gu row-major) with
 *   dgu [P_max, 2I] written tiled; a row of the last pair at or past offsets[E] is
 *   written as zeros.
 * moe_grouped_wgrad_tiled: moe_grouped_wgrad (no row_token) with a, b each
 *   row-major (0) or tiled (1): a_tiled, b_tiled outside {0, 1}: MOE_ERR_INVALID_SHAPE.
 * Shapes as for the row-major calls; P_max must be even where an operand is tiled
 * (MOE_ERR_INVALID_SHAPE otherwise).
 */
moe_status moe_grouped_gemm_tiled(const moe_bf16 *a, const moe_bf16 *w, const int32_t *expert_counts,
                                  const int32_t *expert_offsets, int32_t E, int32_t K, int32_t N, int64_t P_max,
                                  moe_bf16 *c, moe_stream_t stream);
moe_status moe_swiglu_tiled(const moe_bf16 *gu, const int32_t *expert_offsets, int32_t E, int32_t I,
                            int64_t P_max, moe_bf16 *h, moe_stream_t stream);
moe_status moe_swiglu_backward_tiled(const moe_bf16 *dh, const moe_bf16 *gu, const int32_t *expert_offsets,
                                     int32_t E, int32_t I, int64_t P_max, moe_bf16 *dgu, moe_stream_t stream);
moe_status moe_grouped_wgrad_tiled(const moe_bf16 *a, int32_t a_tiled, const moe_bf16 *b, int32_t b_tiled,
                                   const int32_t *expert_counts, const int32_t *expert_offsets, int32_t E, int32_t M,
                                   int32_t N, int64_t P_max, float *dw, moe_stream_t stream);

/*
 * Debug build [prime-rl, Changes: 32-bit row offsets overflowed silently -- a bad
 * index must be reported, not turned into a stray write]. The debug library
 * (libmoe_mi355x_debug.so, built with MOE_DEBUG) exports the same calls; ahead of
 * each call's kernels it enqueues checks of the preconditions the release kernels
 * trust without checking:
 *   moe_route_topk            every logit finite
 *   moe_permute               every top-k id in [0, E), a token's k ids distinct
 *   every call taking expert_offsets   offsets[0] == 0, non-decreasing,
 *                             offsets[E] <= P_max, and (where counts are passed)
 *                             0 <= counts[e] <= offsets[e+1] - offsets[e]
 *   moe_combine, moe_permute_backward, moe_combine_backward   route_row in [-1, P_max)
 *   the gathering gate/up GEMMs   row_token in [-1, T)
 * A failed check stores a code in a device word; from then on every kernel of the
 * library (this call's and later calls') does nothing until moe_debug_reset, so
 * no kernel runs on the bad data and nothing traps. The calls themselves still
 * return MOE_OK (nothing is read back); moe_debug_status reports the word.
 *
 * moe_debug_build:  1 in the debug library, 0 in the release library.
 * moe_debug_status: synchronises `stream`, reads the word: MOE_OK if no check has
 *                   failed, else MOE_ERR_PRECONDITION with moe_last_error_message()
 *                   naming the failed check. The release library returns MOE_OK.
 * moe_debug_reset:  enqueues a clear of the word on `stream` (no-op in release).
 * The word is one per device and process, shared by all streams.
 */
int moe_debug_build(void);
moe_status moe_debug_status(moe_stream_t stream);
moe_status moe_debug_reset(moe_stream_t stream);

/*
 * Measurement probes -- not part of the layer. The chip's own roofs, measured on
 * the device at hand, so kernel times can be placed against them as well as
 * against the published peaks [PocketLLM, Theoretical ceilings / Hardware roofs:
 * a measured copy rate and measured GEMM rates quoted beside the spec].
 *
 * moe_probe_copy: dst[0 .. bytes) = src[0 .. bytes) with a grid-stride kernel of
 * non-temporal 16-byte loads and stores (bytes read + bytes written, each once).
 *   src, dst  device buffers of `bytes` bytes, 16-byte aligned, not overlapping
 *   bytes     a positive multiple of 16, else MOE_ERR_INVALID_SHAPE
 *
 * moe_probe_read: reads src[0 .. bytes) once with the copy's grid-stride walk of
 * non-temporal 16-byte loads and writes only a 16-byte XOR of each thread's loads
 * to sink (the read-only HBM rate).
 *   src          device buffer of `bytes` bytes, 16-byte aligned
 *   bytes        a positive multiple of 16, else MOE_ERR_INVALID_SHAPE
 *   sink         device buffer of at least moe_probe_read_sink_bytes() bytes, 16-byte
 *                aligned (MOE_ERR_WORKSPACE_TOO_SMALL otherwise); its values are meaningless
 *
 * moe_probe_mfma_bf16: a register-only loop of v_mfma_f32_32x32x16_bf16 on every
 * compute unit (8 waves per CU, 4 independent accumulator chains per wave,
 * `iters` rounds); no memory traffic but one float per thread written to sink.
 *   sink         device buffer of at least moe_probe_mfma_sink_floats() floats
 *                (MOE_ERR_WORKSPACE_TOO_SMALL otherwise); its values are meaningless
 *   iters >= 1   (MOE_ERR_INVALID_VALUE otherwise)
 *   *flops       host out: the launch's bf16 flops (2*32*32*16 per MFMA)
 */
moe_status moe_probe_copy(const void *src, void *dst, size_t bytes, moe_stream_t stream);
moe_status moe_probe_read(const void *src, size_t bytes, void *sink, size_t sink_bytes, moe_stream_t stream);
size_t moe_probe_read_sink_bytes(void);
moe_status moe_probe_mfma_bf16(float *sink, int64_t sink_floats, int32_t iters, double *flops,
                               moe_stream_t stream);
int64_t moe_probe_mfma_sink_floats(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
