/*
 * moe.h -- C ABI of the MI355X (gfx950) trainable MoE expert layer.
 *
 * One GPU's share of a fused mixture-of-experts layer, forward and backward.
 * The computation follows the pages that describe Prime Mega MoE:
 *   - MarkTechPost article "Prime Intellect Releases Prime Mega MoE: Trainable
 *     Fused MoE Kernel, 3.11x Faster Forward Pass", section "How does the
 *     fused kernel work?": one call covers the two expert linear layers with
 *     SwiGLU between them and the weighted combine; the backward adds the
 *     missing gradient pass.
 *   - kongchang.com explainer, grouped-GEMM note: routing indices become a
 *     token reorder, then one grouped GEMM call indexes each expert's
 *     differently-sized matrix product by group offsets, then activation and
 *     routing-weighted aggregation.
 *   - ic.work analysis, section on hardware constraints: bias-free gated
 *     experts only, hidden size divisible by 256, intermediate size divisible
 *     by 128; precisions BF16, MXFP8 and blockwise FP8.
 * The router is outside the call (ic.work analysis, section on idealised
 * assumptions: the single-layer benchmark excludes the router), so routing
 * arrives as (topk_idx, topk_w). There is no cross-GPU dispatch.
 *
 * Notation: T tokens, H hidden, I expert intermediate, E experts, k experts
 * per token, M = T*k routed (token, slot) pairs, f = t*k + j the flat pair.
 *
 * Math (fp32 accumulation; SwiGLU a = silu(g)*u, silu(g) = g*sigmoid(g)):
 *   g = W13[e][0:I] x[t],  u = W13[e][I:2I] x[t],  o = W2[e] (silu(g)*u)
 *   y[t] = sum_j topk_w[t,j] * o(t, j)
 * Backward of L = <dY, y>:
 *   d_topk_w[t,j] = <dY[t], o>,  dO = w dY[t],  dA = W2[e]^T dO,
 *   dg = dA*u*sig(g)*(1 + g*(1 - sig(g))),  du = dA*silu(g),
 *   dx[t] += W13[e]^T [dg;du],  dW13[e] += [dg;du] x[t]^T,  dW2[e] += dO a^T.
 *
 * Conventions for every entry point:
 *   - All tensor pointers are device memory owned by the caller; the library
 *     never allocates, frees or synchronises on the forward/backward path.
 *     Tensors are dense and row-major with the shapes given below; every
 *     tensor pointer must be 16-byte aligned.
 *   - `stream` is a hipStream_t (NULL = the null stream); all work is
 *     enqueued on it in order. Results are ready when the stream says so.
 *   - Host-checkable preconditions are checked before anything is launched;
 *     on error the call returns a status and enqueues nothing.
 *   - Expert ids outside [0, E) are dropped (the pair contributes nothing and
 *     gets d_topk_w = 0); the forward records this in a device status word
 *     read back by moe_read_status.
 *   - Calls that share a workspace or saved buffer must not overlap.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_NULL = 1,        /* a required pointer is NULL                       */
  MOE_ERR_SHAPE = 2,       /* H%256, I%128, k<1, k>E, T<0, E<1 or size limits */
  MOE_ERR_ALIGN = 3,       /* a tensor pointer is not 16-byte aligned          */
  MOE_ERR_PRECISION = 4,   /* unknown precision value                          */
  MOE_ERR_ARCH = 5,        /* current device is not gfx950                     */
  MOE_ERR_WORKSPACE = 6,   /* workspace or saved buffer smaller than required  */
  MOE_ERR_LAUNCH = 7,      /* a HIP launch or runtime call failed              */
  MOE_ERR_ROUTING = 8,     /* device: some expert id was outside [0, E)        */
  MOE_ERR_UNSUPPORTED = 9  /* valid request this library does not implement    */
} moe_status;

/* Precision of the expert GEMMs (ic.work analysis, hardware constraints;
 * MarkTechPost article, "How do developers use it?": bf16, mxfp8, fp8 and
 * fp8_bwd = BF16 forward with FP8 backward). The pages fix no number format
 * or scale rule; this library reads them as follows.
 *   FP8 values are OCP E4M3 (bias 7, max 448, round to nearest even,
 *   saturating); every block of values has one power-of-two scale 2^e,
 *   stored as the byte e + 127.
 *   MOE_FP8_BLOCK: activations in 1x128 blocks along the GEMM's reduction
 *     axis, weights in 128x128 tiles; e is the smallest integer with
 *     448 * 2^e >= the block's largest magnitude.
 *   MOE_MXFP8: 1x32 blocks along the reduction axis for every operand;
 *     e = floor(log2(largest magnitude)) - 8.
 *   An all-zero block has e = 0.
 * Quantized operands: x, w*silu(g)*u and both weight stacks in the forward;
 * dY, [dg | du] and the weights (re-blocked for the transposed product
 * under MXFP8) in the backward. By default the weight-gradient GEMMs read
 * the bf16 tensors x, dY, w*silu(g)*u and [dg | du]; with MOE_FLAG_FP8_WGRAD
 * (see moe_shape) they read those four quantized along each expert's rows:
 * every column in blocks of 128 rows (MOE_FP8_BLOCK, MOE_FP8_BWD; pow2 rule)
 * or 32 rows (MOE_MXFP8; MX rule), counted from the expert's first row in
 * permuted order. MOE_FP8_BWD runs the forward of MOE_BF16 and the backward
 * of MOE_FP8_BLOCK.
 *   MOE_FP8_FP4: an inference forward with FP4 weights (the FP8 x FP4 type
 *     of a forward-only fused MoE kernel in the MarkTechPost article's
 *     comparison table). Activations as MOE_MXFP8; W13 and W2 in OCP MX FP4
 *     (E2M1: 0, 0.5, 1, 1.5, 2, 3, 4, 6 and their negatives, round to
 *     nearest even, saturating) in 1x32 blocks along the reduction axis with
 *     e = floor(log2(largest magnitude)) - 2. moe_bwd rejects it
 *     (MOE_ERR_PRECISION), as does MOE_FLAG_FP8_WGRAD. */
/*   MOE_FP8_BLOCK_F32, MOE_FP8_BWD_F32: blockwise FP8 with fp32 block
 *     scales (the blocks of MOE_FP8_BLOCK: 1x128 activations, 128x128
 *     weights). A block with largest magnitude amax > 0 has the scale
 *     s = amax / 448 and inv = 448 / amax (each an fp32 division, correctly
 *     rounded); a value v is stored as the E4M3 code of fl32(v * inv), so
 *     the block maximum becomes +-448; an all-zero block, or one whose
 *     448 / amax overflows fp32 (amax below about 1.3e-36), has s = 1 and
 *     zero codes. The GEMMs run each 128-deep block at unit hardware scale
 *     and add it to the fp32 accumulators times s_x * s_w. A scale array
 *     holds one float per (row, 128 values), in the bytes the E8M0 layout
 *     gives those 128 values' four 32-blocks (the layouts below keep their
 *     sizes). MOE_FP8_BWD_F32 runs the forward of MOE_BF16 and the backward
 *     of MOE_FP8_BLOCK_F32. Both reject MOE_FLAG_FP8_WGRAD
 *     (MOE_ERR_UNSUPPORTED). */
typedef enum moe_precision {
  MOE_BF16 = 0,
  MOE_FP8_BLOCK = 1,
  MOE_MXFP8 = 2,
  MOE_FP8_BWD = 3,
  MOE_FP8_FP4 = 4,
  MOE_FP8_BLOCK_F32 = 5,
  MOE_FP8_BWD_F32 = 6
} moe_precision;

/* Flags of moe_shape.flags. MOE_FLAG_FP8_WGRAD: the weight-gradient GEMMs
 * of an FP8 precision run in FP8 on operands quantized along each expert's
 * rows (see moe_precision); with MOE_BF16 it is MOE_ERR_PRECISION. */
enum { MOE_FLAG_FP8_WGRAD = 1 };

/* Problem description. Limits: 0 <= T, 1 <= E <= 1024, 1 <= k <= E,
 * T*k < 2^31, T*H < 2^31, T*k*I < 2^30, H%256 == 0, I%128 == 0,
 * 256 <= H <= 16384, 128 <= I <= 8192 (the kernels address rows with
 * 32-bit byte offsets); with MOE_FLAG_FP8_WGRAD also T*k < 2^23.
 * num_cus caps how many compute units the persistent GEMMs occupy
 * (0 = all), so that concurrent kernels (e.g. collectives) keep CUs.
 * flags: MOE_FLAG_* bits (unknown bits: MOE_ERR_PRECISION); reserved
 * must be 0 (else MOE_ERR_SHAPE). */
typedef struct moe_shape {
  int64_t T, H, I, E, k;
  int32_t precision; /* moe_precision */
  int32_t num_cus;
  int32_t flags;
  int32_t reserved;
} moe_shape;

/* Byte sizes of the three caller-provided buffers for `s`:
 *   fwd_ws      scratch of moe_fwd (also holds its status word)
 *   saved_bytes what moe_fwd keeps for moe_bwd (permutation, gate/up
 *               pre-activations, activations)
 *   bwd_ws      scratch of moe_bwd
 * Any output pointer may be NULL. Pure host function. */
moe_status moe_workspace_size(const moe_shape* s, size_t* fwd_ws, size_t* saved_bytes,
                              size_t* bwd_ws);

/* Layout of the saved buffer (byte offsets from its start). Pure host. */
typedef struct moe_saved_layout {
  size_t counts;    /* int32 [E]      rows per expert                         */
  size_t offsets;   /* int32 [E+1]    exclusive prefix of counts              */
  size_t row_of;    /* int32 [T*k]    permuted row of pair f, -1 if dropped   */
  size_t src_of;    /* int32 [T*k]    pair f of permuted row r (first M used) */
  size_t wrow;      /* fp32 [T*k]     routing weight of permuted row r        */
  size_t h13;       /* bf16 [T*k,2I]  per permuted row: [g | u] (bf16)        */
  size_t act;       /* bf16 [T*k, I]  per permuted row: w*silu(g)*u, with w   */
                    /*                the pair's routing weight (bf16)        */
  size_t total;
} moe_saved_layout;
moe_status moe_get_saved_layout(const moe_shape* s, moe_saved_layout* out);

/* Quantized weights (E4M3 codes and scale bytes) for the FP8 precisions,
 * made by moe_quantize_weights in one caller-owned buffer. Byte offsets:
 *   w13, w13_scale    forward gate/up: codes [E, 2I, H], scales [E, 2I, H/32]
 *   w2, w2_scale      forward down:    codes [E, H, I],  scales [E, H, I/32]
 *   w2t, w2t_scale    backward dH:     W2^T  codes [E, I, H],  scales [E, I, H/32]
 *   w13t, w13t_scale  backward dX:     W13^T codes [E, H, 2I], scales [E, H, 2I/32]
 * Scales are stored per (row, 32 consecutive codes); a 128-wide or 128x128
 * block repeats its byte in every 32-block it covers. Under the fp32-scale
 * precisions the same bytes hold one float per (row, 128 codes): the
 * 128x128 tile's scale, repeated on each of its rows. MOE_FP8_FP4 stores
 * only the forward parts, as E2M1 codes two per byte (w13 [E, 2I, H/2],
 * w2 [E, H, I/2]; value 2j of a row in the low nibble of byte j). Entries a
 * precision does not use (the forward parts for MOE_FP8_BWD and
 * MOE_FP8_BWD_F32, the backward
 * parts for MOE_FP8_FP4, everything for MOE_BF16) are SIZE_MAX; total is 0
 * for MOE_BF16. Pure host function. */
typedef struct moe_wq_layout {
  size_t w13, w13_scale, w2, w2_scale;
  size_t w2t, w2t_scale, w13t, w13t_scale;
  size_t total;
} moe_wq_layout;
moe_status moe_get_wq_layout(const moe_shape* s, moe_wq_layout* out);

/* Fills `wq` (moe_get_wq_layout().total bytes, 16-byte aligned) with the
 * quantized forms of W13 (bf16 [E, 2I, H]) and W2 (bf16 [E, H, I]) that
 * s->precision uses. Call again whenever the weights change; moe_fwd and
 * moe_bwd read `wq` and never the quantization of stale weights. A no-op
 * returning MOE_OK for MOE_BF16. */
moe_status moe_quantize_weights(const moe_shape* s, const void* W13, const void* W2, void* wq,
                                void* stream);

/* Quantizes bf16 rows in [rows, K] to E4M3 codes [rows, K] and scale bytes
 * [rows, K/32] by the activation rule of s->precision (1x128 blocks for
 * MOE_FP8_BLOCK and MOE_FP8_BWD, 1x32 blocks for MOE_MXFP8; see
 * moe_precision). This is the step moe_fwd applies to x and w*silu(g)*u and
 * moe_bwd to dY and [dg | du]; it is exposed for callers that keep
 * activations in FP8 and for testing. Requires 0 <= rows, 128 <= K <= 65536,
 * K % 128 == 0, rows*K < 2^31; `in` and `codes` 16-byte aligned. Under
 * MOE_FP8_BLOCK_F32 and MOE_FP8_BWD_F32 `scales` holds fp32 scales
 * [rows, K/128] (the same bytes; 4-byte aligned). MOE_ERR_PRECISION for
 * MOE_BF16. */
moe_status moe_quantize_rows(const moe_shape* s, const void* in, int64_t rows, int64_t K, void* codes,
                             void* scales, void* stream);

/* Quantizes the rows of every expert along the rows, column by column: the
 * step moe_bwd applies to x, [dg | du], dY and w*silu(g)*u under
 * MOE_FLAG_FP8_WGRAD (blocks of 128 rows with the pow2 rule for
 * MOE_FP8_BLOCK and MOE_FP8_BWD, 32 rows with the MX rule for MOE_MXFP8; see
 * moe_precision). Exposed for testing.
 *   in      bf16 [*, ld]; the r-th row of expert e is row offsets[e] + r of
 *           `in` (src_of == NULL) or row src_of[offsets[e] + r] / s->k
 *   C       columns quantized (128 <= C <= ld, C % 128 == 0, ld % 8 == 0)
 *   counts, offsets, src_of   int32 [E], [E+1], [T*k] as moe_permute writes
 *   codes   uint8, C * K bytes with K = 128 * (s->T * s->k / 128 + s->E):
 *           expert e's codes [C][Kp_e] start at byte C * poff_e, where Kp_e
 *           is counts[e] rounded up to 128 (codes past counts[e] are zero)
 *           and poff_e the sum of Kp over the experts before e
 *   scales  uint8, C * K / 32 bytes: expert e's bytes [C][Kp_e / 32] at
 *           C * poff_e / 32, one per (column, 32 rows)
 * `in` and `codes` 16-byte aligned. MOE_ERR_PRECISION for MOE_BF16,
 * MOE_ERR_UNSUPPORTED for MOE_FP8_BLOCK_F32 and MOE_FP8_BWD_F32;
 * enqueued on `stream`, the caller owns every buffer. */
moe_status moe_quantize_tokens(const moe_shape* s, const void* in, int64_t ld, int64_t C, const int32_t* counts,
                               const int32_t* offsets, const int32_t* src_of, void* codes, void* scales,
                               void* stream);

/* Expert-contiguous permutation of the routed pairs (kongchang.com explainer,
 * grouped-GEMM note: routing index -> token reorder -> grouped GEMM indexed
 * by group offsets). Integer work, deterministic:
 *   counts[e]  = #{f : topk_idx[f] == e}
 *   offsets    = exclusive prefix sum of counts, offsets[E] = number of
 *                valid pairs
 *   row_of[f]  = offsets[e] + #{f' < f : topk_idx[f'] == e}; -1 if the id
 *                is outside [0, E)
 *   src_of[r]  = f with row_of[f] == r, for r < offsets[E]
 * topk_idx: int32 [T,k]. Outputs: counts int32[E], offsets int32[E+1],
 * row_of int32[T*k], src_of int32[T*k] (entries past offsets[E] unspecified).
 * `scratch` must hold moe_permute_scratch_bytes(s) bytes; its first int32 is
 * the status word (0 or MOE_ERR_ROUTING) after the call. */
size_t moe_permute_scratch_bytes(const moe_shape* s);
moe_status moe_permute(const moe_shape* s, const int32_t* topk_idx, int32_t* counts,
                       int32_t* offsets, int32_t* row_of, int32_t* src_of, void* scratch,
                       void* stream);

/* moe_permute without a caller-provided scratch buffer, for callers that
 * cannot allocate device memory or hand the library a workspace (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * Same permutation and outputs as moe_permute (counts, offsets, row_of,
 * src_of); the status word (MOE_OK or MOE_ERR_ROUTING) goes to `status`, one
 * int32 in device memory (4-byte aligned), written. The chunk table lives in
 * a fixed device array of the library (4 MiB per device, held until the
 * process ends); it never allocates or frees. Limit: ceil(T*k / 1024) *
 * (E + 1) <= 2^20 table entries (e.g. T*k <= 8,323,072 pairs at E = 128,
 * <= 1,047,552 at E = 1024), else MOE_ERR_WORKSPACE and nothing is enqueued.
 * Every call on one device shares that array: calls that overlap on one
 * device (other streams, other threads) race and must not be issued. */
moe_status moe_permute_noalloc(const moe_shape* s, const int32_t* topk_idx, int32_t* counts,
                               int32_t* offsets, int32_t* row_of, int32_t* src_of, int32_t* status,
                               void* stream);

/* Router step before the layer. The pages leave the router outside the
 * measured layer and name that, with uniform random routing, as their
 * benchmark's idealisation (ic.work analysis, section on the benchmark's
 * idealised assumptions); the router itself is not on the pages. Reading:
 *   logits   fp32 [T, E]   a token's expert scores
 *   topk_idx int32 [T, k]  the k experts with the largest logits, in
 *                          descending order, ties to the lower expert id
 *   topk_w   fp32 [T, k]   their softmax probabilities (softmax over all E);
 *                          renorm != 0: divided by their sum (= a softmax
 *                          over the k selected logits)
 * Both outputs are written and can go straight to moe_fwd. Uses s->T, E, k
 * (check as moe_workspace_size); the caller owns every buffer; enqueued on
 * `stream`. */
moe_status moe_route(const moe_shape* s, const float* logits, int32_t renorm, int32_t* topk_idx, float* topk_w,
                     void* stream);

/* Backward of moe_route: d_logits fp32 [T, E] (written) = dL/dlogits given
 * d_topk_w = dL/dtopk_w (fp32 [T, k], e.g. from moe_bwd) and the topk_idx,
 * topk_w moe_route produced from these logits with the same renorm. The
 * selection is piecewise constant in the logits and passes no gradient:
 * renorm: w (d_topk_w - <w, d_topk_w>) on the selected experts, 0 elsewhere;
 * otherwise p (G - <p, G>) with p = softmax(logits) and G = d_topk_w placed
 * on the selected experts. */
moe_status moe_route_bwd(const moe_shape* s, const float* logits, const int32_t* topk_idx, const float* topk_w,
                         const float* d_topk_w, int32_t renorm, float* d_logits, void* stream);

/* Forward of the layer (MarkTechPost article, "How does the fused kernel
 * work?"; kongchang.com explainer, grouped-GEMM note).
 *   x        bf16  [T, H]
 *   topk_idx int32 [T, k]       expert of each pair
 *   topk_w   fp32  [T, k]       routing weight of each pair, used as given
 *   W13      bf16  [E, 2I, H]   rows [0,I) gate (W1), rows [I,2I) up (W3)
 *   W2       bf16  [E, H, I]    (W13 and W2 may be NULL where the forward
 *                               reads only wq: MOE_FP8_BLOCK, MOE_MXFP8,
 *                               MOE_FP8_FP4, MOE_FP8_BLOCK_F32)
 *   wq       quantized weights (moe_quantize_weights of this W13, W2):
 *            required for MOE_FP8_BLOCK and MOE_MXFP8, ignored for
 *            MOE_FP8_BWD, must be NULL for MOE_BF16 (else MOE_ERR_PRECISION)
 *   y        bf16  [T, H]       output (written, not accumulated)
 *   saved    moe_workspace_size().saved_bytes, or NULL for inference only;
 *            when given it is what moe_bwd reads
 *   ws       moe_workspace_size().fwd_ws bytes of scratch
 * Steps: permutation; gate/up grouped GEMM whose epilogue forms
 * w * silu(g) * u (SwiGLU with the routing weight folded in); down grouped
 * GEMM; gather-reduce combine (fp32 sum over ascending j, one bf16
 * rounding). FP8 forwards quantize x before the first GEMM and
 * w * silu(g) * u before the second. */
moe_status moe_fwd(const moe_shape* s, const void* x, const int32_t* topk_idx,
                   const float* topk_w, const void* W13, const void* W2, const void* wq,
                   void* y, void* saved, void* ws, size_t ws_bytes, void* stream);

/* The forward with the router step in front of it, fused with the
 * permutation: one pass routes each token's fp32 logits [T, E] exactly as
 * moe_route with the same renorm (the routing is the step the pages keep out
 * of their measured layer: ic.work analysis, section on the benchmark's
 * idealised assumptions) and counts, per chunk of 1024 pairs, the rows each
 * expert receives, which is the permutation's first pass; the rest is
 * moe_fwd. topk_idx int32 [T, k] and topk_w fp32 [T, k] are outputs here,
 * bit-identical to moe_route's, for moe_bwd and moe_route_bwd. Everything
 * else (buffers, errors, precisions) as moe_fwd; logits may be NULL only
 * when T == 0. */
moe_status moe_fwd_logits(const moe_shape* s, const void* x, const float* logits, int32_t renorm,
                          int32_t* topk_idx, float* topk_w, const void* W13, const void* W2, const void* wq,
                          void* y, void* saved, void* ws, size_t ws_bytes, void* stream);

/* Backward of the layer for L = <dY, y> (ic.work analysis, "From 3.11x to
 * 1.32x": the backward produces activation and weight gradients).
 *   dy       bf16 [T, H]
 *   x, topk_idx, topk_w, W13, W2: as passed to moe_fwd (W13 and W2 may be
 *            NULL for every FP8 precision: its backward reads only wq)
 *   wq       quantized weights: required for every FP8 precision, must be
 *            NULL for MOE_BF16
 *   saved    filled by moe_fwd with the same inputs
 *   dx       bf16 [T, H]        written
 *   d_topk_w fp32 [T, k]        written (0 for dropped pairs)
 *   dW13     bf16 [E, 2I, H]    written (exact zeros for experts with no rows)
 *   dW2      bf16 [E, H, I]     written (exact zeros for experts with no rows)
 *   ws       moe_workspace_size().bwd_ws bytes of scratch
 * Steps: dH grouped GEMM (K = H) with SwiGLU-backward and routing-weight
 * gradient partials fused in its epilogue; dX grouped GEMM (K = 2I);
 * gather-reduce of dx and d_topk_w; per-expert dW13 and dW2 GEMMs whose
 * reduction dimension is that expert's row count. FP8 backwards quantize dY
 * before the dH GEMM and [dg | du] before the dX GEMM; with
 * MOE_FLAG_FP8_WGRAD the weight-gradient GEMMs run in FP8 on x, [dg | du],
 * dY and w*silu(g)*u quantized along each expert's rows (moe_quantize_tokens
 * layout; [dg | du], and dY when k == 1, are quantized along both axes in
 * one pass). Under skewed routing the weight-gradient tiles of the hottest
 * experts, and under balanced routing the tiles of a last round of
 * workgroups that would be at most half full, are cut along the expert's
 * rows into fp32 partials (in bwd_ws) that a second kernel adds in a fixed
 * order: results are deterministic and do not depend on num_cus. */
moe_status moe_bwd(const moe_shape* s, const void* dy, const void* x, const int32_t* topk_idx,
                   const float* topk_w, const void* W13, const void* W2, const void* wq,
                   const void* saved, void* dx, float* d_topk_w, void* dW13, void* dW2, void* ws,
                   size_t ws_bytes, void* stream);

/* Copies the routing status word that moe_fwd left in `fwd_ws` (or that
 * moe_permute left in its scratch) to *out (MOE_OK or MOE_ERR_ROUTING).
 * Synchronises `stream`. */
moe_status moe_read_status(const void* fwd_ws, int32_t* out, void* stream);

/* Human-readable name of a status value (static storage). */
const char* moe_status_string(moe_status st);

/* Optional per-kernel timing. While enabled, every kernel that moe_fwd /
 * moe_bwd / moe_permute launches is bracketed by HIP events recorded on the
 * call's stream. moe_kernel_timing_collect waits for those events, adds up
 * the elapsed times per kernel name, writes at most `max` entries and clears
 * the record. Not for use under graph capture. */
typedef struct moe_kernel_time {
  char name[48];
  int32_t launches;
  double total_ms;
} moe_kernel_time;
moe_status moe_set_kernel_timing(int enable);
moe_status moe_kernel_timing_collect(moe_kernel_time* out, int32_t max, int32_t* n_out);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
