/*
 * moe.h -- C ABI of the MI355X (gfx950) dropless top-k MoE expert layer.
 *
 * One layer, forward and backward, on one GPU: a softmax top-k router, a
 * row-wise dispatch of every (token, slot) straight into its expert's rows,
 * routing metadata that never leaves the GPU, SwiGLU experts run as grouped
 * GEMMs (bf16 or MXFP8 on MFMA, fp32 on the vector units) and a weighted
 * combine.  Sources, by page and section:
 *   - "OLMoE in HF Transformers" walkthrough, section 2 (router) and section 3
 *     (expert layer: 3-D expert weights; per expert gate/up, SiLU(gate)*up,
 *     down, times the top-k weight, index_add back to the token);
 *   - olmoforge README, module table (row-wise expert parallel: token rows
 *     written straight into the expert input buffer; grouped GEMM: the small
 *     per-expert matmuls merged into one kernel; GPU-resident routing table:
 *     metadata stays on the device and the CPU never waits for a copy) and
 *     its MXFP8 snippet (block of 32 with one shared scale, e4m3 max 448);
 *   - OLMo-core 3 release summary (wedoingai), features and technical
 *     principle sections: paired SwiGLU backward, bf16-rounded weight
 *     gradients.
 *
 * Conventions shared by every entry point
 *   - Shapes: T tokens (rows of x), d model width, E experts, f expert
 *     width, k experts per token, R = T*k routed rows.
 *   - All buffers are device memory owned by the caller, dense and row-major,
 *     16-byte aligned.  The library allocates nothing and keeps no state
 *     between calls; a call may use the caller's workspace `ws` (size from
 *     moe_workspace_size) and must not overlap another call using the same
 *     workspace.
 *   - Every call only enqueues kernels on `stream` (a hipStream_t; NULL is
 *     the default stream) and returns; nothing is copied back to the host and
 *     nothing synchronises.  Routing metadata (counts, offsets, rows) is read
 *     on the device by the kernels that need it.
 *   - dtype: MOE_F32 or MOE_BF16, the storage type of x, the weights and every
 *     activation and gradient tensor.  Logits, top-k weights, dw and dlogits
 *     are always float32; indices and metadata are int32.
 *   - prec: MOE_PREC_F32 (dtype must be MOE_F32), MOE_PREC_BF16 (dtype
 *     MOE_BF16) or MOE_PREC_MXFP8 (dtype MOE_BF16; expert forward and dgrad
 *     GEMMs in e4m3 with one power-of-two E8M0 scale per 32 elements along
 *     the contraction axis, weight gradients in bf16).
 *   - Size limits of the grouped GEMMs (their operands are addressed with
 *     32-bit byte offsets from a per-tile or per-expert base; a larger call
 *     returns MOE_ERR_UNSUPPORTED, it never wraps):
 *       one expert's weights:         d * (f + 128) * 2 < 2^32 bytes;
 *       weight gradients (bf16):      R * max(d, 2f) * 2 < 2^32 bytes;
 *       weight gradients (MOE_WGRAD_MX), Kp = sum over experts of n_e rounded
 *       up to 128 (bounded by (R + 127 E + 127) rounded down to 128):
 *                                     256 * Kp < 2^32 and
 *                                     (Kp / 32) * max(d, 2f) < 2^30;
 *       MXFP8 activation scales:      ceil(max(d, 2f) / 128) * 4 * Rp < 2^30
 *                                     (Rp = R rounded up to 16).
 *   - Errors are detected on the host before anything is enqueued and come
 *     back as a negative status; nothing is launched then.  There is no
 *     silent fallback to another precision or algorithm.  Values the host
 *     cannot see are not checked: logits must be finite, and the experts of
 *     one token distinct (duplicates are taken as separate slots).  A
 *     pre-routed topk_idx entry outside [0, E) makes its slot empty: it gets
 *     no row (dest_row -1, not counted), adds nothing to y or dx, and its
 *     dtopk_w is 0 (the rows after offsets[E] are then left unwritten).
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum moe_status {
  MOE_OK = 0,
  MOE_ERR_NULL = -1,        /* a required pointer is NULL */
  MOE_ERR_SHAPE = -2,       /* a size is non-positive, or T*k / sizes overflow int32 */
  MOE_ERR_DTYPE = -3,       /* unknown dtype/prec, or a dtype/prec pair that does not exist */
  MOE_ERR_ALIGN = -4,       /* a pointer is not 16-byte aligned */
  MOE_ERR_WORKSPACE = -5,   /* ws_bytes below moe_workspace_size */
  MOE_ERR_UNSUPPORTED = -6, /* E > 256, k > E, d or f not a multiple of 64, or an operand
                               beyond the GEMM engines' 32-bit offsets (see below) */
  MOE_ERR_LAUNCH = -7,      /* the HIP runtime rejected a launch */
  MOE_ERR_SCRATCH = -8      /* larger than a no-allocation entry point's static scratch */
};

enum moe_dtype { MOE_F32 = 0, MOE_BF16 = 1 };
enum moe_prec { MOE_PREC_F32 = 0, MOE_PREC_BF16 = 1, MOE_PREC_MXFP8 = 2 };

/* moe_route flags */
#define MOE_ROUTE_LOGITS_IN 0x1u   /* logits are an input: x and Wr are not read */
/* moe_route / moe_route_bwd flag: renormalise the top-k weights to sum to 1 */
#define MOE_ROUTE_RENORM 0x4u
/* moe_grouped_ffn_bwd / moe_dispatch_bwd / moe_route_bwd flags */
#define MOE_ACCUMULATE 0x2u        /* add into the output (dW*, dx, dWr) instead of overwriting */
/* moe_grouped_ffn_bwd flag (bf16 layer): dWg, dWu, dWd are float32 buffers */
#define MOE_WGRAD_F32 0x8u
/* moe_grouped_ffn_bwd flag (MXFP8): the weight-gradient GEMMs in MXFP8 too */
#define MOE_WGRAD_MX 0x10u
/* moe_grouped_ffn_fwd / moe_grouped_ffn_bwd flag (MXFP8): the forward quantises
   each weight matrix once for both directions and keeps the backward's codes
   in its workspace, which the backward then reads (see both entry points) */
#define MOE_MX_KEEP_WEIGHTS 0x20u

/* Operation ids for moe_workspace_size. */
enum moe_op {
  MOE_OP_ROUTE = 0, MOE_OP_DISPATCH = 1, MOE_OP_FFN_FWD = 2, MOE_OP_COMBINE = 3,
  MOE_OP_COMBINE_BWD = 4, MOE_OP_FFN_BWD = 5, MOE_OP_DISPATCH_BWD = 6, MOE_OP_ROUTE_BWD = 7,
  MOE_OP_ROUTE_AUX = 8,
  MOE_OP_FFN_BWD_MXW = 9,  /* moe_grouped_ffn_bwd with MOE_WGRAD_MX (its own part) */
  MOE_OP_FFN_FWD_KEEP = 10 /* moe_grouped_ffn_fwd with MOE_MX_KEEP_WEIGHTS */
};

/*
 * moe_route -- router logits, softmax and top-k.
 * HF OLMoE walkthrough, section 2: logits = x . Wr (router weight without
 * bias; the page stores it as (E, d), here it is its transpose Wr[d,E]),
 * softmax over the experts in float32, the top_k experts per token, the
 * softmax probabilities of the chosen experts as weights: as they are (the
 * page's default), or with MOE_ROUTE_RENORM divided by their sum (the page's
 * optional top-k renormalisation).
 *   x[T,d] (dtype), Wr[d,E] (dtype) -> logits[T,E] f32 (written unless
 *   MOE_ROUTE_LOGITS_IN, then read), topk_idx[T,k] i32, topk_w[T,k] f32.
 *   Slots are ordered by (logit desc, expert index asc): ties go to the
 *   lower index; selection is made on the float32 logits.
 *   Limits: 1 <= E <= 256, 1 <= k <= E.  d % 64 == 0 (unless logits are an
 *   input).
 *   Workspace: optional.  With moe_workspace_size(MOE_OP_ROUTE, ...) bytes
 *   (non-zero for bf16 batches of at most 64 tokens with E % 8 == 0) the
 *   small-batch router runs (partial logits over slices of Wr's rows, added
 *   in slice order); without it the general one (a logits kernel over all
 *   of Wr, then the top-k kernel) does.
 */
int moe_route(const void* x, const void* Wr, int T, int d, int E, int k, int dtype,
              unsigned flags, float* logits, int32_t* topk_idx, float* topk_w,
              void* ws, size_t ws_bytes, void* stream);

/*
 * moe_dispatch -- routing metadata and row-wise dispatch.
 * olmoforge README (row-wise expert parallel, GPU-resident routing table):
 * every (token t, slot j) gets one row of its expert's segment and x[t] is
 * copied straight there; there is no separate sort of the activations.
 *   counts[E]     rows per expert
 *   offsets[E+1]  exclusive scan of counts; offsets[E] = R
 *   dest_row[T,k] row of (t, j): offsets[e] + number of tokens t' < t routed
 *                 to e (rows of one expert are in ascending token order)
 *   src_token[R]  inverse map: the token of every row
 *   Xs[R,d]       Xs[dest_row[t,j]] = x[t] (dtype).
 *   Xq, Xq_scale  prec MXFP8 only (ignored, may be NULL, otherwise): the
 *                 rows of Xs block-quantised along d.  Xq[R,d] holds e4m3
 *                 codes (1 byte each); Xq_scale holds the E8M0 bytes (2^E
 *                 stored as E + 127) in groups of four blocks: the scale
 *                 of block b (elements 32b..32b+31) of row r is
 *                 Xq_scale[((b/4)*Rp + r)*4 + b%4], Rp = R rounded up to a
 *                 multiple of 16, ceil(d/128)*4*Rp bytes (the words of a
 *                 partial last group hold unwritten bytes).
 *   Workspace: moe_workspace_size(MOE_OP_DISPATCH, ...).
 */
int moe_dispatch(const void* x, const int32_t* topk_idx, int T, int d, int E, int k,
                 int dtype, int prec, int32_t* counts, int32_t* offsets,
                 int32_t* dest_row, int32_t* src_token, void* Xs, void* Xq, uint8_t* Xq_scale,
                 void* ws, size_t ws_bytes, void* stream);

/*
 * moe_dispatch_noalloc -- moe_dispatch without a caller workspace, for
 * callers that cannot allocate device memory at all: code being captured
 * into a HIP graph, tight serving loops, and harnesses that forbid
 * allocation.  Same arguments, results and errors as moe_dispatch, minus
 * ws / ws_bytes: the per-block expert histograms and their scanned bases
 * (2 * ceil(T/64) * E int32, each table padded to 256 bytes) live in a static
 * device array of 4 MiB that the library holds on every GPU it runs on until
 * the process ends; its address is looked up once per device on the first
 * call made with that device current.  The call itself allocates nothing
 * and, like every entry point, only enqueues kernels on `stream`.
 *   MOE_ERR_SCRATCH: the tables would exceed 4 MiB (about T * E > 2^25, e.g.
 *   T = 524288 tokens at E = 64); use moe_dispatch with a workspace then.
 *   Calls on one GPU share that GPU's scratch (each call overwrites it fully
 *   before reading it, so nothing carries over): two calls that can run at
 *   the same time on one GPU (different streams, no ordering between them)
 *   race on it and must not be issued.
 */
int moe_dispatch_noalloc(const void* x, const int32_t* topk_idx, int T, int d, int E, int k,
                         int dtype, int prec, int32_t* counts, int32_t* offsets,
                         int32_t* dest_row, int32_t* src_token, void* Xs, void* Xq,
                         uint8_t* Xq_scale, void* stream);

/*
 * moe_grouped_ffn_fwd -- all SwiGLU experts as grouped GEMMs.
 * HF OLMoE walkthrough, section 3; olmoforge README (grouped GEMM).  For each
 * expert e and its rows r in [offsets[e], offsets[e+1]):
 *   Hg = Xs.Wg[e], Hu = Xs.Wu[e], A = silu(Hg) * Hu, Ys = A.Wd[e]
 *   Wg, Wu [E,d,f], Wd [E,f,d] (dtype); Hg, Hu, A [R,f], Ys [R,d] (dtype),
 *   stored from float32 accumulators (A from the unrounded Hg, Hu).
 *   offsets is read on the device.  Xs_scale is ignored except for prec
 *   MXFP8, where Xs and Xs_scale are the Xq codes and Xq_scale scales that
 *   moe_dispatch wrote; the weights are block-quantised inside (Wg, Wu along
 *   d, Wd along f) and A along f before the down GEMM.  Workspace:
 *   moe_workspace_size(MOE_OP_FFN_FWD, ...) (0 bytes except for MXFP8).
 *   flags: MOE_MX_KEEP_WEIGHTS (prec MXFP8 only, else MOE_ERR_DTYPE): each
 *   weight matrix is read once and quantised for both directions of the
 *   layer (Wg, Wu along d and along f; Wd along f and along d), and the
 *   backward's codes stay in ws, which must then hold
 *   moe_workspace_size(MOE_OP_FFN_FWD_KEEP, ...) bytes; pass that workspace,
 *   unchanged, to moe_grouped_ffn_bwd with the same flag.  The results are
 *   the same as without the flag (the codes are the same bytes).  0: no flag.
 */
int moe_grouped_ffn_fwd(const void* Xs, const uint8_t* Xs_scale, const int32_t* offsets,
                        int T, int k, int d, int f, int E, const void* Wg, const void* Wu,
                        const void* Wd, int dtype, int prec, unsigned flags, void* Hg, void* Hu,
                        void* A, void* Ys, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_combine -- weighted un-dispatch.
 * HF OLMoE walkthrough, section 3 (multiply by the top-k weight and
 * index_add back to the token): y[t] = sum_j topk_w[t,j] * Ys[dest_row[t,j]],
 * summed in float32 in slot order, stored in dtype.  y[T,d].
 */
int moe_combine(const void* Ys, const float* topk_w, const int32_t* dest_row, int T, int d,
                int k, int dtype, void* y, void* stream);

/*
 * moe_combine_bwd -- backward of moe_combine for upstream gradient dY[T,d].
 * Differentiates the weighted index_add of the HF OLMoE walkthrough,
 * section 3 (each expert output times its top-k weight, added back to the
 * token): for L = sum_t <y[t], dY[t]>,
 *   dYs[dest_row[t,j]] = topk_w[t,j] * dY[t]       (dtype, [R,d])
 *   dtopk_w[t,j]       = <dY[t], Ys[dest_row[t,j]]> (f32, [T,k])
 *   dYs_q, dYs_q_scale (optional; both NULL or both set, bf16 only): the rows
 *   of dYs as stored, block-quantised along d for an MXFP8 backward, laid out
 *   like moe_dispatch's Xq / Xq_scale (codes [R,d]; scale of block b of row r
 *   at dYs_q_scale[((b/4)*Rp + r)*4 + b%4], Rp = R rounded up to 16,
 *   ceil(d/128)*4*Rp bytes).
 */
int moe_combine_bwd(const void* dY, const void* Ys, const float* topk_w,
                    const int32_t* dest_row, int T, int d, int k, int dtype, void* dYs,
                    float* dtopk_w, void* dYs_q, uint8_t* dYs_q_scale, void* stream);

/*
 * moe_grouped_ffn_bwd -- backward of moe_grouped_ffn_fwd.
 * OLMo-core 3 release summary: paired SwiGLU backward (gate and up gradients
 * in one pass), bf16-rounded weight gradients.  Per expert e:
 *   dA  = dYs.Wd[e]^T
 *   dHg = dA * Hu * silu'(Hg), dHu = dA * silu(Hg)  -> dH[R,2f]: columns
 *         [0,f) hold dHg, [f,2f) hold dHu (dtype)
 *   dXs = dHg.Wg[e]^T + dHu.Wu[e]^T                  -> dXs[R,d] (dtype)
 *   dWd[e] = A^T.dYs, dWg[e] = Xs^T.dHg, dWu[e] = Xs^T.dHu, summed in float32
 *   over the expert's rows and stored in dtype (an expert with no rows gets
 *   zeros; with MOE_ACCUMULATE the sum is added to the existing values).
 *   MOE_WGRAD_F32 (same summary: optional FP32 gradient accumulation): the
 *   three weight gradients are float32 buffers, written, or with
 *   MOE_ACCUMULATE added to, without rounding to bf16 (a float32 layer's
 *   gradients are float32 anyway; the flag changes nothing there).
 *   MOE_WGRAD_MX (prec MXFP8 only, else MOE_ERR_DTYPE; olmoforge README,
 *   MXFP8 block quantisation, applied to the weight gradients as well): the
 *   weight-gradient GEMMs run in MXFP8 too, each operand (Xs, dH, A, dYs)
 *   block-quantised along the tokens of each expert in blocks of 32 from
 *   the expert's first row (a last partial block padded with zeros); with
 *   MOE_WGRAD_F32 the gradients are float32.  Workspace:
 *   moe_workspace_size(MOE_OP_FFN_BWD_MXW, ...).
 *   Xs: the dispatched rows in dtype (also for MXFP8).  prec MXFP8: both
 *   operands of the two dgrad GEMMs are block-quantised along their
 *   contraction axis (dYs and Wd along d; dH, Wg, Wu along f); dYs_q /
 *   dYs_q_scale are dYs quantised along d as moe_combine_bwd writes them
 *   (ignored, may be NULL, in other precisions); dH is quantised as the down
 *   dgrad's epilogue writes it; the weight gradients take the unquantised
 *   operands.  Workspace: moe_workspace_size(MOE_OP_FFN_BWD, ...) (0 bytes
 *   except for MXFP8).
 *   MOE_MX_KEEP_WEIGHTS (prec MXFP8 only, else MOE_ERR_DTYPE): ws begins with
 *   the workspace that moe_grouped_ffn_fwd filled with the same flag,
 *   unchanged since (moe_workspace_size(MOE_OP_FFN_FWD_KEEP, ...) bytes),
 *   followed by the backward's own workspace (MOE_OP_FFN_BWD, or
 *   MOE_OP_FFN_BWD_MXW with MOE_WGRAD_MX); ws_bytes covers both.  The
 *   dgrad GEMMs read the weight codes the forward kept instead of quantising
 *   Wg, Wu and Wd again; the results are the same bytes.
 */
int moe_grouped_ffn_bwd(const void* dYs, const void* dYs_q, const uint8_t* dYs_q_scale,
                        const void* Xs, const void* Hg, const void* Hu,
                        const void* A, const int32_t* offsets, int T, int k, int d, int f,
                        int E, const void* Wg, const void* Wu, const void* Wd, int dtype,
                        int prec, unsigned flags, void* dH, void* dXs, void* dWg, void* dWu,
                        void* dWd, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_dispatch_bwd -- backward of moe_dispatch's row copy.  The forward
 * writes each token row straight into the expert rows of its k slots
 * (olmoforge README, module table, row-wise expert parallel; HF OLMoE
 * walkthrough, section 3: hidden_states[token_idx] per expert), so the
 * gradient of x gathers those rows back:
 *   dx[t] = sum_j dXs[dest_row[t,j]]  (float32 sum in slot order, stored in
 *   dtype; with MOE_ACCUMULATE added to dx).  dXs [R,d], dx [T,d] (dtype).
 */
int moe_dispatch_bwd(const void* dXs, const int32_t* dest_row, int T, int d, int k,
                     int dtype, unsigned flags, void* dx, void* stream);

/*
 * moe_route_bwd -- router backward for the weight gradient dtopk_w.
 * Differentiates moe_route (HF OLMoE walkthrough, section 2: logits = x.Wr
 * with no bias, float32 softmax over the experts, the chosen probabilities
 * as weights, optionally renormalised); the top-k choice itself is piecewise
 * constant and has no gradient:
 *   dp[t,e] = dtopk_w[t,j] where e = topk_idx[t,j], else 0; with
 *             MOE_ROUTE_RENORM (weights p/S, S = sum of the chosen p):
 *             dp[t,e_m] = (dtopk_w[t,m] - sum_j dtopk_w[t,j] w[t,j]) / S;
 *             plus aux_dp[e] (optional, [E] f32, from moe_route_aux) for
 *             every token
 *   dlogits = p * (dp - <p, dp>), p = softmax(logits)    (f32 [T,E])
 *   dWr     = x^T . dlogits                               (dtype [d,E])
 *   dx     += dlogits . Wr^T                              (dtype [T,d], always added)
 *   With bf16 the two GEMMs read dlogits rounded to bf16 (held in ws), and
 *   dWr is summed over chunks of tokens into float32 partials (also in ws)
 *   that are added in chunk order: the result does not depend on timing.
 *   Workspace: moe_workspace_size(MOE_OP_ROUTE_BWD, ...).
 */
int moe_route_bwd(const void* x, const void* Wr, const float* logits,
                  const int32_t* topk_idx, const float* dtopk_w, const float* aux_dp, int T,
                  int d, int E, int k, int dtype, unsigned flags, float* dlogits, void* dWr,
                  void* dx, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_route_aux -- load-balancing loss of the router and its gradient.
 * HF OLMoE walkthrough, section 4: load_balancing_loss_func in
 * modeling_olmoe.py (Switch-Transformer-style: expert assignment frequencies
 * times router probabilities, summed, times the expert count), scaled by
 * router_aux_loss_coef (default 0.01) as the causal-LM head does.  With
 * f_e = counts[e] / T (the per-slot assignment frequencies summed over the k
 * slots; counts as written by moe_dispatch) and
 * P_e = (1/T) sum_t softmax(logits[t])[e]:
 *   aux_loss[0] = coef * E * sum_e f_e * P_e             (f32, device; coef*k
 *                 when every expert receives T*k/E slots)
 *   aux_dp[e]   = coef * E * f_e / T                      (f32 [E], the
 *                 gradient with respect to every token's probability of e;
 *                 pass it to moe_route_bwd)
 *   k is checked (1 <= k <= E) and does not enter the formulas.
 *   Sums are in a fixed order (per 64-token block, then over blocks).
 *   Workspace: moe_workspace_size(MOE_OP_ROUTE_AUX, ...).
 */
int moe_route_aux(const float* logits, const int32_t* counts, int T, int E, int k, float coef,
                  float* aux_loss, float* aux_dp, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_check_routing -- device-side check of pre-routed expert indices (the
 * preconditions the host cannot see without a copy; an optional debugging
 * step before moe_dispatch, in the spirit of the pages' convention of
 * failing early rather than silently changing behaviour: OLMo-core 3 release
 * summary, technical principle section).  Enqueues two small kernels that
 * write, once they have run,
 *   report[0] = number of entries of topk_idx[T,k] outside [0, E)
 *   report[1] = number of tokens whose in-range experts are not all distinct
 * (report: 2 int32 in device memory, 16-byte aligned, owned by the caller;
 * read it after the stream reaches this point).  Nothing else is written and
 * nothing synchronises.  E <= 256, else MOE_ERR_UNSUPPORTED.
 */
int moe_check_routing(const int32_t* topk_idx, int T, int E, int k, int32_t* report,
                      void* stream);

/* Workspace bytes an operation needs for these sizes (0 is a valid answer). */
int moe_workspace_size(int op, int T, int d, int E, int f, int k, int dtype, int prec,
                       size_t* bytes);

/* Text of a status code (static storage). */
const char* moe_status_string(int status);

/* Name of the HIP error behind the last MOE_ERR_LAUNCH on this thread, or
   "none" (static storage). */
const char* moe_last_launch_error(void);

/*
 * moe_set_kernel_events -- per-kernel timing hook (observability only).
 * While set (and no filter is set, see moe_set_kernel_filter), every kernel
 * launched by an entry point on the calling thread
 * is followed by hipEventRecord(events[i], stream), i = 0, 1, ... up to
 * `capacity`, and names[i] (when names is not NULL) receives a static label
 * of that kernel; *count (when not NULL) tracks how many were recorded.
 * The events are caller-created hipEvent_t handles.  If a record fails the
 * hook switches itself off and *count becomes -(HIP error code); the kernel
 * launches are not affected.  Pass events = NULL to switch the hook off.
 * This thread-local hook, with its filter, is the only state the library
 * keeps between calls; it is off by default.
 */
int moe_set_kernel_events(void* const* events, const char** names, int capacity, int* count);

/*
 * moe_set_kernel_filter -- narrows the timing hook to one kernel (observability
 * only).  With `name` set (a label as moe_set_kernel_events reports it, at most
 * 63 characters, copied), the hook records, for each launch of that kernel on
 * the calling thread, one event right before it and one right after it
 * (events[2i] and events[2i+1], both labelled), and nothing for other kernels,
 * so that the rest of the work runs without events between its kernels.
 * NULL (the default) times every kernel again.  Returns MOE_ERR_SHAPE for a
 * longer name (the filter is then unchanged).  The filter is thread-local and
 * outlives moe_set_kernel_events calls.
 */
int moe_set_kernel_filter(const char* name);

/*
 * moe_probe_clock -- clock probe (observability only).  Launches `grid`
 * workgroups of 256 threads on `stream`; each runs `iters` rounds of 8
 * independent v_mfma_f32_32x32x16_bf16 per wave on register data (no memory
 * traffic), the load the expert GEMMs put on the matrix cores, and its first
 * thread writes the shader clock counter (s_memtime) and the constant-rate
 * counter (s_memrealtime) before and after that work to
 * ticks[4b .. 4b+3] = {memtime start, memtime end, realtime start, realtime
 * end} (device memory, 16-byte aligned, 4*grid entries, owned by the
 * caller).  With the launch timed by events, (memtime end - start) / time
 * gives the clock under MFMA load, and 8 * 32768 * 4 * iters * grid FLOP /
 * time the sustained dense bf16 MFMA rate.
 */
int moe_probe_clock(unsigned long long* ticks, int grid, int iters, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
