/*
 * moe.h -- C ABI of the single-GPU Mixture-of-Experts FFN layer for MI355X (gfx950).
 *
 * The layer, for each token x_t (a row of `hidden`):
 *   logits  l = W_r x_t (+ optional per-expert logit offset)
 *   scores  s = softmax / sigmoid / sqrt(softplus) of l; selection key s + bias
 *   top-k   ids[t, 0..k-1] in descending key order, gates renormalised over
 *           the selected unbiased scores
 *   y_t     = sum_j g[t,j] * FFN_{ids[t,j]}(x_t) + FFN_shared(x_t)
 *   FFN_e(x) = W2_e (SiLU(W1_e x) (.) W3_e x)
 * Sources (web pages by title and section):
 *   "MoE 的算量与通信" (arganzheng) chapter 二.1-二.3: SwiGLU FFN, router W_r [E, d],
 *       top-k, renormalisation, weighted sum plus shared experts; 七.3: the
 *       selection bias; 五.3: group-limited choice.
 *   "MoE 架构与路由策略" (DeepSeek-V4 notes): equation dsv4-moe-softplus (sigmoid
 *       and sqrt(softplus)), the V3 node-limited routing section, hash routing.
 *   "DeepSeek-V4 MoE: Token 从路由到专家计算" (akiyangdev) sections 二 and 四:
 *       MoEGate weight [n_routed_experts, hidden_size], topk_ids / topk_weights,
 *       HashTopK's tid2eid, w13_weight (gate and up fused) and w2_weight,
 *       the dispatch -> expert core -> combine hand-off.
 *   "Mixture of Experts: Router, Token Dispatch, Grouped GEMM" (111qqz):
 *       router worked example, permuted_token_ids / tokens_per_expert, grouped
 *       GEMM over ragged row counts, index_add_ combine.
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers on the current HIP device, row-major
 *    and contiguous, 16-byte aligned.  Outputs must not alias inputs.  The caller
 *    owns all memory, including the workspace; the library never allocates
 *    device memory, frees or synchronises.  Work is queued on `stream` (a
 *    hipStream_t; NULL is the default stream) and completes asynchronously.
 *    Calls with distinct workspaces may run concurrently.
 *  - The library keeps no state between calls (no streams, events or handles
 *    of its own), except moe_forward_noalloc's static scratch (below).  Every
 *    launch of a call goes to `stream`, in order.
 *  - Floating-point tensors (hidden, weights, expert outputs, out) are float32
 *    when cfg->dtype == MOE_F32 and bfloat16 when MOE_BF16.  Logits, gates, bias
 *    and logit offsets are always float32; accumulation is always float32.
 *  - w13 is [E, 2*d_ff, d]: rows [0, d_ff) are W1 (gate, the SiLU input) and rows
 *    [d_ff, 2*d_ff) are W3 (up).  w2 is [E, d, d_ff].  Shared-expert weights are
 *    one expert's worth: w13_shared [2*d_ff, d], w2_shared [d, d_ff].
 *  - Errors: every argument check runs on the host before any launch, so an
 *    error return means no work was queued.  A failed launch returns
 *    MOE_ERR_HIP; faults inside kernels surface at the caller's next
 *    synchronisation of the stream.  T == 0 is valid and queues nothing.
 *  - Device-side range errors (an expert id outside [0, E) in moe_permute's
 *    input, a token id outside [0, vocab)) are not trapped: such a pair gets no
 *    dispatch row, its dispatch_index entry is -1, and expert_offsets[E] counts
 *    only the valid pairs.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = -1, /* null required pointer, inconsistent sizes */
    MOE_ERR_UNSUPPORTED = -2, /* valid but outside what the kernels handle */
    MOE_ERR_WORKSPACE = -3,   /* workspace too small (see moe_workspace_size) */
    MOE_ERR_HIP = -4,         /* a HIP launch or runtime call failed */
    MOE_ERR_TOO_LARGE = -5    /* moe_forward_noalloc: workspace beyond its static scratch */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;
typedef enum { MOE_SCORE_SOFTMAX = 0, MOE_SCORE_SIGMOID = 1, MOE_SCORE_SQRTSOFTPLUS = 2 } moe_scoring;
typedef enum { MOE_ROUTE_LEARNED = 0, MOE_ROUTE_HASH = 1 } moe_route_mode;

/* Layer shape and routing rule.
 *   T tokens, hidden size d, E routed experts, k selected per token, expert
 *   width d_ff, n_shared in {0, 1} unrouted experts.
 *   Group-limited routing (DeepSeek-V3): n_group > 1 splits the experts into
 *   n_group contiguous groups of E/n_group; each group scores the sum of its
 *   group_topk largest keys; the topk_group best groups stay eligible; then top-k
 *   among them.  n_group = 1 disables it (topk_group, group_topk ignored).
 *   Hash routing (route_mode MOE_ROUTE_HASH): ids are tid2eid[token_ids[t]]
 *   (a [vocab, k] table); gates are the token's affinities at those ids,
 *   renormalised; the bias is unused.
 *   logits_given (moe_route only): 1 = `logits` is an input and the router GEMM
 *   is skipped.
 * Limits: 1 <= k <= min(E, 16); E <= 1024; d, d_ff multiples of 64;
 *   n_group <= 64 with E % n_group == 0, 1 <= topk_group <= n_group,
 *   1 <= group_topk <= E/n_group and k <= topk_group*E/n_group;
 *   T*(k+n_shared)*max(d, d_ff) < 2^31. */
typedef struct moe_config {
    int32_t T, d, E, k, d_ff, n_shared;
    int32_t dtype;      /* moe_dtype */
    int32_t scoring;    /* moe_scoring */
    int32_t route_mode; /* moe_route_mode */
    int32_t n_group, topk_group, group_topk;
    int32_t vocab;        /* hash mode: rows of tid2eid */
    int32_t logits_given; /* moe_route: read logits instead of computing them */
} moe_config;

/* Bytes of workspace moe_forward needs for this configuration (moe_permute and
 * moe_expert_ffn need no more).  Returns MOE_OK or an argument error. */
int moe_workspace_size(const moe_config *cfg, size_t *bytes);

/* Router: logits, affinity scores, (group-limited) top-k and gates.
 *   hidden [T, d], w_router [E, d]  (unused when cfg->logits_given)
 *   logit_offset [E] float32, nullable: added to every token's logits
 *   bias [E] float32, nullable: added to the scores for selection only
 *   token_ids [T] int32, tid2eid [vocab, k] int32: hash mode only
 *   logits [T, E] float32: output (input when cfg->logits_given)
 *   topk_ids [T, k] int32, topk_weights [T, k] float32: outputs, slot j holds
 *   the j-th largest key (equal keys: lower expert id first); in hash mode, the
 *   table's order.  Needs no workspace. */
int moe_route(const moe_config *cfg, const void *hidden, const void *w_router,
              const float *logit_offset, const float *bias, const int32_t *token_ids,
              const int32_t *tid2eid, float *logits, int32_t *topk_ids,
              float *topk_weights, void *stream);

/* Token dispatch: the T*k (token, slot) pairs sorted expert-major, tokens in
 * ascending order inside each expert (a stable sort by expert id).
 *   topk_ids [T, k] int32 (any slot order), topk_weights [T, k] float32
 *   expert_counts [E], expert_offsets [E+1] (exclusive prefix sum; [E] = T*k)
 *   sorted_token_ids [T*k]: token of each dispatch row
 *   sorted_weights [T*k]: gate of each dispatch row
 *   dispatch_index [T, k]: dispatch row of pair (t, j)
 *   workspace: at least moe_workspace_size bytes. */
int moe_permute(const moe_config *cfg, const int32_t *topk_ids, const float *topk_weights,
                int32_t *expert_counts, int32_t *expert_offsets, int32_t *sorted_token_ids,
                float *sorted_weights, int32_t *dispatch_index, void *workspace,
                size_t workspace_bytes, void *stream);

/* Grouped SwiGLU experts over ragged row counts: for every expert e and every
 * dispatch row r in [expert_offsets[e], expert_offsets[e+1]),
 *   expert_out[r] = FFN_e(hidden[sorted_token_ids[r]])   (unweighted)
 * in cfg->dtype.  hidden [T, d]; sorted_token_ids [R]; expert_offsets [E+1]
 * (device; R = expert_offsets[E] <= T*k); w13 [E, 2*d_ff, d]; w2 [E, d, d_ff];
 * expert_out [T*k, d].  The intermediate SiLU(W1 x) (.) W3 x is rounded to
 * cfg->dtype.  For the shared expert, call with E = 1, k = 1, identity rows
 * (sorted_token_ids[t] = t) and offsets {0, T}. */
int moe_expert_ffn(const moe_config *cfg, const void *hidden, const int32_t *sorted_token_ids,
                   const int32_t *expert_offsets, const void *w13, const void *w2,
                   void *expert_out, void *workspace, size_t workspace_bytes, void *stream);

/* The two stages of moe_expert_ffn, callable on their own (the pages' Linear-1
 * with its activation, and Linear-2):
 *   moe_expert_up:   h_out[r] = SiLU(W1_e x) (.) W3_e x,  x = hidden[sorted_token_ids[r]]
 *                    h_out [T*k, d_ff] in cfg->dtype (rounded once from float32)
 *   moe_expert_down: expert_out[r] = W2_e h[r]; h [T*k, d_ff], expert_out [T*k, d]
 * for every expert e and dispatch row r in [expert_offsets[e], expert_offsets[e+1]).
 * Other arguments as for moe_expert_ffn; rows past expert_offsets[E] are untouched. */
int moe_expert_up(const moe_config *cfg, const void *hidden, const int32_t *sorted_token_ids,
                  const int32_t *expert_offsets, const void *w13, void *h_out, void *workspace,
                  size_t workspace_bytes, void *stream);
int moe_expert_down(const moe_config *cfg, const void *h, const int32_t *expert_offsets,
                    const void *w2, void *expert_out, void *workspace, size_t workspace_bytes,
                    void *stream);

/* Weighted combine back into token rows, in a fixed order (deterministic):
 *   out[t] = sum_{j<k} topk_weights[t,j] * expert_out[dispatch_index[t,j]]
 *            + shared_out[t]   (when shared_out is not NULL)
 * summed in float32 in slot order j = 0..k-1, then the shared row; rounded once
 * to cfg->dtype.  expert_out [T*k, d]; shared_out [T, d] nullable; out [T, d].
 * Pairs with dispatch_index -1 are skipped.  Needs no workspace. */
int moe_combine(const moe_config *cfg, const void *expert_out, const int32_t *dispatch_index,
                const float *topk_weights, const void *shared_out, void *out, void *stream);

/* The whole layer in one call: route, permute, grouped experts (routed and
 * shared in the same grouped launches), combine.  Arguments as above;
 * w13_shared / w2_shared are required when cfg->n_shared == 1.
 * topk_ids_out [T, k] and topk_weights_out [T, k] are optional copies of the
 * routing decision (nullable).  out [T, d]. */
int moe_forward(const moe_config *cfg, const void *hidden, const void *w_router,
                const float *logit_offset, const float *bias, const int32_t *token_ids,
                const int32_t *tid2eid, const void *w13, const void *w2,
                const void *w13_shared, const void *w2_shared, void *out,
                int32_t *topk_ids_out, float *topk_weights_out, void *workspace,
                size_t workspace_bytes, void *stream);

/* moe_forward without a caller workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation): the workspace is a static device array of
 * MOE_NOALLOC_SCRATCH_BYTES in the library (one copy per GPU, held until the
 * process ends; its address is looked up once per device on the first call
 * there).  Arguments and results as moe_forward.  A configuration whose
 * workspace (moe_workspace_size) exceeds the scratch returns MOE_ERR_TOO_LARGE
 * before any launch: 64 MiB holds decode-shaped batches, e.g. T up to ~770 at
 * d = 4096, d_ff = 2048, k = 6 with a shared expert.  Nothing in the scratch
 * needs clearing between calls (every region is written before it is read).
 * All calls on one GPU share its scratch: calls that overlap in time on one
 * GPU (two streams, two threads) race and must be serialised by the caller.
 * The call allocates and frees nothing. */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int moe_forward_noalloc(const moe_config *cfg, const void *hidden, const void *w_router,
                        const float *logit_offset, const float *bias, const int32_t *token_ids,
                        const int32_t *tid2eid, const void *w13, const void *w2,
                        const void *w13_shared, const void *w2_shared, void *out,
                        int32_t *topk_ids_out, float *topk_weights_out, void *stream);

/* ---------------------------------------------------------------------------
 * FP8 experts.  Codes are E4M3 (the OCP "FN" encoding: sign, 4 exponent bits with
 * bias 7, 3 mantissa bits, no infinities, largest finite 448; one byte each)
 * with float32 scales ("MoE 架构与路由策略", FP4 QAT section and table
 * dsv4-moe-fp4-vs-fp8: E4M3 with one scale per 128x128 weight tile; table
 * dsv4-moe-stages: the FP8 cast after the SwiGLU activation, between Linear-1
 * and Linear-2; "MoE 的算量与通信" 五.2: FP8 dispatch, BF16 combine).
 *   Weights: w13q [E, 2*d_ff, d] uint8 with w13s [E, 2*d_ff/128, d/128] float32,
 *            w2q [E, d, d_ff] with w2s [E, d/128, d_ff/128]: one scale per
 *            128x128 tile (row-major over tiles).  Shared expert: one expert's worth.
 *   Activations (hidden rows before Linear-1, h after the activation): one scale
 *            per row per 128 columns: codes [rows, K], scales stored
 *            K-block-major, [K/128, rows] (column group g of all rows
 *            together, so the matrix cores' loads read one group's scales of
 *            consecutive rows as contiguous words).
 *   A group's scale is a power of two, 2^e: the smallest with max |x| <= 448 * 2^e
 *   (e >= -126; an all-zero group has scale 1); its codes are E4M3(x * 2^-e),
 *   nearest-even, saturated to +-448.  Power-of-two tile scales keep FP4 (E2M1)
 *   weights with their finer scales exactly representable after the cast to
 *   FP8 (the FP4 QAT section's lossless dequantization), and they are the
 *   scales gfx950's block-scaled matrix cores apply.  A dot product sums each
 *   128-element K block, scales the block sum by the two block scales and
 *   accumulates in float32.
 * The FP8 entry points need cfg->dtype == MOE_BF16 (hidden, router weight,
 * expert_out and out are bfloat16; the router stays bfloat16) and d, d_ff
 * multiples of 128 (else MOE_ERR_UNSUPPORTED), and every operand smaller than
 * 2 GiB.  Workspace: moe_workspace_size covers them. */

/* Quantize the rows of x [n, K] (in_dtype MOE_F32 or MOE_BF16) in groups of 128
 * columns: q [n, K] uint8 codes, scales [K/128, n].  K a multiple of 128 (else
 * MOE_ERR_UNSUPPORTED).  Needs no workspace; n == 0 queues nothing. */
int moe_quantize_fp8_rows(int n, int K, int in_dtype, const void *x, uint8_t *q, float *scales,
                          void *stream);

/* Quantize a matrix w [R, C] (in_dtype) in 128x128 tiles: q [R, C] uint8,
 * scales [R/128, C/128] (row-major over tiles).  R and C multiples of 128.  For
 * stacked expert weights [E, R, C] pass E*R rows.  Needs no workspace. */
int moe_quantize_fp8_blocks(int R, int C, int in_dtype, const void *w, uint8_t *q,
                            float *scales, void *stream);

/* FP8 Linear-1 with the activation and the FP8 cast fused: for every expert e and
 * dispatch row r in [expert_offsets[e], expert_offsets[e+1]),
 *   h = SiLU(W1_e x) (.) W3_e x in float32, x = the codes xq[sorted_token_ids[r]]
 *   with their scales; hq[r], hs[r] = the 128-column-group quantization of h.
 * xq [T, d], xs [d/128, T]; hq [T*k, d_ff] uint8; hs [d_ff/128, T*k]. */
int moe_expert_up_fp8(const moe_config *cfg, const uint8_t *xq, const float *xs,
                      const int32_t *sorted_token_ids, const int32_t *expert_offsets,
                      const uint8_t *w13q, const float *w13s, uint8_t *hq, float *hs,
                      void *workspace, size_t workspace_bytes, void *stream);

/* FP8 Linear-2: expert_out[r] = W2_e h[r] for the same rows, bfloat16 rounded
 * once from float32.  hq [T*k, d_ff], hs [d_ff/128, T*k]; expert_out [T*k, d]. */
int moe_expert_down_fp8(const moe_config *cfg, const uint8_t *hq, const float *hs,
                        const int32_t *expert_offsets, const uint8_t *w2q, const float *w2s,
                        void *expert_out, void *workspace, size_t workspace_bytes,
                        void *stream);

/* The whole layer with FP8 experts: route (bfloat16 router, as moe_forward),
 * quantize the hidden rows, permute, FP8 grouped experts (routed and shared in
 * the same launches), combine (float32 sum, bfloat16 out).  The four shared
 * arguments are required when cfg->n_shared == 1. */
int moe_forward_fp8(const moe_config *cfg, const void *hidden, const void *w_router,
                    const float *logit_offset, const float *bias, const int32_t *token_ids,
                    const int32_t *tid2eid, const uint8_t *w13q, const float *w13s,
                    const uint8_t *w2q, const float *w2s, const uint8_t *w13q_shared,
                    const float *w13s_shared, const uint8_t *w2q_shared,
                    const float *w2s_shared, void *out, int32_t *topk_ids_out,
                    float *topk_weights_out, void *workspace, size_t workspace_bytes,
                    void *stream);

/* ---------------------------------------------------------------------------
 * MXFP4 expert weights ("MoE 架构与路由策略", FP4 QAT section and table
 * dsv4-moe-fp4-vs-fp8: E2M1 codes with one shared scale per 1x32 sub-block;
 * inference uses the FP4 weights directly; FP4 x FP8 products on hardware that
 * multiplies them natively, as gfx950's matrix cores do).  Activations (hidden
 * rows, h) are E4M3 with 1x128 power-of-two scales exactly as for the FP8
 * experts; only the weights change.
 *   Codes: E2M1 (sign, 2 exponent bits with bias 1, 1 mantissa bit; magnitudes
 *   0, 0.5, 1, 1.5, 2, 3, 4, 6; no infinities or NaN), two per byte, element 2j
 *   in the low nibble.  Scales: one E8M0 byte per 32 consecutive elements of a
 *   weight row (value 2^(byte - 127)), the smallest power of two with
 *   max |x| <= 6 * scale (>= 2^-126; 2^0 for an all-zero block); codes are
 *   E2M1(x / scale), nearest-even, saturated to +-6.
 *   Scale layout: for a weight matrix [R, C] the scales are stored
 *   K-block-major, [C/128, R, 4]: for each 128-column block j, each row r's four
 *   bytes (its blocks 4j .. 4j+3).  The matrix cores' loads then read one K
 *   block's scales of consecutive rows as contiguous words.
 *   Code layout: rows are paired.  For a weight matrix [R, C] (R even) the
 *   codes are stored [R/2, C/128, 2, 64]: for row pair i and 128-column block
 *   j, 64 bytes of row 2i then 64 bytes of row 2i+1, so the element (r, c)
 *   sits at byte (r/2)*C + (c/128)*128 + (r%2)*64 + (c%128)/2.  One K block of
 *   two rows fills one whole 128-byte line.  Total size R*C/2 bytes, the size
 *   of the row-major [R, C/2] array it replaces.
 *   Weights: w13q [E, d_ff, d] uint8 (2*d_ff rows in pairs) with w13s
 *            [E, d/128, 2*d_ff, 4] uint8, w2q [E, d/2, d_ff] (d rows in pairs)
 *            with w2s [E, d_ff/128, d, 4].  Shared expert: one
 *            expert's worth.
 * A dot product sums each 32-element block, scales the block sum by the
 * weight block's scale and the activation's 1x128 scale, and accumulates in
 * float32.  Requirements, workspace and errors as for the FP8 entry points. */

/* Quantize n_mat matrices w [n_mat, R, C] (in_dtype MOE_F32 or MOE_BF16) in 1x32
 * blocks: q [n_mat, R/2, C] packed codes in the paired-row code layout above,
 * scales [n_mat, C/128, R, 4] E8M0 bytes.  C a multiple of 128 and R even (else
 * MOE_ERR_UNSUPPORTED).  Needs no workspace; n_mat, R or C == 0 queues nothing. */
int moe_quantize_mxfp4(int n_mat, int R, int C, int in_dtype, const void *w, uint8_t *q,
                       uint8_t *scales, void *stream);

/* Linear-1 + SwiGLU + FP8 cast of h with MXFP4 weights; arguments as for
 * moe_expert_up_fp8 except w13q [E, d_ff, d] (paired rows) and w13s
 * [E, d/128, 2*d_ff, 4]. */
int moe_expert_up_mxfp4(const moe_config *cfg, const uint8_t *xq, const float *xs,
                        const int32_t *sorted_token_ids, const int32_t *expert_offsets,
                        const uint8_t *w13q, const uint8_t *w13s, uint8_t *hq, float *hs,
                        void *workspace, size_t workspace_bytes, void *stream);

/* Linear-2 with MXFP4 weights; arguments as for moe_expert_down_fp8 except w2q
 * [E, d/2, d_ff] (paired rows) and w2s [E, d_ff/128, d, 4]. */
int moe_expert_down_mxfp4(const moe_config *cfg, const uint8_t *hq, const float *hs,
                          const int32_t *expert_offsets, const uint8_t *w2q, const uint8_t *w2s,
                          void *expert_out, void *workspace, size_t workspace_bytes,
                          void *stream);

/* The whole layer with MXFP4 expert weights: the steps of moe_forward_fp8 with
 * the weights above (the shared expert's likewise). */
int moe_forward_mxfp4(const moe_config *cfg, const void *hidden, const void *w_router,
                      const float *logit_offset, const float *bias, const int32_t *token_ids,
                      const int32_t *tid2eid, const uint8_t *w13q, const uint8_t *w13s,
                      const uint8_t *w2q, const uint8_t *w2s, const uint8_t *w13q_shared,
                      const uint8_t *w13s_shared, const uint8_t *w2q_shared,
                      const uint8_t *w2s_shared, void *out, int32_t *topk_ids_out,
                      float *topk_weights_out, void *workspace, size_t workspace_bytes,
                      void *stream);

/* Static description of a status code. */
const char *moe_strerror(int status);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
