/*
 * moe_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow CPU statement of the single-GPU Mixture-of-Experts FFN layer.
 * Only the test suite, the smoke check and the CPU-baseline leg of the
 * benchmark load this library.  The product path never links, imports or calls
 * it, and it shares no code, header, table or helper with the HIP library.
 *
 * Sources (web pages, by title and section):
 *  [P1] "DeepSeek-V4 MoE: Token 从路由到专家计算，再回到原位置" (akiyangdev llm-inference-notes),
 *       sections 二 (Router, TopK, HashTopK) and 四 (Dispatch, expert FFN, Combine).
 *  [P2] "MoE 架构与路由策略" (t6page DeepSeek-V4 notes), equation dsv4-moe-softplus,
 *       the aux-loss-free section, the V3 node-limited routing section and the
 *       hash routing section.
 *  [P3] "MoE 的算量与通信" (arganzheng, moe-compute-and-communication), chapter 二.1-二.3
 *       (SwiGLU FFN, router, top-k renormalisation, weighted sum plus shared experts),
 *       chapter 五.3 (group choice by the sum of each group's top Kr/M scores),
 *       chapter 七.3 (bias used for selection only).
 *  [P4] "Mixture of Experts: Router, Token Dispatch, Grouped GEMM" (111qqz), sections
 *       Router (worked example), Expert (SwiGLU), Token Dispatch, Token Combine.
 *
 * Precision.
 *  - Expert FFNs, logits and the combine are evaluated in double precision from
 *    the inputs as given (bf16 -> double is exact).
 *  - Routing decisions (which experts a token selects) are taken in float, the
 *    precision the GPU kernels decide in: logits are rounded to float, affinities
 *    come from the C library's expf/log1pf/sqrtf, and the selection key is the
 *    float sum score + bias.  Gates are then formed in double from those floats.
 *
 * Readings where the pages are silent (each is also listed in the design notes):
 *  - w13 rows [0, d_ff) are the gate projection W1 (the SiLU input), rows
 *    [d_ff, 2 d_ff) the up projection W3; weights are stored [out, in].
 *  - top-k order: descending key, equal keys go to the lower expert index; the
 *    same rule orders groups.
 *  - softmax routing selects on the raw logits and forms the gates as a softmax
 *    over the selected logits (equal to softmax over all experts followed by
 *    renormalisation over the selected ones).
 *  - sigmoid / sqrt(softplus): gates are the unbiased scores of the selected
 *    experts divided by their sum; if that sum is 0 every gate is 1/k.
 *  - the group stage scores a group by the float sum, in descending order, of its
 *    top `group_topk` biased keys.
 *  - hash routing takes the ids from tid2eid in stored order; its gates are the
 *    affinities of the token's logits at those ids, renormalised (bias unused).
 *  - shared experts are added with weight 1; no routed scaling factor.
 *
 *  - FP8 experts ([P2] FP4 QAT section and table dsv4-moe-fp4-vs-fp8: E4M3 with
 *    one scale per 128x128 weight tile; [P2] table dsv4-moe-stages: activation
 *    then FP8 cast between Linear-1 and Linear-2; [P3] 五.2: FP8 dispatch; [P3]
 *    closing section: promotion to FP32 accumulation every 128 elements).  The
 *    pages fix the weight tile; activations are read as one scale per token per
 *    128 channels (1x128, the K blocks of the weight tiles).  Scales are powers
 *    of two: [P2]'s FP4 QAT section calls FP4 -> FP8 dequantization lossless
 *    when each FP8 tile's FP4 sub-block scales span no more than the FP8
 *    exponent range, which holds only if the FP8 tile scale is a power of two.
 *    A group's scale is the smallest 2^e with max |x| <= 448 * 2^e (e >= -126;
 *    1 for an all-zero group) and a code is E4M3 of x * 2^-e (exact scaling),
 *    rounded to nearest-even.  Products are summed per 128-element K block and
 *    each block sum is scaled by the two block scales (in double here).
 *    h = SiLU(g)*u is rounded to float before it is quantized.
 *  - MXFP4 expert weights ([P2] FP4 QAT section: E2M1 with one scale per 1x32
 *    sub-block, used directly at inference; FP4 x FP8 products): a weight row's
 *    32-element blocks get power-of-two scales (E8M0 bytes) by the FP8 rule with
 *    6 in place of 448, codes rounded to nearest-even; activations and h stay
 *    E4M3 1x128 as above.  Products are summed per 32-element block and scaled
 *    by the block's weight scale and the activation's 1x128 scale.
 *
 * Pins: the tests check this file against the pages' worked examples (router
 * example, two-token toy, dispatch/combine toy, EP4 per-expert counts), closed
 * forms of the affinities, invariants of routing and permutation, a dense SwiGLU
 * FFN for E = 1, k = 1, and a dense masked evaluation of every expert on tiny
 * inputs.  The group stage has no printed example: it is pinned only by its
 * invariants and by an independent array formulation in the tests.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_SOFTMAX 0
#define ORACLE_SIGMOID 1
#define ORACLE_SQRTSOFTPLUS 2

/* element i of a tensor stored as float (dtype 0) or bfloat16 (dtype 1) */
static double elem(const void *p, size_t i, int dtype)
{
    if (dtype == 0)
        return (double)((const float *)p)[i];
    uint32_t bits = (uint32_t)((const uint16_t *)p)[i] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* ---------------------------------------------------------------------------
 * Affinity functions, in float.  [P2] equation dsv4-moe-softplus gives
 * Sigmoid(x) = 1 / (1 + e^-x) and sqrt(Softplus(x)) = sqrt(ln(1 + e^x));
 * ln(1 + e^x) is evaluated as max(x, 0) + log1p(e^-|x|), which is the same
 * number without overflow for large x.
 * ------------------------------------------------------------------------- */
float oracle_affinity(float l, int scoring)
{
    if (scoring == ORACLE_SIGMOID)
        return 1.0f / (1.0f + expf(-l));
    if (scoring == ORACLE_SQRTSOFTPLUS)
        return sqrtf(fmaxf(l, 0.0f) + log1pf(expf(-fabsf(l))));
    return l; /* softmax: selection is on the logit itself */
}

/* index of the best candidate (largest key, lowest index on equal keys) among
   those with ok[i] != 0; -1 if none is left */
static int best_of(int n, const float *key, const unsigned char *ok)
{
    int b = -1;
    for (int i = 0; i < n; ++i)
        if (ok[i] && (b < 0 || key[i] > key[b]))
            b = i;
    return b;
}

/* gates over the selected experts, in double ([P3] 二.2 renormalisation; [P4]
   Router: softmax over the selected logits) */
static void form_gates(int k, const int32_t *sel, const float *logit_row,
                       const float *score_row, int scoring, float *gates)
{
    double g[64];
    double sum = 0.0;
    if (scoring == ORACLE_SOFTMAX) {
        double lmax = -INFINITY;
        for (int j = 0; j < k; ++j)
            if ((double)logit_row[sel[j]] > lmax)
                lmax = (double)logit_row[sel[j]];
        for (int j = 0; j < k; ++j) {
            g[j] = exp((double)logit_row[sel[j]] - lmax);
            sum += g[j];
        }
    } else {
        for (int j = 0; j < k; ++j) {
            g[j] = (double)score_row[sel[j]];
            sum += g[j];
        }
    }
    for (int j = 0; j < k; ++j)
        gates[j] = (sum > 0.0) ? (float)(g[j] / sum) : (float)(1.0 / k);
}

/* ---------------------------------------------------------------------------
 * Learned routing for one token.  Returns 0, or -1 on bad arguments.
 *  key_i = affinity_i + bias_i  ([P3] 七.3: the bias only decides who is chosen)
 *  optional group stage ([P2] V3 node-limited routing, [P3] 五.3): experts form
 *  n_group contiguous groups; a group scores the sum of its top group_topk keys;
 *  the topk_group best groups stay eligible.
 *  top-k by key among eligible experts ([P3] 二.2, [P4] Router).
 *  margin: the smallest gap between consecutive sorted values that decide the
 *  result (keys 1..k+1 among eligible experts, and group scores around the
 *  topk_group cut); tests use it to excuse near-ties.
 * ------------------------------------------------------------------------- */
static int route_one(int E, int k, int scoring, int n_group, int topk_group,
                     int group_topk, const float *l, const float *bias,
                     int32_t *ids, float *gates, float *margin)
{
    float *s = malloc(sizeof(float) * E);
    float *key = malloc(sizeof(float) * E);
    unsigned char *ok = malloc(E);
    float m = INFINITY;
    if (!s || !key || !ok)
        return -1;
    for (int i = 0; i < E; ++i) {
        s[i] = oracle_affinity(l[i], scoring);
        key[i] = bias ? s[i] + bias[i] : s[i];
        ok[i] = 1;
    }
    if (n_group > 1) {
        int G = E / n_group;
        float *gs = malloc(sizeof(float) * n_group);
        unsigned char *gok = malloc(n_group);
        unsigned char *tmp = malloc(G);
        for (int g = 0; g < n_group; ++g) {
            /* sum of this group's group_topk largest keys, largest first */
            memset(tmp, 1, G);
            float acc = 0.0f;
            for (int r = 0; r < group_topk; ++r) {
                int b = best_of(G, key + g * G, tmp);
                acc = (r == 0) ? key[g * G + b] : acc + key[g * G + b];
                tmp[b] = 0;
            }
            gs[g] = acc;
            gok[g] = 1;
        }
        unsigned char *keep = calloc(n_group, 1);
        float prev = 0.0f;
        for (int r = 0; r < topk_group + 1 && r < n_group; ++r) {
            int b = best_of(n_group, gs, gok);
            /* only the cut between kept and dropped groups decides the result */
            if (r == topk_group && prev - gs[b] < m)
                m = prev - gs[b];
            prev = gs[b];
            gok[b] = 0;
            if (r < topk_group)
                keep[b] = 1;
        }
        for (int i = 0; i < E; ++i)
            ok[i] = keep[i / G];
        free(gs);
        free(gok);
        free(tmp);
        free(keep);
    }
    float prev = 0.0f;
    for (int r = 0; r < k + 1; ++r) {
        int b = best_of(E, key, ok);
        if (b < 0) {
            if (r < k) { /* fewer eligible experts than k */
                free(s); free(key); free(ok);
                return -1;
            }
            break;
        }
        if (r > 0 && prev - key[b] < m)
            m = prev - key[b];
        prev = key[b];
        ok[b] = 0;
        if (r < k)
            ids[r] = b;
    }
    form_gates(k, ids, l, s, scoring, gates);
    if (margin)
        *margin = m;
    free(s);
    free(key);
    free(ok);
    return 0;
}

int oracle_route(int T, int E, int k, int scoring, int n_group, int topk_group,
                 int group_topk, const float *logits, const float *bias,
                 int32_t *ids, float *gates, float *margin)
{
    if (T < 0 || E < 1 || k < 1 || k > E || k > 64)
        return -1;
    if (n_group > 1 && (E % n_group || topk_group < 1 || topk_group > n_group ||
                        group_topk < 1 || group_topk > E / n_group))
        return -1;
    for (int t = 0; t < T; ++t)
        if (route_one(E, k, scoring, n_group, topk_group, group_topk,
                      logits + (size_t)t * E, bias, ids + (size_t)t * k,
                      gates + (size_t)t * k, margin ? margin + t : NULL))
            return -1;
    return 0;
}

/* Hash routing ([P1] 二 HashTopK; [P2] hash routing): ids come from the
   token-id table; gates are the token's affinities at those ids, renormalised. */
int oracle_hash_route(int T, int E, int k, int scoring, const float *logits,
                      const int32_t *token_ids, const int32_t *tid2eid, int vocab,
                      int32_t *ids, float *gates)
{
    float *s = malloc(sizeof(float) * E);
    if (!s || k > 64)
        return -1;
    for (int t = 0; t < T; ++t) {
        const float *l = logits + (size_t)t * E;
        int tok = token_ids[t];
        if (tok < 0 || tok >= vocab) {
            free(s);
            return -1;
        }
        for (int j = 0; j < k; ++j) {
            int e = tid2eid[(size_t)tok * k + j];
            if (e < 0 || e >= E) {
                free(s);
                return -1;
            }
            ids[(size_t)t * k + j] = e;
        }
        for (int i = 0; i < E; ++i)
            s[i] = oracle_affinity(l[i], scoring);
        form_gates(k, ids + (size_t)t * k, l, s, scoring, gates + (size_t)t * k);
    }
    free(s);
    return 0;
}

/* ---------------------------------------------------------------------------
 * Token dispatch ([P4] Token Dispatch): the T*k (token, slot) pairs reordered
 * expert-major, tokens ascending inside each expert.  Written as the plain
 * definition: walk the experts in order and, for each, the pairs in token order.
 * dispatch_index[t*k + j] is the row that pair (t, j) lands on.
 * ------------------------------------------------------------------------- */
int oracle_permute(int T, int k, int E, const int32_t *ids, const float *gates,
                   int32_t *counts, int32_t *offsets, int32_t *sorted_tok,
                   float *sorted_w, int32_t *dispatch_index)
{
    int r = 0;
    for (int e = 0; e < E; ++e) {
        offsets[e] = r;
        counts[e] = 0;
        for (int t = 0; t < T; ++t)
            for (int j = 0; j < k; ++j)
                if (ids[(size_t)t * k + j] == e) {
                    sorted_tok[r] = t;
                    sorted_w[r] = gates[(size_t)t * k + j];
                    dispatch_index[(size_t)t * k + j] = r;
                    ++counts[e];
                    ++r;
                }
    }
    offsets[E] = r;
    return (r == T * k) ? 0 : -1; /* every pair must name an expert in [0, E) */
}

/* ---------------------------------------------------------------------------
 * Combine ([P4] Token Combine, index_add_): for every dispatch row r,
 * out[token_of_row[r]] += weight[r] * expert_out[r]; then the shared rows.
 * out must hold zeros (or the value to add onto) on entry.
 * ------------------------------------------------------------------------- */
void oracle_combine(int P, int d, const double *expert_out, const int32_t *token_of_row,
                    const float *weight_of_row, double *out)
{
    for (int r = 0; r < P; ++r) {
        double w = (double)weight_of_row[r];
        double *o = out + (size_t)token_of_row[r] * d;
        const double *x = expert_out + (size_t)r * d;
        for (int i = 0; i < d; ++i)
            o[i] += w * x[i];
    }
}

/* ---------------------------------------------------------------------------
 * One SwiGLU expert ([P3] 二.1; [P1] 四; [P4] Expert):
 *   y = W2 (SiLU(W1 x) (.) W3 x),  SiLU(z) = z / (1 + e^-z)
 * with W1 = w13[0:d_ff], W3 = w13[d_ff:2 d_ff] (each [d_ff, d]) and W2 = w2 [d, d_ff].
 * ------------------------------------------------------------------------- */
void oracle_expert_ffn(int d, int d_ff, const double *x, const void *w13,
                       const void *w2, int dtype, double *y)
{
    double *h = malloc(sizeof(double) * d_ff);
    for (int f = 0; f < d_ff; ++f) {
        double g = 0.0, u = 0.0;
        for (int i = 0; i < d; ++i) {
            g += elem(w13, (size_t)f * d + i, dtype) * x[i];
            u += elem(w13, (size_t)(d_ff + f) * d + i, dtype) * x[i];
        }
        h[f] = g / (1.0 + exp(-g)) * u;
    }
    for (int o = 0; o < d; ++o) {
        double acc = 0.0;
        for (int f = 0; f < d_ff; ++f)
            acc += elem(w2, (size_t)o * d_ff + f, dtype) * h[f];
        y[o] = acc;
    }
    free(h);
}

/* router logits ([P3] 二.2: l = W_r x, W_r is [E, d]) for the listed tokens, in
   double, plus an optional per-expert offset added to every token's logits */
void oracle_logits(int n, const int32_t *rows, int d, int E, const void *hidden,
                   const void *w_router, int dtype, const float *logit_offset,
                   double *logits)
{
    for (int q = 0; q < n; ++q) {
        size_t t = (size_t)rows[q];
        for (int e = 0; e < E; ++e) {
            double acc = 0.0;
            for (int i = 0; i < d; ++i)
                acc += elem(w_router, (size_t)e * d + i, dtype) * elem(hidden, t * d + i, dtype);
            if (logit_offset)
                acc += (double)logit_offset[e];
            logits[(size_t)q * E + e] = acc;
        }
    }
}

/* Route listed token q: logits (double, then float), learned or hash routing.
   Returns the routing status; ids/gates/margin as route_one. */
static int route_listed(int q, const int32_t *rows, int d, int E, int k, int scoring,
                        int route_mode, int n_group, int topk_group, int group_topk,
                        const void *hidden, const void *w_router, int dtype,
                        const float *bias, const float *logit_offset,
                        const int32_t *token_ids, const int32_t *tid2eid, int vocab,
                        int32_t *ids, float *gates, float *margin)
{
    double *lg = malloc(sizeof(double) * E);
    float *lf = malloc(sizeof(float) * E);
    size_t t = (size_t)rows[q];
    oracle_logits(1, rows + q, d, E, hidden, w_router, dtype, logit_offset, lg);
    for (int e = 0; e < E; ++e)
        lf[e] = (float)lg[e];
    int rc;
    *margin = INFINITY;
    if (route_mode == 1)
        rc = oracle_hash_route(1, E, k, scoring, lf, token_ids + t, tid2eid, vocab, ids,
                               gates);
    else
        rc = route_one(E, k, scoring, n_group, topk_group, group_topk, lf, bias, ids, gates,
                       margin);
    free(lg);
    free(lf);
    return rc;
}

/* ---------------------------------------------------------------------------
 * The whole layer for a list of tokens ([P3] 二.2 and 二.3):
 *   y_t = sum_j g[t,j] * FFN_{ids[t,j]}(x_t) + sum_s FFN^shared_s(x_t)
 * Each listed token is routed from its own logits (rounded to float) and its
 * output row is written in double.  w13[e] / w2[e] point at expert e's weights
 * (only the experts the listed tokens select need to be non-NULL); route_mode
 * 0 = learned, 1 = hash.  ids/gates/margin may be NULL.
 * Returns 0, or -1 on bad arguments or a needed expert without weights.
 * ------------------------------------------------------------------------- */
int oracle_layer(int n, const int32_t *rows, int d, int E, int k, int d_ff,
                 int n_shared, int dtype, int scoring, int route_mode, int n_group,
                 int topk_group, int group_topk, const void *hidden,
                 const void *w_router, const float *bias, const float *logit_offset,
                 const int32_t *token_ids, const int32_t *tid2eid, int vocab,
                 const void *const *w13, const void *const *w2,
                 const void *w13_shared, const void *w2_shared, double *out,
                 int32_t *ids_out, float *gates_out, float *margin_out)
{
    int bad = 0;
    if (k < 1 || k > 64 || k > E || n_shared < 0 || n_shared > 1)
        return -1;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int q = 0; q < n; ++q) {
        int32_t ids[64];
        float gates[64], margin;
        double *x = malloc(sizeof(double) * d);
        double *y = malloc(sizeof(double) * d);
        double *o = out + (size_t)q * d;
        size_t t = (size_t)rows[q];
        int rc = route_listed(q, rows, d, E, k, scoring, route_mode, n_group, topk_group,
                              group_topk, hidden, w_router, dtype, bias, logit_offset,
                              token_ids, tid2eid, vocab, ids, gates, &margin);
        for (int i = 0; i < d; ++i) {
            x[i] = elem(hidden, t * d + i, dtype);
            o[i] = 0.0;
        }
        for (int j = 0; !rc && j < k; ++j) {
            if (!w13[ids[j]] || !w2[ids[j]]) {
                rc = -1;
                break;
            }
            oracle_expert_ffn(d, d_ff, x, w13[ids[j]], w2[ids[j]], dtype, y);
            for (int i = 0; i < d; ++i)
                o[i] += (double)gates[j] * y[i];
        }
        if (!rc && n_shared == 1) {
            oracle_expert_ffn(d, d_ff, x, w13_shared, w2_shared, dtype, y);
            for (int i = 0; i < d; ++i)
                o[i] += y[i];
        }
        if (rc)
            bad = 1;
        for (int j = 0; j < k; ++j) {
            if (ids_out)
                ids_out[(size_t)q * k + j] = rc ? -1 : ids[j];
            if (gates_out)
                gates_out[(size_t)q * k + j] = rc ? 0.0f : gates[j];
        }
        if (margin_out)
            margin_out[q] = margin;
        free(x);
        free(y);
    }
    return bad ? -1 : 0;
}

/* ---------------------------------------------------------------------------
 * FP8 E4M3 ([P2] table dsv4-moe-fp4-vs-fp8: 4 exponent bits, 3 mantissa bits).
 * Code layout (the OCP "E4M3FN" encoding): sign bit, exponent field E (bias 7),
 * mantissa field m.  E = 0: m * 2^-9 (subnormal); E = 1..15: (1 + m/8) * 2^(E-7),
 * except E = 15, m = 7, which is NaN; there are no infinities, so the largest
 * finite magnitude is (1 + 6/8) * 2^8 = 448.
 * ------------------------------------------------------------------------- */
double oracle_e4m3_decode(uint8_t c)
{
    int E = (c >> 3) & 15, m = c & 7;
    double v;
    if (E == 15 && m == 7)
        return NAN;
    v = E == 0 ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, E - 7);
    return (c & 0x80) ? -v : v;
}

/* nearest code to a finite float, ties to the even mantissa; magnitudes at or
   past 448 give +-448 */
uint8_t oracle_e4m3_encode(float v)
{
    uint8_t sign = signbit(v) ? 0x80 : 0;
    double a = fabs((double)v);
    if (a >= 448.0)
        return sign | 0x7E;
    if (a < ldexp(1.0, -6)) /* subnormal range: multiples of 2^-9 (8 * 2^-9 is code 0x08) */
        return sign | (uint8_t)nearbyint(a * 512.0);
    int e;
    double fr = frexp(a, &e); /* a = (2 fr) * 2^(e-1), 2 fr in [1, 2) */
    double m = nearbyint((2.0 * fr - 1.0) * 8.0);
    int E = e - 1 + 7;
    if (m == 8.0) {
        m = 0.0;
        ++E;
    }
    unsigned code = ((unsigned)E << 3) | (unsigned)m;
    return sign | (uint8_t)(code > 0x7E ? 0x7E : code);
}

/* Exponent of a group's scale: the smallest e with amax <= top * 2^e, where top
   is the format's largest magnitude (448 for E4M3, 6 for E2M1).  With
   amax = m * 2^k and top = tm * 2^tk (m, tm in [0.5, 1)): e = k - tk if m <= tm,
   else k - tk + 1 (448 = 0.875 * 2^9, 6 = 0.75 * 2^3).  Clamped to e >= -126
   (the scale stays a normal float); an all-zero group gets e = 0. */
static int scale_exp_top(float amax, float top)
{
    if (amax == 0.0f)
        return 0;
    int k, tk;
    float m = frexpf(amax, &k);
    float tm = frexpf(top, &tk);
    int e = k - tk + (m > tm ? 1 : 0);
    return e < -126 ? -126 : e;
}

static int scale_exp(float amax) { return scale_exp_top(amax, 448.0f); }

static uint8_t quantize_one(float x, int e)
{
    float v = ldexpf(x, -e); /* exact: a power-of-two scaling */
    v = v > 448.0f ? 448.0f : (v < -448.0f ? -448.0f : v);
    return oracle_e4m3_encode(v);
}

/* Rows of a float [n, K] matrix in groups of 128 columns (the 1x128 reading for
   activations): s[r, g] = 2^e with e = scale_exp(max |x|), q = E4M3(x / s). */
void oracle_quantize_rows(int n, int K, const float *x, uint8_t *q, float *s)
{
    int G = K / 128;
    for (int r = 0; r < n; ++r)
        for (int g = 0; g < G; ++g) {
            const float *xr = x + (size_t)r * K + (size_t)g * 128;
            float amax = 0.0f;
            for (int i = 0; i < 128; ++i)
                amax = fmaxf(amax, fabsf(xr[i]));
            int e = scale_exp(amax);
            s[(size_t)r * G + g] = ldexpf(1.0f, e);
            for (int i = 0; i < 128; ++i)
                q[(size_t)r * K + (size_t)g * 128 + i] = quantize_one(xr[i], e);
        }
}

/* A [R, C] weight matrix (float or bf16) in 128x128 tiles, one power-of-two
   scale per tile ([P2] FP4 QAT section: FP8 quantized per 128x128 tile):
   s[R/128, C/128]. */
void oracle_quantize_blocks(int R, int C, const void *w, int dtype, uint8_t *q, float *s)
{
    int GC = C / 128;
#pragma omp parallel for collapse(2) schedule(static)
    for (int br = 0; br < R / 128; ++br)
        for (int bc = 0; bc < GC; ++bc) {
            float amax = 0.0f;
            for (int i = 0; i < 128; ++i)
                for (int j = 0; j < 128; ++j) {
                    size_t at = (size_t)(br * 128 + i) * C + (size_t)bc * 128 + j;
                    amax = fmaxf(amax, fabsf((float)elem(w, at, dtype)));
                }
            int e = scale_exp(amax);
            s[(size_t)br * GC + bc] = ldexpf(1.0f, e);
            for (int i = 0; i < 128; ++i)
                for (int j = 0; j < 128; ++j) {
                    size_t at = (size_t)(br * 128 + i) * C + (size_t)bc * 128 + j;
                    q[at] = quantize_one((float)elem(w, at, dtype), e);
                }
        }
}

/* sum_kb sa[kb] * sb[kb] * sum_{k in kb} dec(a_k) dec(b_k), in double: the dot
   product of two FP8 vectors of length K with one scale per 128 elements each */
static double dot_fp8(int K, const uint8_t *a, const float *sa, const uint8_t *b,
                      const float *sb)
{
    double val[256], acc = 0.0;
    for (int c = 0; c < 256; ++c)
        val[c] = oracle_e4m3_decode((uint8_t)c);
    for (int kb = 0; kb < K / 128; ++kb) {
        double part = 0.0;
        for (int i = kb * 128; i < kb * 128 + 128; ++i)
            part += val[a[i]] * val[b[i]];
        acc += (double)sa[kb] * (double)sb[kb] * part;
    }
    return acc;
}

/* ---------------------------------------------------------------------------
 * One SwiGLU expert with FP8 operands.  x: the token's codes xq[d] and scales
 * xs[d/128]; w13q [2 d_ff, d] with tile scales w13s [2 d_ff/128, d/128]; w2q
 * [d, d_ff] with w2s [d/128, d_ff/128].  h = SiLU(g) * u is rounded to float,
 * quantized in 1x128 groups, and the down projection reads those codes.
 * ------------------------------------------------------------------------- */
/* The up half: h = SiLU(g) * u rounded to float, then its 1x128 quantization
   (hq [d_ff] codes, hs [d_ff/128] scales). */
void oracle_expert_up_fp8(int d, int d_ff, const uint8_t *xq, const float *xs,
                          const uint8_t *w13q, const float *w13s, uint8_t *hq, float *hs)
{
    int Gd = d / 128;
    float *h = malloc(sizeof(float) * d_ff);
    float *sb = malloc(sizeof(float) * Gd);
    for (int f = 0; f < d_ff; ++f) {
        for (int kb = 0; kb < Gd; ++kb)
            sb[kb] = w13s[(size_t)(f / 128) * Gd + kb];
        double g = dot_fp8(d, xq, xs, w13q + (size_t)f * d, sb);
        for (int kb = 0; kb < Gd; ++kb)
            sb[kb] = w13s[(size_t)((d_ff + f) / 128) * Gd + kb];
        double u = dot_fp8(d, xq, xs, w13q + (size_t)(d_ff + f) * d, sb);
        h[f] = (float)(g / (1.0 + exp(-g)) * u);
    }
    oracle_quantize_rows(1, d_ff, h, hq, hs);
    free(h);
    free(sb);
}

void oracle_expert_ffn_fp8(int d, int d_ff, const uint8_t *xq, const float *xs,
                           const uint8_t *w13q, const float *w13s, const uint8_t *w2q,
                           const float *w2s, double *y)
{
    int Gd = d / 128, Gf = d_ff / 128;
    uint8_t *hq = malloc(d_ff);
    float *hs = malloc(sizeof(float) * Gf);
    float *sb = malloc(sizeof(float) * (Gd > Gf ? Gd : Gf));
    oracle_expert_up_fp8(d, d_ff, xq, xs, w13q, w13s, hq, hs);
    for (int o = 0; o < d; ++o) {
        for (int kb = 0; kb < Gf; ++kb)
            sb[kb] = w2s[(size_t)(o / 128) * Gf + kb];
        y[o] = dot_fp8(d_ff, hq, hs, w2q + (size_t)o * d_ff, sb);
    }
    free(hq);
    free(hs);
    free(sb);
}

/* ---------------------------------------------------------------------------
 * The layer with FP8 experts: routing exactly as oracle_layer (from the bf16 or
 * float hidden states and router weight); each listed token's hidden row is
 * quantized (1x128, [P3] 五.2 FP8 dispatch) and goes through the FP8 experts;
 * the gated sum is formed in double.  w13q/w13s/w2q/w2s: per-expert pointers
 * (NULL for experts no listed token selects); shared expert likewise.  The
 * weight scales are float32 tile scales (FP8) or E8M0 bytes (MXFP4): the
 * expert function given reads them.
 * ------------------------------------------------------------------------- */
typedef void (*lowp_ffn_fn)(int d, int d_ff, const uint8_t *xq, const float *xs,
                            const uint8_t *w13q, const void *w13s, const uint8_t *w2q,
                            const void *w2s, double *y);

static void ffn_fp8_any(int d, int d_ff, const uint8_t *xq, const float *xs,
                        const uint8_t *w13q, const void *w13s, const uint8_t *w2q,
                        const void *w2s, double *y)
{
    oracle_expert_ffn_fp8(d, d_ff, xq, xs, w13q, (const float *)w13s, w2q, (const float *)w2s, y);
}

static int layer_lowp(lowp_ffn_fn ffn, int n, const int32_t *rows, int d, int E, int k, int d_ff,
                      int n_shared, int dtype, int scoring, int route_mode, int n_group,
                      int topk_group, int group_topk, const void *hidden,
                      const void *w_router, const float *bias, const float *logit_offset,
                      const int32_t *token_ids, const int32_t *tid2eid, int vocab,
                      const uint8_t *const *w13q, const void *const *w13s,
                      const uint8_t *const *w2q, const void *const *w2s,
                      const uint8_t *w13q_sh, const void *w13s_sh, const uint8_t *w2q_sh,
                      const void *w2s_sh, double *out, int32_t *ids_out, float *gates_out,
                      float *margin_out)
{

    int bad = 0;
    if (k < 1 || k > 64 || k > E || n_shared < 0 || n_shared > 1 || d % 128 || d_ff % 128)
        return -1;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int q = 0; q < n; ++q) {
        int32_t ids[64];
        float gates[64], margin;
        float *xf = malloc(sizeof(float) * d);
        uint8_t *xq = malloc(d);
        float *xs = malloc(sizeof(float) * (d / 128));
        double *y = malloc(sizeof(double) * d);
        double *o = out + (size_t)q * d;
        size_t t = (size_t)rows[q];
        int rc = route_listed(q, rows, d, E, k, scoring, route_mode, n_group, topk_group,
                              group_topk, hidden, w_router, dtype, bias, logit_offset,
                              token_ids, tid2eid, vocab, ids, gates, &margin);
        for (int i = 0; i < d; ++i) {
            xf[i] = (float)elem(hidden, t * d + i, dtype);
            o[i] = 0.0;
        }
        oracle_quantize_rows(1, d, xf, xq, xs);
        for (int j = 0; !rc && j < k; ++j) {
            int e = ids[j];
            if (!w13q[e] || !w13s[e] || !w2q[e] || !w2s[e]) {
                rc = -1;
                break;
            }
            ffn(d, d_ff, xq, xs, w13q[e], w13s[e], w2q[e], w2s[e], y);
            for (int i = 0; i < d; ++i)
                o[i] += (double)gates[j] * y[i];
        }
        if (!rc && n_shared == 1) {
            ffn(d, d_ff, xq, xs, w13q_sh, w13s_sh, w2q_sh, w2s_sh, y);
            for (int i = 0; i < d; ++i)
                o[i] += y[i];
        }
        if (rc)
            bad = 1;
        for (int j = 0; j < k; ++j) {
            if (ids_out)
                ids_out[(size_t)q * k + j] = rc ? -1 : ids[j];
            if (gates_out)
                gates_out[(size_t)q * k + j] = rc ? 0.0f : gates[j];
        }
        if (margin_out)
            margin_out[q] = margin;
        free(xf);
        free(xq);
        free(xs);
        free(y);
    }
    return bad ? -1 : 0;
}


int oracle_layer_fp8(int n, const int32_t *rows, int d, int E, int k, int d_ff,
                     int n_shared, int dtype, int scoring, int route_mode, int n_group,
                     int topk_group, int group_topk, const void *hidden,
                     const void *w_router, const float *bias, const float *logit_offset,
                     const int32_t *token_ids, const int32_t *tid2eid, int vocab,
                     const uint8_t *const *w13q, const float *const *w13s,
                     const uint8_t *const *w2q, const float *const *w2s,
                     const uint8_t *w13q_sh, const float *w13s_sh, const uint8_t *w2q_sh,
                     const float *w2s_sh, double *out, int32_t *ids_out, float *gates_out,
                     float *margin_out)
{
    return layer_lowp(ffn_fp8_any, n, rows, d, E, k, d_ff, n_shared, dtype, scoring, route_mode,
                      n_group, topk_group, group_topk, hidden, w_router, bias, logit_offset,
                      token_ids, tid2eid, vocab, w13q, (const void *const *)w13s, w2q,
                      (const void *const *)w2s, w13q_sh, w13s_sh, w2q_sh, w2s_sh, out, ids_out,
                      gates_out, margin_out);
}

/* ---------------------------------------------------------------------------
 * MXFP4 E2M1 ([P2] FP4 QAT section and table dsv4-moe-fp4-vs-fp8: 2 exponent
 * bits and 1 mantissa bit, one shared scale per 1x32 sub-block; [P2]: inference
 * uses the FP4 weights directly, and FP4 x FP8 products are what hardware with
 * native support multiplies).  Code layout (the OCP MX E2M1 element): sign bit 3,
 * exponent field E (bits 2..1, bias 1), mantissa bit m.  E = 0: m / 2; E = 1..3:
 * (1 + m/2) * 2^(E-1).  No infinities or NaN: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6.
 * Weights only: one scale per 32 consecutive elements of a weight row (the K
 * direction of the dot products), a power of two stored as an E8M0 byte
 * (scale = 2^(byte - 127)), chosen as for FP8 with 6 in place of 448.  Two codes
 * per byte, element 2j in the low nibble.  Activations (the hidden rows and h)
 * stay E4M3 with 1x128 scales.
 * ------------------------------------------------------------------------- */
double oracle_e2m1_decode(uint8_t c)
{
    int E = (c >> 1) & 3, m = c & 1;
    double v = E == 0 ? 0.5 * m : ldexp(1.0 + 0.5 * m, E - 1);
    return (c & 8) ? -v : v;
}

/* nearest of the eight magnitudes (searched in order); on a tie the code whose
   mantissa bit is 0; past 6 it stays 6 */
uint8_t oracle_e2m1_encode(float v)
{
    uint8_t sign = signbit(v) ? 8 : 0;
    double a = fabs((double)v);
    if (a >= 6.0) /* saturate (far past 6 the distances below would tie) */
        return sign | 7;
    int best = 0;
    for (int c = 1; c < 8; ++c) {
        double dc = fabs(oracle_e2m1_decode((uint8_t)c) - a);
        double db = fabs(oracle_e2m1_decode((uint8_t)best) - a);
        if (dc < db || (dc == db && (c & 1) == 0))
            best = c;
    }
    return sign | (uint8_t)best;
}

/* A [R, C] weight matrix (float or bf16, C a multiple of 32) in 1x32 blocks:
   q [R, C/2] (two codes per byte), s [R, C/32] E8M0 scale bytes. */
void oracle_quantize_mxfp4(int R, int C, const void *w, int dtype, uint8_t *q, uint8_t *s)
{
    int G = C / 32;
#pragma omp parallel for schedule(static)
    for (int r = 0; r < R; ++r)
        for (int g = 0; g < G; ++g) {
            size_t at = (size_t)r * C + (size_t)g * 32;
            float amax = 0.0f;
            for (int i = 0; i < 32; ++i)
                amax = fmaxf(amax, fabsf((float)elem(w, at + i, dtype)));
            int e = scale_exp_top(amax, 6.0f);
            s[(size_t)r * G + g] = (uint8_t)(e + 127);
            for (int i = 0; i < 32; i += 2) {
                uint8_t lo = oracle_e2m1_encode(ldexpf((float)elem(w, at + i, dtype), -e));
                uint8_t hi = oracle_e2m1_encode(ldexpf((float)elem(w, at + i + 1, dtype), -e));
                q[(at + i) / 2] = (uint8_t)(lo | (hi << 4));
            }
        }
}

/* sum over 32-element blocks b of sa[b / 4] * 2^(sb[b] - 127) * sum_{k in b}
   dec8(a_k) dec4(w_k), in double: an FP8 vector (1x128 scales) against an MXFP4
   weight row */
static double dot_mx(int K, const uint8_t *a, const float *sa, const uint8_t *wq,
                     const uint8_t *sb)
{
    double v8[256], v4[16], acc = 0.0;
    for (int c = 0; c < 256; ++c)
        v8[c] = oracle_e4m3_decode((uint8_t)c);
    for (int c = 0; c < 16; ++c)
        v4[c] = oracle_e2m1_decode((uint8_t)c);
    for (int b = 0; b < K / 32; ++b) {
        double part = 0.0;
        for (int i = b * 32; i < b * 32 + 32; ++i) {
            uint8_t code = (i & 1) ? (uint8_t)(wq[i / 2] >> 4) : (uint8_t)(wq[i / 2] & 15);
            part += v8[a[i]] * v4[code];
        }
        acc += (double)sa[b / 4] * ldexp(1.0, (int)sb[b] - 127) * part;
    }
    return acc;
}

/* One SwiGLU expert with MXFP4 weights: w13q [2 d_ff, d/2] with w13s [2 d_ff,
   d/32]; w2q [d, d_ff/2] with w2s [d, d_ff/32].  x and h as for FP8. */
void oracle_expert_up_mxfp4(int d, int d_ff, const uint8_t *xq, const float *xs,
                            const uint8_t *w13q, const uint8_t *w13s, uint8_t *hq, float *hs)
{
    float *h = malloc(sizeof(float) * d_ff);
    for (int f = 0; f < d_ff; ++f) {
        double g = dot_mx(d, xq, xs, w13q + (size_t)f * (d / 2), w13s + (size_t)f * (d / 32));
        double u = dot_mx(d, xq, xs, w13q + (size_t)(d_ff + f) * (d / 2),
                          w13s + (size_t)(d_ff + f) * (d / 32));
        h[f] = (float)(g / (1.0 + exp(-g)) * u);
    }
    oracle_quantize_rows(1, d_ff, h, hq, hs);
    free(h);
}

void oracle_expert_ffn_mxfp4(int d, int d_ff, const uint8_t *xq, const float *xs,
                             const uint8_t *w13q, const uint8_t *w13s, const uint8_t *w2q,
                             const uint8_t *w2s, double *y)
{
    uint8_t *hq = malloc(d_ff);
    float *hs = malloc(sizeof(float) * (d_ff / 128));
    oracle_expert_up_mxfp4(d, d_ff, xq, xs, w13q, w13s, hq, hs);
    for (int o = 0; o < d; ++o)
        y[o] = dot_mx(d_ff, hq, hs, w2q + (size_t)o * (d_ff / 2), w2s + (size_t)o * (d_ff / 32));
    free(hq);
    free(hs);
}

static void ffn_mxfp4_any(int d, int d_ff, const uint8_t *xq, const float *xs,
                          const uint8_t *w13q, const void *w13s, const uint8_t *w2q,
                          const void *w2s, double *y)
{
    oracle_expert_ffn_mxfp4(d, d_ff, xq, xs, w13q, (const uint8_t *)w13s, w2q,
                            (const uint8_t *)w2s, y);
}

/* The layer with MXFP4 expert weights (the FP8 layer's steps; weight scales are
   E8M0 bytes) */
int oracle_layer_mxfp4(int n, const int32_t *rows, int d, int E, int k, int d_ff,
                       int n_shared, int dtype, int scoring, int route_mode, int n_group,
                       int topk_group, int group_topk, const void *hidden,
                       const void *w_router, const float *bias, const float *logit_offset,
                       const int32_t *token_ids, const int32_t *tid2eid, int vocab,
                       const uint8_t *const *w13q, const uint8_t *const *w13s,
                       const uint8_t *const *w2q, const uint8_t *const *w2s,
                       const uint8_t *w13q_sh, const uint8_t *w13s_sh, const uint8_t *w2q_sh,
                       const uint8_t *w2s_sh, double *out, int32_t *ids_out, float *gates_out,
                       float *margin_out)
{
    return layer_lowp(ffn_mxfp4_any, n, rows, d, E, k, d_ff, n_shared, dtype, scoring,
                      route_mode, n_group, topk_group, group_topk, hidden, w_router, bias,
                      logit_offset, token_ids, tid2eid, vocab, w13q, (const void *const *)w13s,
                      w2q, (const void *const *)w2s, w13q_sh, w13s_sh, w2q_sh, w2s_sh, out,
                      ids_out, gates_out, margin_out);
}

/* ---------------------------------------------------------------------------
 * One expert over a list of token rows (test convenience): y[q] = FFN_e(x_t)
 * for t = tokens[q], each row exactly as oracle_expert_ffn evaluates it (the
 * rows are independent; OpenMP over rows).  hidden [T, d] in dtype.
 * ------------------------------------------------------------------------- */
void oracle_expert_rows(int n, const int32_t *tokens, int d, int d_ff, const void *hidden,
                        int dtype, const void *w13, const void *w2, double *y)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int q = 0; q < n; ++q) {
        double *x = malloc(sizeof(double) * d);
        size_t t = (size_t)tokens[q];
        for (int i = 0; i < d; ++i)
            x[i] = elem(hidden, t * d + i, dtype);
        oracle_expert_ffn(d, d_ff, x, w13, w2, dtype, y + (size_t)q * d);
        free(x);
    }
}

/* The same with FP8 (fmt 0: E4M3 weights, float tile scales) or MXFP4 (fmt 1:
   E2M1 weights, E8M0 block scales) expert weights: each token's hidden row is
   rounded to float and quantized 1x128 as in the FP8 layer, then goes through
   the low-precision expert. */
void oracle_expert_rows_lowp(int fmt, int n, const int32_t *tokens, int d, int d_ff,
                             const void *hidden, int dtype, const uint8_t *w13q,
                             const void *w13s, const uint8_t *w2q, const void *w2s, double *y)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int q = 0; q < n; ++q) {
        float *xf = malloc(sizeof(float) * d);
        uint8_t *xq = malloc(d);
        float *xs = malloc(sizeof(float) * (d / 128));
        size_t t = (size_t)tokens[q];
        for (int i = 0; i < d; ++i)
            xf[i] = (float)elem(hidden, t * d + i, dtype);
        oracle_quantize_rows(1, d, xf, xq, xs);
        if (fmt == 0)
            ffn_fp8_any(d, d_ff, xq, xs, w13q, w13s, w2q, w2s, y + (size_t)q * d);
        else
            ffn_mxfp4_any(d, d_ff, xq, xs, w13q, w13s, w2q, w2s, y + (size_t)q * d);
        free(xf);
        free(xq);
        free(xs);
    }
}

/* set the number of OpenMP threads later parallel loops use (timing on one core) */
void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    omp_set_num_threads(n > 0 ? n : 1);
#else
    (void)n;
#endif
}

/* number of OpenMP threads the layer loop runs on (reported with timings) */
int oracle_num_threads(void)
{
    int n = 1;
#ifdef _OPENMP
#pragma omp parallel
    {
#pragma omp single
        n = omp_get_num_threads();
    }
#endif
    return n;
}
