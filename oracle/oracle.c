/*
 * oracle.c -- plain, slow, CPU reference of the MoE routing hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library (moe_routing_amd/)
 * includes, links or calls this file.  It may be loaded only by the tests, by
 * the smoke check and by the CPU-baseline leg of the benchmark.  It shares no
 * source with the HIP path: every rounding rule, table and loop below is
 * written here from the definitions, independently of the kernels.
 *
 * Sources (web pages; cited by title and section):
 *   [P1] "刚刚！DeepSeek开源高性能GPU算子库TileKernels" (147227.xyz), item
 *        "moe/（14个算子）": top-k gating, expert scoring, token-to-expert
 *        mapping, fused expand/reduce, tensor-parallel mask; 256 experts with
 *        8 active per token (DeepSeek-V3).
 *   [P2] "剛剛，DeepSeek開始頻繁更新：Tile Kernels、DeepEP V2" (yhxrc.cn),
 *        feature list (gating, MoE routing, per-token FP8 quantisation) and
 *        section "性能表現" (8K tokens, hidden 7168, top-8, FP8 dispatch,
 *        BF16 combine).
 *   [P5] "DeepSeek 的 GPU 内核帝国：从 TileLang DSL 到 Engram 条件记忆…"
 *        (zhichai.net), section "第三层：TileKernels", subsection
 *        "MoE TopK 门控" listing: per token, num_topk rounds of
 *        (max, argmax with a min-index reducer), winner masked to -inf,
 *        winners stored in round order; unused lanes padded with -inf.
 *   DeepSeek-V3 gating as used for the DeepSeek-V3-shaped workload: sigmoid
 *        scores, a per-expert bias used for selection only, group score =
 *        sum of the group's top-2 biased scores, keep the top-4 of 8 groups,
 *        top-8 experts among them, weights = unbiased scores normalised and
 *        scaled by 2.5.
 *   OCP 8-bit Floating Point Specification (OFP8): the E4M3 format (bias 7,
 *        largest finite 448, subnormals m*2^-9, S.1111.111 = NaN, no Inf).
 *
 * Precision: the pages fix none.  Weights and the combine are evaluated in
 * fp64.  Where floating point decides an integer -- the expert selection and
 * the FP8 codes -- the decision is taken in fp32, the kernels' precision:
 *   - selection keys use the fp32 sigmoid pinned below (orc_sigmoid_f32);
 *   - the FP8 quotient is the IEEE fp32 quotient x/scale;
 *   - the stand-in expert output is computed in fp32 before its bf16 rounding.
 * Compile with -O2 -ffp-contract=off and without -ffast-math so that every
 * fp32 operation below is one IEEE-rounded operation.
 *
 * Pins (tests/test_oracle_*.py): every function here is checked against
 * something other than itself -- brute force on tiny inputs, torch library
 * routines (stable sort, bincount, cumsum, float8/bfloat16 casts), fp64/exact
 * rational arithmetic, closed forms and invariants.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* bit views                                                                 */
/* ------------------------------------------------------------------------ */
static float f32_of_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t bits_of_f32(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* A bf16 value is the upper half of an fp32 pattern, so widening is exact. */
float orc_bf16_to_f32(uint16_t h) { return f32_of_bits((uint32_t)h << 16); }

/* ------------------------------------------------------------------------ */
/* bf16 rounding: nearest bf16 to a real number, ties to even significand,   */
/* IEEE overflow to infinity.  bf16 = 1 sign, 8 exponent, 7 stored bits.     */
/* ------------------------------------------------------------------------ */
uint16_t orc_bf16_from_f64(double v)
{
    if (isnan(v)) return 0x7FC0;
    const uint16_t sign = signbit(v) ? 0x8000u : 0u;
    const double a = fabs(v);
    if (isinf(a)) return sign | 0x7F80u;
    /* spacing of bf16 values around a */
    double ulp;
    if (a < ldexp(1.0, -126)) {
        ulp = ldexp(1.0, -133);                 /* subnormal spacing */
    } else {
        int e;
        frexp(a, &e);                            /* a = m * 2^e, m in [0.5, 1) */
        ulp = ldexp(1.0, e - 8);                 /* 8 significant bits */
    }
    const double n_lo = floor(a / ulp);          /* a/ulp exact (power of two) */
    const double lo = n_lo * ulp, hi = lo + ulp; /* lo <= a < hi, both exact */
    const double d_lo = a - lo, d_hi = hi - a;
    double r;
    if (d_lo < d_hi) r = lo;
    else if (d_hi < d_lo) r = hi;
    else r = (fmod(n_lo, 2.0) == 0.0) ? lo : hi;  /* tie: even significand */
    if (r >= ldexp(1.0, 128)) return sign | 0x7F80u;  /* beyond the largest finite */
    return sign | (uint16_t)(bits_of_f32((float)r) >> 16);  /* (float)r is exact */
}

uint16_t orc_bf16_from_f32(float f) { return orc_bf16_from_f64((double)f); }

/* ------------------------------------------------------------------------ */
/* OCP E4M3 (E4M3FN): decode table and nearest-value encoder.                */
/* ------------------------------------------------------------------------ */
/* Value of the non-negative code c in 0..126 (c = 0 eeee mmm). */
static double e4m3_mag(int c)
{
    const int e = (c >> 3) & 15, m = c & 7;
    if (e == 0) return ldexp((double)m, -9);         /* subnormal: m * 2^-9 */
    return ldexp((double)(8 + m), e - 10);           /* (1 + m/8) * 2^(e-7) */
}

double orc_e4m3_to_f64(uint8_t q)
{
    const int c = q & 0x7F;
    if (c == 0x7F) return NAN;
    const double m = e4m3_mag(c);
    return (q & 0x80) ? -m : m;
}

/* Nearest E4M3 value to v, ties to the even code (= even significand), sign
 * kept (so -0 and tiny negatives give 0x80), magnitudes at or above the
 * largest finite value saturate to 448.  NaN input gives the NaN code. */
uint8_t orc_e4m3_from_f32(float v)
{
    const uint8_t sign = signbit(v) ? 0x80 : 0x00;
    if (isnan(v)) return sign | 0x7F;
    const double a = fabs((double)v);
    if (a >= 448.0) return sign | 0x7E;
    /* codes 0..126 have strictly increasing magnitudes: bisect for the
     * largest code whose magnitude is <= a */
    int lo = 0, hi = 126;          /* mag(lo) <= a < mag(hi) */
    while (hi - lo > 1) {
        const int mid = (lo + hi) / 2;
        if (e4m3_mag(mid) <= a) lo = mid; else hi = mid;
    }
    const double d_lo = a - e4m3_mag(lo), d_hi = e4m3_mag(hi) - a;  /* exact */
    int c;
    if (d_lo < d_hi) c = lo;
    else if (d_hi < d_lo) c = hi;
    else c = (lo & 1) ? hi : lo;
    return sign | (uint8_t)c;
}

/* ------------------------------------------------------------------------ */
/* Pinned fp32 exponential and sigmoid.                                      */
/*                                                                           */
/* Top-k indices must be reproducible bit for bit, and sigmoid scores of     */
/* nearby experts differ by 0-2 ulp often enough that any two different     */
/* fp32 sigmoid codes would pick different experts.  So the score is pinned  */
/* to one fixed sequence of IEEE fp32 operations:                            */
/*   Cody & Waite argument reduction (Software Manual for the Elementary     */
/*   Functions, 1980) with a two-word ln 2, then the degree-7 Taylor         */
/*   polynomial of e^r in Horner form with fused multiply-adds.              */
/*     n = rint(RN(y * RN(log2 e)))                                          */
/*     r = fma(-n, LN2_HI, y);  r = fma(-n, LN2_LO, r)                        */
/*     p = sum_{i=0..7} RN(1/i!) r^i   (Horner, highest degree first)        */
/*     E(y) = p * 2^n ;  E(y) = +inf for y > 88 ; E(y) = 0 for y < -86       */
/*   sigmoid(x) = 1 / (1 + E(-x))  with IEEE round-to-nearest division.      */
/* LN2_HI is ln 2 truncated to 16 significant bits, so n * LN2_HI is exact   */
/* for |n| <= 128; LN2_LO = RN(ln 2 - LN2_HI).  The range cuts keep p * 2^n  */
/* a normal number, so no step depends on denormal handling.                 */
/* ------------------------------------------------------------------------ */
static const float kLog2e = 0x1.715476p+0f;   /* RN(log2 e) */
static const float kLn2Hi = 0x1.62e4p-1f;     /* ln 2 truncated to 16 bits */
static const float kLn2Lo = 0x1.7f7d1cp-20f;  /* RN(ln 2 - kLn2Hi) */
static const float kInvFact[8] = {            /* RN(1/i!) */
    0x1p+0f, 0x1p+0f, 0x1p-1f, 0x1.555556p-3f,
    0x1.555556p-5f, 0x1.111112p-7f, 0x1.6c16c2p-10f, 0x1.a01a02p-13f,
};

float orc_exp_f32(float y)
{
    if (y > 88.0f) return INFINITY;
    if (y < -86.0f) return 0.0f;
    const float n = rintf(y * kLog2e);
    float r = fmaf(-n, kLn2Hi, y);
    r = fmaf(-n, kLn2Lo, r);
    float p = kInvFact[7];
    for (int i = 6; i >= 0; --i) p = fmaf(p, r, kInvFact[i]);
    return ldexpf(p, (int)n);
}

float orc_sigmoid_f32(float x) { return 1.0f / (1.0f + orc_exp_f32(-x)); }

/* ------------------------------------------------------------------------ */
/* Route: score, optional group limit, top-k selection, weights.             */
/* ------------------------------------------------------------------------ */
enum { ORC_SOFTMAX = 0, ORC_SIGMOID = 1 };

/* Selection key of one expert (fp32).
 *  softmax: the logit itself.  Softmax is strictly increasing in the logit,
 *           so the experts with the k largest softmax scores are the experts
 *           with the k largest logits; selecting on logits avoids ties that
 *           fp32 rounding of probabilities would create.
 *  sigmoid: pinned fp32 sigmoid, plus the bias when one is given (fp32 add). */
float orc_route_key(float logit, int score, const float* bias, int e)
{
    if (score == ORC_SOFTMAX) return logit;
    const float s = orc_sigmoid_f32(logit);
    return bias ? s + bias[e] : s;
}

/* Route T tokens.  Per token (one row of E logits):
 *   1. key_e for every expert;
 *   2. if n_groups > 1: E splits into n_groups groups of consecutive experts;
 *      group score = fp32 sum, largest first, of the group's group_topn
 *      largest keys; the topk_groups groups with the largest scores stay
 *      eligible (ties -> lower group); experts of the other groups are not;
 *   3. k rounds: the eligible, not yet chosen expert with the largest key is
 *      chosen, ties -> lower expert index (the listing's max + min-index
 *      argmax, winner masked before the next round); round j fills slot j;
 *   4. weights, fp64:
 *      sigmoid: s_j = 1/(1+exp(-x_j)), unbiased;
 *               renormalize: w_j = s_j / sum_i s_i * route_scale,
 *               else         w_j = s_j * route_scale;
 *      softmax: renormalize: w_j = exp(x_j - x_0) / sum_i exp(x_i - x_0)
 *                            * route_scale (softmax restricted to the k
 *                            chosen experts; x_0 is the first chosen logit),
 *               else         w_j = exp(x_j - m) / sum_e exp(x_e - m)
 *                            * route_scale over all E experts, m = max logit.
 * Returns 0, or -1 for an argument combination the definition does not cover. */
int orc_route(const float* logits, const float* bias, int T, int E, int k,
              int score, int n_groups, int topk_groups, int group_topn,
              int renormalize, double route_scale,
              int32_t* topk_idx, double* topk_w)
{
    if (T < 0 || E < 1 || k < 1 || k > E) return -1;
    if (n_groups < 1 || E % n_groups != 0) return -1;
    const int gs = E / n_groups;
    if (n_groups > 1) {
        if (topk_groups < 1 || topk_groups > n_groups) return -1;
        if (group_topn < 1 || group_topn > gs) return -1;
        if (topk_groups * gs < k) return -1;
    }
    float* key = (float*)malloc(sizeof(float) * (size_t)E);
    int* eligible = (int*)malloc(sizeof(int) * (size_t)E);
    int* taken = (int*)malloc(sizeof(int) * (size_t)E);
    float* gscore = (float*)malloc(sizeof(float) * (size_t)n_groups);
    int* gtaken = (int*)malloc(sizeof(int) * (size_t)n_groups);
    float* tmp = (float*)malloc(sizeof(float) * (size_t)gs);
    if (!key || !eligible || !taken || !gscore || !gtaken || !tmp) {
        free(key); free(eligible); free(taken); free(gscore); free(gtaken); free(tmp);
        return -1;
    }
    for (int t = 0; t < T; ++t) {
        const float* x = logits + (size_t)t * E;
        for (int e = 0; e < E; ++e) {
            key[e] = orc_route_key(x[e], score, bias, e);
            eligible[e] = 1;
            taken[e] = 0;
        }
        if (n_groups > 1) {
            for (int g = 0; g < n_groups; ++g) {
                /* group_topn largest keys of the group, by repeated max */
                for (int i = 0; i < gs; ++i) tmp[i] = key[g * gs + i];
                float sum = 0.0f;
                for (int r = 0; r < group_topn; ++r) {
                    int best = -1;
                    for (int i = 0; i < gs; ++i)
                        if (tmp[i] == tmp[i] && (best < 0 || tmp[i] > tmp[best])) best = i;
                    if (best < 0) break;
                    sum = (r == 0) ? tmp[best] : sum + tmp[best];
                    tmp[best] = NAN;           /* used */
                }
                gscore[g] = sum;
                gtaken[g] = 0;
            }
            for (int r = 0; r < topk_groups; ++r) {
                int best = -1;
                for (int g = 0; g < n_groups; ++g)
                    if (!gtaken[g] && (best < 0 || gscore[g] > gscore[best])) best = g;
                gtaken[best] = 1;
            }
            for (int e = 0; e < E; ++e) eligible[e] = gtaken[e / gs];
        }
        int32_t* idx = topk_idx + (size_t)t * k;
        for (int j = 0; j < k; ++j) {
            int best = -1;
            for (int e = 0; e < E; ++e)
                if (eligible[e] && !taken[e] && (best < 0 || key[e] > key[best])) best = e;
            taken[best] = 1;
            idx[j] = best;
        }
        double* w = topk_w + (size_t)t * k;
        if (score == ORC_SIGMOID) {
            double s_sum = 0.0;
            for (int j = 0; j < k; ++j) {
                w[j] = 1.0 / (1.0 + exp(-(double)x[idx[j]]));
                s_sum += w[j];
            }
            for (int j = 0; j < k; ++j)
                w[j] = renormalize ? w[j] / s_sum * route_scale : w[j] * route_scale;
        } else if (renormalize) {
            const double x0 = (double)x[idx[0]];
            double z = 0.0;
            for (int j = 0; j < k; ++j) { w[j] = exp((double)x[idx[j]] - x0); z += w[j]; }
            for (int j = 0; j < k; ++j) w[j] = w[j] / z * route_scale;
        } else {
            double m = (double)x[0];
            for (int e = 1; e < E; ++e) if ((double)x[e] > m) m = (double)x[e];
            double z = 0.0;
            for (int e = 0; e < E; ++e) z += exp((double)x[e] - m);
            for (int j = 0; j < k; ++j) w[j] = exp((double)x[idx[j]] - m) / z * route_scale;
        }
    }
    free(key); free(eligible); free(taken); free(gscore); free(gtaken); free(tmp);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Load-balance statistics and loss over one batch of T tokens (the          */
/* load-balancing loss computation of TileKernels' moe/ module), in the      */
/* form DeepSeek-V3 trains with:                                             */
/*   count_e = number of routes (t, j) with topk_idx[t,j] = e                 */
/*   f_e     = E / (k T) * count_e            (1 for a perfectly even load)   */
/*   p_{t,e} = normalised score of e for token t: sigmoid scores divided by    */
/*             their sum over all E experts, or the softmax probabilities     */
/*   P_e     = (1/T) sum_t p_{t,e}                                            */
/*   loss    = sum_e f_e P_e                   (the caller applies its weight)*/
/* Sigmoid scores are the pinned fp32 orc_sigmoid_f32 (the same scores the   */
/* route ranks on); everything after them is fp64.  Softmax is fp64.         */
/* ------------------------------------------------------------------------ */
int orc_balance_loss(const float* logits, int T, int E, int k, int score,
                     const int32_t* topk_idx, double* f, double* P, double* loss)
{
    if (T < 1 || E < 1 || k < 1) return -1;
    double* p = (double*)malloc(sizeof(double) * (size_t)E);
    int64_t* count = (int64_t*)calloc((size_t)E, sizeof(int64_t));
    if (!p || !count) { free(p); free(count); return -1; }
    for (int e = 0; e < E; ++e) P[e] = 0.0;
    for (int t = 0; t < T; ++t) {
        const float* x = logits + (size_t)t * E;
        double z = 0.0;
        if (score == ORC_SIGMOID) {
            for (int e = 0; e < E; ++e) { p[e] = (double)orc_sigmoid_f32(x[e]); z += p[e]; }
        } else {
            double m = (double)x[0];
            for (int e = 1; e < E; ++e) if ((double)x[e] > m) m = (double)x[e];
            for (int e = 0; e < E; ++e) { p[e] = exp((double)x[e] - m); z += p[e]; }
        }
        for (int e = 0; e < E; ++e) P[e] += p[e] / z;
        for (int j = 0; j < k; ++j) {
            const int32_t e = topk_idx[(size_t)t * k + j];
            if (e >= 0 && e < E) count[e] += 1;
        }
    }
    double l = 0.0;
    for (int e = 0; e < E; ++e) {
        P[e] /= (double)T;
        f[e] = (double)E / ((double)k * (double)T) * (double)count[e];
        l += f[e] * P[e];
    }
    *loss = l;
    free(p); free(count);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Map: local mask, per-expert counts, exclusive offsets, stable positions.  */
/*                                                                           */
/* A route (t, j) is local when lo <= topk_idx[t,j] < hi (the mask of the    */
/* experts one expert-parallel rank owns; [0, E) keeps every route).  A      */
/* repeated expert id within one token's row is routed only at its first     */
/* occurrence; later repeats are treated like masked routes.                 */
/*   counts[e-lo]  = number of local routes to e                             */
/*   offsets       = exclusive prefix sum of counts; offsets[hi-lo] = R      */
/*   pos[t,j]      = offsets[e-lo] + (number of earlier tokens t' < t routed  */
/*                   to e): expert-contiguous rows in token order (stable);  */
/*                   -1 for a route that is not local                         */
/*   row_src[pos]  = t  (the token each expanded row came from)              */
/* Routes that are not local keep their weights; nothing is renormalised, so */
/* partial combines of different ranks add up to the full combine.           */
/* ------------------------------------------------------------------------ */
int orc_map(const int32_t* topk_idx, int T, int k, int E, int lo, int hi,
            int32_t* counts, int32_t* offsets, int32_t* pos, int32_t* row_src)
{
    if (T < 0 || k < 1 || E < 1 || lo < 0 || hi > E || lo >= hi) return -1;
    const int nl = hi - lo;
    for (int i = 0; i < nl; ++i) counts[i] = 0;
    for (int t = 0; t < T; ++t)
        for (int j = 0; j < k; ++j) {
            const int32_t e = topk_idx[(size_t)t * k + j];
            int first = 1;
            for (int jj = 0; jj < j; ++jj)
                if (topk_idx[(size_t)t * k + jj] == e) first = 0;
            if (first && e >= lo && e < hi) counts[e - lo] += 1;
        }
    offsets[0] = 0;
    for (int i = 0; i < nl; ++i) offsets[i + 1] = offsets[i] + counts[i];
    int32_t* cursor = (int32_t*)calloc((size_t)nl, sizeof(int32_t));
    if (!cursor) return -1;
    for (int t = 0; t < T; ++t)
        for (int j = 0; j < k; ++j) {
            const int32_t e = topk_idx[(size_t)t * k + j];
            int first = 1;
            for (int jj = 0; jj < j; ++jj)
                if (topk_idx[(size_t)t * k + jj] == e) first = 0;
            int32_t p = -1;
            if (first && e >= lo && e < hi) {
                p = offsets[e - lo] + cursor[e - lo];
                cursor[e - lo] += 1;
                if (row_src) row_src[p] = t;
            }
            pos[(size_t)t * k + j] = p;
        }
    free(cursor);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Map with expert segments aligned for a grouped GEMM: expert e's rows      */
/* start at a multiple of `align` and its segment holds                       */
/* roundup(counts[e], align) rows:                                           */
/*   offsets[0] = 0, offsets[e+1] = offsets[e] + roundup(counts[e], align)   */
/*   pos[t,j]   = offsets[e] + (number of earlier tokens routed to e)         */
/*   row_src[r] = t for the rows routes land on, -1 for padding rows, for    */
/*                r < offsets[hi-lo]                                          */
/* align = 1 is orc_map.                                                     */
/* ------------------------------------------------------------------------ */
int orc_map_aligned(const int32_t* topk_idx, int T, int k, int E, int lo, int hi, int align,
                    int32_t* counts, int32_t* offsets, int32_t* pos, int32_t* row_src)
{
    if (T < 0 || k < 1 || E < 1 || lo < 0 || hi > E || lo >= hi || align < 1) return -1;
    const int nl = hi - lo;
    for (int i = 0; i < nl; ++i) counts[i] = 0;
    for (int t = 0; t < T; ++t)
        for (int j = 0; j < k; ++j) {
            const int32_t e = topk_idx[(size_t)t * k + j];
            int first = 1;
            for (int jj = 0; jj < j; ++jj)
                if (topk_idx[(size_t)t * k + jj] == e) first = 0;
            if (first && e >= lo && e < hi) counts[e - lo] += 1;
        }
    offsets[0] = 0;
    for (int i = 0; i < nl; ++i) {
        const int32_t padded = ((counts[i] + align - 1) / align) * align;
        offsets[i + 1] = offsets[i] + padded;
    }
    if (row_src)
        for (int32_t r = 0; r < offsets[nl]; ++r) row_src[r] = -1;
    int32_t* cursor = (int32_t*)calloc((size_t)nl, sizeof(int32_t));
    if (!cursor) return -1;
    for (int t = 0; t < T; ++t)
        for (int j = 0; j < k; ++j) {
            const int32_t e = topk_idx[(size_t)t * k + j];
            int first = 1;
            for (int jj = 0; jj < j; ++jj)
                if (topk_idx[(size_t)t * k + jj] == e) first = 0;
            int32_t p = -1;
            if (first && e >= lo && e < hi) {
                p = offsets[e - lo] + cursor[e - lo];
                cursor[e - lo] += 1;
                if (row_src) row_src[p] = t;
            }
            pos[(size_t)t * k + j] = p;
        }
    free(cursor);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Per-token 1x128 FP8 quantisation of one row of H bf16 values.             */
/* For each block b of 128 consecutive columns:                              */
/*   amax  = max |x| over the block (bf16 -> fp32 is exact), at least 1e-4f   */
/*   scale = RN32(amax / 448)                                                */
/*   q_c   = E4M3(RN32(x_c / scale))                                         */
/* H must be a multiple of 128.                                              */
/* ------------------------------------------------------------------------ */
void orc_quant_row(const uint16_t* x, int H, uint8_t* q, float* scales)
{
    for (int b = 0; b < H / 128; ++b) {
        float amax = 0.0f;
        for (int c = b * 128; c < b * 128 + 128; ++c) {
            const float a = fabsf(orc_bf16_to_f32(x[c]));
            if (a > amax) amax = a;
        }
        if (amax < 1e-4f) amax = 1e-4f;
        const float scale = amax / 448.0f;
        scales[b] = scale;
        for (int c = b * 128; c < b * 128 + 128; ++c)
            q[c] = orc_e4m3_from_f32(orc_bf16_to_f32(x[c]) / scale);
    }
}

/* ------------------------------------------------------------------------ */
/* Expand: each local route (t, j) gets row pos[t,j] = copy of token t.       */
/* mode 0: bf16 rows, bitwise copies.                                        */
/* mode 1: FP8 rows: token t is quantised once (orc_quant_row) and the same  */
/*         bytes and block scales are written to every one of its rows.      */
/* Rows with pos < 0 or pos >= rows_capacity are skipped.                    */
/* ------------------------------------------------------------------------ */
int orc_expand(const uint16_t* x, int T, int H, int k, const int32_t* pos, int mode,
               int64_t rows_capacity, void* out, float* scales)
{
    if (T < 0 || H < 1 || k < 1) return -1;
    if (mode == 1 && H % 128 != 0) return -1;
    uint8_t* q = (uint8_t*)malloc((size_t)H);
    float* sc = (float*)malloc(sizeof(float) * (size_t)(H / 128 + 1));
    if (!q || !sc) { free(q); free(sc); return -1; }
    const int nb = H / 128;
    for (int t = 0; t < T; ++t) {
        const uint16_t* xt = x + (size_t)t * H;
        if (mode == 1) orc_quant_row(xt, H, q, sc);
        for (int j = 0; j < k; ++j) {
            const int64_t r = pos[(size_t)t * k + j];
            if (r < 0 || r >= rows_capacity) continue;
            if (mode == 0) {
                memcpy((uint16_t*)out + (size_t)r * H, xt, sizeof(uint16_t) * (size_t)H);
            } else {
                memcpy((uint8_t*)out + (size_t)r * H, q, (size_t)H);
                memcpy(scales + (size_t)r * nb, sc, sizeof(float) * (size_t)nb);
            }
        }
    }
    free(q); free(sc);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Stand-in expert (end-to-end harness): dequantise and scale.               */
/*   y[r,c] = bf16(RN32(RN32(dec(q[r,c]) * scales[r, c/128]) * mult))        */
/* computed in fp32, the precision of the device harness kernel.             */
/* ------------------------------------------------------------------------ */
void orc_standin(const uint8_t* xq, const float* scales, int64_t rows, int H, float mult,
                 uint16_t* y)
{
    const int nb = H / 128;
    for (int64_t r = 0; r < rows; ++r)
        for (int c = 0; c < H; ++c) {
            const float d = (float)orc_e4m3_to_f64(xq[(size_t)r * H + c]);  /* exact */
            const float v = d * scales[(size_t)r * nb + c / 128];
            y[(size_t)r * H + c] = orc_bf16_from_f32(v * mult);
        }
}

/* ------------------------------------------------------------------------ */
/* Reduce (combine): out[t] = bf16( sum_j w[t,j] * y[pos[t,j]] ) over the     */
/* routes with 0 <= pos < rows, summed in slot order j = 0..k-1 in fp64 and   */
/* rounded once to bf16.  A token with no such route gets +0.                */
/* ------------------------------------------------------------------------ */
int orc_reduce(const uint16_t* y, int64_t rows, const int32_t* pos, const float* w,
               int T, int k, int H, uint16_t* out)
{
    if (T < 0 || k < 1 || H < 1) return -1;
    double* acc = (double*)malloc(sizeof(double) * (size_t)H);
    if (!acc) return -1;
    for (int t = 0; t < T; ++t) {
        for (int c = 0; c < H; ++c) acc[c] = 0.0;
        for (int j = 0; j < k; ++j) {
            const int64_t r = pos[(size_t)t * k + j];
            if (r < 0 || r >= rows) continue;
            const double wj = (double)w[(size_t)t * k + j];
            const uint16_t* yr = y + (size_t)r * H;
            for (int c = 0; c < H; ++c) acc[c] += wj * (double)orc_bf16_to_f32(yr[c]);
        }
        for (int c = 0; c < H; ++c) out[(size_t)t * H + c] = orc_bf16_from_f64(acc[c]);
    }
    free(acc);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Per-token 1x128 FP8 quantisation of one row of n fp32 values (the same    */
/* codec as orc_quant_row, on fp32 input).  n must be a multiple of 128.     */
/*   amax  = max |a| over the block, at least 1e-4f                          */
/*   scale = RN32(amax / 448);  q_c = E4M3(RN32(a_c / scale))                */
/* ------------------------------------------------------------------------ */
void orc_quant_f32_row(const float* a, int n, uint8_t* q, float* scales)
{
    for (int b = 0; b < n / 128; ++b) {
        float amax = 0.0f;
        for (int c = b * 128; c < b * 128 + 128; ++c) {
            const float m = fabsf(a[c]);
            if (m > amax) amax = m;
        }
        if (amax < 1e-4f) amax = 1e-4f;
        const float scale = amax / 448.0f;
        scales[b] = scale;
        for (int c = b * 128; c < b * 128 + 128; ++c) q[c] = orc_e4m3_from_f32(a[c] / scale);
    }
}

/* ------------------------------------------------------------------------ */
/* Weight of each expanded row: row_w[pos[t,j]] = w[t,j] for every route     */
/* with 0 <= pos < rows; rows no route points at keep 0.                     */
/* ------------------------------------------------------------------------ */
void orc_row_weights(const int32_t* pos, const float* w, int T, int k, int64_t rows, float* row_w)
{
    for (int64_t r = 0; r < rows; ++r) row_w[r] = 0.0f;
    for (int t = 0; t < T; ++t)
        for (int j = 0; j < k; ++j) {
            const int64_t r = pos[(size_t)t * k + j];
            if (r >= 0 && r < rows) row_w[r] = w[(size_t)t * k + j];
        }
}

/* ------------------------------------------------------------------------ */
/* SwiGLU activation fused with per-token 1x128 FP8 quantisation (the        */
/* SwiGLU and FP8 quantisation fusion of TileKernels' quant/ module), with   */
/* an optional per-row weight (the routing weight of the expanded row).      */
/* Row r of h holds 2*I bf16 values: gate g = h[r, 0..I), up u = h[r, I..2I).*/
/* In fp32, one IEEE operation per step:                                     */
/*   s = sigmoid(g)  (the pinned orc_sigmoid_f32)                            */
/*   a = RN(RN(g * s) * u);  weighted: a = RN(a * row_w[r])                  */
/* then a is quantised with orc_quant_f32_row into out[r] (I codes) and      */
/* scales[r] (I/128).  I must be a multiple of 128.                          */
/* ------------------------------------------------------------------------ */
int orc_swiglu_quant(const uint16_t* h, int64_t rows, int I, const float* row_w, uint8_t* out,
                     float* scales)
{
    if (rows < 0 || I < 128 || I % 128 != 0) return -1;
    float* a = (float*)malloc(sizeof(float) * (size_t)I);
    if (!a) return -1;
    for (int64_t r = 0; r < rows; ++r) {
        const uint16_t* hr = h + (size_t)r * 2 * I;
        for (int c = 0; c < I; ++c) {
            const float g = orc_bf16_to_f32(hr[c]);
            const float u = orc_bf16_to_f32(hr[I + c]);
            const float s = orc_sigmoid_f32(g);
            float v = (g * s) * u;
            if (row_w) v = v * row_w[r];
            a[c] = v;
        }
        orc_quant_f32_row(a, I, out + (size_t)r * I, scales + (size_t)r * (I / 128));
    }
    free(a);
    return 0;
}

/* The fp32 activations alone (before quantisation), for the pins. */
int orc_swiglu_f32(const uint16_t* h, int64_t rows, int I, const float* row_w, float* a)
{
    if (rows < 0 || I < 1) return -1;
    for (int64_t r = 0; r < rows; ++r) {
        const uint16_t* hr = h + (size_t)r * 2 * I;
        for (int c = 0; c < I; ++c) {
            const float g = orc_bf16_to_f32(hr[c]);
            const float u = orc_bf16_to_f32(hr[I + c]);
            float v = (g * orc_sigmoid_f32(g)) * u;
            if (row_w) v = v * row_w[r];
            a[(size_t)r * I + c] = v;
        }
    }
    return 0;
}

/* The transposed half of the SwiGLU + FP8 + transpose fusion: the same      */
/* activations a (rows, I) quantised along the other axis, i.e. a^T (I, rows)*/
/* with 1x128 blocks along its rows (128 consecutive tokens of one channel):*/
/*   out_t[c, r] = E4M3(RN32(a[r, c] / scale_t[c, r/128])),                  */
/*   scale_t[c, b] = RN32(max(max_{r in block b} |a[r, c]|, 1e-4) / 448).    */
/* rows must be a multiple of 128.  out_t (I, rows), scales_t (I, rows/128).  */
int orc_swiglu_quant_t(const uint16_t* h, int64_t rows, int I, const float* row_w,
                       uint8_t* out_t, float* scales_t)
{
    if (rows < 0 || rows % 128 != 0 || I < 1) return -1;
    float* a = (float*)malloc(sizeof(float) * (size_t)rows * (size_t)I);
    float* col = (float*)malloc(sizeof(float) * (size_t)(rows > 0 ? rows : 1));
    if (!a || !col) { free(a); free(col); return -1; }
    orc_swiglu_f32(h, rows, I, row_w, a);
    for (int c = 0; c < I; ++c) {
        for (int64_t r = 0; r < rows; ++r) col[r] = a[(size_t)r * I + c];
        orc_quant_f32_row(col, (int)rows, out_t + (size_t)c * rows, scales_t + (size_t)c * (rows / 128));
    }
    free(a); free(col);
    return 0;
}


/* ------------------------------------------------------------------------ */
/* Other granularities of the quantisation codec (TileKernels' quant/ module */
/* lists per-token, per-block and per-channel FP8 and FP4).  Inputs are bf16 */
/* matrices (rows, cols), row-major.                                          */
/* ------------------------------------------------------------------------ */

/* Power-of-two block scale for FP8: the smallest 2^e with 448 * 2^e >= amax */
/* (amax clamped >= 1e-4), found from amax's binary exponent: with            */
/* amax = m * 2^x, m in [0.5, 1) and 448 = 0.875 * 2^9,                       */
/* amax / 448 <= 2^(x-9) exactly when m <= 0.875.                             */
float orc_pow2_scale_e4m3(float amax)
{
    if (amax < 1e-4f) amax = 1e-4f;
    int x;
    const float m = frexpf(amax, &x);
    return ldexpf(1.0f, m <= 0.875f ? x - 9 : x - 8);
}

/* Per-token 1x128 FP8 of a (rows, cols) matrix, cols % 128 == 0; scales     */
/* (rows, cols/128).  pow2 = 0: scale = RN32(amax/448) (orc_quant_row);       */
/* pow2 = 1: scale = orc_pow2_scale_e4m3(amax), q = E4M3(x * (1/scale))       */
/* (exact: a power of two).                                                   */
void orc_quant_1x128(const uint16_t* x, int64_t rows, int cols, int pow2, uint8_t* q,
                     float* scales)
{
    for (int64_t r = 0; r < rows; ++r) {
        const uint16_t* xr = x + (size_t)r * cols;
        uint8_t* qr = q + (size_t)r * cols;
        float* sr = scales + (size_t)r * (cols / 128);
        if (!pow2) { orc_quant_row(xr, cols, qr, sr); continue; }
        for (int b = 0; b < cols / 128; ++b) {
            float amax = 0.0f;
            for (int c = b * 128; c < b * 128 + 128; ++c) {
                const float a = fabsf(orc_bf16_to_f32(xr[c]));
                if (a > amax) amax = a;
            }
            const float scale = orc_pow2_scale_e4m3(amax);
            sr[b] = scale;
            for (int c = b * 128; c < b * 128 + 128; ++c)
                qr[c] = orc_e4m3_from_f32(orc_bf16_to_f32(xr[c]) / scale);
        }
    }
}

/* Per-block 128x128 FP8 (weights): one scale per tile of 128 rows x 128    */
/* columns (the last tile row may be shorter), scale = RN32(max(amax,1e-4)/448)*/
/* q = E4M3(RN32(x/scale)).  cols % 128 == 0; scales (ceil(rows/128), cols/128)*/
void orc_quant_128x128(const uint16_t* x, int64_t rows, int cols, uint8_t* q, float* scales)
{
    const int64_t tr = (rows + 127) / 128;
    for (int64_t bi = 0; bi < tr; ++bi)
        for (int bj = 0; bj < cols / 128; ++bj) {
            const int64_t r1 = (bi + 1) * 128 < rows ? (bi + 1) * 128 : rows;
            float amax = 0.0f;
            for (int64_t r = bi * 128; r < r1; ++r)
                for (int c = bj * 128; c < bj * 128 + 128; ++c) {
                    const float a = fabsf(orc_bf16_to_f32(x[(size_t)r * cols + c]));
                    if (a > amax) amax = a;
                }
            if (amax < 1e-4f) amax = 1e-4f;
            const float scale = amax / 448.0f;
            scales[(size_t)bi * (cols / 128) + bj] = scale;
            for (int64_t r = bi * 128; r < r1; ++r)
                for (int c = bj * 128; c < bj * 128 + 128; ++c)
                    q[(size_t)r * cols + c] = orc_e4m3_from_f32(orc_bf16_to_f32(x[(size_t)r * cols + c]) / scale);
        }
}

/* Per-channel FP8: one scale per column over all rows,                      */
/* scale = RN32(max(amax,1e-4)/448), q = E4M3(RN32(x/scale)); scales (cols).  */
void orc_quant_per_channel(const uint16_t* x, int64_t rows, int cols, uint8_t* q, float* scales)
{
    for (int c = 0; c < cols; ++c) {
        float amax = 0.0f;
        for (int64_t r = 0; r < rows; ++r) {
            const float a = fabsf(orc_bf16_to_f32(x[(size_t)r * cols + c]));
            if (a > amax) amax = a;
        }
        if (amax < 1e-4f) amax = 1e-4f;
        scales[c] = amax / 448.0f;
    }
    for (int64_t r = 0; r < rows; ++r)
        for (int c = 0; c < cols; ++c)
            q[(size_t)r * cols + c] = orc_e4m3_from_f32(orc_bf16_to_f32(x[(size_t)r * cols + c]) / scales[c]);
}

/* FP4 E2M1 (OCP MX element format): sign, 2 exponent bits (bias 1), 1       */
/* mantissa bit; magnitudes of codes 0..7 = 0, 0.5, 1, 1.5, 2, 3, 4, 6.       */
double orc_e2m1_to_f64(uint8_t c)
{
    static const double mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
    const double m = mag[c & 7];
    return (c & 8) ? -m : m;
}

/* Nearest E2M1 value, ties to the even code (= even mantissa bit), sign kept,*/
/* magnitudes beyond 6 saturate to 6.  NaN gives +-6 (no NaN code exists).   */
uint8_t orc_e2m1_from_f32(float v)
{
    const uint8_t sign = signbit(v) ? 8 : 0;
    const double a = fabs((double)v);
    if (isnan(v) || a >= 6.0) return sign | 7;
    int best = 0;
    for (int c = 1; c < 8; ++c) {
        const double dc = fabs(a - orc_e2m1_to_f64((uint8_t)c));
        const double db = fabs(a - orc_e2m1_to_f64((uint8_t)best));
        if (dc < db || (dc == db && (c & 1) == 0)) best = c;
    }
    return sign | (uint8_t)best;
}

/* FP4 with 1x32 blocks and power-of-two scales (OCP MX-style): per block,   */
/* amax clamped >= 1e-4, X = 2^(floor(log2 amax) - 2) (2 = the largest E2M1  */
/* exponent), codes E2M1(x / X) (exact division), saturating.  cols % 32 == 0;*/
/* codes two per byte, column 2i in the low nibble; q (rows, cols/2),        */
/* scales (rows, cols/32) as fp32 powers of two.                              */
void orc_quant_fp4_1x32(const uint16_t* x, int64_t rows, int cols, uint8_t* q, float* scales)
{
    for (int64_t r = 0; r < rows; ++r)
        for (int b = 0; b < cols / 32; ++b) {
            const uint16_t* xb = x + (size_t)r * cols + (size_t)b * 32;
            float amax = 0.0f;
            for (int c = 0; c < 32; ++c) {
                const float a = fabsf(orc_bf16_to_f32(xb[c]));
                if (a > amax) amax = a;
            }
            if (amax < 1e-4f) amax = 1e-4f;
            int e;
            frexpf(amax, &e);                        /* amax = m * 2^e, m in [0.5, 1) */
            const float scale = ldexpf(1.0f, (e - 1) - 2);
            scales[(size_t)r * (cols / 32) + b] = scale;
            for (int c = 0; c < 32; c += 2) {
                const uint8_t lo = orc_e2m1_from_f32(orc_bf16_to_f32(xb[c]) / scale);
                const uint8_t hi = orc_e2m1_from_f32(orc_bf16_to_f32(xb[c + 1]) / scale);
                q[(size_t)r * (cols / 2) + (size_t)b * 16 + c / 2] = (uint8_t)(lo | (hi << 4));
            }
        }
}

void orc_e2m1_from_f32_n(const float* v, int64_t n, uint8_t* q)
{
    for (int64_t i = 0; i < n; ++i) q[i] = orc_e2m1_from_f32(v[i]);
}

/* Element-wise helpers over arrays, for the codec pins. */
void orc_e4m3_from_f32_n(const float* v, int64_t n, uint8_t* q)
{
    for (int64_t i = 0; i < n; ++i) q[i] = orc_e4m3_from_f32(v[i]);
}
void orc_bf16_from_f32_n(const float* v, int64_t n, uint16_t* h)
{
    for (int64_t i = 0; i < n; ++i) h[i] = orc_bf16_from_f32(v[i]);
}
void orc_bf16_from_f64_n(const double* v, int64_t n, uint16_t* h)
{
    for (int64_t i = 0; i < n; ++i) h[i] = orc_bf16_from_f64(v[i]);
}
void orc_sigmoid_f32_n(const float* x, int64_t n, float* s)
{
    for (int64_t i = 0; i < n; ++i) s[i] = orc_sigmoid_f32(x[i]);
}
void orc_exp_f32_n(const float* x, int64_t n, float* s)
{
    for (int64_t i = 0; i < n; ++i) s[i] = orc_exp_f32(x[i]);
}
