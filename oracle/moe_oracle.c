/*
 * moe_oracle.c -- reference definition of one MoE layer's forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke check and the benchmark's
 * CPU-baseline leg may load this library.  The product path never calls it and
 * shares no code, header, table or constant with it.
 *
 * What it computes is the plain layer, written out loop by loop in fp64:
 *   logits  = x . W_r^T                          (router; fp64 sum, one rounding to fp32)
 *   idx     = the k largest logits per token     (ties -> lower expert id)
 *   gates   = softmax of the selected logits     (renormalised over the k; or the
 *                                                 full-softmax probabilities if renorm=0)
 *   perm    = stable counting sort of the T*k routed rows by expert
 *   out[t]  = sum_j gates[t,j] * FFN_{idx[t,j]}(x[t]),  j ascending,
 *   FFN_e(v) = W_down[e] . (silu(W_gate[e] . v) * (W_up[e] . v)),  silu(a) = a / (1 + exp(-a))
 *
 * The expert cache and the q* split never enter here: the method is exact,
 * so placement of an expert (GPU slot, streamed copy, or host CPU) changes no
 * result.  Sources: FreeToken paper explainer (ta-paperlens), section "Design:
 * two-tier expert memory" (GPU memory affects performance only); techfeed
 * summary of "Meet FreeToken" (MarkTechPost), section "Bandwidth-adaptive
 * execution (q* policy)" (partial sums added at the end, no router change and
 * no approximation).  Routing k of E experts per token: explainer section
 * "MoE opens one door and closes another".  Softmax/top-k gating, SwiGLU and
 * the counting-sort permutation are not on the pages; they are the standard
 * definitions, with the readings listed at each function.
 *
 * Weight encodings: fp32, bf16 (upper 16 bits of an fp32), and MXFP4 (OCP
 * Microscaling Formats v1.0: E2M1 elements, E8M0 scale per 32 consecutive
 * elements along the reduction dimension, element 2i in the low nibble of
 * byte i).  Every encoding is decoded exactly to fp64.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -shared -fPIC (no fast-math).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_MXFP4 = 2 };

/* ---- exact decoding of stored values --------------------------------------- */

static double bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* E2M1: sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0; exponent 0 is subnormal. */
double orc_e2m1(unsigned nib)
{
    unsigned s = (nib >> 3) & 1u, e = (nib >> 1) & 3u, m = nib & 1u;
    double mag = (e == 0) ? 0.5 * (double)m : ldexp(1.0 + 0.5 * (double)m, (int)e - 1);
    return s ? -mag : mag;
}

/* E8M0: 2^(s - 127); s = 255 is NaN. */
double orc_e8m0(uint8_t s)
{
    return s == 255 ? NAN : ldexp(1.0, (int)s - 127);
}

/* Element (r, c) of a weight matrix with `cols` columns (the reduction dim). */
double orc_weight(int dtype, const void *w, const uint8_t *scales, long r, long c, long cols)
{
    if (dtype == ORC_F32)
        return (double)((const float *)w)[r * cols + c];
    if (dtype == ORC_BF16)
        return bf16_to_double(((const uint16_t *)w)[r * cols + c]);
    /* MXFP4 */
    uint8_t byte = ((const uint8_t *)w)[r * (cols / 2) + c / 2];
    unsigned nib = (c & 1) ? (unsigned)(byte >> 4) : (unsigned)(byte & 15u);
    return orc_e2m1(nib) * orc_e8m0(scales[r * (cols / 32) + c / 32]);
}

/* The same MXFP4 matrix [rows][cols] written as bf16 bit patterns: element
 * (r, c) is orc_weight's exact value of it, stored in bf16.  An E2M1 value
 * (at most two significant bits) times 2^(s - 127) fits bf16 exactly for
 * every scale byte s up to 252 (bf16 has fp32's exponent range); the return
 * value counts the elements that do not (they are stored rounded), so a
 * caller that gets 0 holds the very values the MXFP4 path computes with and
 * can run the bf16 path in their place, fp64 for fp64, at bf16 decoding cost. */
long orc_mxfp4_to_bf16(const uint8_t *w, const uint8_t *scales, long rows, long cols, uint16_t *out)
{
    long bad = 0;
#pragma omp parallel for schedule(static) reduction(+ : bad)
    for (long r = 0; r < rows; ++r)
        for (long c = 0; c < cols; ++c) {
            double v = orc_weight(ORC_MXFP4, w, scales, r, c, cols);
            float f = (float)v;
            uint32_t u;
            memcpy(&u, &f, sizeof u);
            if (!isnan(v) && ((double)f != v || (u & 0xffffu) != 0))
                ++bad;
            out[r * cols + c] = (uint16_t)(u >> 16);
        }
    return bad;
}

static double act(int a_dtype, const void *x, long r, long c, long cols)
{
    if (a_dtype == ORC_F32)
        return (double)((const float *)x)[r * cols + c];
    return bf16_to_double(((const uint16_t *)x)[r * cols + c]);
}

/* ---- router ---------------------------------------------------------------- */

/* logits[t][e] = fp32( sum_i x[t][i] * W_r[e][i] ), summed in fp64.
 * Products of two bf16 or two fp32 values are exact in fp64; the one rounding
 * to fp32 is the precision the top-k decision is taken in. */
void orc_logits(int a_dtype, const void *x, const void *wr, int T, int d, int E, float *logits)
{
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t)
        for (int e = 0; e < E; ++e) {
            double s = 0.0;
            for (int i = 0; i < d; ++i)
                s += act(a_dtype, x, t, i, d) * act(a_dtype, wr, e, i, d);
            logits[(long)t * E + e] = (float)s;
        }
}

/* A logit as routing reads it: NaN is taken as -infinity (in the order and in
 * the softmax); -0 and +0 compare equal. */
static double route_val(float v)
{
    return isnan(v) ? -INFINITY : (double)v;
}

/* Top-k and gates for every token.
 * Selection: k rounds, each taking the largest logit not yet taken; a strict
 * ">" comparison in ascending id order keeps the lower expert id on ties.
 * Gates: renorm=1 -> softmax over the k selected logits;
 *        renorm=0 -> softmax over all E logits, read at the selected ones.
 * Both use the largest logit as the shift, which does not change the value. */
void orc_route(const float *logits, int T, int E, int k, int renorm, int32_t *idx, double *gates)
{
    for (int t = 0; t < T; ++t) {
        const float *l = logits + (long)t * E;
        char *taken = (char *)calloc((size_t)E, 1);
        for (int j = 0; j < k; ++j) {
            int best = -1;
            for (int e = 0; e < E; ++e)
                if (!taken[e] && (best < 0 || route_val(l[e]) > route_val(l[best])))
                    best = e;
            taken[best] = 1;
            idx[(long)t * k + j] = best;
        }
        free(taken);
        double mx = route_val(l[idx[(long)t * k]]);
        double denom = 0.0;
        if (renorm)
            for (int j = 0; j < k; ++j)
                denom += exp(route_val(l[idx[(long)t * k + j]]) - mx);
        else
            for (int e = 0; e < E; ++e)
                denom += exp(route_val(l[e]) - mx);
        for (int j = 0; j < k; ++j)
            gates[(long)t * k + j] = exp(route_val(l[idx[(long)t * k + j]]) - mx) / denom;
    }
}

/* Stable counting sort of the R = T*k routed rows by expert.
 * Row f = t*k + j is routed to idx[f].  counts[e] = number of rows routed to e;
 * offsets = exclusive prefix sum (E+1 entries); perm lists the rows of expert 0,
 * then of expert 1, ..., each group in ascending f; pos is the inverse of perm. */
void orc_permute(const int32_t *idx, int T, int k, int E, int32_t *counts, int32_t *offsets,
                 int32_t *perm, int32_t *pos)
{
    long R = (long)T * k;
    for (int e = 0; e < E; ++e)
        counts[e] = 0;
    for (long f = 0; f < R; ++f)
        counts[idx[f]]++;
    offsets[0] = 0;
    for (int e = 0; e < E; ++e)
        offsets[e + 1] = offsets[e] + counts[e];
    long r = 0;
    for (int e = 0; e < E; ++e)
        for (long f = 0; f < R; ++f)
            if (idx[f] == e) {
                perm[r] = (int32_t)f;
                pos[f] = (int32_t)r;
                ++r;
            }
}

/* ---- experts and combine --------------------------------------------------- */

/* One expert applied to one token vector v (fp64, length d):
 *   a_i = sum_c W_gate[i][c] v_c,  b_i = sum_c W_up[i][c] v_c,
 *   h_i = silu(a_i) * b_i,         y_o = sum_i W_down[o][i] h_i. */
void orc_expert_ffn(int w_dtype, const void *wg, const void *wu, const void *wd, const uint8_t *sg,
                    const uint8_t *su, const uint8_t *sd, int d, int I, const double *v, double *y)
{
    double *h = (double *)malloc(sizeof(double) * (size_t)I);
    for (int i = 0; i < I; ++i) {
        double a = 0.0, b = 0.0;
        for (int c = 0; c < d; ++c) {
            a += orc_weight(w_dtype, wg, sg, i, c, d) * v[c];
            b += orc_weight(w_dtype, wu, su, i, c, d) * v[c];
        }
        h[i] = a / (1.0 + exp(-a)) * b;
    }
    for (int o = 0; o < d; ++o) {
        double s = 0.0;
        for (int i = 0; i < I; ++i)
            s += orc_weight(w_dtype, wd, sd, o, i, I) * h[i];
        y[o] = s;
    }
    free(h);
}

/* Layer output for the listed tokens:
 *   out[s][:] = sum_{j=0..k-1} gates[t][j] * FFN_{idx[t][j]}(x[t]),  t = tokens[s].
 * Expert e's tensors are wg[e], wu[e], wd[e] (and scales sg/su/sd for MXFP4;
 * those arrays may be NULL otherwise).  Tokens are independent, so they are
 * spread over OpenMP threads; each token's sum runs in ascending j. */
void orc_moe_tokens(int w_dtype, int a_dtype, const void *x, int d, int I, int k,
                    const void *const *wg, const void *const *wu, const void *const *wd,
                    const uint8_t *const *sg, const uint8_t *const *su, const uint8_t *const *sd,
                    const int32_t *idx, const double *gates, const int32_t *tokens, int n_tokens,
                    double *out)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int s = 0; s < n_tokens; ++s) {
        int t = tokens[s];
        double *v = (double *)malloc(sizeof(double) * (size_t)d);
        double *y = (double *)malloc(sizeof(double) * (size_t)d);
        for (int c = 0; c < d; ++c)
            v[c] = act(a_dtype, x, t, c, d);
        double *o = out + (long)s * d;
        for (int c = 0; c < d; ++c)
            o[c] = 0.0;
        for (int j = 0; j < k; ++j) {
            int e = idx[(long)t * k + j];
            double g = gates[(long)t * k + j];
            orc_expert_ffn(w_dtype, wg[e], wu[e], wd[e], sg ? sg[e] : NULL, su ? su[e] : NULL,
                           sd ? sd[e] : NULL, d, I, v, y);
            for (int c = 0; c < d; ++c)
                o[c] += g * y[c];
        }
        free(v);
        free(y);
    }
}
