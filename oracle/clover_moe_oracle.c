/*
 * clover_moe_oracle.c -- CPU oracle for the block-restricted sparse-MoE FFN.
 *
 * TEST INFRASTRUCTURE ONLY (see clover_moe_oracle.h).  Plain C, plain loops,
 * no blocking or fusion beyond what each step's definition states.  Built with
 * -ffp-contract=off so that every floating-point operation written here is
 * the one executed.
 *
 * Stages, in the order the pages describe the layer:
 *   1. router logits                 (CMF model card, introduction: 256 experts, top-8)
 *   2. softmax over all experts      (same)
 *   3. block routing mass            (CMF model card, "Usage": the experts holding 90%
 *                                     of the block's routing weight; InfiniLM PR #604
 *                                     "Summary": block coreset routing)
 *   4. coreset = smallest mass-ordered prefix reaching the threshold
 *   5. restricted top-k + renormalised gates (InfiniLM PR #604 "Motivation": top-4
 *                                     preview routing; "Notes for Reviewers": full-route
 *                                     replay = unrestricted routing)
 *   6. per-expert counts and the expert-major row order
 *   7. routed SwiGLU experts + the shared expert, gate-weighted sum (CMF model card,
 *                                     introduction: one shared expert besides the routed ones)
 */
#include "clover_moe_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------ */
/* exp for the routing softmax.                                              */
/*                                                                           */
/* Cody & Waite (1980) argument reduction: d = n*ln2 + r with n = rint(d/ln2) */
/* and ln2 split into a head with trailing zero bits (so n*head is exact for */
/* |n| < 2^11) and a tail; then exp(r) by its Taylor series to degree 13     */
/* (truncation < 2^-53 for |r| <= ln2/2), evaluated by Horner with fma, and  */
/* exp(d) = 2^n * exp(r).  Constants, derived from ln 2 and i!:              */
/*   1/ln2    correctly rounded                                             */
/*   ln2 head = the double nearest ln 2 with its low 11 mantissa bits zeroed */
/*   ln2 tail = (ln 2 - head) correctly rounded                             */
/*   1/i!     correctly rounded, i = 0..13                                   */
/* ------------------------------------------------------------------------ */

static const double ORC_INV_LN2 = 0x1.71547652b82fep+0;
static const double ORC_LN2_HEAD = 0x1.62e42fefa3800p-1;
static const double ORC_LN2_TAIL = 0x1.ef35793c76730p-45;

static double orc_inv_factorial(int i)
{
    double f = 1.0; /* i! is exact in fp64 for i <= 18 */
    for (int j = 2; j <= i; ++j) f *= (double)j;
    return 1.0 / f; /* one correctly rounded division */
}

void orc_exp_constants(double out[17])
{
    out[0] = ORC_INV_LN2;
    out[1] = ORC_LN2_HEAD;
    out[2] = ORC_LN2_TAIL;
    for (int i = 0; i <= 13; ++i) out[3 + i] = orc_inv_factorial(i);
}

double orc_exp(double d)
{
    static double coef[14];
    static int ready = 0;
    if (!ready) { /* benign race: every thread writes the same values */
        for (int i = 0; i <= 13; ++i) coef[i] = orc_inv_factorial(i);
        ready = 1;
    }
    if (d < -708.0) return 0.0; /* below this exp(d) leaves the normal range */
    double n = rint(d * ORC_INV_LN2);
    double r = fma(-n, ORC_LN2_HEAD, d);
    r = fma(-n, ORC_LN2_TAIL, r);
    double poly = coef[13];
    for (int i = 12; i >= 0; --i) poly = fma(poly, r, coef[i]);
    return ldexp(poly, (int)n);
}

/* ------------------------------------------------------------------------ */
/* storage decoding (all exact in fp64)                                      */
/* ------------------------------------------------------------------------ */

double orc_bf16_to_double(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* OCP FP8 E4M3 ("e4m3fn"): 1 sign, 4 exponent (bias 7), 3 mantissa bits; no
 * infinities; S.1111.111 is NaN; largest finite magnitude 448. */
double orc_e4m3_to_double(uint8_t code)
{
    int sign = code >> 7;
    int expo = (code >> 3) & 0xF;
    int mant = code & 0x7;
    double mag;
    if (expo == 0xF && mant == 0x7) return NAN;
    if (expo == 0)
        mag = ldexp((double)mant, -9);            /* mant/8 * 2^(1-7) */
    else
        mag = ldexp(8.0 + (double)mant, expo - 10); /* (1+mant/8) * 2^(expo-7) */
    return sign ? -mag : mag;
}

/* OCP FP4 E2M1 (low 4 bits of `code`): 1 sign, 2 exponent (bias 1), 1
 * mantissa bit; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6; no NaN or infinity. */
double orc_e2m1_to_double(uint8_t code)
{
    int sign = (code >> 3) & 1;
    int expo = (code >> 1) & 0x3;
    int mant = code & 0x1;
    double mag = expo == 0 ? 0.5 * mant : ldexp(1.0 + 0.5 * mant, expo - 1);
    return sign ? -mag : mag;
}

/* OCP E8M0 scale: 2^(s-127), s in 0..254; 255 is NaN. */
double orc_e8m0_to_double(uint8_t s)
{
    return s == 255 ? NAN : ldexp(1.0, (int)s - 127);
}

/* ------------------------------------------------------------------------ */
/* fp8 activations (the library's opt-in W8A8 mode; not a step of the pages: */
/* their fp8 experts run with bf16 activations, InfiniLM PR #584,            */
/* "Benchmark").  Activations enter each expert GEMM as MXFP8, the layout of  */
/* the OCP Microscaling (MX) format: E4M3 elements with one E8M0 power-of-two */
/* scale per 32 consecutive elements of a row.  The scale of a group is the   */
/* smallest 2^e that keeps its largest magnitude within 448 (the largest     */
/* E4M3 value), so no element saturates; each element is v / 2^e rounded to  */
/* the nearest E4M3 value, ties to the even code.  x is bf16 already; h is    */
/* held in bf16 (round to nearest even) before it is rounded to MXFP8.        */
/* ------------------------------------------------------------------------ */

/* v rounded to bf16 (8 significant bits, round to nearest, ties to even) */
double orc_round_bf16(double v)
{
    if (v == 0.0 || isnan(v) || isinf(v)) return v;
    int ex;
    frexp(v, &ex);                            /* |v| = f * 2^ex, f in [0.5, 1) */
    double q = ldexp(v, 8 - ex);              /* 8 significant bits left of the point */
    double r = nearbyint(q);                  /* default rounding: to nearest, ties to even */
    return ldexp(r, ex - 8);
}

/* The E4M3 code nearest to v (ties to the even code), by comparing v with
 * every finite non-negative code value; the sign bit is v's. */
uint8_t orc_e4m3_encode(double v)
{
    double a = fabs(v);
    int best = 0;
    double bd = INFINITY;
    for (int c = 0; c <= 0x7E; ++c) {
        double d = fabs(orc_e4m3_to_double((uint8_t)c) - a);
        if (d < bd || (d == bd && (c & 1) == 0)) {
            bd = d;
            best = c;
        }
    }
    return (uint8_t)(best | (signbit(v) ? 0x80 : 0x00));
}

/* the scale exponent of a group whose largest magnitude is amax: the
 * smallest e in [-127, 127] with amax <= 448 * 2^e (-127 for amax 0) */
int orc_mx8_scale_exp(double amax)
{
    for (int e = -127; e <= 127; ++e)
        if (amax <= ldexp(448.0, e)) return e;
    return 127;
}

/* out[0..n) = v rounded to MXFP8 and back (n a multiple of 32) */
void orc_mx8_round(const double* v, int n, double* out)
{
    for (int g = 0; g < n; g += 32) {
        double amax = 0.0;
        for (int i = 0; i < 32; ++i) amax = fmax(amax, fabs(v[g + i]));
        int e = orc_mx8_scale_exp(amax);
        for (int i = 0; i < 32; ++i)
            out[g + i] = ldexp(orc_e4m3_to_double(orc_e4m3_encode(ldexp(v[g + i], -e))), e);
    }
}

static double act_value(int dtype, const void* x, size_t i)
{
    if (dtype == ORC_BF16) return orc_bf16_to_double(((const uint16_t*)x)[i]);
    return (double)((const float*)x)[i];
}

/* Widen row `row` of a [rows, cols] weight matrix to fp64.  fp8 values are
 * code * scale[row/128][col/128]; fp4 values are code * 2^(s-127) with s the
 * E8M0 byte [row][col/32]; both products are exact in fp64. */
static void widen_weight_row(int dtype, const void* w, const void* scale, int cols,
                             int row, double* dst)
{
    size_t base = (size_t)row * (size_t)cols;
    for (int c = 0; c < cols; ++c) {
        switch (dtype) {
        case ORC_F32: dst[c] = (double)((const float*)w)[base + c]; break;
        case ORC_BF16: dst[c] = orc_bf16_to_double(((const uint16_t*)w)[base + c]); break;
        case ORC_FP4_E2M1: {
            uint8_t byte = ((const uint8_t*)w)[(base + (size_t)c) / 2];
            uint8_t code = (c & 1) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 0xF);
            uint8_t s = ((const uint8_t*)scale)[(size_t)row * (size_t)(cols / 32) + (size_t)(c / 32)];
            dst[c] = orc_e2m1_to_double(code) * orc_e8m0_to_double(s);
            break;
        }
        default: {
            const float* sc = (const float*)scale;
            double s = (double)sc[(size_t)(row / 128) * (size_t)(cols / 128) + (size_t)(c / 128)];
            dst[c] = orc_e4m3_to_double(((const uint8_t*)w)[base + c]) * s;
        }
        }
    }
}

/* ------------------------------------------------------------------------ */
/* 1. router logits                                                          */
/*                                                                           */
/* l[r,e] = sum_h x[r,h] * Wr[e,h] (+ b[e]), in fp32 under a fixed order:    */
/* h is split into 8 contiguous chunks [j*H/8, (j+1)*H/8) (integer division); */
/* each chunk accumulates ascending h with fp32 fma from +0; the 8 partials  */
/* combine pairwise (j += j+4, then j += j+2, then j += j+1); the bias, when */
/* present, is one final fp32 add.                                           */
/* ------------------------------------------------------------------------ */

void orc_router_logits(const orc_problem* p, const void* x, const float* router_w,
                       const float* router_b, float* logits, int threads)
{
    const int H = p->hidden, E = p->num_experts;
    const int N = p->block_rows * p->num_blocks;
#ifdef _OPENMP
    if (threads > 0) omp_set_num_threads(threads);
#pragma omp parallel for schedule(static)
#endif
    for (int r = 0; r < N; ++r) {
        float* xrow = (float*)malloc(sizeof(float) * (size_t)H);
        for (int h = 0; h < H; ++h) xrow[h] = (float)act_value(p->act_dtype, x, (size_t)r * H + h);
        for (int e = 0; e < E; ++e) {
            const float* wrow = router_w + (size_t)e * H;
            float part[8];
            for (int j = 0; j < 8; ++j) {
                int lo = (int)(((long)j * H) / 8), hi = (int)(((long)(j + 1) * H) / 8);
                float acc = 0.0f;
                for (int h = lo; h < hi; ++h) acc = fmaf(xrow[h], wrow[h], acc);
                part[j] = acc;
            }
            for (int s = 4; s >= 1; s /= 2)
                for (int j = 0; j < s; ++j) part[j] = part[j] + part[j + s];
            float l = part[0];
            if (router_b) l = l + router_b[e];
            logits[(size_t)r * E + e] = l;
        }
        free(xrow);
    }
    (void)threads;
}

/* ------------------------------------------------------------------------ */
/* 2. softmax over all E experts of each row, in fp64.                       */
/* u = exp(l - max_row); Z = sum_e u (8 contiguous chunks of e, ascending    */
/* within a chunk, pairwise combine as for the logits); p = u / Z.           */
/* ------------------------------------------------------------------------ */

void orc_softmax(const orc_problem* p, const float* logits, double* u, double* prob)
{
    const int E = p->num_experts;
    const int N = p->block_rows * p->num_blocks;
    for (int r = 0; r < N; ++r) {
        const float* l = logits + (size_t)r * E;
        double* ur = u + (size_t)r * E;
        float m = l[0];
        for (int e = 1; e < E; ++e)
            if (l[e] > m) m = l[e];
        for (int e = 0; e < E; ++e) ur[e] = orc_exp((double)l[e] - (double)m);
        double part[8];
        for (int j = 0; j < 8; ++j) {
            int lo = (j * E) / 8, hi = ((j + 1) * E) / 8;
            double acc = 0.0;
            for (int e = lo; e < hi; ++e) acc = acc + ur[e];
            part[j] = acc;
        }
        for (int s = 4; s >= 1; s /= 2)
            for (int j = 0; j < s; ++j) part[j] = part[j] + part[j + s];
        double Z = part[0];
        if (prob)
            for (int e = 0; e < E; ++e) prob[(size_t)r * E + e] = ur[e] / Z;
    }
}

/* ------------------------------------------------------------------------ */
/* 3. block routing mass: mass[b,e] = sum of p[r,e] over the block's rows,   */
/* rows ascending, fp64.  Block b is rows [b*R, (b+1)*R).  Only the rows     */
/* evaluated in this pass count (live[r] != 0; NULL = all).                  */
/* ------------------------------------------------------------------------ */

void orc_block_mass(const orc_problem* p, const double* prob, const uint8_t* live, double* mass)
{
    const int E = p->num_experts, R = p->block_rows;
    for (int b = 0; b < p->num_blocks; ++b)
        for (int e = 0; e < E; ++e) {
            double acc = 0.0;
            for (int r = b * R; r < (b + 1) * R; ++r)
                if (!live || live[r]) acc = acc + prob[(size_t)r * E + e];
            mass[(size_t)b * E + e] = acc;
        }
}

/* ------------------------------------------------------------------------ */
/* 4. coreset: experts ordered by (mass desc, id asc); total = sequential    */
/* fp64 sum in that order; the coreset is the shortest prefix whose          */
/* sequential fp64 cumulative sum reaches tau * total (one fp64 multiply),   */
/* i.e. the smallest expert set carrying that share of the block's routing.  */
/* tau >= 1 is the unrestricted ("full route") case: all experts.            */
/* ------------------------------------------------------------------------ */

static const double* g_sort_mass; /* used only by the qsort comparator */

static int by_mass_desc_id_asc(const void* a, const void* b)
{
    int ea = *(const int32_t*)a, eb = *(const int32_t*)b;
    double ma = g_sort_mass[ea], mb = g_sort_mass[eb];
    if (ma > mb) return -1;
    if (ma < mb) return 1;
    return (ea < eb) ? -1 : (ea > eb);
}

int orc_coreset(const double* mass, int num_experts, float tau, int32_t* ids)
{
    for (int e = 0; e < num_experts; ++e) ids[e] = e;
    g_sort_mass = mass;
    qsort(ids, (size_t)num_experts, sizeof(int32_t), by_mass_desc_id_asc);
    if (tau >= 1.0f) return num_experts;
    double total = 0.0;
    for (int i = 0; i < num_experts; ++i) total = total + mass[ids[i]];
    double thr = (double)tau * total;
    double cum = 0.0;
    for (int m = 1; m <= num_experts; ++m) {
        cum = cum + mass[ids[m - 1]];
        if (cum >= thr) return m;
    }
    return num_experts;
}

/* ------------------------------------------------------------------------ */
/* 5. restricted top-k: the k_eff = min(k, |C|) coreset experts with the     */
/* largest fp32 logits, ordered by (logit desc, id asc).  Gates renormalise  */
/* the softmax numerators over the chosen slots: U = sum of u in slot order  */
/* (fp64), g_j = (float)(u_j / U).                                           */
/* ------------------------------------------------------------------------ */

int orc_row_topk(const float* logits_row, const double* u_row, const uint8_t* in_set,
                 int num_experts, int top_k, int32_t* idx, float* gates)
{
    int k_eff = 0;
    for (int j = 0; j < top_k; ++j) {
        int best = -1;
        for (int e = 0; e < num_experts; ++e) {
            if (!in_set[e]) continue;
            int taken = 0;
            for (int t = 0; t < k_eff; ++t)
                if (idx[t] == e) taken = 1;
            if (taken) continue;
            if (best < 0 || logits_row[e] > logits_row[best]) best = e; /* ties keep the lower id */
        }
        if (best < 0) break;
        idx[k_eff++] = best;
    }
    double U = 0.0;
    for (int j = 0; j < k_eff; ++j) U = U + u_row[idx[j]];
    for (int j = 0; j < k_eff; ++j) gates[j] = (float)(u_row[idx[j]] / U);
    for (int j = k_eff; j < top_k; ++j) {
        idx[j] = -1;
        gates[j] = 0.0f;
    }
    return k_eff;
}

/* ------------------------------------------------------------------------ */
/* 7. expert FFN in fp64: z = W13 x; a = z[0:I]; v = z[I:2I];                 */
/* h = a * sigmoid(a) * v; y = W2 h.                                          */
/* ------------------------------------------------------------------------ */

void orc_expert_ffn(int hidden, int inter, int wdtype, const void* w13, const void* w13_scale,
                    const void* w2, const void* w2_scale, const double* xrow, double* y)
{
    double* wrow = (double*)malloc(sizeof(double) * (size_t)(hidden > inter ? hidden : inter));
    double* z = (double*)malloc(sizeof(double) * 2 * (size_t)inter);
    double* h = (double*)malloc(sizeof(double) * (size_t)inter);
    for (int i = 0; i < 2 * inter; ++i) {
        widen_weight_row(wdtype, w13, w13_scale, hidden, i, wrow);
        double acc = 0.0;
        for (int c = 0; c < hidden; ++c) acc += wrow[c] * xrow[c];
        z[i] = acc;
    }
    for (int i = 0; i < inter; ++i) {
        double a = z[i], v = z[inter + i];
        h[i] = a * (1.0 / (1.0 + exp(-a))) * v;
    }
    for (int o = 0; o < hidden; ++o) {
        widen_weight_row(wdtype, w2, w2_scale, inter, o, wrow);
        double acc = 0.0;
        for (int i = 0; i < inter; ++i) acc += wrow[i] * h[i];
        y[o] = acc;
    }
    free(wrow);
    free(z);
    free(h);
}

/* orc_expert_ffn with fp8 activations: xq is the input row already rounded
 * to MXFP8; h is rounded to bf16 and then to MXFP8 before the down GEMM. */
void orc_expert_ffn_mx8(int hidden, int inter, int wdtype, const void* w13, const void* w13_scale,
                        const void* w2, const void* w2_scale, const double* xq, double* y)
{
    double* wrow = (double*)malloc(sizeof(double) * (size_t)(hidden > inter ? hidden : inter));
    double* z = (double*)malloc(sizeof(double) * 2 * (size_t)inter);
    double* h = (double*)malloc(sizeof(double) * (size_t)inter);
    double* hq = (double*)malloc(sizeof(double) * (size_t)inter);
    for (int i = 0; i < 2 * inter; ++i) {
        widen_weight_row(wdtype, w13, w13_scale, hidden, i, wrow);
        double acc = 0.0;
        for (int c = 0; c < hidden; ++c) acc += wrow[c] * xq[c];
        z[i] = acc;
    }
    for (int i = 0; i < inter; ++i) {
        double a = z[i], v = z[inter + i];
        h[i] = orc_round_bf16(a * (1.0 / (1.0 + exp(-a))) * v);
    }
    orc_mx8_round(h, inter, hq);
    for (int o = 0; o < hidden; ++o) {
        widen_weight_row(wdtype, w2, w2_scale, inter, o, wrow);
        double acc = 0.0;
        for (int i = 0; i < inter; ++i) acc += wrow[i] * hq[i];
        y[o] = acc;
    }
    free(wrow);
    free(z);
    free(h);
    free(hq);
}

/* bytes of a [rows, cols] weight matrix, and of its scales, in `dtype` storage */
static size_t matrix_bytes(int dtype, size_t rows, size_t cols)
{
    switch (dtype) {
    case ORC_F32: return rows * cols * 4;
    case ORC_BF16: return rows * cols * 2;
    case ORC_FP4_E2M1: return rows * cols / 2;
    default: return rows * cols;
    }
}

static size_t scale_bytes(int dtype, size_t rows, size_t cols)
{
    if (dtype == ORC_FP8_E4M3) return (rows / 128) * (cols / 128) * 4;
    if (dtype == ORC_FP4_E2M1) return rows * (cols / 32);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* whole call                                                               */
/* ------------------------------------------------------------------------ */

int orc_forward(const orc_problem* p, const orc_weights* w, const void* x,
                float tau, int top_k, double* out, orc_routing* rt,
                const uint8_t* row_mask, int threads)
{
    return orc_forward_ex(p, w, x, tau, top_k, 0, NULL, out, rt, row_mask, threads);
}

static int forward_common(const orc_problem* p, const orc_weights* w, const void* x,
                          float tau, int top_k, int expert_budget, const uint8_t* live,
                          double* out, orc_routing* rt, const uint8_t* row_mask, int threads,
                          int act_fp8);

int orc_forward_ex(const orc_problem* p, const orc_weights* w, const void* x,
                   float tau, int top_k, int expert_budget, const uint8_t* live,
                   double* out, orc_routing* rt, const uint8_t* row_mask, int threads)
{
    return forward_common(p, w, x, tau, top_k, expert_budget, live, out, rt, row_mask, threads, 0);
}

int orc_forward_ex_act8(const orc_problem* p, const orc_weights* w, const void* x,
                        float tau, int top_k, int expert_budget, const uint8_t* live,
                        double* out, orc_routing* rt, const uint8_t* row_mask, int threads)
{
    if (p->weight_dtype != ORC_FP8_E4M3 || p->act_dtype != ORC_BF16) return 6;
    if (p->hidden % 32 || p->inter % 32 || p->shared_inter % 32) return 6;
    return forward_common(p, w, x, tau, top_k, expert_budget, live, out, rt, row_mask, threads, 1);
}

static int forward_common(const orc_problem* p, const orc_weights* w, const void* x,
                          float tau, int top_k, int expert_budget, const uint8_t* live,
                          double* out, orc_routing* rt, const uint8_t* row_mask, int threads,
                          int act_fp8)
{
    const int H = p->hidden, E = p->num_experts, I = p->inter, Is = p->shared_inter;
    const int R = p->block_rows, B = p->num_blocks, N = R * B, K = top_k;
    if (H <= 0 || E <= 0 || I <= 0 || Is < 0 || R <= 0 || B <= 0) return 1;
    if (K < 1 || K > E) return 2;
    if (!(tau > 0.0f && tau <= 1.0f)) return 3;
    if (expert_budget < 0 || expert_budget > E) return 5;
    if (p->weight_dtype == ORC_FP8_E4M3 &&
        (H % 128 || I % 128 || Is % 128 || !w->w13_scale || !w->w2_scale)) return 4;
    if (p->weight_dtype == ORC_FP4_E2M1 &&
        (H % 32 || I % 32 || Is % 32 || !w->w13_scale || !w->w2_scale)) return 4;

    float* logits = (float*)malloc(sizeof(float) * (size_t)N * E);
    double* u = (double*)malloc(sizeof(double) * (size_t)N * E);
    double* prob = (double*)malloc(sizeof(double) * (size_t)N * E);
    double* mass = (double*)malloc(sizeof(double) * (size_t)B * E);
    int32_t* ids = (int32_t*)malloc(sizeof(int32_t) * (size_t)B * E);
    int32_t* csize = (int32_t*)malloc(sizeof(int32_t) * (size_t)B);
    int32_t* idx = (int32_t*)malloc(sizeof(int32_t) * (size_t)N * K);
    float* gates = (float*)malloc(sizeof(float) * (size_t)N * K);
    uint8_t* in_set = (uint8_t*)malloc((size_t)E);

    /* 1-3 */
    orc_router_logits(p, x, w->router_w, w->router_b, logits, threads);
    orc_softmax(p, logits, u, prob);
    orc_block_mass(p, prob, live, mass);

    /* 4-5, block by block: coreset, budget cut, top-k of the live rows */
    for (int b = 0; b < B; ++b) {
        int32_t* bid = ids + (size_t)b * E;
        int m = orc_coreset(mass + (size_t)b * E, E, tau, bid);
        if (expert_budget > 0 && m > expert_budget) m = expert_budget;
        int any_live = 0;
        for (int r = b * R; r < (b + 1) * R; ++r) any_live |= !live || live[r];
        if (!any_live) m = 0;
        csize[b] = m;
        for (int i = m; i < E; ++i) bid[i] = -1;
        memset(in_set, 0, (size_t)E);
        for (int i = 0; i < m; ++i) in_set[bid[i]] = 1;
        for (int r = b * R; r < (b + 1) * R; ++r) {
            if (live && !live[r]) {
                for (int j = 0; j < K; ++j) {
                    idx[(size_t)r * K + j] = -1;
                    gates[(size_t)r * K + j] = 0.0f;
                }
                continue;
            }
            orc_row_topk(logits + (size_t)r * E, u + (size_t)r * E, in_set, E, K,
                         idx + (size_t)r * K, gates + (size_t)r * K);
        }
    }

    /* 6. counts, offsets and the stable expert-major order of (row, slot) */
    if (rt) {
        if (rt->expert_counts || rt->expert_offsets || rt->perm) {
            int32_t* cnt = (int32_t*)calloc((size_t)E, sizeof(int32_t));
            for (int i = 0; i < N * K; ++i)
                if (idx[i] >= 0) cnt[idx[i]]++;
            if (rt->expert_counts) memcpy(rt->expert_counts, cnt, sizeof(int32_t) * (size_t)E);
            if (rt->expert_offsets) {
                int32_t run = 0;
                for (int e = 0; e < E; ++e) {
                    rt->expert_offsets[e] = run;
                    run += cnt[e];
                }
                rt->expert_offsets[E] = run;
            }
            if (rt->perm) {
                int pos = 0;
                for (int e = 0; e < E; ++e)
                    for (int i = 0; i < N * K; ++i)
                        if (idx[i] == e) rt->perm[pos++] = i;
                for (; pos < N * K; ++pos) rt->perm[pos] = -1;
            }
            free(cnt);
        }
        if (rt->topk_idx) memcpy(rt->topk_idx, idx, sizeof(int32_t) * (size_t)N * K);
        if (rt->gates) memcpy(rt->gates, gates, sizeof(float) * (size_t)N * K);
        if (rt->coreset_ids) memcpy(rt->coreset_ids, ids, sizeof(int32_t) * (size_t)B * E);
        if (rt->coreset_size) memcpy(rt->coreset_size, csize, sizeof(int32_t) * (size_t)B);
        if (rt->logits) memcpy(rt->logits, logits, sizeof(float) * (size_t)N * E);
        if (rt->block_mass) memcpy(rt->block_mass, mass, sizeof(double) * (size_t)B * E);
    }

    /* 7. FFN of every (row, slot) plus the shared expert, fp64 */
    if (out) {
        const int wd = p->weight_dtype;
        const size_t w13_b = matrix_bytes(wd, (size_t)2 * I, (size_t)H);
        const size_t w2_b = matrix_bytes(wd, (size_t)H, (size_t)I);
        const size_t w13_sb = scale_bytes(wd, (size_t)2 * I, (size_t)H);
        const size_t w2_sb = scale_bytes(wd, (size_t)H, (size_t)I);
#ifdef _OPENMP
        if (threads > 0) omp_set_num_threads(threads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
        for (int r = 0; r < N; ++r) {
            if ((row_mask && !row_mask[r]) || (live && !live[r])) continue;
            double* xr = (double*)malloc(sizeof(double) * (size_t)H);
            double* y = (double*)malloc(sizeof(double) * (size_t)H);
            double* acc = out + (size_t)r * H;
            for (int c = 0; c < H; ++c) xr[c] = act_value(p->act_dtype, x, (size_t)r * H + c);
            if (act_fp8) orc_mx8_round(xr, H, xr);  /* in place: each group is read before written */
            for (int c = 0; c < H; ++c) acc[c] = 0.0;
            if (Is > 0 && w->shared_w13 && w->shared_w2) {
                if (act_fp8)
                    orc_expert_ffn_mx8(H, Is, p->weight_dtype, w->shared_w13, w->shared_w13_scale,
                                       w->shared_w2, w->shared_w2_scale, xr, y);
                else
                    orc_expert_ffn(H, Is, p->weight_dtype, w->shared_w13, w->shared_w13_scale,
                                   w->shared_w2, w->shared_w2_scale, xr, y);
                for (int c = 0; c < H; ++c) acc[c] += y[c];
            }
            for (int j = 0; j < K; ++j) {
                int e = idx[(size_t)r * K + j];
                if (e < 0) continue;
                const char* w13e = (const char*)w->w13 + (size_t)e * w13_b;
                const char* w2e = (const char*)w->w2 + (size_t)e * w2_b;
                const char* s13 = w13_sb ? (const char*)w->w13_scale + (size_t)e * w13_sb : NULL;
                const char* s2 = w2_sb ? (const char*)w->w2_scale + (size_t)e * w2_sb : NULL;
                if (act_fp8) orc_expert_ffn_mx8(H, I, wd, w13e, s13, w2e, s2, xr, y);
                else orc_expert_ffn(H, I, wd, w13e, s13, w2e, s2, xr, y);
                double g = (double)gates[(size_t)r * K + j];
                for (int c = 0; c < H; ++c) acc[c] += g * y[c];
            }
            free(xr);
            free(y);
        }
    }

    free(logits);
    free(u);
    free(prob);
    free(mass);
    free(ids);
    free(csize);
    free(idx);
    free(gates);
    free(in_set);
    return 0;
}
