/*
 * clover_moe_oracle.h -- CPU oracle for the block-restricted sparse-MoE FFN.
 *
 * TEST INFRASTRUCTURE ONLY.  This is a plain, slow, single-purpose CPU
 * implementation used to check the HIP library.  Only the tests, the smoke
 * check and the benchmark's CPU-baseline leg may load it; the product path
 * never does.  It shares no code, header, table or constant with the HIP
 * library (include/clover_moe.h and the package's csrc/).
 *
 * Every pointer is a host pointer.  Arrays are row-major and contiguous.
 *
 * What it follows (pages are cited by title and section):
 *  - Clover-35B-A3B-Preview CMF model card, introduction: 256 routed
 *    experts, top-8 per token, plus one shared expert; answers written in
 *    32-token blocks refined by repeated denoising passes.
 *  - same card, "Usage": each block may use only the experts that together
 *    hold 90% of the block's routing weight; the block size is 8, 16 or 32.
 *  - same card, "Performance": each denoising pass runs the model forward
 *    once over the whole 32-row block.
 *  - InfiniLM PR #604 (Clover on Hygon), "Summary" and "Motivation": block
 *    coreset routing in the preview pass, top-4 preview routing, full-route
 *    replay after the approximate preview.
 *  - InfiniLM PR #584 (Qwen MTP with FP8 block weights), "Benchmark" and
 *    "Notes": E4M3 weights in 128x128 blocks, BF16 activations, aligned
 *    block loading.
 *
 * The pages give no arithmetic for the routing steps.  Because the expert
 * sets, indices and counts must agree bit for bit with the GPU, the routing
 * steps follow a fixed arithmetic contract (summation orders, precisions, an
 * exp written from the Cody-Waite reduction plus a Taylor polynomial); the
 * FFN has an exact definition and is evaluated in fp64.
 */
#ifndef CLOVER_MOE_ORACLE_H
#define CLOVER_MOE_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* storage dtype codes.  ORC_FP4_E2M1: 4-bit E2M1 codes, two per byte (low
 * nibble first), with one E8M0 scale byte (2^(s-127)) per 32 consecutive
 * elements of a row (OCP Microscaling MXFP4; a stand-in for the 4-bit
 * experts of the CMF model card, "Files", whose own layout is not given). */
enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_FP8_E4M3 = 2, ORC_FP4_E2M1 = 3 };

typedef struct {
    int hidden;        /* H */
    int num_experts;   /* E */
    int inter;         /* I  */
    int shared_inter;  /* Is (0 = no shared expert) */
    int block_rows;    /* rows per block */
    int num_blocks;    /* B */
    int act_dtype;     /* ORC_F32 or ORC_BF16 (x) */
    int weight_dtype;  /* ORC_F32, ORC_BF16 or ORC_FP8_E4M3 (expert weights) */
} orc_problem;

/* Scales: fp8: fp32 per 128x128 block, [rows/128, cols/128] per matrix;
 * fp4: uint8 E8M0 per 32 elements of a row, [rows, cols/32] per matrix. */
typedef struct {
    const float* router_w;         /* [E,H] fp32 */
    const float* router_b;         /* [E] fp32 or NULL */
    const void* w13;               /* [E,2I,H]: rows 0..I-1 gate, I..2I-1 up */
    const void* w13_scale;         /* fp8: [E,2I/128,H/128] fp32; fp4: [E,2I,H/32] uint8 */
    const void* w2;                /* [E,H,I] */
    const void* w2_scale;          /* fp8: [E,H/128,I/128] fp32; fp4: [E,H,I/32] uint8 */
    const void* shared_w13;        /* [2Is,H] or NULL */
    const void* shared_w13_scale;  /* fp8: [2Is/128,H/128]; fp4: [2Is,H/32] */
    const void* shared_w2;         /* [H,Is] or NULL */
    const void* shared_w2_scale;   /* fp8: [H/128,Is/128]; fp4: [H,Is/32] */
} orc_weights;

/* ---- scalar building blocks (exposed so the tests can pin them) ---- */

/* exp(d) for d <= 0 by Cody-Waite reduction and a degree-13 Taylor polynomial. */
double orc_exp(double d);
/* the constants orc_exp uses: [0]=1/ln2, [1]=ln2 head, [2]=ln2 tail, [3..16]=1/i!, i=0..13 */
void orc_exp_constants(double out[17]);
double orc_bf16_to_double(uint16_t bits);
double orc_e4m3_to_double(uint8_t code);
double orc_e2m1_to_double(uint8_t code);   /* low 4 bits */
double orc_e8m0_to_double(uint8_t s);      /* 2^(s-127); s = 255 is NaN */

/* ---- fp8 activations (the library's opt-in W8A8 mode) ----
 * Not a step of the pages (their fp8 experts take bf16 activations,
 * InfiniLM PR #584, "Benchmark").  MXFP8 is the OCP Microscaling layout:
 * E4M3 elements, one E8M0 power-of-two scale per 32 consecutive elements of
 * a row; here the scale is the smallest 2^e with max|v| <= 448 * 2^e (no
 * element saturates) and elements round to nearest, ties to the even code. */
double orc_round_bf16(double v);            /* to bf16, nearest, ties to even */
uint8_t orc_e4m3_encode(double v);          /* nearest E4M3 code, ties to even */
int orc_mx8_scale_exp(double amax);         /* smallest e in [-127,127], amax <= 448*2^e */
void orc_mx8_round(const double* v, int n, double* out);  /* n % 32 == 0; out may be v */

/* ---- routing stages ---- */

/* logits[N,E] (fp32) under the chunked fp32 summation contract. */
void orc_router_logits(const orc_problem* p, const void* x, const float* router_w,
                       const float* router_b, float* logits, int threads);

/* u[N,E] = exp(l - max_row) and p[N,E] = u / Z_row (fp64). */
void orc_softmax(const orc_problem* p, const float* logits, double* u, double* prob);

/* mass[B,E] = sum over each block's rows (ascending) of prob.  live[N]
 * (NULL = every row) marks the rows evaluated in this pass; the others add
 * nothing. */
void orc_block_mass(const orc_problem* p, const double* prob, const uint8_t* live, double* mass);

/* Coreset of one block: writes ids[0..m-1] (experts by mass desc, id asc),
 * returns m.  tau >= 1 selects all E experts. */
int orc_coreset(const double* mass, int num_experts, float tau, int32_t* ids);

/* Restricted top-k and gates of one row.  in_set[e] != 0 marks coreset
 * members.  Writes idx[k] (unused slots -1) and gates[k] (unused 0); returns k_eff. */
int orc_row_topk(const float* logits_row, const double* u_row, const uint8_t* in_set,
                 int num_experts, int top_k, int32_t* idx, float* gates);

/* ---- whole call ---- */

typedef struct {
    int32_t* topk_idx;       /* [N,k] */
    float* gates;            /* [N,k] */
    int32_t* coreset_ids;    /* [B,E], -1 padded */
    int32_t* coreset_size;   /* [B] */
    int32_t* expert_counts;  /* [E] */
    int32_t* expert_offsets; /* [E+1] exclusive prefix of counts */
    int32_t* perm;           /* [N*k]: row*k+slot in expert-major stable order, -1 padded */
    float* logits;           /* [N,E] */
    double* block_mass;      /* [B,E] */
} orc_routing;

/* Full forward.  out[N,H] is fp64.  If row_mask is non-NULL only rows with
 * row_mask[r] != 0 get their FFN output computed (routing is always done for
 * every row); other rows of `out` are left untouched.  Any routing pointer
 * may be NULL.  Returns 0 on success, nonzero on invalid arguments. */
int orc_forward(const orc_problem* p, const orc_weights* w, const void* x,
                float tau, int top_k, double* out, orc_routing* routing,
                const uint8_t* row_mask, int threads);

/* orc_forward with an expert budget and live rows (InfiniLM PR #604,
 * "Summary" and "Motivation": expert-budget / live-row reuse, the live rows
 * refreshed in full every few passes by the caller).
 *  - expert_budget: 0 = none, else 1..E; a block's coreset is cut to its
 *    first expert_budget experts (mass order) after the threshold cut.
 *  - live_rows[N] (NULL = all live): a row with 0 is resolved and reuses its
 *    cached output: it adds nothing to its block's mass, gets no route
 *    (idx -1, gate 0) and its row of `out` is left untouched.  A block with
 *    no live row has an empty coreset. */
int orc_forward_ex(const orc_problem* p, const orc_weights* w, const void* x,
                   float tau, int top_k, int expert_budget, const uint8_t* live_rows,
                   double* out, orc_routing* routing, const uint8_t* row_mask, int threads);

/* orc_forward_ex with fp8 activations: every row of x is rounded to MXFP8
 * before the expert GEMMs, and each expert's h is rounded to bf16 and then
 * to MXFP8 before its down GEMM (orc_expert_ffn_mx8).  Routing is unchanged.
 * fp8 weights with bf16 x only (else returns 6). */
int orc_forward_ex_act8(const orc_problem* p, const orc_weights* w, const void* x,
                        float tau, int top_k, int expert_budget, const uint8_t* live_rows,
                        double* out, orc_routing* routing, const uint8_t* row_mask, int threads);

/* fp64 SwiGLU FFN of one expert with fp8 activations: xq[H] already MXFP8;
 * h rounded to bf16, then to MXFP8, before W2. */
void orc_expert_ffn_mx8(int hidden, int inter, int wdtype, const void* w13, const void* w13_scale,
                        const void* w2, const void* w2_scale, const double* xq, double* y);

/* fp64 SwiGLU FFN of one expert weight set on one input row (widened to fp64):
 * y[H] = W2 * (silu(W13[0:I] x) * (W13[I:2I] x)).  wdtype as in orc_problem. */
void orc_expert_ffn(int hidden, int inter, int wdtype, const void* w13, const void* w13_scale,
                    const void* w2, const void* w2_scale, const double* xrow, double* y);

#ifdef __cplusplus
}
#endif
#endif
