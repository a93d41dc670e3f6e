/*
 * clover_moe.h -- C ABI of the block-restricted sparse mixture-of-experts FFN
 * for MI355X (gfx950).
 *
 * The operation (one MoE layer evaluated on a denoising pass of a
 * block-diffusion language model):
 *
 *   Clover-35B-A3B-Preview CMF model card, introduction: every token is
 *   routed to the top 8 of 256 experts, and a shared expert is always
 *   applied; answers are written in 32-token blocks that are re-run pass
 *   after pass until no mask token remains.
 *   Same card, "Usage": during those passes a block may use only the experts
 *   that together hold 90% of the block's routing weight; the block size can
 *   be 8, 16 or 32.
 *   InfiniLM PR #604 (Clover on Hygon), "Summary", "Motivation" and "Notes for
 *   Reviewers": block coreset routing in the preview pass, top-4 preview
 *   routing, and a full-route replay after the approximate preview
 *   (mass_threshold = 1.0 here).
 *   InfiniLM PR #584 (Qwen MTP with FP8 block weights), "Benchmark" and
 *   "Notes": E4M3 weights in 128x128 blocks with BF16 activations, aligned
 *   block loading.
 *
 * For a call with B blocks of R rows (N = B*R rows), H hidden, E routed
 * experts, top-k, expert intermediate I and shared intermediate Is:
 *
 *   1. logits l[r,e] = x[r,:] . Wr[e,:] (+ b[e])                     fp32
 *   2. p[r,:] = softmax(l[r,:]) over all E experts                   fp64
 *   3. mass[b,e] = sum of p[r,e] over the rows of block b             fp64
 *   4. coreset C_b = smallest prefix of experts ordered by (mass desc,
 *      id asc) whose cumulative mass reaches mass_threshold * total;
 *      mass_threshold = 1 selects all experts
 *   5. per row: the min(k, |C_b|) experts of C_b with the largest logits
 *      (ties: lower id), gates renormalised over the chosen slots
 *   6. out[r] = SwiGLU_shared(x[r]) + sum_j gate[r,j] * SwiGLU_{e_j}(x[r]),
 *      SwiGLU_e(x) = W2_e (silu(W13_e[0:I] x) * (W13_e[I:2I] x))
 *
 * Steps 1-5 follow a fixed arithmetic contract (summation orders, fp32 fma
 * for the logits, fp64 softmax with a Cody-Waite exp) so that expert sets,
 * indices, gates and counts are reproducible bit for bit by any conforming
 * implementation.  Step 6 accumulates in fp32 on MFMA; it matches an exact
 * evaluation within a tolerance (bf16 and 4-bit weights: max |err| <=
 * 2e-2 max|ref| and sum|err| <= 5e-3 sum|ref|; fp8 weights: max |err| <=
 * 6e-2 max|ref|).
 *
 * Conventions
 *  - Every pointer argument of clover_moe_block_forward, and every pointer in
 *    the structs, is a DEVICE pointer unless stated otherwise; the struct
 *    objects themselves live in host memory.  Arrays are row-major and
 *    contiguous (expert weights may instead be MFMA panels, see
 *    cmoe_layout).  Device pointers must be 16-byte aligned.
 *  - Ownership: the caller allocates and frees everything, including the
 *    workspace (clover_moe_block_forward_noalloc uses a static array of the
 *    library instead).  The library allocates no memory, keeps no pointer after the
 *    call returns, never synchronises the host and never changes the current
 *    device.  Buffers must stay valid until the work queued on `stream`
 *    completes.
 *  - Inputs are never written.  `out` and the workspace must not overlap any
 *    input.
 *  - Errors (InfiniLM PR #604, "Notes for Reviewers": options the
 *    implementation does not support are refused explicitly, and a
 *    conversion that would be wrong is refused before anything is written):
 *    every argument is checked before any work is queued and before any byte
 *    is written; an invalid call returns a nonzero status and leaves every
 *    buffer untouched.  There is no silent fallback to another dtype, shape
 *    or path.  clover_moe_last_error() then holds a thread-local
 *    description.  Faults inside kernels surface at the caller's next
 *    synchronisation.
 *  - Non-finite inputs are not checked; their results are undefined.
 *  - Thread safety: calls are independent; the library has no global
 *    mutable state apart from the thread-local error text and the per-GPU
 *    scratch array of clover_moe_block_forward_noalloc (calls of that entry
 *    point must not overlap on one GPU).
 *  - A call queues kernels on `stream` and nothing else (no memset, no
 *    allocation, no host synchronisation), so it can be captured in a HIP
 *    graph; replays reproduce the eager results bit for bit.
 */
#ifndef CLOVER_MOE_H
#define CLOVER_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    CMOE_OK = 0,
    CMOE_ERR_NULL = 1,        /* a required pointer is NULL */
    CMOE_ERR_VALUE = 2,       /* a value is out of its domain (threshold, top_k, sizes) */
    CMOE_ERR_UNSUPPORTED = 3, /* a valid but unsupported shape or dtype combination */
    CMOE_ERR_ALIGN = 4,       /* a device pointer is not 16-byte aligned */
    CMOE_ERR_ALIAS = 5,       /* out / workspace / routing outputs overlap an input or each other */
    CMOE_ERR_WORKSPACE = 6,   /* workspace is NULL or smaller than clover_moe_workspace_size() */
    CMOE_ERR_HIP = 7          /* the HIP runtime refused a launch */
} cmoe_status;

typedef enum {
    CMOE_F32 = 0,
    CMOE_BF16 = 1,
    CMOE_FP8_E4M3 = 2, /* OCP E4M3 ("e4m3fn", max 448), with fp32 128x128 block scales */
    CMOE_FP4_E2M1 = 3  /* 4-bit experts (CMF model card, "Files"; its own layout is not
                          given, the stand-in is OCP Microscaling MXFP4): E2M1 codes, two
                          per byte, low nibble first, and one E8M0 scale byte 2^(s-127),
                          s = 1..254, per 32 consecutive elements of a row */
} cmoe_dtype;

/* Shapes and dtypes (host struct). */
typedef struct {
    int32_t hidden;       /* H: multiple of 128, 128..16384 */
    int32_t num_experts;  /* E: 1..256 */
    int32_t inter;        /* I: multiple of 128, 128..8192 */
    int32_t shared_inter; /* Is: 0 (no shared expert) or a multiple of 128, <= 8192 */
    int32_t block_rows;   /* R: 8, 16 or 32 for diffusion blocks (CMF model card, "Usage": block
                             size knob); 1, 2 or 4 for autoregressive decode (llama.cpp PR
                             #31306: the model in AR mode) and for verifying 1-4 drafted
                             candidates (InfiniLM PR #584, "Summary") */
    int32_t num_blocks;   /* B: 1..1024; N = B*R rows, block b is rows [b*R, (b+1)*R) */
    int32_t act_dtype;    /* cmoe_dtype of x and out: CMOE_F32 or CMOE_BF16 */
    int32_t weight_dtype; /* cmoe_dtype of the expert weights.  Supported pairs
                             (act, weight): (F32, F32), (BF16, BF16), (BF16, FP8_E4M3),
                             (BF16, FP4_E2M1) */
} cmoe_problem;

/* Storage of the expert weight matrices w13, w2, shared_w13 and shared_w2
 * (cmoe_weights.layout; one layout for all four).
 *
 *  CMOE_LAYOUT_ROWS:   [rows, cols] row-major, as described in cmoe_weights.
 *  CMOE_LAYOUT_PANELS: MFMA panels, the order in which the expert GEMMs read
 *                      the weights (16 rows at a time, 16 bytes per lane, 64
 *                      lanes per load), so that every load a wave issues is
 *                      1 KiB of whole, consecutive cache lines.  Made from the
 *                      row-major matrices by clover_moe_pack_weights, which
 *                      defines the byte order.  The kernels give every lane
 *                      the same weight bytes in the same registers in either
 *                      layout, so the results are bit-identical.
 * Scale arrays are row-major in both layouts. */
typedef enum {
    CMOE_LAYOUT_ROWS = 0,
    CMOE_LAYOUT_PANELS = 1
} cmoe_layout;

/* Weights (host struct of device pointers). */
/* Weight matrices are [rows, cols] row-major in weight_dtype (or MFMA panels
 * of those, see cmoe_layout); for FP4_E2M1 that is rows*cols/2 bytes.  Scale
 * arrays: FP8_E4M3: fp32, one per 128x128 block, [rows/128, cols/128] per
 * matrix; FP4_E2M1: uint8 E8M0, one per 32 elements of a row, [rows, cols/32]
 * per matrix; other dtypes: ignored. */
typedef struct {
    const float* router_w;        /* [E,H] fp32, required */
    const float* router_b;        /* [E] fp32 per-expert logit bias, or NULL */
    const void* w13;              /* [E,2I,H] weight_dtype: rows 0..I-1 gate, I..2I-1 up */
    const void* w13_scale;        /* fp8: [E,2I/128,H/128] fp32; fp4: [E,2I,H/32] uint8 */
    const void* w2;               /* [E,H,I] weight_dtype (down projection) */
    const void* w2_scale;         /* fp8: [E,H/128,I/128] fp32; fp4: [E,H,I/32] uint8 */
    const void* shared_w13;       /* [2Is,H] weight_dtype; required when Is > 0 */
    const void* shared_w13_scale; /* fp8: [2Is/128,H/128]; fp4: [2Is,H/32] */
    const void* shared_w2;        /* [H,Is] weight_dtype; required when Is > 0 */
    const void* shared_w2_scale;  /* fp8: [H/128,Is/128]; fp4: [H,Is/32] */
    int32_t layout;               /* cmoe_layout of w13, w2, shared_w13, shared_w2 */
} cmoe_weights;

/* Optional routing outputs (host struct of device pointers; each may be NULL). */
typedef struct {
    int32_t* topk_idx;       /* [N,k] chosen experts per slot, -1 for unused slots */
    float* gates;            /* [N,k] renormalised gates, 0 for unused slots */
    int32_t* coreset_ids;    /* [B,E] coreset of each block, by (mass desc, id asc), -1 padded */
    int32_t* coreset_size;   /* [B] |C_b| */
    int32_t* expert_counts;  /* [E] number of (row, slot) pairs routed to each expert */
    int32_t* expert_offsets; /* [E+1] exclusive prefix sum of expert_counts */
    int32_t* perm;           /* [N*k] row*k+slot of each routed pair in expert-major order
                                (experts ascending, then row ascending), -1 padded */
    float* logits;           /* [N,E] router logits */
    double* block_mass;      /* [B,E] routing mass of each expert in each block */
} cmoe_routing;

/* Options of one call (host struct; pass NULL for the defaults: no budget,
 * every row live).  They follow the expert-budget / live-row reuse of
 * InfiniLM PR #604 ("Summary"; "Motivation": live rows refreshed in full
 * every five passes, which is the caller's schedule: a refresh pass passes
 * live_rows = NULL).
 *
 *  expert_budget: 0 = none, else 1..E.  Each block's coreset is cut to its
 *                 first expert_budget experts in (mass desc, id asc) order,
 *                 after the threshold cut; coreset_size reports the cut size.
 *  live_rows:     [N] uint8, device, 16-byte aligned, or NULL = every row
 *                 live.  A row with 0 is resolved: it reuses the caller's
 *                 cached output (its row of `out` is not written), adds
 *                 nothing to its block's routing mass and takes no route
 *                 (topk_idx -1, gates 0).  A block with no live row has an
 *                 empty coreset (size 0, ids -1).  Its logits are still
 *                 computed.
 *  activation_fp8: 0 (default) or 1.  With 1, the expert GEMMs take their
 *                 activations in fp8 too (W8A8): x and h are rounded to
 *                 OCP MXFP8 (E4M3 codes, one E8M0 power-of-two scale per 32
 *                 consecutive elements of a row, the smallest scale that
 *                 keeps the group's largest magnitude within 448, codes
 *                 rounded to nearest even) and multiplied on the fp8
 *                 matrix cores.  The fp8 weights of InfiniLM PR #584
 *                 ("Benchmark") are served with bf16 activations; this is
 *                 an opt-in trade of accuracy for speed, checked against
 *                 the same oracle at a looser bound.  Only for fp8 weights
 *                 with bf16 activations, inter 512, shared_inter 0 or 512,
 *                 hidden 512, 1024 or 2048 and calls with many routed rows
 *                 per expert (work tiles of 32 rows or more: N*top_k above
 *                 about 4/3 E routed pairs);
 *                 other calls return CMOE_ERR_UNSUPPORTED.  Router, routing
 *                 and combine are unchanged.
 */
typedef struct {
    int32_t expert_budget;
    const uint8_t* live_rows;
    int32_t activation_fp8;
} cmoe_options;

/* Bytes of device workspace clover_moe_block_forward needs for this problem
 * and top_k (InfiniLM PR #604, "Checklist": mask, state and workspace bounds
 * and their lifetime are part of the checked contract).  Host-only; queues no
 * work.  Writes *bytes on success.
 *
 *  problem: host pointer; validated exactly as clover_moe_block_forward does
 *  top_k:   1..min(8, E)
 *  bytes:   host pointer, written on success only
 * Lifetime: the workspace is caller-owned device memory; a call may use it
 * until the work queued on its stream completes, and keeps nothing in it
 * between calls (its contents on entry do not matter).  Two calls whose
 * work may overlap in time need two workspaces.
 * Errors: CMOE_ERR_NULL (problem or bytes is NULL), and the CMOE_ERR_VALUE /
 * CMOE_ERR_UNSUPPORTED codes of the problem checks. */
cmoe_status clover_moe_workspace_size(const cmoe_problem* problem, int32_t top_k, size_t* bytes);

/* One MoE layer over B blocks (steps 1-6 above), queued on `stream`.
 *
 *  problem, weights, routing: host pointers to the structs above (routing may be NULL)
 *  x:               [N,H] act_dtype, device
 *  mass_threshold:  share of the block's routing mass the coreset must carry,
 *                   in (0, 1]; 1.0 = unrestricted top-k ("full route")
 *  top_k:           1..min(8, E); 4 = "preview" routing, 8 = the model's routing
 *  out:             [N,H] act_dtype, device; written, rounded once from fp32
 *  workspace:       device scratch of at least clover_moe_workspace_size() bytes;
 *                   its contents on entry do not matter
 *  stream:          hipStream_t to queue the work on (NULL = the default stream)
 */
cmoe_status clover_moe_block_forward(const cmoe_problem* problem, const cmoe_weights* weights,
                                     const void* x, float mass_threshold, int32_t top_k,
                                     void* out, const cmoe_routing* routing,
                                     void* workspace, size_t workspace_bytes, void* stream);

/* clover_moe_block_forward with options (see cmoe_options; NULL = none).
 * Errors: expert_budget outside [0, E] or activation_fp8 other than 0 or 1 is
 * CMOE_ERR_VALUE; activation_fp8 = 1 on a call it does not cover is
 * CMOE_ERR_UNSUPPORTED; a live_rows range that is misaligned or overlaps an
 * output is CMOE_ERR_ALIGN / CMOE_ERR_ALIAS. */
cmoe_status clover_moe_block_forward_ex(const cmoe_problem* problem, const cmoe_weights* weights,
                                        const void* x, float mass_threshold, int32_t top_k,
                                        const cmoe_options* options, void* out,
                                        const cmoe_routing* routing, void* workspace,
                                        size_t workspace_bytes, void* stream);

/* Largest workspace of clover_moe_block_forward_noalloc, in bytes (128 MiB:
 * enough for 64 blocks of 32 rows at H 2048, 256 experts, top-8, I 512). */
#define CLOVER_MOE_NOALLOC_MAX_WORKSPACE (128u * 1024u * 1024u)

/* clover_moe_block_forward_ex without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, serving loops
 * that must not call hipMalloc, harnesses that forbid allocation).
 *
 * The workspace is a static device array of CLOVER_MOE_NOALLOC_MAX_WORKSPACE
 * bytes inside the library, one per GPU, held from the first use on that GPU
 * until the process ends.  The call allocates nothing (no hipMalloc, no
 * hipFree, no allocating library routine); the first call on a device looks up
 * that device's array address once.
 *
 * Arguments and results are those of clover_moe_block_forward_ex; `stream`
 * must belong to the current device (NULL = its default stream).  Every call
 * on one GPU shares that GPU's array, which keeps the last call's contents
 * (no call depends on them): calls whose work may overlap on one GPU (other
 * streams, other threads) race and give undefined results; serialise them.
 * Errors: those of clover_moe_block_forward_ex; CMOE_ERR_WORKSPACE when the
 * problem needs more than CLOVER_MOE_NOALLOC_MAX_WORKSPACE bytes (see
 * clover_moe_workspace_size); CMOE_ERR_VALUE when the stream belongs to
 * another device; CMOE_ERR_HIP when the array's address cannot be taken. */
cmoe_status clover_moe_block_forward_noalloc(const cmoe_problem* problem, const cmoe_weights* weights,
                                             const void* x, float mass_threshold, int32_t top_k,
                                             const cmoe_options* options, void* out,
                                             const cmoe_routing* routing, void* stream);

/* Number of kernel stages clover_moe_block_forward queues, in order:
 * 0 router logits, 1 per-block routing (softmax, mass, coreset, top-k, gates;
 * a one-block call also builds the row permutation and the GEMM work list in
 * the same kernel, a call of several blocks in two kernels after it),
 * 2 gate/up GEMM + SwiGLU (with fp8 activations, after rounding x to MXFP8),
 * 3 down GEMM, 4 gate-weighted combine with the shared expert (empty when the
 * down GEMM writes `out` itself, see cmoe_plan_info). */
#define CLOVER_MOE_NUM_STAGES 5

/* Same operation as clover_moe_block_forward_ex, for profiling: records
 * stage_events[i] (i = 0..CLOVER_MOE_NUM_STAGES-1) on `stream` right before
 * stage i is queued and stage_events[CLOVER_MOE_NUM_STAGES] after the last
 * one.  stage_events points to n_events = CLOVER_MOE_NUM_STAGES + 1 host
 * hipEvent_t handles created by the caller (hipEventCreate); the library only
 * records them.  The elapsed time between events i and i+1 is the device time
 * of stage i. */
cmoe_status clover_moe_block_forward_staged(const cmoe_problem* problem, const cmoe_weights* weights,
                                            const void* x, float mass_threshold, int32_t top_k,
                                            const cmoe_options* options, void* out,
                                            const cmoe_routing* routing,
                                            void* workspace, size_t workspace_bytes, void* stream,
                                            void* const* stage_events, int32_t n_events);

/* Which grouped-GEMM kernels a call runs (InfiniLM PR #604, "Benchmark /
 * Performance Impact": the cost of each phase is measured apart from the
 * rest; a caller that times the stages of clover_moe_block_forward_staged
 * learns from this which kernel each stage timed).  Host-only: no device
 * work and no device needed.  The choice depends only on the problem's
 * shape and dtypes, top_k and options->activation_fp8. */
typedef enum {
    CMOE_GEMM_REGISTER = 0,     /* 16-row work tiles, operands in registers */
    CMOE_GEMM_LDS_TILED = 1,    /* taller tiles, activation tile staged in LDS */
    CMOE_GEMM_PERSISTENT = 2,   /* one workgroup per CU, runs of tiles */
    CMOE_GEMM_DOWN_COMBINE = 3  /* down GEMM and combine in one kernel (few routed pairs) */
} cmoe_gemm_kind;

typedef struct {
    int32_t tile_rows;      /* rows of a grouped-GEMM work tile: 16, 32, 64, 96 or 128 */
    int32_t gate_up;        /* cmoe_gemm_kind of stage 2 */
    int32_t down;           /* cmoe_gemm_kind of stage 3 */
    int32_t y_bytes;        /* bytes per element of the per-pair down outputs (2: bf16, 4: fp32) */
    int32_t kernels;        /* kernels queued per call */
} cmoe_plan_info;

/* Fills *info for a call of clover_moe_block_forward_ex with these
 * arguments.  options may be NULL (defaults); its live_rows pointer is not
 * read.  Errors: those of clover_moe_workspace_size, CMOE_ERR_NULL when info
 * is NULL, CMOE_ERR_VALUE for an activation_fp8 other than 0 or 1 and
 * CMOE_ERR_UNSUPPORTED when activation_fp8 = 1 does not cover the call (the
 * statuses clover_moe_block_forward_ex returns for them). */
cmoe_status clover_moe_plan_info(const cmoe_problem* problem, int32_t top_k, const cmoe_options* options,
                                 cmoe_plan_info* info);

/* Rearranges row-major expert weight matrices into MFMA panels
 * (CMOE_LAYOUT_PANELS).  Queued on `stream`; one pass over the bytes, nothing
 * converted or rounded, so packing is done once when the weights are loaded.
 *
 * Layout: a matrix of `rows` rows of `row_bytes` bytes becomes rows/16 panels
 * of 16 rows, stored one after another; panel p is row_bytes/64 units of
 * 1 KiB, and byte 16*l + b (l = 0..63, b = 0..15) of unit q of panel p is byte
 * 64*q + 16*(l/16) + b of panel row l%16.  Panel row i is matrix row 16p + i
 * when gate_up = 0 (w2, shared_w2).  When gate_up = 1 (w13, shared_w13:
 * rows = 2*inter, gate rows then up rows) panel p pairs gate and up: panel
 * row i is gate row 8p + i for i < 8 and up row inter + 8p + i - 8 for i >= 8.
 *
 *  src:       [count, rows, row_bytes] bytes, device, 16-byte aligned:
 *             count row-major matrices (w13 [E,2I,H] with count = E, w2 [E,H,I],
 *             or a shared matrix with count = 1)
 *  dst:       the same number of bytes, device, 16-byte aligned, not
 *             overlapping src; written
 *  count:     number of matrices, >= 1
 *  rows:      a multiple of 16
 *  row_bytes: a multiple of 64 (cols * bits per element / 8)
 *  gate_up:   1 for w13 and shared_w13, 0 for w2 and shared_w2
 *  stream:    hipStream_t (NULL = the default stream)
 * Errors: CMOE_ERR_NULL, CMOE_ERR_VALUE (a size outside its domain),
 * CMOE_ERR_ALIGN, CMOE_ERR_ALIAS (src and dst overlap), CMOE_ERR_HIP. */
cmoe_status clover_moe_pack_weights(const void* src, void* dst, int64_t count, int32_t rows,
                                    int32_t row_bytes, int32_t gate_up, void* stream);

/* Error reporting (InfiniLM PR #604, "Notes for Reviewers": unsupported
 * options are refused explicitly, so a caller must be able to tell why).
 *
 * clover_moe_status_string: static text of a status code (any value; unknown
 * codes give "unknown status").  The pointer is to static storage: never
 * freed, valid for the life of the process, safe from any thread.
 *
 * clover_moe_last_error: text describing the last non-OK status returned on
 * the calling thread (which argument, which value, which limit).  The
 * pointer is owned by the library and stays valid until the next call into
 * the library on the same thread; successful calls leave it unchanged. */
const char* clover_moe_status_string(cmoe_status status);
const char* clover_moe_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* CLOVER_MOE_H */
