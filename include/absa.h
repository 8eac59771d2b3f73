/*
 * absa.h - AB-Attention sampled block-sparse attention for AMD MI355X (gfx950).
 *
 * The method (AB-Attention) is described by two web pages:
 *   [edumints]  edumints blog, "AB-Attention: Video Difuzyon Transformer'larini
 *               Hizlandirmak Icin Dogru Blok Dikkat Mekanizmasi", sections
 *               "attention bottleneck" and "three innovations";
 *   [hamidun]   hamidun news, "AB-Attention speeds up video generation up to
 *               2.23x and skips 92% of attention compute" (Arabic), section
 *               "three techniques in AB-Attention" with its IBCS, SIP and
 *               kernel paragraphs.
 *
 * Per (batch b, head h, query block r) the library
 *   1. averages the 4 keys of every KV block                 [hamidun, IBCS]
 *   2. clusters the 128 queries of the block into C weighted
 *      centroids with a fixed number of Lloyd iterations, in
 *      the original token order                              [hamidun, IBCS;
 *                                                             edumints, IBCS]
 *   3. scores every KV block by the weighted softmax attention
 *      of the centroids toward its mean key                  [hamidun, IBCS]
 *   4. sets inclusion probabilities proportional to score,
 *      capped at 1 and summing to the budget, draws blocks
 *      with Philox4x32-10 and keeps -ln(p) as a logit offset [hamidun, SIP]
 *   5. runs softmax attention over the gathered 4-token blocks
 *      with the offsets added to the logits                  [hamidun, SIP and
 *                                                             kernel paragraphs]
 * Steps 1-4 build a plan, which the pages rebuild once every 4 denoising steps
 * and reuse in between [hamidun, kernel paragraph]; step 5 runs every step.
 * A dense flash-attention kernel from the same code is the comparator.
 *
 * Conventions for every call:
 *   - Tensor pointers are device pointers owned by the caller, contiguous
 *     [B, H, N, d] row-major, element type given by absa_dtype. Outputs have
 *     the inputs' dtype.
 *   - Supported shapes: d in {64, 128}; N a multiple of 4 with
 *     4 <= N <= 2^21; B, H >= 1 with B*H*ceil(N/128) < 2^31.
 *   - Work is queued on the given HIP stream (NULL = the null stream) and
 *     returns at once, except absa_plan_create / absa_plan_from_scores /
 *     absa_plan_import (which block until the plan is built) and the
 *     export calls (which copy to host memory).
 *   - Arguments are validated before any HIP call; a rejected call touches
 *     no device state. No C++ exception crosses this interface.
 *   - On failure a call returns a non-zero absa_status and records a detail
 *     message readable through absa_last_error() on the same thread.
 *   - Plans are immutable after creation and may be shared by concurrent
 *     attention calls; the caller must not destroy a plan while work that
 *     uses it is in flight.
 */
#ifndef ABSA_H
#define ABSA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The enums below cross the ABI as 32-bit integers. A C caller may pass any
 * int, so in C++ they carry a fixed underlying type: every int32 value is then
 * a valid value of the type, and an out-of-range one reaches the argument
 * checks (ABSA_ERR_UNSUPPORTED / ABSA_ERR_INVALID_ARG) instead of being
 * undefined behaviour. */
#ifdef __cplusplus
#define ABSA_ENUM_BASE : int32_t
#else
#define ABSA_ENUM_BASE
#endif

typedef enum absa_status ABSA_ENUM_BASE {
    ABSA_OK = 0,
    ABSA_ERR_INVALID_ARG = 1,   /* null pointer, value out of range, bad scores */
    ABSA_ERR_UNSUPPORTED = 2,   /* valid request this build does not implement  */
    ABSA_ERR_OUT_OF_MEMORY = 3, /* device allocation failed                     */
    ABSA_ERR_DEVICE = 4,        /* a HIP call failed                            */
    ABSA_ERR_PLAN_MISMATCH = 5  /* plan built for another (B, H, N, d)          */
} absa_status;

typedef enum absa_dtype ABSA_ENUM_BASE {
    ABSA_BF16 = 0,              /* bfloat16 storage; MFMA inputs as stored         */
    ABSA_F32 = 1                /* float32 storage; rounded to bf16 for the MFMA   */
} absa_dtype;

typedef struct absa_plan_s* absa_plan;

/* Sampling design of a plan (step 4). Both take each KV block with the same
 * capped probability p and weight it by 1/p [hamidun, SIP paragraph]:
 *   POISSON     one independent draw per block (Philox uniform u < p); the
 *               count per query block is K only in expectation.
 *   SYSTEMATIC  a fixed-size design for the pages' fixed budget per query
 *               block: sizes P = floor(p 2^40), one Philox uniform U per
 *               query block, and block j is taken iff a point U + k 2^40
 *               falls in its cumulative interval [P_0+..+P_{j-1},
 *               P_0+..+P_j). The count is K (K - 1 or K + 1 only where
 *               rounding left the fixed-point total off K 2^40), each block
 *               is taken with probability P 2^-40 exactly, and that is the
 *               p the plan records and weights by. */
typedef enum absa_sampling ABSA_ENUM_BASE {
    ABSA_SAMPLING_POISSON = 0,
    ABSA_SAMPLING_SYSTEMATIC = 1
} absa_sampling;

/* Plan parameters. query_block must be 128 and kv_block 4 (the sizes the
 * pages give: [hamidun, IBCS paragraph] 128-query blocks, [hamidun, kernel
 * paragraph] KV blocks of at most 4 tokens). n_clusters in [1, 16]
 * (pages: 8; the k-means keeps a row's centroids in registers and LDS and
 * the score tiles take 32 centroid slots, so larger counts return
 * ABSA_ERR_UNSUPPORTED); kmeans_iters in [1, 64] (pages: a fixed count, not stated;
 * default 4). budget_blocks = K, the KV blocks each query block samples in
 * expectation, in [1, N/4]. seed = the sampler's 64-bit Philox key; a plan
 * rebuilt at a later step takes a new seed. sampling = an absa_sampling
 * value (default POISSON). keep_intermediates != 0 keeps
 * the mean keys, centroids, weights and scores on the device for
 * absa_plan_export_intermediate; otherwise they are freed when the plan is
 * built. fused != 0 builds the plan with the second score pass and the SIP
 * count in one kernel [hamidun, IBCS paragraph into the SIP paragraph]: a
 * workgroup computes the scores of two query blocks into on-chip memory and
 * runs their water-filling and draws from there, so no score row goes
 * through device memory. The plan is bit-identical to the default path's.
 * It needs n_clusters <= 8, M = N/4 <= 20224 and keep_intermediates = 0
 * (ABSA_ERR_UNSUPPORTED otherwise). */
typedef struct absa_plan_params {
    int32_t query_block;
    int32_t kv_block;
    int32_t n_clusters;
    int32_t kmeans_iters;
    int64_t budget_blocks;
    uint64_t seed;
    int32_t keep_intermediates;
    int32_t sampling;           /* absa_sampling */
    int32_t fused;              /* 0: two score passes, then SIP; else fused */
} absa_plan_params;

/* Which retained intermediate absa_plan_export_intermediate copies. */
typedef enum absa_intermediate ABSA_ENUM_BASE {
    ABSA_INTER_MEAN_KEYS = 0,   /* float [B, H, M, d], M = N/4                   */
    ABSA_INTER_CENTROIDS = 1,   /* float [B, H, QB, C, d], QB = ceil(N/128)       */
    ABSA_INTER_WEIGHTS = 2,     /* float [B, H, QB, C]                            */
    ABSA_INTER_SCORES = 3       /* float [B, H, QB, M]                            */
} absa_intermediate;

/* Fill *out with the defaults: 128, 4, 8 clusters, 4 iterations, budget 1,
 * seed 0, keep_intermediates 0, POISSON sampling, fused 0. Returns
 * ABSA_ERR_INVALID_ARG on NULL. */
absa_status absa_plan_params_init(absa_plan_params* out);

/* Build a plan from Q and K: mean keys, IBCS k-means and scores, then SIP
 * probabilities, Philox draws and HT log-weights (steps 1-4 above). The
 * scores are within 1e-4 relative of their fp64 definition while the
 * centroid logits |c.kbar| / sqrt(d) stay below about 300 (the score
 * contraction runs on 22-bit block floating point operands, so its error
 * grows with the largest logit of the 4 query blocks sharing a tile).
 * q, k: device [B, H, N, d] of dtype. On success *out owns device memory
 * until absa_plan_destroy. The call synchronises the stream twice: once to
 * read the number of sampled blocks (the size of the plan's arrays, which
 * the host allocates), and once when the plan is complete (the build's
 * temporaries live in a per-device workspace that the next build reuses).
 * It returns with the plan complete, usable on any stream. B*H must not
 * exceed 65535 (ABSA_ERR_UNSUPPORTED). */
absa_status absa_plan_create(const void* q, const void* k, absa_dtype dtype,
                             int64_t B, int64_t H, int64_t N, int64_t d,
                             const absa_plan_params* params, void* hip_stream,
                             absa_plan* out);

/* Build a plan from caller-supplied IBCS scores (SIP only, step 4).
 * scores_dev: device float [B, H, QB, M]; every score must lie in [0, 1] and
 * every row must sum to less than 2, else ABSA_ERR_INVALID_ARG (checked on
 * the device, reported when the call returns). sampling: an absa_sampling
 * value, else ABSA_ERR_INVALID_ARG. Given the same fp32 scores, seed and
 * design, the plan (row pointers, indices, p) is bit-identical to the
 * documented fixed-point rule. Blocks like absa_plan_create. */
absa_status absa_plan_from_scores(const float* scores_dev, int64_t B, int64_t H,
                                  int64_t N, int64_t d, int64_t budget_blocks,
                                  uint64_t seed, int32_t sampling, void* hip_stream,
                                  absa_plan* out);

/* Build a plan from a host CSR: rowptr int64 [rows+1] (rowptr[0] = 0,
 * non-decreasing), idx int32 [nnz] strictly ascending within each row and in
 * [0, M), logw float [nnz] finite, p double [nnz] or NULL (then stored as
 * exp(-logw)). rows = B*H*ceil(N/128). The arrays are copied; the caller
 * keeps ownership. Blocks until the copy is done. */
absa_status absa_plan_import(const int64_t* rowptr, const int32_t* idx,
                             const float* logw, const double* p,
                             int64_t B, int64_t H, int64_t N, int64_t d,
                             void* hip_stream, absa_plan* out);

/* Shape of a plan; any output pointer may be NULL. shape4 receives
 * (B, H, N, d). */
absa_status absa_plan_info(absa_plan plan, int64_t* shape4, int64_t* rows,
                           int64_t* M, int64_t* nnz);

/* Copy the plan to host buffers sized from absa_plan_info: rowptr [rows+1],
 * idx [nnz], logw [nnz], p [nnz]; any pointer may be NULL. Synchronous. */
absa_status absa_plan_export(absa_plan plan, int64_t* rowptr, int32_t* idx,
                             float* logw, double* p);

/* Device address of the plan's retained IBCS scores, float [B, H, QB, M]
 * (QB = ceil(N/128), M = N/4, rows summing to 1), in *scores_dev; NULL when
 * the plan was built without keep_intermediates or by
 * absa_plan_from_scores / absa_plan_import. The memory belongs to the plan
 * (valid until absa_plan_destroy; do not write to it). It can be handed to
 * absa_plan_from_scores on the device, e.g. to draw a new plan from the
 * same scores with another seed or budget [hamidun, kernel paragraph: a
 * plan serves several steps]. ABSA_ERR_INVALID_ARG on NULL arguments. */
absa_status absa_plan_scores(absa_plan plan, const float** scores_dev);

/* Copy count elements starting at element offset of a retained intermediate
 * (see absa_intermediate) to host memory. ABSA_ERR_INVALID_ARG if the plan
 * did not keep intermediates or the range is out of bounds. Synchronous. */
absa_status absa_plan_export_intermediate(absa_plan plan, absa_intermediate which,
                                          int64_t offset, int64_t count, float* dst);

/* Gathered block-sparse attention (step 5): for every query of row (b,h,r),
 * softmax over the keys of the plan's KV blocks of that row with logit
 * z = q.k / sqrt(d) + logw(block), times V. o: device [B, H, N, d] of
 * dtype. A row whose plan holds no block gets zeros. bf16 MFMA products,
 * fp32 accumulation and softmax. q, k and v must be finite: a NaN or an
 * infinity among them gives an unspecified output (no error is reported).
 * (B, H, N, d) restate the tensors' shape, which the plan fixes:
 * ABSA_ERR_PLAN_MISMATCH if they differ from the plan's, so a tensor of
 * another layer is caught before any kernel runs. fp32 inputs are first
 * rounded to bf16 into temporaries from the library's memory pool. */
absa_status absa_sparse_attention(absa_plan plan, const void* q, const void* k,
                                  const void* v, void* o, absa_dtype dtype,
                                  int64_t B, int64_t H, int64_t N, int64_t d,
                                  void* hip_stream);

/* absa_sparse_attention for callers that cannot allocate device memory
 * (code under stream capture, serving loops, harnesses that forbid it):
 * the same arguments, kernels and result, and it calls no allocator. fp32
 * inputs are rounded to bf16 into a static scratch array that every device
 * the library runs on holds for the life of the process (24 MiB), so they
 * may hold at most 2^22 elements per tensor (B*H*N*d), else
 * ABSA_ERR_UNSUPPORTED; bf16 inputs use no scratch and have no limit. All
 * calls on one device share that scratch: fp32 calls that overlap in time
 * on one device (on different streams) race and give unspecified outputs.
 * Under stream capture the plan records no use, so the caller keeps the
 * plan alive while the captured work may run. */
absa_status absa_sparse_attention_noalloc(absa_plan plan, const void* q, const void* k,
                                          const void* v, void* o, absa_dtype dtype,
                                          int64_t B, int64_t H, int64_t N, int64_t d,
                                          void* hip_stream);

/* Dense softmax(Q K^T / sqrt(d)) V with the same tiles and arithmetic as
 * absa_sparse_attention (the comparator); q, k and v must be finite. */
absa_status absa_dense_attention(const void* q, const void* k, const void* v, void* o,
                                 absa_dtype dtype, int64_t B, int64_t H, int64_t N,
                                 int64_t d, void* hip_stream);

/* Free a plan (NULL is a no-op). Does not wait: the plan's device memory
 * goes back to the library's pool for that device (see
 * absa_release_cached_memory) in stream order, after the latest attention
 * call on the plan on each stream that used it. Work the caller queued on
 * the plan by other routes (a captured graph) must be finished first. */
void absa_plan_destroy(absa_plan plan);

/* The library allocates plans from one stream-ordered memory pool per
 * device, which keeps freed memory for the next plan instead of returning it
 * to the driver, and keeps one plan-building workspace per device for the
 * temporaries of absa_plan_create / absa_plan_from_scores (it grows to the
 * largest build: about 2.9 GB at B=1, H=40, N=75,600, d=128). This call
 * waits for the current device to go idle, frees that device's workspace
 * (unless a build on another thread holds it) and returns all cached, unused
 * pool memory to the system; live plans keep theirs. ABSA_ERR_DEVICE on a
 * HIP failure. */
absa_status absa_release_cached_memory(void);

/* Static name of a status code. */
const char* absa_status_string(absa_status status);

/* Detail message of the last failed call on this thread ("" if none). */
const char* absa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ABSA_H */
