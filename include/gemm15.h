/*
 * gemm15.h -- C ABI of the gemm15 dense GEMM library for AMD MI355X (gfx950).
 *
 * The library computes the row-major product
 *
 *     C[M x N] = epi( A[M x K] x B[K x N] )
 *
 * with element (i, k) of A at A[i*K + k], (k, j) of B at B[k*N + j] and (i, j)
 * of C at C[i*N + j] (tutorial page "from CUDA tile parallelism to GEMM
 * kernels", section 4.1; SGEMM page, section 1.1). A and B are both FP16, both
 * BF16 or both FP32. Products and sums are FP32 whatever the input type
 * (DeepGEMM page, section 3.4: 16-bit inputs, FP32 accumulation). The work is
 * 2*M*N*K floating-point operations (SGEMM page, section 1.1).
 *
 * The optional epilogue runs on the FP32 accumulator in registers before the
 * single store of C (DeepGEMM page, section 1.2: activation, residual add and
 * vector scale fused into the GEMM instead of a second pass over C):
 *
 *     v = acc;  v *= scale (SCALE);  v += bias[j] (BIAS);
 *     v = GELU(v) = v * Phi(v) (GELU, exact-erf form);  v += resid[i][j] (RESID);
 *     C[i][j] = round_to_out_dtype(v)   (round to nearest, ties to even)
 *
 * GELU is evaluated in FP32: for FP32 output to within about 1e-7 |v| of the
 * exact-erf value; for BF16 / FP16 output (which rounds to 16 bits afterwards)
 * with a shorter fit, to within 2.5e-5 |v| and 6.1e-5 relative, a few percent of
 * the 16-bit rounding step.
 *
 * Plans: gemm_plan_create chooses a kernel configuration for the problem shape
 * from size buckets and caches the choice per exact shape, so repeated shapes
 * hit the cache (DeepGEMM page, sections 2.3 and 4.3: different tile parameters
 * per size bucket, a small-tile path for small M or N, cached configurations).
 *
 * Conventions of every entry point below:
 *  - All pointers to matrix data are DEVICE pointers (memory of the GPU that is
 *    current on the calling thread). The caller allocates and owns them; the
 *    library never frees or synchronises them and writes only C (and a
 *    workspace passed to it).
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    gemm_run* only enqueue work on it and return; results are ready when the
 *    stream reaches that point.
 *  - Errors are negative gemm_status codes; the creating calls return NULL and
 *    record the code for gemm_last_error(). No call aborts the process; launch
 *    failures are read back with hipGetLastError (tutorial page, section 7: check
 *    the error state after every launch).
 *  - Plans hold host state only; no call allocates device memory (scratch comes
 *    from a workspace the caller passes in). A plan is immutable after creation and
 *    may be run concurrently from several host threads and streams; runs that use a
 *    workspace need one workspace each while they overlap.
 *  - Debug aids read from the environment: GEMM15_LOG=1 prints each plan's
 *    configuration choice to stderr; GEMM15_POISON=1 makes every run fill C with NaN
 *    first (C with 4-byte aligned rows, and not when the residual shares C's memory),
 *    so elements a kernel leaves unwritten show (tutorial page, section 7: NaN
 *    results from unwritten or unsynchronised memory); GEMM15_FORCE_CONFIG=<name>
 *    forces one configuration for every plan.
 */
#ifndef GEMM15_H
#define GEMM15_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types of A and B (both the same), of C and of the residual. */
typedef enum gemm_dtype { GEMM_F32 = 0, GEMM_F16 = 1, GEMM_BF16 = 2 } gemm_dtype;

/* Epilogue flags, applied in the order SCALE, BIAS, GELU, RESID. */
enum {
  GEMM_EPI_BIAS = 1u,  /* v += bias[j]; bias is FP32 of length N, shared by all rows */
  GEMM_EPI_GELU = 2u,  /* v = v * Phi(v), Phi the standard normal CDF */
  GEMM_EPI_RESID = 4u, /* v += resid[i][j]; resid is M x N row-major of type out_dtype */
  GEMM_EPI_SCALE = 8u  /* v *= scale */
};

/* The epilogue of a plan. Passing NULL means {0, 1.0f, GEMM_F32}: plain C in FP32. */
typedef struct gemm_epilogue {
  uint32_t flags;    /* GEMM_EPI_* bits */
  float scale;       /* multiplier when GEMM_EPI_SCALE is set */
  int32_t out_dtype; /* gemm_dtype of C and of resid */
} gemm_epilogue;

typedef enum gemm_status {
  GEMM_OK = 0,
  GEMM_ERR_SHAPE = -1,     /* a dimension < 1, or a grid or index too large */
  GEMM_ERR_DTYPE = -2,     /* unknown dtype, out_dtype or epilogue flag */
  GEMM_ERR_NULL = -3,      /* NULL A, B or C, or NULL bias / resid when its flag is set */
  GEMM_ERR_ALIGN = -4,     /* a pointer not aligned to its element size */
  GEMM_ERR_NO_DEVICE = -5, /* no HIP device is visible */
  GEMM_ERR_HIP = -6,       /* a HIP runtime call or a kernel launch failed */
  GEMM_ERR_PLAN = -7,      /* NULL plan, or a plan used on another device than its own */
  GEMM_ERR_NOMEM = -8,     /* host or device memory for a plan could not be allocated */
  GEMM_ERR_CONFIG = -9,    /* a forced configuration does not exist or does not fit */
  GEMM_ERR_ARG = -10,      /* another invalid argument (batch < 1, a bad stride, ...) */
  GEMM_ERR_WORKSPACE = -11 /* the workspace passed is smaller than the plan needs, or the
                              plan has no configuration that runs without one */
} gemm_status;

/* Storage of the right operand B. */
enum {
  GEMM_B_KN = 0, /* B is K x N row-major (C = A B) */
  GEMM_B_NK = 1  /* B is given transposed: Bt is N x K row-major, C = A Bt^T (a linear
                    layer's weight in [out, in] order, or K of attention scores Q K^T) */
};

typedef struct gemm_plan gemm_plan;

/*
 * Create a plan for C = epi(A x B) with A M x K and B K x N of type `dtype`.
 * Chooses the kernel configuration (shape-bucket rules, exact-shape cache) for
 * the device current on the calling thread. Host work only: the plan owns no
 * device memory. A configuration that splits K (fp32 partial sums), or that
 * copies operands whose rows are not 16-byte multiples (K or N not a multiple
 * of 8, of 4 for fp32) into zero-padded rows, needs device scratch that the caller
 * passes to gemm_run_ws (size from gemm_plan_workspace_bytes). Rows that are not
 * 16-byte multiples with K <= 64 and M x N >= 2^22 need no copies: the one-slice
 * streaming kernel then reads them through registers (the "_u" configurations,
 * which take A and B at any element alignment and batch stride, with C and the
 * residual 4-byte aligned).
 * Returns NULL on error (see gemm_last_error()).
 */
gemm_plan* gemm_plan_create(int64_t M, int64_t N, int64_t K, int32_t dtype,
                            const gemm_epilogue* epi);

/*
 * As gemm_plan_create, with two extra inputs:
 *  batch_hint  expected batch of gemm_run_strided_batched calls (>= 1); the
 *              configuration is chosen for that many independent products.
 *  config      -1: choose automatically; otherwise the index of a configuration
 *              listed by gemm_config_name (GEMM_ERR_CONFIG if it cannot run this
 *              problem). Used by tuning sweeps and by tests of each kernel.
 */
gemm_plan* gemm_plan_create_ex(int64_t M, int64_t N, int64_t K, int32_t dtype,
                               const gemm_epilogue* epi, int64_t batch_hint, int32_t config);

/*
 * As gemm_plan_create_ex, with the storage of B: GEMM_B_KN (B is K x N row-major,
 * as for gemm_plan_create) or GEMM_B_NK (the B argument of gemm_run* is then Bt,
 * N x K row-major, and the plan computes C = epi(A Bt^T)). This is the operand
 * order of a linear layer whose weight is stored [out, in] (tutorial page,
 * section 2: Y = X W^T + b) and of attention scores Q K^T with K stored [S x D],
 * so no transposed copy is needed. With GEMM_B_NK both operands are K-contiguous,
 * as the matrix core reads them, and both stream straight into LDS.
 * Every dtype takes GEMM_B_NK (fp32: the f32d kernels with Bt slices loaded like
 * A's). It needs 16-byte aligned A, Bt and C base pointers and batch strides at
 * run time (GEMM_ERR_ALIGN otherwise); when K is not a multiple of 8 (4 for fp32)
 * a run with a workspace first copies A and Bt into zero-padded rows there
 * (without one: GEMM_ERR_WORKSPACE).
 * GEMM_ERR_ARG for another b_layout.
 */
gemm_plan* gemm_plan_create_layout(int64_t M, int64_t N, int64_t K, int32_t dtype,
                                   const gemm_epilogue* epi, int64_t batch_hint, int32_t config,
                                   int32_t b_layout);

/*
 * Device scratch, in bytes, that gemm_run_ws and gemm_run_strided_batched_ws use
 * for this plan (0 for most plans): the fp32 partial sums of a plan that splits K
 * (split x M x N floats, or split x rows x N for the few-row kernel), or the
 * zero-padded copies of A and/or B of a plan with padded operands (each copy's
 * rows rounded up to 8 elements, the B copy at the next 256-byte boundary).
 * Batch items of one call reuse it in stream order. Returns the size, or a
 * negative status (GEMM_ERR_PLAN for NULL).
 */
int64_t gemm_plan_workspace_bytes(const gemm_plan* plan);

/*
 * Enqueue C = epi(A x B) on `stream`.
 *  A      device, M x K row-major, plan dtype
 *  B      device, K x N row-major, plan dtype (N x K row-major for a GEMM_B_NK plan)
 *  bias   device, N FP32 values; required iff GEMM_EPI_BIAS, else ignored
 *  resid  device, M x N row-major of out_dtype; required iff GEMM_EPI_RESID, else
 *         ignored. resid may equal C (each element is read before it is written).
 *  C      device, M x N row-major of out_dtype; must not overlap A or B
 * Returns GEMM_OK, or GEMM_ERR_PLAN / _NULL / _ALIGN / _HIP. Pointers need only
 * element alignment; 16-byte aligned rows take the vector-load kernels.
 * Without a workspace, a plan that would use one runs its configuration that
 * needs none: the same kernel with K unsplit, or the scalar-load kernel in place
 * of padded copies (GEMM_ERR_WORKSPACE for a transposed-B plan with padded
 * operands, which has none). Nothing is allocated or copied.
 */
int gemm_run(const gemm_plan* plan, const void* A, const void* B, const float* bias,
             const void* resid, void* C, void* stream);

/*
 * gemm_run with caller-provided device scratch: `workspace` (256-byte aligned,
 * GEMM_ERR_ALIGN otherwise) of `workspace_bytes` >= gemm_plan_workspace_bytes(plan)
 * (GEMM_ERR_WORKSPACE otherwise); NULL with 0 bytes behaves as gemm_run. The
 * caller owns it; it must stay allocated until the run completes on `stream`, and
 * runs that overlap in time (other streams) need separate workspaces. Its contents
 * on entry do not matter: every byte a run reads back it has written first.
 * This is the path of the plan's chosen configuration (split-K partial sums, or
 * padded operand copies made into the workspace before the product).
 */
int gemm_run_ws(const gemm_plan* plan, const void* A, const void* B, const float* bias,
                const void* resid, void* C, void* workspace, int64_t workspace_bytes,
                void* stream);

/*
 * Enqueue `batch` independent products C_b = epi(A_b x B_b), b = 0..batch-1, with
 * A_b = A + b*strideA, B_b = B + b*strideB, C_b = C + b*strideC and residual
 * resid + b*strideR (strides in ELEMENTS of the respective type; a stride of 0
 * shares one operand across the batch). bias is shared by the whole batch.
 * This is the batched QK^T product of attention: per (batch, head) an
 * [S x D] x [D x S] GEMM (tutorial page, section 2; DeepGEMM page, section 1.1).
 * Same pointer rules and errors as gemm_run, plus GEMM_ERR_ARG for batch < 1 or a
 * negative stride.
 */
int gemm_run_strided_batched(const gemm_plan* plan, int64_t batch, const void* A,
                             int64_t strideA, const void* B, int64_t strideB, const float* bias,
                             const void* resid, int64_t strideR, void* C, int64_t strideC,
                             void* stream);

/*
 * For callers that cannot allocate memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): gemm_run_strided_batched with the
 * plan's chosen configuration, its scratch taken from a fixed array the library
 * holds on each GPU it runs on (gemm_noalloc_scratch_bytes() = 16 MiB, kept until
 * the process ends) instead of a caller workspace. The call allocates nothing and
 * calls no allocating routine. Every call on one GPU shares that GPU's array: calls
 * that overlap in time (other streams) race and must not be issued. Nothing in it
 * needs to start at zero (each run writes every byte it reads back). Same arguments
 * and errors as gemm_run_strided_batched, plus GEMM_ERR_WORKSPACE when the plan needs
 * more scratch than the array holds.
 */
int gemm_run_noalloc(const gemm_plan* plan, int64_t batch, const void* A, int64_t strideA,
                     const void* B, int64_t strideB, const float* bias, const void* resid,
                     int64_t strideR, void* C, int64_t strideC, void* stream);

/* Bytes of the per-GPU scratch array gemm_run_noalloc uses. */
int64_t gemm_noalloc_scratch_bytes(void);

/* gemm_run_strided_batched with caller-provided scratch, as gemm_run_ws. */
int gemm_run_strided_batched_ws(const gemm_plan* plan, int64_t batch, const void* A,
                                int64_t strideA, const void* B, int64_t strideB,
                                const float* bias, const void* resid, int64_t strideR, void* C,
                                int64_t strideC, void* workspace, int64_t workspace_bytes,
                                void* stream);

/*
 * Row softmax between the two batched products of attention (tutorial page,
 * section 2: attention is Q K^T, a softmax, then the product with V; DeepGEMM
 * page, section 3.4: the softmax denominator must be accumulated in FP32):
 *
 *     P[r][c] = exp(scale*S[r][c] - m_r) / sum_c' exp(scale*S[r][c'] - m_r),
 *     m_r = max_c scale*S[r][c]
 *
 * S      device, rows x cols FP32, row r at S + r*ld_s (ld_s >= cols, elements);
 *        the scores as gemm_run_strided_batched leaves them (rows = batch * M)
 * P      device, rows x cols of p_dtype (GEMM_F32, GEMM_F16 or GEMM_BF16), row r at
 *        P + r*ld_p; computed in FP32 and rounded once (nearest, ties to even).
 *        P must not overlap S.
 * scale  a finite multiplier applied to S before the softmax (1 for the plain form)
 * Enqueues one kernel on `stream` (a hipStream_t as void*; NULL = default) and
 * returns GEMM_OK, or GEMM_ERR_SHAPE (rows or cols < 1), GEMM_ERR_ARG (ld_s or
 * ld_p < cols, scale not finite), GEMM_ERR_DTYPE, GEMM_ERR_NULL, GEMM_ERR_ALIGN
 * (S not 4-byte or P not element aligned), GEMM_ERR_NO_DEVICE, GEMM_ERR_HIP.
 * Inputs are expected finite; a row whose scaled scores are all -inf has no
 * softmax and yields NaN.
 */
int gemm_softmax_rows(const float* S, int64_t rows, int64_t cols, int64_t ld_s, float scale,
                      void* P, int64_t ld_p, int32_t p_dtype, void* stream);

/*
 * The attention probabilities in one kernel: per batch item b,
 *
 *     P_b = softmax_rows(scale * Q_b K_b^T)      (as gemm_softmax_rows)
 *
 * i.e. the first product of attention and the softmax after it (tutorial page,
 * section 2) with the scores kept in FP32 registers: each workgroup holds whole
 * rows (32 query rows x every key), takes their maximum and the FP32 sum of
 * exp(s - max) there (DeepGEMM page, section 3.4), and writes P once, so the FP32
 * score matrix is never written to or read back from memory.
 *
 * Q      device, batch x M x D row-major of dtype (GEMM_BF16 or GEMM_F16), items
 *        contiguous (item b at Q + b*M*D)
 * Kmat   device, per item the keys: with k_layout GEMM_B_KN their transpose K^T,
 *        D x N row-major; with GEMM_B_NK the keys themselves, N x D row-major
 *        (a linear layer's [out x in] weight); item b at Kmat + b*N*D
 * P      device, batch x M x N row-major of p_dtype (GEMM_F32, GEMM_F16 or GEMM_BF16),
 *        computed in FP32 and rounded once (nearest, ties to even); must not
 *        overlap Q or Kmat
 * Limits: 1 <= N <= 512 keys and 8 <= D <= 64 (D % 8 == 0); with GEMM_B_KN also
 * N % 8 == 0; Q and Kmat 16-byte aligned, P aligned to its element; one item's
 * Q and P each under 2 GiB. scale finite.
 * Enqueues one kernel on `stream` (NULL = default) and returns GEMM_OK, or
 * GEMM_ERR_SHAPE (batch, M < 1, N or D out of range), GEMM_ERR_ARG (k_layout,
 * scale), GEMM_ERR_DTYPE, GEMM_ERR_NULL, GEMM_ERR_ALIGN, GEMM_ERR_NO_DEVICE,
 * GEMM_ERR_HIP. Q and Kmat must hold finite values.
 */
int gemm_attention_probs(const void* Q, const void* Kmat, int64_t batch, int64_t M, int64_t N,
                         int64_t D, int32_t dtype, int32_t k_layout, float scale, void* P,
                         int32_t p_dtype, void* stream);

/* Release a plan (host memory only). NULL is ignored. Runs already enqueued do not
 * use the plan object and may still be pending. */
void gemm_plan_destroy(gemm_plan* plan);

/* The status of the last failing gemm_plan_create* call on this thread (tutorial
 * page, section 7: report every failure to the caller). */
int gemm_last_error(void);

/* A static English message for a status code (never NULL; tutorial page, section 7). */
const char* gemm_strerror(int status);

/*
 * Write a one-line description of the plan (configuration name, tile, grid,
 * LDS bytes, split, workspace bytes) into buf (always NUL-terminated when
 * len > 0): the configuration the shape-bucket choice made (DeepGEMM page,
 * section 2.3), for logs and tuning. Returns the number of characters the full
 * line needs, or a negative status.
 */
int gemm_plan_describe(const gemm_plan* plan, char* buf, size_t len);

/* ---------------- host-only introspection (no GPU needed) ------------------ */

/* The hardware facts configuration choice depends on. */
typedef struct gemm_device_desc {
  int32_t cu_count;  /* compute units (256 on MI355X) */
  int32_t lds_bytes; /* LDS per workgroup (163840 on gfx950) */
} gemm_device_desc;

/* What a configuration choice resolves to. */
typedef struct gemm_choice {
  int32_t config;    /* index for gemm_config_name / gemm_plan_create_ex */
  int32_t kind;      /* 0 simple, 1 mfma16, 2 fp32 mfma, 3 few-row split-K, 4 optimisation-
                        ladder rung (by name only), 5 one K slice streaming over tiles */
  int32_t bm, bn, bk;
  int32_t threads;
  int32_t lds_bytes;
  int32_t split;     /* K split factor (1 = none): the few-row kernel's, or a tile
                        product's run as split-K partial sums */
  int64_t workgroups;
  int32_t packed;    /* bit 0: A, bit 1: B copied into 16-byte-padded rows before the kernel */
} gemm_choice;

/*
 * Choose a configuration for a problem on a described device, without touching
 * a GPU, through the same rules and exact-shape cache gemm_plan_create uses.
 * `aligned16` says whether A, B and C will be 16-byte aligned (the allocator's
 * usual guarantee). Returns GEMM_OK or a negative status.
 */
int gemm_select(const gemm_device_desc* dev, int64_t M, int64_t N, int64_t K, int32_t dtype,
                const gemm_epilogue* epi, int64_t batch_hint, int32_t aligned16,
                gemm_choice* out);

/* gemm_select for a given storage of B (GEMM_B_KN or GEMM_B_NK). */
int gemm_select_layout(const gemm_device_desc* dev, int64_t M, int64_t N, int64_t K,
                       int32_t dtype, const gemm_epilogue* epi, int64_t batch_hint,
                       int32_t aligned16, int32_t b_layout, gemm_choice* out);

/* Number of configurations compiled into the library. */
int gemm_config_count(void);

/* Name of configuration i (NULL when out of range). */
const char* gemm_config_name(int32_t i);

/* Exact-shape cache counters since load (any pointer may be NULL). */
void gemm_cache_stats(int64_t* hits, int64_t* misses, int64_t* entries);

#ifdef __cplusplus
}
#endif

#endif /* GEMM15_H */
