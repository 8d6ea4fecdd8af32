/*
 * fp32gemm -- true-fp32 GEMM for AMD Instinct MI355X (gfx950).
 *
 *     C = alpha * op(A) * op(B) + beta * C
 *
 * Operation: the general matrix multiply as defined in "Optimising fp32 GEMM
 * on A100", section "What is GEMM?" (A is M x K, B is K x N, C is M x N,
 * alpha and beta scalars), with the BLAS-style argument list of "CuTe-ly
 * writing an SM86 SGEMM", section "host-side setup" (m, n, k, alpha, A, ldA,
 * B, ldB, beta, C, ldC, stream), extended by the two transpose flags.
 *
 * Arithmetic: binary32 inputs, binary32 products and accumulation on the
 * matrix cores (v_mfma_f32_32x32x2_f32, v_mfma_f32_16x16x4_f32) or on the
 * vector ALU, binary32
 * output. Nothing is converted to a narrower format.
 *
 * Storage convention: ROW-MAJOR with explicit leading dimensions (elements).
 *   op(A)(i,k) = A[i*lda + k]  when transA == FG_OP_N  (A stored M x K, lda >= K)
 *   op(A)(i,k) = A[k*lda + i]  when transA == FG_OP_T  (A stored K x M, lda >= M)
 *   op(B)(k,j) = B[k*ldb + j]  when transB == FG_OP_N  (B stored K x N, ldb >= N)
 *   op(B)(k,j) = B[j*ldb + k]  when transB == FG_OP_T  (B stored N x K, ldb >= K)
 *   C(i,j)     = C[i*ldc + j]                          (ldc >= N)
 * A column-major caller computes C^T = op(B)^T op(A)^T by swapping the
 * operands (and M with N).
 *
 * Ownership: the caller owns every buffer. A, B and C are device pointers
 * (e.g. from hipMalloc or a framework's allocator). The library allocates,
 * frees and copies nothing and keeps no workspace of its own (split-K takes
 * one from the caller), apart from the fixed device array that
 * fg_sgemm_splitk_noalloc uses instead. C must not overlap A or B.
 *
 * Streams: work is enqueued on `stream` (NULL = the null stream) and the call
 * returns without synchronising; C is complete once the stream reaches that
 * point. The library holds no per-stream state; calls are thread-safe.
 *
 * Errors: no exception or abort crosses this boundary. Invalid arguments are
 * reported before any GPU work is enqueued, and fg_last_bad_arg() then gives
 * the 1-based position of the first bad argument (BLAS numbering below).
 * fg_last_error() gives a message for the last failure on the calling thread.
 */
#ifndef FP32GEMM_H
#define FP32GEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same opaque type as HIP's hipStream_t, so HIP callers can pass theirs. */
typedef struct ihipStream_t* hipStream_t;

typedef enum fg_op { FG_OP_N = 0, FG_OP_T = 1 } fg_op;

typedef enum fg_status {
    FG_OK = 0,
    FG_ERR_INVALID_ARG = 1, /* an argument is out of its domain; nothing enqueued */
    FG_ERR_HIP = 2,         /* the HIP runtime reported an error (launch, device query) */
    FG_ERR_UNSUPPORTED = 3  /* valid BLAS arguments this library cannot run, e.g. a
                               device that is not gfx950 or a leading dimension
                               above FG_MAX_LD */
} fg_status;

/* Kernel families. */
typedef enum fg_kind {
    FG_KIND_MFMA = 1,  /* matrix-core contraction, v_mfma_f32_32x32x2_f32 or
                          v_mfma_f32_16x16x4_f32 (fg_config.mr) */
    FG_KIND_VALU = 2,  /* vector-ALU v_fma_f32 outer products (comparison path) */
    FG_KIND_SKINNY = 3 /* few rows of C (the GEMV shape, memory-bound): streams
                          op(B) once per block of rows, up to 64 on the matrix
                          cores (v_mfma_f32_16x16x4_f32, rows padded to 16) or
                          up to 8 on the vector ALU; chosen automatically only
                          up to 512 rows, and forced calls with more than
                          524280 rows return FG_ERR_UNSUPPORTED */
} fg_kind;

/* Largest leading dimension (elements) the kernels address with 32-bit
 * offsets. Larger values return FG_ERR_UNSUPPORTED. */
#define FG_MAX_LD 2097152

/* One entry of the tile-configuration table. */
typedef struct fg_config {
    int32_t id;        /* position in the table (0 .. fg_num_configs()-1) */
    int32_t kind;      /* fg_kind */
    int32_t bm, bn;    /* output tile of one workgroup (FG_KIND_SKINNY: rows per
                          block, and columns per workgroup when B is K x N) */
    int32_t bk;        /* depth of one k-tile staged in LDS */
    int32_t wm, wn;    /* output tile of one wavefront (MFMA) or thread (VALU) */
    int32_t threads;   /* work-items per workgroup */
    int32_t stages;    /* LDS buffers in the k-tile ring */
    int32_t lds_bytes; /* LDS per workgroup */
    int32_t mr;        /* FG_KIND_MFMA: edge of the instruction's output block,
                          32 (v_mfma_f32_32x32x2_f32) or 16
                          (v_mfma_f32_16x16x4_f32); 0 for the other kinds */
    char name[40];
} fg_config;

/*
 * fg_sgemm: C = alpha * op(A) * op(B) + beta * C on `stream`.
 *
 * Arguments (BLAS positions used by fg_last_bad_arg):
 *   1 transA, 2 transB : FG_OP_N or FG_OP_T
 *   3 M, 4 N, 5 K      : >= 0
 *   6 alpha
 *   7 A, 8 lda         : lda >= max(1, transA == FG_OP_N ? K : M)
 *   9 B, 10 ldb        : ldb >= max(1, transB == FG_OP_N ? N : K)
 *   11 beta
 *   12 C, 13 ldc       : ldc >= max(1, N)
 *   14 stream
 * A and B must be non-NULL when M, N and K are all > 0 and alpha != 0;
 * C must be non-NULL when M and N are > 0.
 *
 * Quick returns (BLAS convention; no kernel reads A or B):
 *   M == 0 or N == 0                       -> FG_OK, nothing enqueued
 *   (K == 0 or alpha == 0) and beta == 1   -> FG_OK, nothing enqueued
 *   (K == 0 or alpha == 0) otherwise       -> C = beta * C
 * When beta == 0, C is not read: NaN or Inf in C does not reach the result.
 */
fg_status fg_sgemm(fg_op transA, fg_op transB, int64_t M, int64_t N, int64_t K,
                   float alpha, const float* A, int64_t lda,
                   const float* B, int64_t ldb, float beta,
                   float* C, int64_t ldc, hipStream_t stream);

/*
 * fg_sgemm_ex: fg_sgemm with the tile configuration forced.
 * config_id = -1 selects automatically (same as fg_sgemm); otherwise it must
 * be a valid table index (else FG_ERR_INVALID_ARG, bad argument 15).
 */
fg_status fg_sgemm_ex(fg_op transA, fg_op transB, int64_t M, int64_t N, int64_t K,
                      float alpha, const float* A, int64_t lda,
                      const float* B, int64_t ldb, float beta,
                      float* C, int64_t ldc, hipStream_t stream,
                      int32_t config_id);

/*
 * fg_sgemm_splitk: fg_sgemm with the K dimension split across workgroups,
 * for shapes whose M x N grid of output tiles is too small to fill the GPU
 * (split-K as described in "Matmul II: register blocking, warp tiling,
 * tensor cores", section 8: several blocks share one output tile and their
 * partial sums are added).
 *
 * Each of S slices sums a contiguous range of k into a dense M x N binary32
 * partial in `workspace` (slice s at workspace + s*M*N floats); a second
 * kernel then writes C = alpha * (P_0 + P_1 + ... + P_{S-1}) + beta * C,
 * adding the slices in ascending order, so repeated calls give identical
 * bits. Both kernels run on `stream`.
 *
 * Arguments 1-13 as for fg_sgemm, then:
 *   14 splits          : 0 = choose (at most what the workspace holds),
 *                        1 = no split (same as fg_sgemm), S > 1 = S slices
 *                        (capped at the number of k-tiles of the
 *                        entry used)
 *   15 workspace       : device memory owned by the caller, 4-byte aligned
 *                        (16-byte alignment enables 128-bit accesses); may be
 *                        NULL when splits == 1 (or splits == 0: then no split)
 *   16 workspace_bytes : at least fg_sgemm_splitk_workspace_size(M, N, S) for
 *                        the S actually used, else FG_ERR_INVALID_ARG
 *   17 stream
 * The workspace must not overlap A, B or C and must not be used by another
 * call that may run at the same time.
 */
fg_status fg_sgemm_splitk(fg_op transA, fg_op transB, int64_t M, int64_t N, int64_t K,
                          float alpha, const float* A, int64_t lda,
                          const float* B, int64_t ldb, float beta,
                          float* C, int64_t ldc, int32_t splits,
                          void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * fg_sgemm_splitk_noalloc: fg_sgemm_splitk for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc). The partial slices go to a scratch array that is
 * part of the library's device code: each GPU the library runs on holds one
 * copy of FG_NOALLOC_SCRATCH_MAX bytes from module load until the process
 * ends. The call itself allocates and frees nothing (no hipMalloc, no
 * library routine that allocates).
 *
 * Arguments 1-13 as for fg_sgemm, then:
 *   14 splits : 0 = choose (at most what the scratch holds), 1 = no split,
 *               S > 1 = S slices; M * N * S * 4 bytes above
 *               FG_NOALLOC_SCRATCH_MAX is FG_ERR_INVALID_ARG (bad argument
 *               14), reported before any device call
 *   15 stream
 * Results are those of fg_sgemm_splitk with the same split count.
 * Sharing: every call on one GPU uses that GPU's single scratch array, which
 * keeps the last call's partial sums (each call writes every slice element
 * it reads back, so nothing needs clearing). Calls that can overlap on one
 * GPU -- on different streams, or from different host threads without
 * ordering -- race on it; serialise them (one stream, or events).
 */
#define FG_NOALLOC_SCRATCH_MAX (32u << 20)
fg_status fg_sgemm_splitk_noalloc(fg_op transA, fg_op transB, int64_t M, int64_t N,
                                  int64_t K, float alpha, const float* A, int64_t lda,
                                  const float* B, int64_t ldb, float beta,
                                  float* C, int64_t ldc, int32_t splits, hipStream_t stream);

/* FG_NOALLOC_SCRATCH_MAX as the library was built with it. Host only. */
size_t fg_sgemm_splitk_noalloc_max_bytes(void);

/* Activations of the fused epilogue (binary32). */
typedef enum fg_activation {
    FG_ACT_NONE = 0,
    FG_ACT_RELU = 1, /* max(x, 0); NaN stays NaN */
    FG_ACT_GELU = 2, /* x * Phi(x) = x * (1 + erf(x / sqrt(2))) / 2 (erf form) */
    FG_ACT_SILU = 3  /* x * sigma(x) = x / (1 + exp(-x)) */
} fg_activation;

/* Operations fused after the product; every vector is device memory owned by
 * the caller (any 4-byte alignment), or NULL for the neutral value. */
typedef struct fg_epilogue {
    const float* row_scale; /* r, M floats (NULL: ones) */
    const float* col_scale; /* c, N floats (NULL: ones) */
    const float* row_bias;  /* u, M floats (NULL: zeros) */
    const float* col_bias;  /* w, N floats (NULL: zeros) */
    int32_t activation;     /* fg_activation */
} fg_epilogue;

/*
 * fg_sgemm_fused: the GEMM with an epilogue fused into its store, as in the
 * closing remarks of "Optimising fp32 GEMM on A100", section "Performance
 * comparison" (operations after a GEMM are fused into it as an epilogue):
 *
 *     C(i,j) = act( alpha * r_i * c_j * (op(A) op(B))(i,j) + beta * C(i,j) + u_i + w_j )
 *
 * evaluated in binary32 in that order. Per-row / per-column scales, biases
 * and the activation set are this library's choice of epilogue (the page
 * names none).
 *
 * Arguments 1-13 as for fg_sgemm, then:
 *   14 epilogue  : NULL (plain GEMM) or a description as above; an activation
 *                  outside fg_activation is rejected
 *   15 stream
 *   16 config_id : -1 = automatic, else a table index (as fg_sgemm_ex)
 * Quick returns as for fg_sgemm, except that with any epilogue operation
 * (K == 0 or alpha == 0) and beta == 1 still runs: C = act(C + u_i + w_j).
 * With beta == 0, C is not read. No split-K here.
 */
fg_status fg_sgemm_fused(fg_op transA, fg_op transB, int64_t M, int64_t N, int64_t K,
                         float alpha, const float* A, int64_t lda,
                         const float* B, int64_t ldb, float beta,
                         float* C, int64_t ldc, const fg_epilogue* epilogue,
                         hipStream_t stream, int32_t config_id);

/* Formats of the quantised second output. */
typedef enum fg_quant_kind {
    FG_QUANT_NONE = 0,
    FG_QUANT_BF16 = 1,    /* uint16 codes: the bfloat16 nearest to C(i,j), ties to
                             even; overflow rounds to infinity, infinities stay,
                             every NaN becomes 0x7FC0 */
    FG_QUANT_INT8_ROW = 2 /* int8 codes: clamp(round_half_even(fl32(C(i,j) * s_i)),
                             -128, 127) with the caller's factor s_i of row i
                             (e.g. 127 / max_j |C(i,j)|); NaN gives 0 */
} fg_quant_kind;

/* Where and how fg_sgemm_quant writes Q. */
typedef struct fg_quant {
    int32_t kind;            /* fg_quant_kind */
    void* out;               /* Q: device memory owned by the caller, M rows of
                                ldq elements (2 bytes each for FG_QUANT_BF16, 1
                                for FG_QUANT_INT8_ROW); must not overlap A, B, C */
    int64_t ldq;             /* elements, >= max(1, N) */
    const float* row_factor; /* FG_QUANT_INT8_ROW: s, M floats (device memory) */
} fg_quant;

/*
 * fg_sgemm_quant: fg_sgemm_fused that also writes a quantised copy of the
 * result to a second buffer, in the same store ("Optimising fp32 GEMM on
 * A100", section "Performance comparison": quantisation is among the
 * operations fused into a GEMM's epilogue). C is written exactly as
 * fg_sgemm_fused writes it (binary32); then Q(i,j) = quantize(C(i,j)) for
 * every 0 <= i < M, 0 <= j < N, from that binary32 value. Elements of Q's
 * rows past N are not touched. 4-element-aligned rows of Q (ldq a multiple
 * of 4, out aligned to 4 elements) are written with vector stores.
 *
 * Arguments 1-13 as for fg_sgemm, then:
 *   14 epilogue  : NULL or as for fg_sgemm_fused
 *   15 quant     : NULL or kind FG_QUANT_NONE: same as fg_sgemm_fused; else
 *                  out non-NULL (when M, N > 0), ldq >= max(1, N) and at most
 *                  FG_MAX_LD, row_factor non-NULL for FG_QUANT_INT8_ROW
 *   16 stream
 *   17 config_id : -1 = automatic among the entries that write Q, else a
 *                  table index; the entries that do not (the vector-ALU
 *                  kernels, and matrix-core tiles whose accumulators take more
 *                  than 128 registers per lane: the 256 x 256 tile) are
 *                  FG_ERR_INVALID_ARG here
 * Quick returns as for fg_sgemm_fused, except that (K == 0 or alpha == 0)
 * with beta == 1 still writes Q (from C as it is). No split-K here.
 */
fg_status fg_sgemm_quant(fg_op transA, fg_op transB, int64_t M, int64_t N, int64_t K,
                         float alpha, const float* A, int64_t lda,
                         const float* B, int64_t ldb, float beta,
                         float* C, int64_t ldc, const fg_epilogue* epilogue,
                         const fg_quant* quant, hipStream_t stream, int32_t config_id);

/*
 * fg_sgemm_streamk: fg_sgemm with stream-K style scheduling of the last,
 * partial round of output tiles ("Matmul II: register blocking, warp tiling,
 * tensor cores", section 8: split-K when the tiles cannot fill the machine,
 * here only for the tiles that would otherwise run in a round of their own).
 *
 * The table entry is the one fg_sgemm would use. Its tiles that fill whole
 * rounds of resident workgroups run as usual; the remaining tiles (when they
 * would fill at most three quarters of a round, and the cost model expects
 * the split to gain at least 3%; see fg_set_streamk_policy in
 * fp32gemm_tune.h) are each split along K into
 * S slices, S chosen so that tiles x S fill one round, the partial sums go to
 * per-(tile, slice) slots of `workspace`, and a last kernel adds each tile's
 * slices in ascending order (repeated calls give identical bits) and applies
 * alpha and beta. Otherwise, or when the workspace holds fewer than two
 * slices per tail tile, it runs exactly as fg_sgemm.
 *
 * Arguments 1-13 as for fg_sgemm, then:
 *   14 workspace       : device memory owned by the caller, 16-byte aligned,
 *                        or NULL (then no split); must not overlap A, B or C
 *                        or be used by a call that may run at the same time
 *   15 workspace_bytes : its size; fg_sgemm_streamk_workspace_size gives what
 *                        the full plan needs (less is never an error: fewer
 *                        slices, or none)
 *   16 stream
 */
fg_status fg_sgemm_streamk(fg_op transA, fg_op transB, int64_t M, int64_t N, int64_t K,
                           float alpha, const float* A, int64_t lda,
                           const float* B, int64_t ldb, float beta,
                           float* C, int64_t ldc, void* workspace, size_t workspace_bytes,
                           hipStream_t stream);

/* Workspace bytes fg_sgemm_streamk would use for this call (the plan
 * depends on the shape and on the 16-byte alignment of A, B, lda and ldb;
 * pointers are inspected, never dereferenced). 0 when no tail is split or
 * the arguments are invalid. Host only. */
size_t fg_sgemm_streamk_workspace_size(fg_op transA, fg_op transB, int64_t M, int64_t N,
                                       int64_t K, const float* A, int64_t lda,
                                       const float* B, int64_t ldb);

/* Bytes of workspace fg_sgemm_splitk needs for `splits` slices of an M x N
 * result (0 when splits <= 1 or the result is empty). Host only. */
size_t fg_sgemm_splitk_workspace_size(int64_t M, int64_t N, int32_t splits);

/* Size of the tile-configuration table. Host only; no GPU needed. */
int32_t fg_num_configs(void);

/* Copy table entry `id` to *out. FG_ERR_INVALID_ARG if id is out of range or
 * out is NULL. Host only. */
fg_status fg_get_config(int32_t id, fg_config* out);

/*
 * The configuration fg_sgemm would use for this call with beta == 0 (shape,
 * layouts and the 16-byte alignment of the pointers and leading dimensions),
 * without launching anything; with beta != 0 the cost of reading C can change
 * the choice (fg_select_config_ex in fp32gemm_tune.h takes beta, a split-K
 * request and a quantised output). Pointers are only inspected, never
 * dereferenced; they may be NULL (then treated as 16-byte aligned). Same
 * validation as fg_sgemm. Host only.
 */
fg_status fg_select_config(fg_op transA, fg_op transB, int64_t M, int64_t N,
                           int64_t K, const float* A, int64_t lda,
                           const float* B, int64_t ldb, const float* C,
                           int64_t ldc, fg_config* out);

/* 1-based BLAS position of the first invalid argument of the last failing
 * call on this thread, or 0. */
int32_t fg_last_bad_arg(void);

/* Message for the last failure on this thread ("" if none). */
const char* fg_last_error(void);

/* Static name of a status code. */
const char* fg_status_string(fg_status status);

/* Version of this interface (incremented on incompatible changes). */
int32_t fg_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FP32GEMM_H */
