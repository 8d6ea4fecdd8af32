/*
 * fp32gemm_tune -- hooks for tuning the tile-configuration table offline.
 * Host only; no GPU is needed for any of these.
 *
 * fg_sgemm picks a table entry with a cost model (see fg_select_config). For
 * every matrix-core entry the model holds two efficiencies: `eff`, the
 * fraction of the fp32 matrix peak one wave reaches with its SIMD full, and
 * `eff1`, the same with one wave per SIMD; the few-row entry has one (`eff`
 * divides its modelled time per step of K, `eff1` is ignored there). The
 * library starts from a
 * generated table of them (fg_tuned.inc, written by the package's autotune
 * module from timings of every entry on a grid of shapes), following the
 * empirical configuration search of "How to get a matmul kernel into the
 * top percentile (worklog)", section "Extra" (retune per GPU) and "Matmul
 * II: register blocking, warp tiling, tensor cores", section 8 (a library
 * carries a family of tile variants and chooses one per shape).
 *
 * Errors as in fp32gemm.h: fg_last_bad_arg() / fg_last_error().
 */
#ifndef FP32GEMM_TUNE_H
#define FP32GEMM_TUNE_H

#include "fp32gemm.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * The model's estimate, in seconds, of one call of M x N x K with table
 * entry config_id and `splits` split-K slices (values below 1 mean 1);
 * beta_zero != 0 when beta == 0. Matrix-core and few-row entries only;
 * returns -1 for a vector-ALU entry, an id out of range or a negative size.
 * The layout flags do not enter the present model.
 */
double fg_estimate_seconds(int64_t M, int64_t N, int64_t K, int32_t config_id, int32_t splits,
                           int32_t beta_zero);

/* The efficiencies of entry config_id (arguments 2, 3: outputs, non-NULL).
 * FG_ERR_INVALID_ARG (bad argument 1) for a vector-ALU entry (not modelled)
 * or an id out of range. */
fg_status fg_get_efficiency(int32_t config_id, double* eff, double* eff1);

/*
 * Replace the efficiencies of entry config_id (matrix-core or few-row) for
 * this process (both in (0, 1]). Every later selection, on every thread, uses them. For
 * tuners: a production build takes its values from fg_tuned.inc.
 */
fg_status fg_set_efficiency(int32_t config_id, double eff, double eff1);

/*
 * Raster order of the matrix-core kernels for every later call in this
 * process (for measurements, e.g. of how much each part of the order saves;
 * the defaults are what the library is tuned with):
 *   1 group_m   : output tiles are visited in bands of group_m tile rows,
 *                 column by column inside a band (0 = the default: 4 when B
 *                 is stored K x N, 8 when it is stored N x K; 1 = plain
 *                 row-major order); at most 4096
 *   2 xcd_remap : 1 (default) renumbers workgroups so that each of the 8
 *                 XCDs receives a contiguous run of tiles (when the grid is a
 *                 multiple of 8); 0 keeps the hardware's round-robin order
 * Process-wide; FG_ERR_INVALID_ARG outside these ranges. Results do not
 * depend on it (every tile computes the same sums in any order).
 */
fg_status fg_set_raster(int32_t group_m, int32_t xcd_remap);

/*
 * Workgroup size of the few-row kernel for B stored K x N (for measurements):
 * 0 (default) picks 512 work-items when the grid has at most one workgroup
 * per CU and 256 otherwise; 256, 512 or 1024 force that size for every later
 * call in this process. FG_ERR_INVALID_ARG otherwise.
 */
fg_status fg_set_few_row_threads(int32_t threads);

/*
 * Which kernel the few-row entry runs: 0 (the default) the vector-ALU kernel
 * up to 4 rows of C and the matrix-core kernel (rows padded to blocks of 16)
 * above; 1 always the vector-ALU kernel; 2 always the matrix-core kernel.
 * Process-wide, for tests and measurements. FG_ERR_INVALID_ARG otherwise.
 */
fg_status fg_set_few_row_kernel(int32_t kernel);

/*
 * As fg_select_config (fp32gemm.h), for a call that also writes a quantised
 * output of kind quant_kind (fg_quant_kind, argument 12): the entry
 * fg_sgemm_quant would run with config_id -1 (entries without the quantised
 * store are passed over). Argument 13: output. Host only.
 */
fg_status fg_select_config_quant(fg_op transA, fg_op transB, int64_t M, int64_t N, int64_t K,
                                 const float* A, int64_t lda, const float* B, int64_t ldb,
                                 const float* C, int64_t ldc, int32_t quant_kind,
                                 fg_config* out);

/*
 * The table entry and split-K slice count a call with config_id -1 runs,
 * from everything that decides them (fg_select_config takes beta = 0 and no
 * split): beta (argument 10; with beta != 0 the cost of reading C enters the
 * choice), splits (13) as fg_sgemm_splitk takes it (1: fg_sgemm, no split;
 * 0: the library's count, bounded by the workspace; > 1: that count, also
 * bounded by K as the call bounds it), workspace_bytes (14; 0 = no
 * workspace) and quant_kind (15, fg_quant_kind: the entry fg_sgemm_quant
 * runs). *out (16) receives the entry, *splits_out (17, may be NULL) the
 * slices the call runs (1 = none). The same validation and the same errors
 * as the call: FG_ERR_INVALID_ARG (bad argument 14) when the workspace holds
 * fewer slices than a requested count needs. Stream-K calls plan their own
 * split (fg_sgemm_streamk_workspace_size). Pointers are only inspected.
 * Host only.
 */
fg_status fg_select_config_ex(fg_op transA, fg_op transB, int64_t M, int64_t N, int64_t K,
                              const float* A, int64_t lda, const float* B, int64_t ldb,
                              float beta, const float* C, int64_t ldc, int32_t splits,
                              size_t workspace_bytes, int32_t quant_kind, fg_config* out,
                              int32_t* splits_out);

/*
 * Constants shared by the cost models of the table entries (fitted together
 * with the entries' efficiencies by the tuner and compiled in; settable for
 * a refit). FG_ERR_INVALID_ARG for an unknown constant (argument 1) or a
 * value outside its domain (argument 2: positive; at most 1 for fractions).
 */
typedef enum fg_model_constant {
    FG_MODEL_LAUNCH = 0,        /* seconds per further kernel launch */
    FG_MODEL_STORE_BW = 1,      /* bytes/s at which C tiles leave the CUs */
    FG_MODEL_STORE_EXPOSED = 2, /* fraction of those stores not hidden when several
                                   workgroups share a SIMD */
    FG_MODEL_STREAM_BW = 3,     /* bytes/s of one pass over the operands */
    FG_MODEL_SPLIT_BW = 4,      /* bytes/s of split-K and stream-K partial slices */
    FG_MODEL_FEW_FIXED = 5,     /* seconds of fixed cost of the few-row entry */
    FG_MODEL_FEW_MFMA = 6,      /* fraction of the matrix peak the few-row matrix-core
                                   kernel reaches on its padded rows */
    FG_MODEL_COUNT = 7
} fg_model_constant;
fg_status fg_get_model_constant(int32_t which, double* value);
fg_status fg_set_model_constant(int32_t which, double value);

/* The current raster settings (arguments 1, 2: outputs, non-NULL); group_m 0
 * means the default of each layout. */
fg_status fg_get_raster(int32_t* group_m, int32_t* xcd_remap);

/*
 * When fg_sgemm_streamk splits the last, partial round of tiles: policy 0
 * (the default) only when the cost model expects it to beat the plain call
 * by at least 3%; policy 1 whenever that round is at most three quarters
 * full (for tests and measurements). Process-wide. FG_ERR_INVALID_ARG for
 * any other value.
 */
fg_status fg_set_streamk_policy(int32_t policy);

#ifdef __cplusplus
}
#endif

#endif /* FP32GEMM_TUNE_H */
