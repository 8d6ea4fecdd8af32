// Internal interface between the host dispatcher (fg_api.cpp) and the
// kernel translation units. Not part of the public C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp32gemm.h"

namespace fg {

// Everything a GEMM kernel needs, passed by value as the kernel argument.
// Element counts and leading dimensions are in floats.
struct GemmParams {
    const float* A;
    const float* B;
    float* C;
    int32_t M, N, K;
    int32_t lda, ldb, ldc;
    float alpha, beta;
    int64_t a_extent;  // floats from A to one past the last element read
    int64_t b_extent;
    int64_t c_extent;
    int32_t tiles_m, tiles_n;
    int32_t group_m;   // tile rows per raster group
    int32_t flags;     // FLAG_* below
    // Split-K: workgroup (tile, blockIdx.y = s) sums k-tiles
    // [s * kt_per_split, (s + 1) * kt_per_split) and writes its result to
    // C + s * c_split_stride. One split: kt_per_split covers all of K and
    // c_split_stride is 0.
    int32_t kt_per_split;
    int64_t c_split_stride;
    // First tile id of the launch (grouped raster order); 0 for a whole GEMM.
    int32_t tile_base;
    // Fused epilogue (FLAG_EPI): C = act(alpha * r_i * c_j * acc + beta * C
    // + u_i + w_j). A null vector means ones (scales) or zeros (biases).
    const float* row_scale;  // r, M floats
    const float* col_scale;  // c, N floats
    const float* row_bias;   // u, M floats
    const float* col_bias;   // w, N floats
    int32_t act;             // ACT_* below
    // Quantised second output (FLAG_QUANT, which comes with FLAG_EPI): Q(i, j)
    // = quantize(final C(i, j)) at qout + (i * ldq + j) elements of QUANT_*.
    void* qout;
    int32_t ldq;
    int32_t qkind;           // QUANT_* below
    const float* qscale;     // QUANT_INT8_ROW: s_i, M floats
    int64_t q_extent;        // elements from qout to one past the last one written
};

enum : int32_t { QUANT_NONE = 0, QUANT_BF16 = 1, QUANT_INT8_ROW = 2 };

enum : int32_t { ACT_NONE = 0, ACT_RELU = 1, ACT_GELU = 2, ACT_SILU = 3 };

enum : int32_t {
    FLAG_VEC_A = 1,    // A rows start 16-byte aligned: 128-bit loads allowed
    FLAG_VEC_B = 2,
    FLAG_VEC_C = 4,    // C rows start 16-byte aligned: 128-bit loads/stores
    FLAG_BETA0 = 8,    // beta == 0: C is written, never read
    FLAG_XCD_REMAP = 16,  // remap workgroup ids so each XCD gets a contiguous tile range
    FLAG_VEC2_C = 32,  // C rows start 8-byte aligned: 64-bit loads/stores
    FLAG_EPI = 64,     // apply the fused epilogue (scales, biases, activation)
    FLAG_TILE_WS = 128,  // write each (tile, split) partial to its own dense
                         // BM x BN slot of C (ldc = BN): slot
                         // (tile id - tile_base) * splits + split
    FLAG_QUANT = 256,  // also write Q = quantize(C) (set together with FLAG_EPI)
    FLAG_VEC_Q = 512,  // Q rows start aligned to 4 elements: vector stores
};

// Launchers: enqueue one kernel on `stream`; return the HIP launch status.
// For the matrix-core kernels `id` is the table id of a line of the
// instance list (fg_mfma_instances.inc); for the others `variant` indexes the
// family's compile-time shapes. trans_a / trans_b select the operand layouts.
hipError_t launch_mfma(int id, int trans_a, int trans_b, const GemmParams& p,
                       hipStream_t stream);
// The same on an explicit grid: `tiles` workgroups along x (tile ids
// p.tile_base ..), `splits` along y (k ranges of p.kt_per_split k-tiles).
hipError_t launch_mfma_tiles(int id, int trans_a, int trans_b, const GemmParams& p,
                             int32_t tiles, int32_t splits, hipStream_t stream);
hipError_t launch_valu(int variant, int trans_a, int trans_b, const GemmParams& p,
                       hipStream_t stream);
// Few-row GEMM (memory-bound): op(B) streamed once per block of rows, on the
// vector ALU (blocks of up to 8 rows) or on the matrix cores (blocks of up to
// 64 rows). threads: workgroup size of the vector-ALU K x N form (0:
// automatic); kernel: 0 automatic (few_rows_on_valu), 1 vector ALU, 2 matrix
// cores.
// The automatic choice, from measurements on one MI355X (us at N = K = 8192,
// vector ALU / matrix cores): B stored K x N, one row 42.9 / 40.7, 4 rows
// 46.1 / 41.7, 8 rows 51.3 / 43.3; B stored N x K, one row 40.1 / 44.0, 4
// rows 41.6 / 43.9, 5 rows 55.0 / 43.6, 8 rows 57.0 / 44.1.
inline bool few_rows_on_valu(int64_t M, int trans_b) { return trans_b && M <= 4; }
hipError_t launch_skinny(int trans_a, int trans_b, const GemmParams& p, hipStream_t stream,
                         int threads = 0, int kernel = 0);
// C = beta * C (beta == 0: C = 0 without reading it); for K == 0 or alpha == 0.
// With FLAG_EPI: C = act(beta * C + u_i + w_j).
hipError_t launch_scale(const GemmParams& p, hipStream_t stream);
// Split-K reduction: C = alpha * sum_{s < splits} W_s + beta * C, where W_s is
// the dense M x N slice W + s * M * N; the sum runs in ascending s. With
// FLAG_EPI the fused epilogue is applied to that sum.
hipError_t launch_splitk_reduce(const float* W, int32_t splits, const GemmParams& p,
                                hipStream_t stream);
// Stream-K tail reduction: for tiles [p.tile_base, p.tile_base + count) of a
// bm x bn tiling, C = epilogue(sum_{s < splits} slot(tile, s)) with the slots
// written by an FLAG_TILE_WS launch (summed in ascending s).
hipError_t launch_tile_reduce(const float* W, int32_t splits, int32_t count, int32_t bm,
                              int32_t bn, const GemmParams& p, hipStream_t stream);
// Device address (this device's copy) and size of the scratch of
// fg_sgemm_splitk_noalloc (FG_NOALLOC_SCRATCH_MAX bytes), looked up
// once per device with the device current (fg_noalloc.hip).
hipError_t noalloc_scratch(void** ptr, size_t* bytes);

// Machine probes (fg_probe.hip): an MFMA-only loop and a streaming read.
hipError_t launch_probe_mfma(int workgroups, int iters, float* out, hipStream_t stream);
hipError_t launch_probe_read(const float* x, int64_t n4, int workgroups, float* out,
                             hipStream_t stream);
// One direct-to-LDS load of `bytes` (4 or 16) per lane, lanes reversed, LDS
// copied out (fg_probe.hip).
hipError_t launch_probe_lds_dma(const float* src, int bytes, float* out, hipStream_t stream);

}  // namespace fg
