/*
 * fp32gemm_probe -- machine probes that sit beside the GEMM in the same
 * library: the attainable fp32 matrix-core rate and HBM read rate of the
 * device, each measured by a kernel that does nothing else. A GEMM's
 * fraction of peak can then be quoted against the published figures and
 * against these measured ceilings. None of this is needed to call fg_sgemm.
 *
 * Same conventions as fp32gemm.h: device pointers owned by the caller, work
 * enqueued on `stream` without synchronising, errors reported through
 * fg_status / fg_last_bad_arg() / fg_last_error(), nothing enqueued when an
 * argument is rejected.
 */
#ifndef FP32GEMM_PROBE_H
#define FP32GEMM_PROBE_H

#include "fp32gemm.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * fg_probe_mfma: `workgroups` workgroups of four waves; every wave runs
 * `iterations` rounds of four independent v_mfma_f32_32x32x2_f32 chains on
 * register operands (no memory traffic), then each work-item stores one
 * float to out[workgroup * 256 + work-item] (the sum of its accumulators).
 *   1 workgroups : 1 .. 65536
 *   2 iterations : 1 .. 16777216
 *   3 out        : device memory for workgroups * 256 floats
 *   4 stream
 * Floating-point operations performed: fg_probe_mfma_flops(workgroups,
 * iterations) = workgroups * 4 * iterations * 4 * 4096.
 */
fg_status fg_probe_mfma(int32_t workgroups, int32_t iterations, float* out, hipStream_t stream);
double fg_probe_mfma_flops(int32_t workgroups, int32_t iterations);

/*
 * fg_probe_read: read n floats of x once with 128-bit loads (grid-stride over
 * `workgroups` workgroups of four waves) and store one partial sum per wave
 * to out[workgroup * 4 + wave]. Bytes read from memory: 4 * n.
 *   1 x          : device memory, 16-byte aligned (may be NULL when n == 0)
 *   2 n          : >= 0, a multiple of 4
 *   3 workgroups : 1 .. 65536
 *   4 out        : device memory for workgroups * 4 floats
 *   5 stream
 */
fg_status fg_probe_read(const float* x, int64_t n, int32_t workgroups, float* out,
                        hipStream_t stream);

/*
 * fg_probe_lds_dma: the lane layout of gfx950's direct-to-LDS buffer load,
 * which the GEMM's loader relies on (lane L's W = bytes_per_lane / 4 floats
 * written to LDS floats W L .. W L + W - 1 of the instruction's base). One
 * wave issues one such load in which lane L reads src[(63 - L) W ..], then
 * copies the 64 W floats of LDS to out; with that layout
 * out[W L + e] = src[(63 - L) W + e].
 *   1 src            : device memory, 64 * W floats
 *   2 bytes_per_lane : 4 (buffer_load_dword ... lds) or 16 (dwordx4)
 *   3 out            : device memory, 64 * W floats
 *   4 stream
 */
fg_status fg_probe_lds_dma(const float* src, int32_t bytes_per_lane, float* out,
                           hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* FP32GEMM_PROBE_H */
