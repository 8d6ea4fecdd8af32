// Machine probes: the attainable fp32 matrix-core rate and HBM read rate of
// the device, measured with kernels that do nothing else. A GEMM's fraction
// of peak is quoted against both the published figures and these.
//
//   * mfma_probe_kernel: every wave runs `iters` rounds of four independent
//     v_mfma_f32_32x32x2_f32 chains (4096 FLOP each) on register operands,
//     with no memory traffic in the loop. One lane sum per thread is stored
//     at the end so the chains cannot be removed.
//   * read_probe_kernel: a grid-stride read of n floats with 128-bit loads,
//     16 KiB per workgroup per pass, one partial sum per wave stored.
//   * lds_dma_probe_kernel: the lane layout of one direct-to-LDS buffer load
//     (the GEMM loader assumes lane L's W floats land at LDS float W L).
#include "fg_device.h"

namespace fg {
namespace {

constexpr int kProbeThreads = 256;

__global__ void __launch_bounds__(kProbeThreads) mfma_probe_kernel(int iters, float* out) {
    // Operands in (0, 1): each MFMA adds at most 2 to an accumulator, so the
    // sums stay finite for any iteration count the host allows.
    const float a = 0.25f + (threadIdx.x & 63) * (1.0f / 512.0f);
    const float b = 0.75f - (threadIdx.x & 63) * (1.0f / 512.0f);
    f16v acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc[j], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[j][r];
    out[(int64_t)blockIdx.x * kProbeThreads + threadIdx.x] = s;
}

__global__ void __launch_bounds__(kProbeThreads) read_probe_kernel(const f4* __restrict__ x,
                                                                   int64_t n4, float* out) {
    // Each pass, a workgroup reads 4 x 256 consecutive 16-byte vectors (16 KiB,
    // four loads in flight per thread); the grid then strides past them.
    constexpr int kChunk = 4 * kProbeThreads;
    const int64_t stride = (int64_t)gridDim.x * kChunk;
    float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
    int64_t base = (int64_t)blockIdx.x * kChunk;
    for (; base + kChunk <= n4; base += stride) {
        const f4* p = x + base + threadIdx.x;
        const f4 v0 = p[0], v1 = p[kProbeThreads], v2 = p[2 * kProbeThreads], v3 = p[3 * kProbeThreads];
        s0 += (v0[0] + v0[1]) + (v0[2] + v0[3]);
        s1 += (v1[0] + v1[1]) + (v1[2] + v1[3]);
        s2 += (v2[0] + v2[1]) + (v2[2] + v2[3]);
        s3 += (v3[0] + v3[1]) + (v3[2] + v3[3]);
    }
    // At most one partial chunk is left, and only the workgroup whose turn it
    // is reaches it (base < n4 < base + kChunk).
    if (base < n4) {
        for (int64_t i = base + threadIdx.x; i < n4; i += kProbeThreads) {
            const f4 v = x[i];
            s0 += (v[0] + v[1]) + (v[2] + v[3]);
        }
    }
    float s = (s0 + s1) + (s2 + s3);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
    if ((threadIdx.x & 63) == 0) out[(int64_t)blockIdx.x * (kProbeThreads / 64) + (threadIdx.x >> 6)] = s;
}

// One wave, one direct-to-LDS buffer load of BYTES per lane: lane L fetches
// the W = BYTES / 4 floats at src[(63 - L) W ..] (lanes reversed, so that any
// other placement shows), then the wave copies the 64 W floats of the LDS
// buffer, prefilled with -1, to out.
template <int BYTES>
__global__ void __launch_bounds__(64) lds_dma_probe_kernel(const float* src, float* out) {
    constexpr int W = BYTES / 4;
    __shared__ float buf[64 * W];
    const int lane = threadIdx.x;
    for (int i = lane; i < 64 * W; i += 64) buf[i] = -1.f;
    __syncthreads();
    const __amdgpu_buffer_rsrc_t r = make_rsrc(src, 64 * W);
#if defined(__HIP_DEVICE_COMPILE__)
    const uint32_t voff = (uint32_t)((63 - lane) * W) * 4u;
    auto* lds = (__attribute__((address_space(3))) void*)buf;
    if constexpr (BYTES == 16)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds, 16, voff, 0, 0, 0);
    else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds, 4, voff, 0, 0, 0);
#else
    (void)r;
#endif
    __builtin_amdgcn_s_waitcnt(0);  // vmcnt, expcnt and lgkmcnt all zero
    __syncthreads();
    for (int i = lane; i < 64 * W; i += 64) out[i] = buf[i];
}

}  // namespace

hipError_t launch_probe_lds_dma(const float* src, int bytes, float* out, hipStream_t stream) {
    if (bytes == 16)
        hipLaunchKernelGGL(lds_dma_probe_kernel<16>, dim3(1), dim3(64), 0, stream, src, out);
    else if (bytes == 4)
        hipLaunchKernelGGL(lds_dma_probe_kernel<4>, dim3(1), dim3(64), 0, stream, src, out);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_probe_mfma(int workgroups, int iters, float* out, hipStream_t stream) {
    hipLaunchKernelGGL(mfma_probe_kernel, dim3(workgroups), dim3(kProbeThreads), 0, stream, iters,
                       out);
    return hipGetLastError();
}

hipError_t launch_probe_read(const float* x, int64_t n4, int workgroups, float* out,
                             hipStream_t stream) {
    hipLaunchKernelGGL(read_probe_kernel, dim3(workgroups), dim3(kProbeThreads), 0, stream,
                       reinterpret_cast<const f4*>(x), n4, out);
    return hipGetLastError();
}

}  // namespace fg
