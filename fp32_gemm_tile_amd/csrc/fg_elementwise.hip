// The memory-bound kernels around the GEMM proper:
//   * scale: C = beta * C (C = 0 without reading C when beta == 0), the
//     whole result when K == 0 or alpha == 0 (with the fused epilogue:
//     C = act(beta * C + u_i + w_j); with a quantised output, Q from it);
//   * split-K reduction: C = alpha * (W_0 + W_1 + ... + W_{S-1}) + beta * C,
//     summing the per-split partial products in ascending split order, so
//     the result does not depend on scheduling; the fused epilogue, when
//     asked for, is applied to that sum.
//   * stream-K tail reduction: the same sum over the per-tile partial slots
//     of a split tail of tiles, in ascending split order.
// All walk their window with a grid-stride loop; every index is inside
// the caller's buffers by construction, so plain global accesses are used.
#include "fg_device.h"

namespace fg {
namespace {

__global__ void __launch_bounds__(256) scale_kernel(GemmParams p) {
    const int64_t total = (int64_t)p.M * p.N;
    const bool beta0 = p.flags & FLAG_BETA0;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total;
         t += (int64_t)gridDim.x * blockDim.x) {
        const int64_t i = t / p.N, j = t - i * p.N;
        float* c = p.C + i * p.ldc + j;
        float o = beta0 ? 0.f : p.beta * *c;
        if (p.flags & FLAG_EPI) o = epi_finish(p, o, i, j);
        if (p.flags & FLAG_QUANT) quant_store1(p, i, j, o);
        *c = o;
    }
}

// VEC: N % 4 == 0, W 16-byte aligned and C rows 16-byte aligned, so each
// thread handles four consecutive columns with 128-bit accesses.
template <bool VEC>
__global__ void __launch_bounds__(256) splitk_reduce_kernel(const float* __restrict__ W,
                                                            int splits, GemmParams p) {
    const int64_t mn = (int64_t)p.M * p.N;
    const bool beta0 = p.flags & FLAG_BETA0;
    constexpr int V = VEC ? 4 : 1;
    const int64_t units = mn / V;
    for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < units;
         u += (int64_t)gridDim.x * blockDim.x) {
        const int64_t e = u * V;  // first element (row-major in the dense slices)
        const int64_t i = e / p.N, j = e - i * p.N;
        float* c = p.C + i * p.ldc + j;
        if constexpr (VEC) {
            f4 acc = *reinterpret_cast<const f4*>(W + e);
            for (int s = 1; s < splits; ++s) acc = acc + *reinterpret_cast<const f4*>(W + s * mn + e);
            const f4 cin = beta0 ? f4{0.f, 0.f, 0.f, 0.f} : *reinterpret_cast<const f4*>(c);
            f4 out;
#pragma unroll
            for (int q = 0; q < 4; ++q) out[q] = epilogue_value(p, acc[q], cin[q], beta0, i, j + q);
            *reinterpret_cast<f4*>(c) = out;
        } else {
            float acc = W[e];
            for (int s = 1; s < splits; ++s) acc += W[s * mn + e];
            *c = epilogue_value(p, acc, beta0 ? 0.f : *c, beta0, i, j);
        }
    }
}

// Stream-K tail: one thread per 4 consecutive columns of one row of one
// tile. The tile's S partial slots (dense bm x bn, ascending split order) are
// summed, then alpha / beta / the fused epilogue applied and C written.
// bn is a multiple of 4 and the slots are 16-byte aligned (host checks).
__global__ void __launch_bounds__(256) tile_reduce_kernel(const float* __restrict__ W,
                                                          int splits, int count, int bm, int bn,
                                                          GemmParams p) {
    const int quads = bn / 4;
    const int64_t per_tile = (int64_t)bm * quads;
    const int64_t units = per_tile * count;
    const int64_t slot = (int64_t)bm * bn;
    const bool beta0 = p.flags & FLAG_BETA0;
    const bool vec_c = p.flags & FLAG_VEC_C;
    for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < units;
         u += (int64_t)gridDim.x * blockDim.x) {
        const int t = (int)(u / per_tile);
        const int within = (int)(u - (int64_t)t * per_tile);
        const int r = within / quads, c4 = within - r * quads;
        int tm, tn;
        tile_coords(p.tile_base + t, p, tm, tn);
        const int64_t i = (int64_t)tm * bm + r, j = (int64_t)tn * bn + 4 * c4;
        if (i >= p.M || j >= p.N) continue;
        const float* w = W + (int64_t)t * splits * slot + (int64_t)r * bn + 4 * c4;
        f4 acc = *reinterpret_cast<const f4*>(w);
        for (int sp = 1; sp < splits; ++sp) acc = acc + *reinterpret_cast<const f4*>(w + sp * slot);
        float* c = p.C + i * p.ldc + j;
        if (vec_c && j + 3 < p.N) {
            const f4 cin = beta0 ? f4{0.f, 0.f, 0.f, 0.f} : *reinterpret_cast<const f4*>(c);
            f4 out;
#pragma unroll
            for (int q = 0; q < 4; ++q) out[q] = epilogue_value(p, acc[q], cin[q], beta0, i, j + q);
            *reinterpret_cast<f4*>(c) = out;
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (j + q < p.N) c[q] = epilogue_value(p, acc[q], beta0 ? 0.f : c[q], beta0, i, j + q);
        }
    }
}

unsigned grid_for(int64_t units) {
    int64_t blocks = (units + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    if (blocks < 1) blocks = 1;
    return (unsigned)blocks;
}

}  // namespace

hipError_t launch_scale(const GemmParams& p, hipStream_t s) {
    hipLaunchKernelGGL(scale_kernel, dim3(grid_for((int64_t)p.M * p.N)), dim3(256), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_splitk_reduce(const float* W, int32_t splits, const GemmParams& p,
                                hipStream_t s) {
    const int64_t mn = (int64_t)p.M * p.N;
    const bool vec = (p.N % 4 == 0) && (((uintptr_t)W & 15u) == 0) && (p.flags & FLAG_VEC_C);
    if (vec)
        hipLaunchKernelGGL(splitk_reduce_kernel<true>, dim3(grid_for(mn / 4)), dim3(256), 0, s,
                           W, splits, p);
    else
        hipLaunchKernelGGL(splitk_reduce_kernel<false>, dim3(grid_for(mn)), dim3(256), 0, s, W,
                           splits, p);
    return hipGetLastError();
}

hipError_t launch_tile_reduce(const float* W, int32_t splits, int32_t count, int32_t bm,
                              int32_t bn, const GemmParams& p, hipStream_t s) {
    const int64_t units = (int64_t)count * bm * (bn / 4);
    hipLaunchKernelGGL(tile_reduce_kernel, dim3(grid_for(units)), dim3(256), 0, s, W, splits,
                       count, bm, bn, p);
    return hipGetLastError();
}

}  // namespace fg
