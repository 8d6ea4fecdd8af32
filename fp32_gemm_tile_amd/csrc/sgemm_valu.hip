// SGEMM on the vector ALU (v_fma_f32): the comparison path for the matrix-core
// kernel.
//
// This is the register-blocked outer-product kernel of "Matmul II: register
// blocking, warp tiling, tensor cores", sections 3-4 (each thread owns a
// TM x TN block of C; at every k it reads TM values of A and TN of B from
// LDS and does TM*TN multiply-adds; A is kept transposed in LDS as As[k][m]
// so both operand reads are 128-bit), laid out for 64-wide wavefronts: a
// thread's TM rows are TM/4 groups of 4 consecutive rows spaced BM/(TM/4)
// apart (likewise columns), so each 128-bit LDS read of a wavefront covers
// distinct banks and each group of 4 columns is one 128-bit store.
//
// k-tiles of BK = 8 go through a 2-buffer LDS ring with register staging
// (load k-tile t+1 into registers while computing k-tile t; one barrier per
// k-tile). Every output element accumulates its k terms in ascending order
// with one fused multiply-add each.
#include "fg_device.h"

namespace fg {
namespace {

constexpr int kVBK = 8;

template <int BM, int BN, int TM, int TN, int TA, int TB>
__global__ void __launch_bounds__((BM / TM) * (BN / TN))
sgemm_valu_kernel(GemmParams p) {
    constexpr int TY = BM / TM, TX = BN / TN, NT = TY * TX;
    constexpr int GM = TM / 4, GN = TN / 4;          // groups of 4 rows / cols
    constexpr int SM = BM / GM, SN = BN / GN;        // spacing of the groups
    constexpr int A_VECS = BM * kVBK / 4, B_VECS = BN * kVBK / 4;
    constexpr int A_VPT = (A_VECS + NT - 1) / NT, B_VPT = (B_VECS + NT - 1) / NT;
    static_assert(TM % 4 == 0 && TN % 4 == 0, "thread tile in groups of 4");

    __shared__ f4 smem[(2 * BM * kVBK + 2 * BN * kVBK) / 4];
    float* sA = reinterpret_cast<float*>(smem);   // [2][BK][BM]
    float* sB = sA + 2 * BM * kVBK;                // [2][BK][BN]

    int tm, tn;
    map_tile(blockIdx.x, gridDim.x, p, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int tid = threadIdx.x;
    const int ty = tid / TX, tx = tid % TX;
    const bool vec_a = p.flags & FLAG_VEC_A, vec_b = p.flags & FLAG_VEC_B;
    const bool a_rows_in = m0 + BM <= p.M, b_rows_in = n0 + BN <= p.N;

    const int64_t a_org = TA ? (int64_t)m0 : (int64_t)m0 * p.lda;
    const int64_t a_kstep = TA ? (int64_t)kVBK * p.lda : (int64_t)kVBK;
    const int64_t b_org = TB ? (int64_t)n0 * p.ldb : (int64_t)n0;
    const int64_t b_kstep = TB ? (int64_t)kVBK : (int64_t)kVBK * p.ldb;

    f4 ra[A_VPT], rb[B_VPT];

    // Vector v of a k-tile: for a k-contiguous operand, tile row = v / 2
    // (m or n), k = 4 * (v % 2); for an mn-contiguous one, k = v / (BX/4),
    // m or n = 4 * (v % (BX/4)).
    auto load_tiles = [&](int kt) {
        const int k0 = kt * kVBK, k_left = p.K - k0;
        const bool k_in = k0 + kVBK <= p.K;
        const int64_t ao = a_org + kt * a_kstep, bo = b_org + kt * b_kstep;
        const __amdgpu_buffer_rsrc_t rsa = make_rsrc(p.A + ao, p.a_extent - ao);
        const __amdgpu_buffer_rsrc_t rsb = make_rsrc(p.B + bo, p.b_extent - bo);
        const f4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int q = 0; q < A_VPT; ++q) {
            const int v = tid + NT * q;
            if (v >= A_VECS) break;
            int rr, cc;  // row along the strided direction, first contiguous element
            if (TA) { rr = v / (BM / 4); cc = 4 * (v % (BM / 4)); }
            else    { rr = v / 2;        cc = 4 * (v % 2); }
            const uint32_t off = (uint32_t)(rr * p.lda + cc) * 4u;
            const bool fast = vec_a && k_in && a_rows_in;
            const int rows_left = TA ? k_left : p.M - m0;
            const int len = TA ? p.M - m0 : k_left;
            ra[q] = fast ? ld4(rsa, off)
                         : (rr < rows_left ? ld4_guard(rsa, off, cc, len, vec_a) : z);
        }
#pragma unroll
        for (int q = 0; q < B_VPT; ++q) {
            const int v = tid + NT * q;
            if (v >= B_VECS) break;
            int rr, cc;
            if (TB) { rr = v / 2;        cc = 4 * (v % 2); }
            else    { rr = v / (BN / 4); cc = 4 * (v % (BN / 4)); }
            const uint32_t off = (uint32_t)(rr * p.ldb + cc) * 4u;
            const bool fast = vec_b && k_in && b_rows_in;
            const int rows_left = TB ? p.N - n0 : k_left;
            const int len = TB ? k_left : p.N - n0;
            rb[q] = fast ? ld4(rsb, off)
                         : (rr < rows_left ? ld4_guard(rsb, off, cc, len, vec_b) : z);
        }
    };

    // Registers -> LDS as [k][m] and [k][n] (transposing k-contiguous operands).
    auto store_tiles = [&](int buf) {
        float* a = sA + buf * BM * kVBK;
        float* b = sB + buf * BN * kVBK;
#pragma unroll
        for (int q = 0; q < A_VPT; ++q) {
            const int v = tid + NT * q;
            if (v >= A_VECS) break;
            if (TA) {
                const int k = v / (BM / 4), m = 4 * (v % (BM / 4));
                *reinterpret_cast<f4*>(a + k * BM + m) = ra[q];
            } else {
                const int m = v / 2, k = 4 * (v % 2);
#pragma unroll
                for (int j = 0; j < 4; ++j) a[(k + j) * BM + m] = ra[q][j];
            }
        }
#pragma unroll
        for (int q = 0; q < B_VPT; ++q) {
            const int v = tid + NT * q;
            if (v >= B_VECS) break;
            if (TB) {
                const int n = v / 2, k = 4 * (v % 2);
#pragma unroll
                for (int j = 0; j < 4; ++j) b[(k + j) * BN + n] = rb[q][j];
            } else {
                const int k = v / (BN / 4), n = 4 * (v % (BN / 4));
                *reinterpret_cast<f4*>(b + k * BN + n) = rb[q];
            }
        }
    };

    float acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = 0.f;

    const int nk = (p.K + kVBK - 1) / kVBK;
    if (nk > 0) {
        load_tiles(0);
        store_tiles(0);
        if (nk > 1) load_tiles(1);
        __syncthreads();
    }
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        const float* a = sA + cur * BM * kVBK;
        const float* b = sB + cur * BN * kVBK;
#pragma unroll
        for (int k = 0; k < kVBK; ++k) {
            float av[TM], bv[TN];
#pragma unroll
            for (int g = 0; g < GM; ++g) {
                f4 v = *reinterpret_cast<const f4*>(a + k * BM + g * SM + 4 * ty);
                av[4 * g] = v[0]; av[4 * g + 1] = v[1]; av[4 * g + 2] = v[2]; av[4 * g + 3] = v[3];
            }
#pragma unroll
            for (int g = 0; g < GN; ++g) {
                f4 v = *reinterpret_cast<const f4*>(b + k * BN + g * SN + 4 * tx);
                bv[4 * g] = v[0]; bv[4 * g + 1] = v[1]; bv[4 * g + 2] = v[2]; bv[4 * g + 3] = v[3];
            }
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) acc[i][j] = __builtin_fmaf(av[i], bv[j], acc[i][j]);
        }
        if (kt + 1 < nk) {
            store_tiles(cur ^ 1);
            if (kt + 2 < nk) load_tiles(kt + 2);
        }
        __syncthreads();
    }

    const int64_t c_org = (int64_t)m0 * p.ldc + n0;
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(p.C + c_org, p.c_extent - c_org);
    const bool beta0 = p.flags & FLAG_BETA0;
    const bool vec_c = (p.flags & FLAG_VEC_C) && a_rows_in && b_rows_in;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int row = (i / 4) * SM + 4 * ty + (i % 4);
        if (m0 + row >= p.M) continue;
#pragma unroll
        for (int g = 0; g < GN; ++g) {
            const int col = g * SN + 4 * tx;
            const uint32_t off = (uint32_t)(row * p.ldc + col) * 4u;
            if (vec_c) {
                const f4 cin = beta0 ? f4{0.f, 0.f, 0.f, 0.f} : ld4(rc, off);
                f4 o;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    o[j] = epilogue_value<false>(p, acc[i][4 * g + j], cin[j], beta0, (int64_t)m0 + row,
                                          (int64_t)n0 + col + j);
                st4(rc, off, o);
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if (n0 + col + j < p.N) {
                        const float cin = beta0 ? 0.f : ld1(rc, off + 4 * j);
                        st1(rc, off + 4 * j,
                            epilogue_value<false>(p, acc[i][4 * g + j], cin, beta0, (int64_t)m0 + row,
                                           (int64_t)n0 + col + j));
                    }
                }
            }
        }
    }
}

template <int BM, int BN, int TM, int TN>
hipError_t launch_valu_shape(int ta, int tb, const GemmParams& p, hipStream_t s) {
    const dim3 grid(p.tiles_m * p.tiles_n), block((BM / TM) * (BN / TN));
    if (ta == 0 && tb == 0)
        hipLaunchKernelGGL((sgemm_valu_kernel<BM, BN, TM, TN, 0, 0>), grid, block, 0, s, p);
    else if (ta == 0 && tb == 1)
        hipLaunchKernelGGL((sgemm_valu_kernel<BM, BN, TM, TN, 0, 1>), grid, block, 0, s, p);
    else if (ta == 1 && tb == 0)
        hipLaunchKernelGGL((sgemm_valu_kernel<BM, BN, TM, TN, 1, 0>), grid, block, 0, s, p);
    else
        hipLaunchKernelGGL((sgemm_valu_kernel<BM, BN, TM, TN, 1, 1>), grid, block, 0, s, p);
    return hipGetLastError();
}

}  // namespace

// Variants (must match the VALU rows of the configuration table):
//   0: 128 x 128 workgroup tile, 8 x 8 per thread (256 threads)
//   1:  64 x  64 workgroup tile, 4 x 4 per thread (256 threads)
hipError_t launch_valu(int variant, int ta, int tb, const GemmParams& p, hipStream_t s) {
    switch (variant) {
        case 0: return launch_valu_shape<128, 128, 8, 8>(ta, tb, p, s);
        case 1: return launch_valu_shape<64, 64, 4, 4>(ta, tb, p, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace fg
