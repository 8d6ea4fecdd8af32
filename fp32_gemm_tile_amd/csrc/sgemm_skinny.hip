// SGEMM for few rows of C (M small: the decode shape of "Matmul II: register
// blocking, warp tiling, tensor cores", section 8, where the kernel is a
// memory-bound GEMV and the game is bytes).
//
// With M <= 8 the product reads every element of op(B) once and does only
// 2*M flops per element, so the bound is HBM bandwidth, not the matrix
// cores: this kernel streams op(B) with coalesced 128-bit loads, keeps MR
// (1, 2, 4 or 8) rows of results per thread in registers, and reduces the
// per-thread partial sums in a fixed order (deterministic results). Larger M
// runs as ceil(M / MR) row blocks (blockIdx.y), each streaming op(B) again.
//
// Two layouts of op(B):
//   * B stored K x N (n contiguous): a workgroup owns 32 columns; lane
//     (g = lane % 8) loads columns 4g..4g+3 of one k row, the 32 lane-rows
//     of the workgroup (8 per wave) step through k together, so each wave
//     load covers 8 rows x 128 contiguous bytes. Partial sums over the 32
//     k classes are reduced with lane shuffles, then across waves in LDS.
//   * B stored N x K (k contiguous): a wave owns 4 columns and its 64 lanes
//     read 256 consecutive k of each (one 1 KiB load per column); the 64
//     lane partials of every (row, column) are reduced with shuffles.
// op(A) is read with ordinary (cached) loads: it is M x K, small next to B.
// Every global access goes through a buffer resource bounded by the matrix.
#include "fg_device.h"

namespace fg {
namespace {

constexpr int kSkinnyThreads = 256;
constexpr int kUnrollMN = 8;  // k steps in flight per lane (B stored K x N)
constexpr int kUnrollK = 2;   // 256-deep k blocks in flight per column (B stored N x K)

// op(A)(i, k) for the rows of this block; rows past M read as 0.
template <int MR, bool TA>
__device__ __forceinline__ void load_a(__amdgpu_buffer_rsrc_t ra, int lda, int rows_left, int k,
                                       float (&a)[MR]) {
#pragma unroll
    for (int m = 0; m < MR; ++m) {
        const uint32_t off = (uint32_t)(TA ? k * lda + m : m * lda + k) * 4u;
        a[m] = m < rows_left ? ld1(ra, off) : 0.f;
    }
}

// Sum of v over the lanes whose index differs only in the bits of `mask`
// (xor butterfly; every lane of a group ends with the same value).
template <int MASK>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1)
        if (MASK & o) v += __shfl_xor(v, o, 64);
    return v;
}

// PIPE: software-pipelined k loop (two blocks of op(B) in flight per wave,
// more registers); for grids of at most a few workgroups per CU, where the
// loads' latency is not hidden by other workgroups.
// NT: work-items per workgroup (256, 512 or 1024): its NT / 8 k classes split
// K inside the workgroup, so a larger workgroup keeps more of op(B) in flight
// per CU when the grid has about one workgroup per CU.
template <int MR, int TA, bool VEC, bool PIPE, int NT>
__global__ void __launch_bounds__(NT) skinny_mn_kernel(GemmParams p) {
    // B stored K x N. Workgroup: columns [n0, n0 + 32), rows [m0, m0 + MR).
    constexpr int NW = NT / 64;
    constexpr int NCLS = NT / 8;  // k classes
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane & 7;                 // column group: 4 columns
    const int rcls = (lane >> 3) + 8 * wave;  // k class 0 .. NCLS-1
    const int n0 = blockIdx.x * 32, m0 = blockIdx.y * MR;
    const int rows_left = p.M - m0;

    float acc[MR][4];
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[m][j] = 0.f;

    // With several rows, the block's op(A) values go through LDS: thread t
    // loads k = kb + t of every row once (coalesced for A stored M x K) and
    // each lane then reads the MR values of its k with 128-bit LDS reads,
    // instead of MR scattered global loads per k. Two buffers: one barrier
    // per k block.
    constexpr int KB = NCLS * kUnrollMN;  // k per block
    constexpr bool STAGE_A = MR > 1;
    __shared__ __attribute__((aligned(16))) float sa[STAGE_A ? 2 : 1][KB][MR];

    // Loads of k block kb: this thread's op(A) values for the LDS stage (issued
    // first, so that waiting for them leaves the B loads in flight) and its
    // kUnrollMN 128-bit pieces of op(B). Past K both read as 0.
    auto load_block = [&](int kb, float (&astage)[MR], f4 (&b)[kUnrollMN]) {
        // Buffer resources based at this k block keep the 32-bit offsets small.
        const int64_t a_org = TA ? (int64_t)kb * p.lda + m0 : (int64_t)m0 * p.lda + kb;
        const int64_t b_org = (int64_t)kb * p.ldb + n0;
        const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.A + a_org, p.a_extent - a_org);
        const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.B + b_org, p.b_extent - b_org);
        if constexpr (STAGE_A) {
            const int kk = threadIdx.x;
            if (kb + kk < p.K) {
                load_a<MR, TA>(ra, p.lda, rows_left, kk, astage);
            } else {
#pragma unroll
                for (int m = 0; m < MR; ++m) astage[m] = 0.f;
            }
        }
#pragma unroll
        for (int u = 0; u < kUnrollMN; ++u) {
            const int kk = rcls + NCLS * u;  // k - kb
            const uint32_t off = (uint32_t)(kk * p.ldb + 4 * g) * 4u;
            const f4 z = {0.f, 0.f, 0.f, 0.f};
            b[u] = kb + kk < p.K ? ld4_guard(rb, off, 4 * g, p.N - n0, VEC) : z;
        }
    };
    // The FMAs of k block kb (op(A) from LDS buffer `it & 1`, or from memory
    // for one row).
    auto compute_block = [&](int kb, int it, const float (&astage)[MR], const f4 (&b)[kUnrollMN]) {
        if constexpr (STAGE_A) {
            float* dst = &sa[it & 1][threadIdx.x][0];
#pragma unroll
            for (int m = 0; m < MR; ++m) dst[m] = astage[m];
            lds_barrier();
        }
        const int64_t a_org = TA ? (int64_t)kb * p.lda + m0 : (int64_t)m0 * p.lda + kb;
        const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.A + a_org, p.a_extent - a_org);
#pragma unroll
        for (int u = 0; u < kUnrollMN; ++u) {
            const int kk = rcls + NCLS * u;
            float a[MR];
            if constexpr (STAGE_A) {
                const float* src = &sa[it & 1][kk][0];
#pragma unroll
                for (int m = 0; m < MR; m += 4) {
                    if constexpr (MR >= 4) {
                        const f4 v = *reinterpret_cast<const f4*>(src + m);
                        a[m] = v[0]; a[m + 1] = v[1]; a[m + 2] = v[2]; a[m + 3] = v[3];
                    } else {
                        const f2 v = *reinterpret_cast<const f2*>(src);
                        a[0] = v[0]; a[1] = v[1];
                    }
                }
            } else if (kb + kk < p.K) {
                load_a<MR, TA>(ra, p.lda, rows_left, kk, a);
            } else {
#pragma unroll
                for (int m = 0; m < MR; ++m) a[m] = 0.f;
            }
#pragma unroll
            for (int m = 0; m < MR; ++m)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[m][j] = __builtin_fmaf(a[m], b[u][j], acc[m][j]);
        }
    };

    // Software pipeline over k blocks: the loads of block i + 1 are issued
    // before the FMAs of block i, so that each wave keeps two blocks of
    // op(B) in flight (two register sets, used alternately).
    // Without PIPE, one block at a time.
    if constexpr (PIPE) {
        float as0[MR], as1[MR];
        f4 b0[kUnrollMN], b1[kUnrollMN];
        if (p.K > 0) load_block(0, as0, b0);
        int it = 0;
        for (int kb = 0; kb < p.K; kb += 2 * KB, it += 2) {
            if (kb + KB < p.K) load_block(kb + KB, as1, b1);
            compute_block(kb, it, as0, b0);
            if (kb + KB >= p.K) break;
            if (kb + 2 * KB < p.K) load_block(kb + 2 * KB, as0, b0);
            compute_block(kb + KB, it + 1, as1, b1);
        }
    } else {
        int it = 0;
        for (int kb = 0; kb < p.K; kb += KB, ++it) {
            float as[MR];
            f4 b[kUnrollMN];
            load_block(kb, as, b);
            compute_block(kb, it, as, b);
        }
    }

    // Reduce over the 8 k classes of a wave (lane bits 3-5), then over the
    // waves through LDS, always in the same order.
    __shared__ float red[NW][MR][32];
    static_assert(KB == NT, "one staged k per thread");
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float s = group_sum<0x38>(acc[m][j]);
            if (lane < 8) red[wave][m][4 * g + j] = s;
        }
    __syncthreads();
    // One element of the MR x 32 block per thread (row t / 32, column t % 32):
    // the wave sums in fixed order, then the epilogue and a coalesced store.
    static_assert(MR * 32 <= NT, "one thread per element");
    {
        const int m = threadIdx.x >> 5, col = threadIdx.x & 31;
        if (m < MR && m < rows_left && col < p.N - n0) {
            float s = red[0][m][col];
#pragma unroll
            for (int w = 1; w < NW; ++w) s += red[w][m][col];
            const int64_t c_org = (int64_t)m0 * p.ldc + n0;
            const __amdgpu_buffer_rsrc_t rc = make_rsrc(p.C + c_org, p.c_extent - c_org);
            const bool beta0 = p.flags & FLAG_BETA0;
            const uint32_t off = (uint32_t)(m * p.ldc + col) * 4u;
            const float cin = beta0 ? 0.f : ld1(rc, off);
            st1(rc, off, epilogue_value(p, s, cin, beta0, (int64_t)m0 + m, (int64_t)n0 + col));
        }
    }
}

template <int MR, int TA, bool VEC>
__global__ void __launch_bounds__(kSkinnyThreads) skinny_k_kernel(GemmParams p) {
    // B stored N x K. Wave w of the workgroup: columns n0 + 4w .. n0 + 4w + 3,
    // rows [m0, m0 + MR); lane L reads k = kb + 4L .. 4L + 3 of each column.
    constexpr int NW = kSkinnyThreads / 64;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n0 = (blockIdx.x * NW + wave) * 4, m0 = blockIdx.y * MR;
    const int rows_left = p.M - m0, cols_left = p.N - n0;

    const bool vec_a = !TA && (p.flags & FLAG_VEC_A);
    float acc[MR][4];
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[m][c] = 0.f;

    for (int kb = 0; kb < p.K; kb += 256 * kUnrollK) {
        // Buffer resources based at this k block keep the 32-bit offsets small.
        const int64_t a_org = TA ? (int64_t)kb * p.lda + m0 : (int64_t)m0 * p.lda + kb;
        const int64_t b_org = (int64_t)n0 * p.ldb + kb;
        const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.A + a_org, p.a_extent - a_org);
        const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.B + b_org, p.b_extent - b_org);
        const int k_left = p.K - kb;
        f4 b[kUnrollK][4];
#pragma unroll
        for (int u = 0; u < kUnrollK; ++u) {
            const int kk = 256 * u + 4 * lane;  // k - kb
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const f4 z = {0.f, 0.f, 0.f, 0.f};
                const uint32_t off = (uint32_t)(c * p.ldb + kk) * 4u;
                b[u][c] = c < cols_left ? ld4_guard(rb, off, kk, k_left, VEC) : z;
            }
        }
#pragma unroll
        for (int u = 0; u < kUnrollK; ++u) {
            const int kk = 256 * u + 4 * lane;
            f4 a[MR];
            if (vec_a) {
#pragma unroll
                for (int m = 0; m < MR; ++m) {
                    const f4 z = {0.f, 0.f, 0.f, 0.f};
                    a[m] = m < rows_left ? ld4_guard(ra, (uint32_t)(m * p.lda + kk) * 4u, kk,
                                                     k_left, true)
                                         : z;
                }
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float t[MR];
                    if (kk + e < k_left) {
                        load_a<MR, TA>(ra, p.lda, rows_left, kk + e, t);
                    } else {
#pragma unroll
                        for (int m = 0; m < MR; ++m) t[m] = 0.f;
                    }
#pragma unroll
                    for (int m = 0; m < MR; ++m) a[m][e] = t[m];
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int m = 0; m < MR; ++m)
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        acc[m][c] = __builtin_fmaf(a[m][e], b[u][c][e], acc[m][c]);
        }
    }

    // Every lane ends up with every sum; lane 4m + c keeps element (m, c) and
    // the MR x 4 elements go through the epilogue side by side.
    float mine = 0.f;
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const float s = group_sum<0x3F>(acc[m][c]);
            if (lane == 4 * m + c) mine = s;
        }
    const int m = lane >> 2, c = lane & 3;
    if (m < MR && m < rows_left && c < cols_left) {
        const int64_t c_org = (int64_t)m0 * p.ldc + n0;
        const __amdgpu_buffer_rsrc_t rc = make_rsrc(p.C + c_org, p.c_extent - c_org);
        const bool beta0 = p.flags & FLAG_BETA0;
        const uint32_t off = (uint32_t)(m * p.ldc + c) * 4u;
        const float cin = beta0 ? 0.f : ld1(rc, off);
        st1(rc, off, epilogue_value(p, mine, cin, beta0, (int64_t)m0 + m, (int64_t)n0 + c));
    }
}

template <int MR, int NT>
void launch_mn(int ta, bool vec_b, bool pipe_req, dim3 grid, const GemmParams& p, hipStream_t s) {
    const dim3 block(NT);
    constexpr bool kCanPipe = NT < 1024;  // see launch_mr
    const bool pipe = kCanPipe && pipe_req;
    if (ta == 0) {
        if (vec_b) {
            if (pipe) hipLaunchKernelGGL((skinny_mn_kernel<MR, 0, true, kCanPipe, NT>), grid, block, 0, s, p);
            else hipLaunchKernelGGL((skinny_mn_kernel<MR, 0, true, false, NT>), grid, block, 0, s, p);
        } else {
            if (pipe) hipLaunchKernelGGL((skinny_mn_kernel<MR, 0, false, kCanPipe, NT>), grid, block, 0, s, p);
            else hipLaunchKernelGGL((skinny_mn_kernel<MR, 0, false, false, NT>), grid, block, 0, s, p);
        }
    } else {
        if (vec_b) {
            if (pipe) hipLaunchKernelGGL((skinny_mn_kernel<MR, 1, true, kCanPipe, NT>), grid, block, 0, s, p);
            else hipLaunchKernelGGL((skinny_mn_kernel<MR, 1, true, false, NT>), grid, block, 0, s, p);
        } else {
            if (pipe) hipLaunchKernelGGL((skinny_mn_kernel<MR, 1, false, kCanPipe, NT>), grid, block, 0, s, p);
            else hipLaunchKernelGGL((skinny_mn_kernel<MR, 1, false, false, NT>), grid, block, 0, s, p);
        }
    }
}

template <int MR>
hipError_t launch_mr(int ta, int tb, const GemmParams& p, hipStream_t s, int threads) {
    const bool vec_b = p.flags & FLAG_VEC_B;
    const int rblocks = (p.M + MR - 1) / MR;
    const dim3 block(kSkinnyThreads);
    if (tb == 0) {  // B stored K x N
        const dim3 grid((p.N + 31) / 32, rblocks);
        const int64_t wgs = (int64_t)grid.x * grid.y;
        // Workgroup size: `threads` when the caller forces one, else 512
        // work-items when the grid has at most one workgroup per CU (twice
        // the waves split K and keep more loads in flight), else 256.
        // Measured on one MI355X (GB/s at 256 / 512 / 1024 work-items):
        // 8 x 8192 x 8192 4377 / 5377 / 5350; 1 x 8192 x 8192 6266 / 6492 /
        // 6201; 32 x 8192 x 8192 (1024 workgroups) 2816 / 2145 / 1507.
        const int nt = threads > 0 ? threads : (wgs <= 256 ? 512 : 256);
        // Pipelined while the whole grid is resident at once (up to 3
        // workgroups of 256 per CU, the pipelined kernel's occupancy, or two
        // of 512;
        // measured: 8 x 4096 x 4096 36.5 -> 32.8 us, 8 x 8192 x 8192 67.6 ->
        // 62.6 us); beyond that the extra registers cost a round of
        // workgroups (64 x 4096 x 4096, 1024 workgroups: 49 us plain, 69
        // pipelined). With one row the loop is light enough that the plain
        // one streams as fast (1 x 8192 x 8192: 44.1 us plain, 45.8 pipelined).
        // (1024 work-items leave a wave 128 registers: too few for the
        // second register set, so that size is never pipelined)
        const int64_t resident = nt == 512 ? 512 : 3 * 256;
        const bool pipe = MR > 1 && nt < 1024 && wgs <= resident;
        if (nt == 1024)
            launch_mn<MR, 1024>(ta, vec_b, pipe, grid, p, s);
        else if (nt == 512)
            launch_mn<MR, 512>(ta, vec_b, pipe, grid, p, s);
        else
            launch_mn<MR, 256>(ta, vec_b, pipe, grid, p, s);
    } else {  // B stored N x K
        const int cols_per_wg = 4 * (kSkinnyThreads / 64);
        const dim3 grid((p.N + cols_per_wg - 1) / cols_per_wg, rblocks);
        if (ta == 0) {
            if (vec_b) hipLaunchKernelGGL((skinny_k_kernel<MR, 0, true>), grid, block, 0, s, p);
            else hipLaunchKernelGGL((skinny_k_kernel<MR, 0, false>), grid, block, 0, s, p);
        } else {
            if (vec_b) hipLaunchKernelGGL((skinny_k_kernel<MR, 1, true>), grid, block, 0, s, p);
            else hipLaunchKernelGGL((skinny_k_kernel<MR, 1, false>), grid, block, 0, s, p);
        }
    }
    return hipGetLastError();
}

}  // namespace

// Rows per block: 1, 2, 4 or 8 (the smallest power of two >= M, capped at 8).
// threads: workgroup size of the K x N kernel (0 = automatic, else 256, 512
// or 1024).
hipError_t launch_skinny(int ta, int tb, const GemmParams& p, hipStream_t s, int threads) {
    if (p.M <= 1) return launch_mr<1>(ta, tb, p, s, threads);
    if (p.M <= 2) return launch_mr<2>(ta, tb, p, s, threads);
    if (p.M <= 4) return launch_mr<4>(ta, tb, p, s, threads);
    return launch_mr<8>(ta, tb, p, s, threads);
}

}  // namespace fg
