// SGEMM for few rows of C (M small: the decode shape of "Matmul II: register
// blocking, warp tiling, tensor cores", section 8, where the kernel is a
// memory-bound GEMV and the game is bytes).
//
// With a few rows the product reads every element of op(B) once and does only
// 2M flops per element, so the bound is HBM bandwidth: every kernel here
// streams op(B) once per block of rows with coalesced 128-bit loads and
// reduces partial sums in a fixed order (deterministic results).
//   * few_rows_mfma_kernel (the default): the products on
//     v_mfma_f32_16x16x4_f32 with the rows padded to blocks of 16 (up to 64
//     rows per pass), 16 waves of a workgroup splitting K for the same
//     columns, for either layout of op(B);
//   * skinny_mn_kernel (vector ALU, B stored K x N): 32 columns per
//     workgroup, 4 per lane, k-row classes down K, op(A) staged in LDS;
//   * skinny_k_kernel (vector ALU, B stored N x K; the automatic choice for
//     at most 4 rows): each wave reads 256 consecutive k of a column per
//     load, several waves split K for the same columns.
// op(A) is read with ordinary (cached) loads: it is M x K, small next to B.
// Every global access goes through a buffer resource bounded by the matrix.
#include "fg_device.h"

namespace fg {
namespace {

constexpr int kSkinnyThreads = 256;
constexpr int kUnrollMN = 8;  // k steps in flight per lane (B stored K x N)

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
// BIG: buffer resources rebased per k step (see load_block).
template <int MR, int TA, bool VEC, bool PIPE, int NT, bool BIG>
__global__ void __launch_bounds__(NT) skinny_mn_kernel(GemmParams p) {
    // B stored K x N. Workgroup: columns [n0, n0 + 32), rows [m0, m0 + MR).
    constexpr int NW = NT / 64;
    constexpr int NCLS = NT / 8;  // k classes
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
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
        // Buffer resources are based at this k block, or with BIG (a leading
        // dimension so large that 32-bit byte offsets across a whole block
        // could pass 2^32) close to each access: this wave's k range of
        // op(A), each k step of op(B).
        if constexpr (STAGE_A) {
            const int ka = BIG ? kb + 64 * wave : kb;
            const int kt = BIG ? lane : (int)threadIdx.x;  // k - ka
            const int64_t a_org = TA ? (int64_t)ka * p.lda + m0 : (int64_t)m0 * p.lda + ka;
            const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.A + a_org, p.a_extent - a_org);
            if (ka + kt < p.K) {
                load_a<MR, TA>(ra, p.lda, rows_left, kt, astage);
            } else {
#pragma unroll
                for (int m = 0; m < MR; ++m) astage[m] = 0.f;
            }
        }
        const int64_t b_blk = (int64_t)kb * p.ldb + n0;
        const __amdgpu_buffer_rsrc_t rb_blk = make_rsrc(p.B + b_blk, p.b_extent - b_blk);
#pragma unroll
        for (int u = 0; u < kUnrollMN; ++u) {
            const int ku = kb + NCLS * u;  // first k of this step
            const f4 z = {0.f, 0.f, 0.f, 0.f};
            if constexpr (BIG) {
                const int64_t b_org = (int64_t)ku * p.ldb + n0;
                const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.B + b_org, p.b_extent - b_org);
                const uint32_t off = (uint32_t)(rcls * p.ldb + 4 * g) * 4u;
                b[u] = ku + rcls < p.K ? ld4_guard(rb, off, 4 * g, p.N - n0, VEC) : z;
            } else {
                const uint32_t off = (uint32_t)((ku - kb + rcls) * p.ldb + 4 * g) * 4u;
                b[u] = ku + rcls < p.K ? ld4_guard(rb_blk, off, 4 * g, p.N - n0, VEC) : z;
            }
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
                const int ku = BIG ? kb + NCLS * u : kb;
                const int64_t a_org = TA ? (int64_t)ku * p.lda + m0 : (int64_t)m0 * p.lda + ku;
                const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.A + a_org, p.a_extent - a_org);
                load_a<MR, TA>(ra, p.lda, rows_left, kb + kk - ku, a);
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

// B stored N x K. CW: columns per wave; KW: waves that share those columns
// and split K between them (k blocks taken round robin, partial sums reduced
// in LDS in a fixed order); UK: 256-deep k steps per block; PIPE: the loads
// of the next block are issued before the FMAs of this one (two register
// sets).
template <int MR, int TA, bool VEC, int CW, int KW, int UK, bool PIPE>
__global__ void __launch_bounds__(kSkinnyThreads) skinny_k_kernel(GemmParams p) {
    // Wave w of the workgroup: columns n0 .. n0 + CW - 1 of column group
    // w / KW, k blocks j with j % KW == w % KW; rows [m0, m0 + MR). Lane L
    // reads k = kb + 256 u + 4L .. 4L + 3 of each column.
    constexpr int NW = kSkinnyThreads / 64;
    static_assert(NW % KW == 0, "waves split evenly over column groups");
    constexpr int NG = NW / KW;  // column groups per workgroup
    constexpr int KB = 256 * UK;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int grp = wave / KW, phase = wave % KW;
    const int n0 = (blockIdx.x * NG + grp) * CW, m0 = blockIdx.y * MR;
    const int rows_left = p.M - m0, cols_left = p.N - n0;
    const bool vec_a = !TA && (p.flags & FLAG_VEC_A);

    float acc[MR][CW];
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int c = 0; c < CW; ++c) acc[m][c] = 0.f;

    // One block's loads: op(A) first, then op(B), so that waiting for this
    // block leaves the next block's loads (issued later) in flight. Past K
    // everything reads as 0. Buffer resources are based at each 256-deep k
    // step, so the 32-bit offsets stay below 256 * lda * 4 bytes.
    auto load_block = [&](int kb, f4 (&a)[UK][MR], f4 (&b)[UK][CW]) {
#pragma unroll
        for (int u = 0; u < UK; ++u) {
            const int ku = kb + 256 * u, kk = 4 * lane, left = p.K - ku;
            const int64_t a_org = TA ? (int64_t)ku * p.lda + m0 : (int64_t)m0 * p.lda + ku;
            const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.A + a_org, p.a_extent - a_org);
            const f4 z = {0.f, 0.f, 0.f, 0.f};
            if (vec_a) {
#pragma unroll
                for (int m = 0; m < MR; ++m)
                    a[u][m] = m < rows_left
                                  ? ld4_guard(ra, (uint32_t)(m * p.lda + kk) * 4u, kk, left, true)
                                  : z;
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float t[MR];
                    if (kk + e < left) {
                        load_a<MR, TA>(ra, p.lda, rows_left, kk + e, t);
                    } else {
#pragma unroll
                        for (int m = 0; m < MR; ++m) t[m] = 0.f;
                    }
#pragma unroll
                    for (int m = 0; m < MR; ++m) a[u][m][e] = t[m];
                }
            }
        }
        const int64_t b_org = (int64_t)n0 * p.ldb + kb;
        const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.B + b_org, p.b_extent - b_org);
        const int k_left = p.K - kb;
#pragma unroll
        for (int u = 0; u < UK; ++u) {
            const int kk = 256 * u + 4 * lane;  // k - kb
#pragma unroll
            for (int c = 0; c < CW; ++c) {
                const f4 z = {0.f, 0.f, 0.f, 0.f};
                const uint32_t off = (uint32_t)(c * p.ldb + kk) * 4u;
                b[u][c] = c < cols_left ? ld4_guard(rb, off, kk, k_left, VEC) : z;
            }
        }
    };
    auto compute_block = [&](const f4 (&a)[UK][MR], const f4 (&b)[UK][CW]) {
#pragma unroll
        for (int u = 0; u < UK; ++u)
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int m = 0; m < MR; ++m)
#pragma unroll
                    for (int c = 0; c < CW; ++c)
                        acc[m][c] = __builtin_fmaf(a[u][m][e], b[u][c][e], acc[m][c]);
    };

    const int k0 = phase * KB;
    constexpr int KSTEP = KW * KB;
    if constexpr (PIPE) {
        f4 a0[UK][MR], a1[UK][MR], b0[UK][CW], b1[UK][CW];
        if (k0 < p.K) load_block(k0, a0, b0);
        for (int kb = k0; kb < p.K; kb += 2 * KSTEP) {
            if (kb + KSTEP < p.K) load_block(kb + KSTEP, a1, b1);
            compute_block(a0, b0);
            if (kb + KSTEP >= p.K) break;
            if (kb + 2 * KSTEP < p.K) load_block(kb + 2 * KSTEP, a0, b0);
            compute_block(a1, b1);
        }
    } else {
        for (int kb = k0; kb < p.K; kb += KSTEP) {
            f4 a[UK][MR], b[UK][CW];
            load_block(kb, a, b);
            compute_block(a, b);
        }
    }

    // Every lane ends up with every sum of its wave; lane CW m + c keeps
    // element (m, c). With KW > 1 the waves of a column group add their
    // partial sums in phase order through LDS; the first wave of the group
    // then runs the MR x CW elements through the epilogue side by side.
    static_assert(MR * CW <= 64, "one lane per element");
    float mine = 0.f;
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int c = 0; c < CW; ++c) {
            const float s = group_sum<0x3F>(acc[m][c]);
            if (lane == CW * m + c) mine = s;
        }
    if constexpr (KW > 1) {
        __shared__ float red[NW][64];
        red[wave][lane] = mine;
        __syncthreads();
        if (phase != 0) return;
#pragma unroll
        for (int w = 1; w < KW; ++w) mine += red[wave + w][lane];
    }
    const int m = lane / CW, c = lane % CW;
    if (m < MR && m < rows_left && c < cols_left) {
        const int64_t c_org = (int64_t)m0 * p.ldc + n0;
        const __amdgpu_buffer_rsrc_t rc = make_rsrc(p.C + c_org, p.c_extent - c_org);
        const bool beta0 = p.flags & FLAG_BETA0;
        const uint32_t off = (uint32_t)(m * p.ldc + c) * 4u;
        const float cin = beta0 ? 0.f : ld1(rc, off);
        st1(rc, off, epilogue_value(p, mine, cin, beta0, (int64_t)m0 + m, (int64_t)n0 + c));
    }
}

template <int MR, int TA, int CW, int KW, int UK, bool PIPE>
void launch_k(bool vec_b, const GemmParams& p, hipStream_t s) {
    constexpr int cols_per_wg = CW * (kSkinnyThreads / 64) / KW;
    const dim3 grid((p.N + cols_per_wg - 1) / cols_per_wg, (p.M + MR - 1) / MR);
    const dim3 block(kSkinnyThreads);
    if (vec_b) hipLaunchKernelGGL((skinny_k_kernel<MR, TA, true, CW, KW, UK, PIPE>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((skinny_k_kernel<MR, TA, false, CW, KW, UK, PIPE>), grid, block, 0, s, p);
}

template <int MR, int NT, bool BIG>
void launch_mn(int ta, bool vec_b, bool pipe_req, dim3 grid, const GemmParams& p, hipStream_t s) {
    const dim3 block(NT);
    constexpr bool kCanPipe = NT < 1024 && !BIG;  // see launch_mr
    const bool pipe = kCanPipe && pipe_req;
    if (ta == 0) {
        if (vec_b) {
            if (pipe) hipLaunchKernelGGL((skinny_mn_kernel<MR, 0, true, kCanPipe, NT, BIG>), grid, block, 0, s, p);
            else hipLaunchKernelGGL((skinny_mn_kernel<MR, 0, true, false, NT, BIG>), grid, block, 0, s, p);
        } else {
            if (pipe) hipLaunchKernelGGL((skinny_mn_kernel<MR, 0, false, kCanPipe, NT, BIG>), grid, block, 0, s, p);
            else hipLaunchKernelGGL((skinny_mn_kernel<MR, 0, false, false, NT, BIG>), grid, block, 0, s, p);
        }
    } else {
        if (vec_b) {
            if (pipe) hipLaunchKernelGGL((skinny_mn_kernel<MR, 1, true, kCanPipe, NT, BIG>), grid, block, 0, s, p);
            else hipLaunchKernelGGL((skinny_mn_kernel<MR, 1, true, false, NT, BIG>), grid, block, 0, s, p);
        } else {
            if (pipe) hipLaunchKernelGGL((skinny_mn_kernel<MR, 1, false, kCanPipe, NT, BIG>), grid, block, 0, s, p);
            else hipLaunchKernelGGL((skinny_mn_kernel<MR, 1, false, false, NT, BIG>), grid, block, 0, s, p);
        }
    }
}

template <int MR>
hipError_t launch_mr(int ta, int tb, const GemmParams& p, hipStream_t s, int threads) {
    const bool vec_b = p.flags & FLAG_VEC_B;
    const int rblocks = (p.M + MR - 1) / MR;
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
        // Byte offsets inside one k block (8 nt rows of op(B), and of op(A)
        // when it is stored K x M) must stay below 2^32; past that (ld of
        // about 2^17 and up at 1024 work-items, 2^19 at 256) the kernel that
        // rebases per k step runs instead, with 256 work-items.
        const int64_t ld = std::max<int64_t>(p.ldb, ta ? p.lda : 0);
        const bool fits = ((int64_t)nt * kUnrollMN + 1) * ld * 4 < (1ll << 32);
        if (!fits)
            launch_mn<MR, 256, true>(ta, vec_b, false, grid, p, s);
        else if (nt == 1024)
            launch_mn<MR, 1024, false>(ta, vec_b, pipe, grid, p, s);
        else if (nt == 512)
            launch_mn<MR, 512, false>(ta, vec_b, pipe, grid, p, s);
        else
            launch_mn<MR, 256, false>(ta, vec_b, pipe, grid, p, s);
    } else {  // B stored N x K
        // Columns per wave, waves per column group, k steps per block and
        // pipelining, measured on one MI355X (us, B stored N x K):
        //   one row: 4, 4, 1, pipelined: 1 x 8192 x 8192 50.8 -> 39.1
        //     (4 columns on one wave, one k step, not pipelined, before);
        //   2 or 4 rows: 4, 4, 2, plain: 4 x 8192 x 8192 54.9 -> 42.2;
        //   8 rows: 4, 2, 1, pipelined: 8 x 8192 x 8192 65.4 -> 58.1,
        //     8 x 4096 x 4096 29.5 -> 18.3;
        //   8 rows, A stored K x M (one scalar load per element of op(A),
        //   so more columns share each): 8, 1, 1, pipelined: 8 x 8192 x 8192
        //   240.7 -> 128.7.
        if (ta == 0) {
            if constexpr (MR == 1) launch_k<MR, 0, 4, 4, 1, true>(vec_b, p, s);
            else if constexpr (MR < 8) launch_k<MR, 0, 4, 4, 2, false>(vec_b, p, s);
            else launch_k<MR, 0, 4, 2, 1, true>(vec_b, p, s);
        } else {
            if constexpr (MR < 8) launch_k<MR, 1, 8, 4, 1, true>(vec_b, p, s);
            else launch_k<MR, 1, 8, 1, 1, true>(vec_b, p, s);
        }
    }
    return hipGetLastError();
}

// ---- 5 to a few dozen rows on the matrix cores ------------------------------
// With more than a handful of rows the vector-ALU kernels above are bound by
// their FMAs and op(A) reads, not by HBM (8 x 8192 x 8192 NT: 58 us, 4.6
// TB/s). Here every product goes through v_mfma_f32_16x16x4_f32 with the
// rows of C padded to RB blocks of 16 (M <= 16 RB per grid row):
//   * lane l gives op(A)(16 b + l % 16, k) and op(B)(k, column) for
//     k = k0 + KPL (l / 16) + s at step s of a 4 KPL-deep k block; the KPL k
//     of a lane are consecutive (the sum over k is order-free), so op(A)
//     stored M x K and op(B) stored N x K are read with 128-bit loads along k;
//   * op(B) stored K x N: a lane's CS columns CS (l % 16) + c are one CS-wide
//     load per k row (column set c of the instruction holds them);
//   * lane l ends with rows 4 (l / 16) + r, r < 4, of its column.
// A workgroup of 16 waves owns 16 CS columns; wave w takes k blocks w,
// w + 16, ... (UB blocks per round of loads), and the 16 partial tiles are
// added in LDS in wave order (deterministic) before the epilogue.
constexpr int kFewWaves = 16;
// k per lane per block (B stored K x N, N x K), registers of loaded operands
// per round, pipelined rounds. Measured on one MI355X against 4, 4, 48, plain
// (us): 8 x 8192^2 NN 44.8 -> 43.2, NT 57.7 -> 48.2; 32 x 8192^2 NN 67.6 ->
// 60.6, NT 75.4 -> 67.9; 8 x 32000 x 4096 NT 125.1 -> 112.3; k per lane 16
// was slower (NT 50.9) and pipelined 64-row blocks spill, so those run plain.
constexpr int kFewKplMN = 8, kFewKplK = 8, kFewRegs = 64;
constexpr bool kFewPipe = true;

template <int RB, int CS, int TA, int TB, bool VEC, int KPL, int UB, bool PIPE>
__global__ void __launch_bounds__(64 * kFewWaves) few_rows_mfma_kernel(GemmParams p) {
    // KPL: k per lane per block (a block is 4 KPL deep: lane group g = l / 16
    // holds k0 + KPL g .. KPL g + KPL - 1); UB: blocks per round of loads;
    // PIPE: the next round's loads are issued before this round's MFMAs (two
    // register sets).
    constexpr int KB = 4 * KPL;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int li = lane & 15, g = lane >> 4;
    const int n0 = blockIdx.x * 16 * CS, m0 = blockIdx.y * 16 * RB;
    const int nblk = (p.K + KB - 1) / KB;
    const bool vec_a = !TA && (p.flags & FLAG_VEC_A);

    f4 acc[RB][CS];
#pragma unroll
    for (int b = 0; b < RB; ++b)
#pragma unroll
        for (int c = 0; c < CS; ++c) acc[b][c] = f4{0.f, 0.f, 0.f, 0.f};

    // Loads of the UB k blocks jb, jb + 16, ... (blocks past K read as 0).
    // Buffer resources are based at each block, so offsets stay below
    // 64 * ld * 4 bytes.
    auto load_round = [&](int jb, float (&av)[UB][RB][KPL], float (&bv)[UB][CS][KPL]) {
#pragma unroll
        for (int u = 0; u < UB; ++u) {
            const int k0 = (jb + kFewWaves * u) * KB;
            const int kl = p.K - k0 - KPL * g;  // this lane's k inside K: min(KPL, kl)
            const int64_t a_org = TA ? (int64_t)k0 * p.lda + m0 : (int64_t)m0 * p.lda + k0;
            const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.A + a_org, p.a_extent - a_org);
#pragma unroll
            for (int b = 0; b < RB; ++b) {
                const int m = 16 * b + li;
                if (m0 + m >= p.M) {
#pragma unroll
                    for (int s = 0; s < KPL; ++s) av[u][b][s] = 0.f;
                } else if constexpr (TA == 0) {
#pragma unroll
                    for (int j = 0; j < KPL; j += 4) {
                        const f4 v = ld4_guard(ra, (uint32_t)(m * p.lda + KPL * g + j) * 4u, j, kl,
                                               vec_a);
#pragma unroll
                        for (int s = 0; s < 4; ++s) av[u][b][j + s] = v[s];
                    }
                } else {
#pragma unroll
                    for (int s = 0; s < KPL; ++s)
                        av[u][b][s] =
                            s < kl ? ld1(ra, (uint32_t)((KPL * g + s) * p.lda + m) * 4u) : 0.f;
                }
            }
            if constexpr (TB == 0) {  // op(B) stored K x N
                const int64_t b_org = (int64_t)k0 * p.ldb + n0;
                const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.B + b_org, p.b_extent - b_org);
                const int cl = p.N - n0 - CS * li;  // this lane's columns inside N: min(CS, cl)
#pragma unroll
                for (int s = 0; s < KPL; ++s) {
                    const uint32_t off = (uint32_t)((KPL * g + s) * p.ldb + CS * li) * 4u;
                    const bool in = s < kl;
                    if constexpr (CS == 4) {
                        const f4 v = in ? ld4_guard(rb, off, 0, cl, VEC) : f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int c = 0; c < 4; ++c) bv[u][c][s] = v[c];
                    } else if constexpr (CS == 2) {
                        f2 v = {0.f, 0.f};
                        if (in && VEC && cl >= 2) {
                            v = ld2(rb, off);
                        } else if (in) {
                            if (cl > 0) v[0] = ld1(rb, off);
                            if (cl > 1) v[1] = ld1(rb, off + 4);
                        }
                        bv[u][0][s] = v[0];
                        bv[u][1][s] = v[1];
                    } else {
                        bv[u][0][s] = in && cl > 0 ? ld1(rb, off) : 0.f;
                    }
                }
            } else {  // op(B) stored N x K
                const int64_t b_org = (int64_t)n0 * p.ldb + k0;
                const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.B + b_org, p.b_extent - b_org);
#pragma unroll
                for (int c = 0; c < CS; ++c) {
                    const int n = 16 * c + li;
#pragma unroll
                    for (int j = 0; j < KPL; j += 4) {
                        const f4 v = n0 + n < p.N ? ld4_guard(rb, (uint32_t)(n * p.ldb + KPL * g + j) * 4u,
                                                              j, kl, VEC)
                                                  : f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int s = 0; s < 4; ++s) bv[u][c][j + s] = v[s];
                    }
                }
            }
        }
    };
    auto mfma_round = [&](const float (&av)[UB][RB][KPL], const float (&bv)[UB][CS][KPL]) {
#pragma unroll
        for (int u = 0; u < UB; ++u)
#pragma unroll
            for (int s = 0; s < KPL; ++s)
#pragma unroll
                for (int b = 0; b < RB; ++b)
#pragma unroll
                    for (int c = 0; c < CS; ++c)
                        acc[b][c] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[u][b][s], bv[u][c][s],
                                                                         acc[b][c], 0, 0, 0);
    };
    constexpr int STEP = kFewWaves * UB;  // blocks per round of the workgroup
    if constexpr (PIPE) {
        float a0[UB][RB][KPL], b0[UB][CS][KPL], a1[UB][RB][KPL], b1[UB][CS][KPL];
        if (wave < nblk) load_round(wave, a0, b0);
        for (int jb = wave; jb < nblk; jb += 2 * STEP) {
            if (jb + STEP < nblk) load_round(jb + STEP, a1, b1);
            mfma_round(a0, b0);
            if (jb + STEP >= nblk) break;
            if (jb + 2 * STEP < nblk) load_round(jb + 2 * STEP, a0, b0);
            mfma_round(a1, b1);
        }
    } else {
        for (int jb = wave; jb < nblk; jb += STEP) {
            float av[UB][RB][KPL], bv[UB][CS][KPL];
            load_round(jb, av, bv);
            mfma_round(av, bv);
        }
    }

    // The 16 waves' partial tiles through LDS, added in wave order; element
    // (q, l) = accumulator register r of (row block b, column set c) of lane l,
    // q = 4 (CS b + c) + r.
    constexpr int NQ = RB * CS * 4;
    __shared__ float red[kFewWaves][NQ][64];
#pragma unroll
    for (int b = 0; b < RB; ++b)
#pragma unroll
        for (int c = 0; c < CS; ++c)
#pragma unroll
            for (int r = 0; r < 4; ++r) red[wave][4 * (CS * b + c) + r][lane] = acc[b][c][r];
    __syncthreads();
    const int64_t c_org = (int64_t)m0 * p.ldc + n0;
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(p.C + c_org, p.c_extent - c_org);
    const bool beta0 = p.flags & FLAG_BETA0;
    for (int t = threadIdx.x; t < NQ * 64; t += 64 * kFewWaves) {
        const int q = t >> 6, l = t & 63;
        const int r = q & 3, c = (q >> 2) % CS, b = (q >> 2) / CS;
        const int row = 16 * b + 4 * (l >> 4) + r;
        const int col = TB == 0 ? CS * (l & 15) + c : 16 * c + (l & 15);
        if (m0 + row < p.M && n0 + col < p.N) {
            float sum = red[0][q][l];
#pragma unroll
            for (int w = 1; w < kFewWaves; ++w) sum += red[w][q][l];
            const uint32_t off = (uint32_t)(row * p.ldc + col) * 4u;
            const float cin = beta0 ? 0.f : ld1(rc, off);
            st1(rc, off, epilogue_value(p, sum, cin, beta0, (int64_t)m0 + row, (int64_t)n0 + col));
        }
    }
}

template <int RB, int CS, int TA, int TB>
void launch_few_mfma_t(bool vec_b, const GemmParams& p, hipStream_t s) {
    constexpr int KPL = TB == 0 ? kFewKplMN : kFewKplK;
    constexpr bool PIPE = kFewPipe && RB < 4;
    // Blocks per round: as many as kFewRegs registers of loaded operands
    // hold (per register set).
    constexpr int UB0 = kFewRegs / ((RB + CS) * KPL * (PIPE ? 2 : 1));
    constexpr int UB = UB0 < 1 ? 1 : UB0;
    const dim3 grid((p.N + 16 * CS - 1) / (16 * CS), (p.M + 16 * RB - 1) / (16 * RB));
    const dim3 block(64 * kFewWaves);
    if (vec_b) hipLaunchKernelGGL((few_rows_mfma_kernel<RB, CS, TA, TB, true, KPL, UB, PIPE>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((few_rows_mfma_kernel<RB, CS, TA, TB, false, KPL, UB, PIPE>), grid, block, 0, s, p);
}

template <int RB, int CS>
void launch_few_mfma_cs(int ta, int tb, bool vec_b, const GemmParams& p, hipStream_t s) {
    if (ta == 0) {
        if (tb == 0) launch_few_mfma_t<RB, CS, 0, 0>(vec_b, p, s);
        else launch_few_mfma_t<RB, CS, 0, 1>(vec_b, p, s);
    } else {
        if (tb == 0) launch_few_mfma_t<RB, CS, 1, 0>(vec_b, p, s);
        else launch_few_mfma_t<RB, CS, 1, 1>(vec_b, p, s);
    }
}

// Row blocks of 16 per grid row: one up to 16 rows, two up to 32, else four
// (M past 64 runs ceil(M / 64) grid rows, each streaming op(B)). Two column sets per
// wave (32 columns per workgroup) once that still gives 256 workgroups.
hipError_t launch_few_mfma(int ta, int tb, const GemmParams& p, hipStream_t s) {
    const bool vec_b = p.flags & FLAG_VEC_B;
    const bool two_sets = p.N >= 32 * 256;
    if (p.M <= 16) {
        if (two_sets) launch_few_mfma_cs<1, 2>(ta, tb, vec_b, p, s);
        else launch_few_mfma_cs<1, 1>(ta, tb, vec_b, p, s);
    } else if (p.M <= 32) {
        if (two_sets) launch_few_mfma_cs<2, 2>(ta, tb, vec_b, p, s);
        else launch_few_mfma_cs<2, 1>(ta, tb, vec_b, p, s);
    } else {
        if (two_sets) launch_few_mfma_cs<4, 2>(ta, tb, vec_b, p, s);
        else launch_few_mfma_cs<4, 1>(ta, tb, vec_b, p, s);
    }
    return hipGetLastError();
}

}  // namespace

// kernel: 0 = automatic (few_rows_on_valu), 1 = vector ALU, 2 = matrix
// cores. Vector ALU rows per block: 1, 2, 4 or 8 (the smallest power of two
// >= M, capped at 8). threads: workgroup size of its K x N kernel (0 =
// automatic, else 256, 512 or 1024).
hipError_t launch_skinny(int ta, int tb, const GemmParams& p, hipStream_t s, int threads,
                         int kernel) {
    if (kernel == 2 || (kernel == 0 && !few_rows_on_valu(p.M, tb)))
        return launch_few_mfma(ta, tb, p, s);
    if (p.M <= 1) return launch_mr<1>(ta, tb, p, s, threads);
    if (p.M <= 2) return launch_mr<2>(ta, tb, p, s, threads);
    if (p.M <= 4) return launch_mr<4>(ta, tb, p, s, threads);
    return launch_mr<8>(ta, tb, p, s, threads);
}

}  // namespace fg
