// True-fp32 SGEMM on the gfx950 matrix cores (v_mfma_f32_32x32x2_f32).
//
// Structure (the block-tile / warp-tile / thread-tile hierarchy of "Matmul
// II: register blocking, warp tiling, tensor cores", sections 1, 5 and 7,
// rebuilt for 64-wide wavefronts and the MFMA register layout):
//
//   workgroup tile BM x BN, k-tiles of BK = 16 staged in a 2-buffer LDS ring;
//   wavefront tile WM x WN = (MB x 32) x (NB x 32), i.e. MB x NB accumulator
//   blocks of 32 x 32, 16 fp32 registers per lane each;
//   one v_mfma_f32_32x32x2_f32 per block and k-step of 2.
//
// k mapping. One MFMA consumes two k values: lanes 0-31 supply k-index 0 and
// lanes 32-63 k-index 1 (A: lane l holds A[l%32][l/32]; B: lane l holds
// B[l/32][l%32]). Summation order is free, so inside a 16-deep k-tile the
// instruction at k-step s (0..7) takes k = s for lanes 0-31 and k = 8 + s for
// lanes 32-63. A lane then needs k = 8h .. 8h+7 of its row across the eight
// k-steps: two 128-bit LDS reads when the tile is stored k-contiguous.
//
// Interleaved blocks. Inside a wave tile, block b of the N direction holds
// columns NB*j + b (j = lane % 32) instead of 32*b + j; likewise rows MB*i + a
// for the M direction. A lane's operands for all NB blocks at one k are then
// NB consecutive floats of an n-contiguous LDS row (one 128-bit read for
// NB = 4), and its results for those blocks are NB consecutive columns of C
// (one 128-bit store), which is the wide-store epilogue of "CuTe-ly writing
// an SM86 SGEMM", section "wide epilogue instructions", obtained here from
// the block assignment alone.
//
// LDS layouts per operand:
//   * mn-contiguous in global memory (A^T stored K x M, or B stored K x N):
//     LDS row = one k, BX floats; lanes read consecutive addresses.
//   * k-contiguous (A stored M x K, or B^T stored N x K): LDS row = one m (or
//     n), 16 floats. Rows are placed in "physical" order so that the 32 rows
//     read by one instruction are consecutive, and the four 16-byte chunks of
//     a row are XOR-swizzled with bits 1-2 of the physical row, so eight
//     consecutive rows' chunk c land in eight distinct 16-byte bank groups
//     (the XOR swizzle of "CuTe-ly writing an SM86 SGEMM", section "swizzles
//     & shared memory", at 16-byte granularity).
//
// Pipeline (one barrier per k-tile): while the MFMAs of k-tile t run from LDS
// buffer t%2, the registers already hold k-tile t+1 loaded from global
// memory; they are written to buffer (t+1)%2 after the MFMAs are issued and
// the loads for k-tile t+2 are started. Buffer (t+1)%2 was last read in
// iteration t-1, which the barrier closing that iteration protects.
//
// Edges: interior tiles use unguarded 128-bit buffer loads; tiles that cross
// M, N or K (and operands whose rows are not 16-byte aligned) use guarded
// loads that read out-of-range elements as zero. Every global access goes
// through a buffer resource bounded by the matrix's extent, so no access can
// leave the caller's allocation.
#include "fg_device.h"

namespace fg {
namespace {

constexpr int kBK = 16;

// One operand's share of a k-tile and how this thread loads and reads it.
//   BX: tile extent in M (for A) or N (for B); WX: wave extent; XB: blocks per
//   wave; MN: operand is mn-contiguous in global memory; NT: threads.
template <int BX, int WX, int XB, bool MN, int NT>
struct Operand {
    static constexpr int kStage = BX * kBK;    // floats per LDS buffer
    static constexpr int kVecs = kStage / 4;   // 16-byte vectors per k-tile
    static constexpr int kVPT = kVecs / NT;    // vectors per thread
    static_assert(kVecs % NT == 0, "tile must split evenly over threads");
    static_assert(XB == 1 || XB == 2 || XB == 4, "1, 2 or 4 blocks per wave");
    static_assert(WX == 32 * XB, "wave extent is XB blocks of 32");

    uint32_t goff[kVPT];  // byte offset inside the k-tile (global)
    int lds[kVPT];        // float offset inside one LDS buffer
    int row[kVPT];        // k row (MN) or m/n row (k-contiguous) within the tile
    int col[kVPT];        // first element along the contiguous direction
    f4 reg[kVPT];

    // Physical LDS row of logical tile row x (k-contiguous layout) and back.
    __device__ static int phys_to_logical(int pr) {
        const int w = pr / WX, within = pr % WX;
        const int a = within / 32, i = within % 32;
        return w * WX + i * XB + a;
    }
    __device__ static int swz(int pr) { return (pr >> 1) & 3; }

    __device__ void init(int tid, int ld) {
#pragma unroll
        for (int q = 0; q < kVPT; ++q) {
            const int v = tid + NT * q;
            if constexpr (MN) {
                const int r = v / (BX / 4), c = v % (BX / 4);
                row[q] = r;
                col[q] = 4 * c;
                lds[q] = r * BX + 4 * c;
                goff[q] = (uint32_t)(r * ld + 4 * c) * 4u;
            } else {
                const int pr = v / 4, c = v % 4;
                const int x = phys_to_logical(pr);
                row[q] = x;
                col[q] = 4 * c;
                lds[q] = pr * kBK + 4 * (c ^ swz(pr));
                goff[q] = (uint32_t)(x * ld + 4 * c) * 4u;
            }
        }
    }

    // rows_left: valid tile rows (k rows for MN, m/n rows otherwise);
    // len: valid elements along the contiguous direction.
    __device__ void load(__amdgpu_buffer_rsrc_t r, bool fast, bool vec, int rows_left,
                         int len) {
        if (fast) {
#pragma unroll
            for (int q = 0; q < kVPT; ++q) reg[q] = ld4(r, goff[q]);
        } else {
#pragma unroll
            for (int q = 0; q < kVPT; ++q) {
                f4 z = {0.f, 0.f, 0.f, 0.f};
                reg[q] = row[q] < rows_left ? ld4_guard(r, goff[q], col[q], len, vec) : z;
            }
        }
    }

    __device__ void store_lds(float* buf) const {
#pragma unroll
        for (int q = 0; q < kVPT; ++q) *reinterpret_cast<f4*>(buf + lds[q]) = reg[q];
    }

    // Operands of this lane for all 8 k-steps and XB blocks:
    // frag[s][x] = op(X) at k = 8h + s, block x, lane position i.
    __device__ static void read_frags(const float* buf, int wbase, int i, int h,
                                      float (&frag)[kBK / 2][XB]) {
        if constexpr (MN) {
#pragma unroll
            for (int s = 0; s < kBK / 2; ++s) {
                const float* p = buf + (8 * h + s) * BX + wbase + XB * i;
                if constexpr (XB == 4) {
                    f4 v = *reinterpret_cast<const f4*>(p);
                    frag[s][0] = v[0]; frag[s][1] = v[1]; frag[s][2] = v[2]; frag[s][3] = v[3];
                } else if constexpr (XB == 2) {
                    f2 v = *reinterpret_cast<const f2*>(p);
                    frag[s][0] = v[0]; frag[s][1] = v[1];
                } else {
                    frag[s][0] = *p;
                }
            }
        } else {
#pragma unroll
            for (int x = 0; x < XB; ++x) {
                const int pr = wbase + 32 * x + i;
                const float* rowp = buf + pr * kBK;
                f4 lo = *reinterpret_cast<const f4*>(rowp + 4 * ((2 * h) ^ swz(pr)));
                f4 hi = *reinterpret_cast<const f4*>(rowp + 4 * ((2 * h + 1) ^ swz(pr)));
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    frag[s][x] = lo[s];
                    frag[s + 4][x] = hi[s];
                }
            }
        }
    }
};

template <int BM, int BN, int WAVES_M, int WAVES_N, int TA, int TB>
__global__ void __launch_bounds__(64 * WAVES_M * WAVES_N)
sgemm_mfma_kernel(GemmParams p) {
    constexpr int NT = 64 * WAVES_M * WAVES_N;
    constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
    constexpr int MB = WM / 32, NB = WN / 32;
    constexpr bool A_MN = (TA == 1);  // A stored K x M
    constexpr bool B_MN = (TB == 0);  // B stored K x N
    using OpA = Operand<BM, WM, MB, A_MN, NT>;
    using OpB = Operand<BN, WN, NB, B_MN, NT>;

    __shared__ f4 smem[(2 * OpA::kStage + 2 * OpB::kStage) / 4];
    float* sA = reinterpret_cast<float*>(smem);
    float* sB = sA + 2 * OpA::kStage;

    int tm, tn;
    map_tile(blockIdx.x, gridDim.x, p, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wave_m = wave / WAVES_N, wave_n = wave % WAVES_N;
    const int li = lane & 31, lh = lane >> 5;

    const bool vec_a = p.flags & FLAG_VEC_A, vec_b = p.flags & FLAG_VEC_B;
    const bool mn_interior = (m0 + BM <= p.M) && (n0 + BN <= p.N);
    const bool a_rows_in = m0 + BM <= p.M, b_rows_in = n0 + BN <= p.N;

    // Element offset of the tile origin (row m0 / column n0, k = 0) and of
    // one k-tile step, per operand.
    const int64_t a_org = A_MN ? (int64_t)m0 : (int64_t)m0 * p.lda;
    const int64_t a_kstep = A_MN ? (int64_t)kBK * p.lda : (int64_t)kBK;
    const int64_t b_org = B_MN ? (int64_t)n0 : (int64_t)n0 * p.ldb;
    const int64_t b_kstep = B_MN ? (int64_t)kBK * p.ldb : (int64_t)kBK;

    OpA opa;
    OpB opb;
    opa.init(tid, p.lda);
    opb.init(tid, p.ldb);

    const int nk = (p.K + kBK - 1) / kBK;

    auto load_tiles = [&](int kt) {
        const int k0 = kt * kBK;
        const int64_t ao = a_org + kt * a_kstep, bo = b_org + kt * b_kstep;
        const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.A + ao, p.a_extent - ao);
        const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.B + bo, p.b_extent - bo);
        const bool k_in = k0 + kBK <= p.K;
        const int k_left = p.K - k0;
        if constexpr (A_MN)
            opa.load(ra, vec_a && k_in && a_rows_in, vec_a, k_left, p.M - m0);
        else
            opa.load(ra, vec_a && k_in && a_rows_in, vec_a, p.M - m0, k_left);
        if constexpr (B_MN)
            opb.load(rb, vec_b && k_in && b_rows_in, vec_b, k_left, p.N - n0);
        else
            opb.load(rb, vec_b && k_in && b_rows_in, vec_b, p.N - n0, k_left);
    };

    f16v acc[MB][NB];
#pragma unroll
    for (int a = 0; a < MB; ++a)
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

    if (nk > 0) {
        load_tiles(0);
        opa.store_lds(sA);
        opb.store_lds(sB);
        if (nk > 1) load_tiles(1);
        __syncthreads();
    }

    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        const float* bufA = sA + cur * OpA::kStage;
        const float* bufB = sB + cur * OpB::kStage;
        float fa[kBK / 2][MB], fb[kBK / 2][NB];
        OpA::read_frags(bufA, wave_m * WM, li, lh, fa);
        OpB::read_frags(bufB, wave_n * WN, li, lh, fb);
#pragma unroll
        for (int s = 0; s < kBK / 2; ++s)
#pragma unroll
            for (int a = 0; a < MB; ++a)
#pragma unroll
                for (int b = 0; b < NB; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[s][a], fb[s][b],
                                                                     acc[a][b], 0, 0, 0);
        if (kt + 1 < nk) {
            opa.store_lds(sA + (cur ^ 1) * OpA::kStage);
            opb.store_lds(sB + (cur ^ 1) * OpB::kStage);
            if (kt + 2 < nk) load_tiles(kt + 2);
        }
        __syncthreads();
    }

    // Epilogue: C = alpha * acc + beta * C, 128-bit where possible.
    // Accumulator register r of a 32x32 block, lane (i = lane%32, h = lane/32),
    // holds block row 8*(r/4) + 4*h + r%4 and block column i.
    const int64_t c_org = (int64_t)m0 * p.ldc + n0;
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(p.C + c_org, p.c_extent - c_org);
    const bool beta0 = p.flags & FLAG_BETA0;
    const bool vec_c = (p.flags & FLAG_VEC_C) && NB == 4;
    const float alpha = p.alpha, beta = p.beta;
    const int col0 = wave_n * WN + NB * li;  // first of this lane's NB columns
    const int cols_left = p.N - n0 - col0;
#pragma unroll
    for (int a = 0; a < MB; ++a) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int brow = 8 * (r / 4) + 4 * lh + (r % 4);
            const int row = wave_m * WM + MB * brow + a;
            if (m0 + row >= p.M) continue;
            const uint32_t off = (uint32_t)(row * p.ldc + col0) * 4u;
            float v[NB];
#pragma unroll
            for (int b = 0; b < NB; ++b) v[b] = alpha * acc[a][b][r];
            if (vec_c && mn_interior) {
                f4 o = {v[0], v[1], v[2], v[3]};
                if (!beta0) {
                    f4 c = ld4(rc, off);
                    o = o + beta * c;
                }
                st4(rc, off, o);
            } else {
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    if (b < cols_left) {
                        float o = v[b];
                        if (!beta0) o += beta * ld1(rc, off + 4 * b);
                        st1(rc, off + 4 * b, o);
                    }
                }
            }
        }
    }
}

template <int BM, int BN, int WAVES_M, int WAVES_N>
hipError_t launch_shape(int ta, int tb, const GemmParams& p, hipStream_t s) {
    const dim3 grid(p.tiles_m * p.tiles_n), block(64 * WAVES_M * WAVES_N);
    if (ta == 0 && tb == 0)
        hipLaunchKernelGGL((sgemm_mfma_kernel<BM, BN, WAVES_M, WAVES_N, 0, 0>), grid, block, 0, s, p);
    else if (ta == 0 && tb == 1)
        hipLaunchKernelGGL((sgemm_mfma_kernel<BM, BN, WAVES_M, WAVES_N, 0, 1>), grid, block, 0, s, p);
    else if (ta == 1 && tb == 0)
        hipLaunchKernelGGL((sgemm_mfma_kernel<BM, BN, WAVES_M, WAVES_N, 1, 0>), grid, block, 0, s, p);
    else
        hipLaunchKernelGGL((sgemm_mfma_kernel<BM, BN, WAVES_M, WAVES_N, 1, 1>), grid, block, 0, s, p);
    return hipGetLastError();
}

}  // namespace

// Variants (must match the MFMA rows of the configuration table):
//   0: 256 x 256, 2 x 2 waves of 128 x 128
//   1: 256 x 128, 2 x 1 waves of 128 x 128
//   2: 128 x 128, 1 wave  of 128 x 128
//   3:  64 x 128, 1 wave  of  64 x 128
//   4:  32 x 128, 1 wave  of  32 x 128
hipError_t launch_mfma(int variant, int ta, int tb, const GemmParams& p, hipStream_t s) {
    switch (variant) {
        case 0: return launch_shape<256, 256, 2, 2>(ta, tb, p, s);
        case 1: return launch_shape<256, 128, 2, 1>(ta, tb, p, s);
        case 2: return launch_shape<128, 128, 1, 1>(ta, tb, p, s);
        case 3: return launch_shape<64, 128, 1, 1>(ta, tb, p, s);
        case 4: return launch_shape<32, 128, 1, 1>(ta, tb, p, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace fg
