// True-fp32 SGEMM on the gfx950 matrix cores: the kernel template behind
// every matrix-core table entry. Each entry is one instance of it, compiled in
// its own translation unit (sgemm_mfma_inst.hip) from the instance list
// fg_mfma_instances.inc.
//
// Structure (the block-tile / warp-tile / thread-tile hierarchy of "Matmul
// II: register blocking, warp tiling, tensor cores", sections 1, 5 and 7,
// rebuilt for 64-wide wavefronts and the MFMA register layout):
//
//   workgroup tile BM x BN, k-tiles of BK (8, 16 or 32) staged in LDS;
//   wavefront tile WM x WN = (MB x MR) x (NB x MR), i.e. MB x NB accumulator
//   blocks of MR x MR;
//   MR = 32: one v_mfma_f32_32x32x2_f32 per block and k-step (2 k values),
//            16 fp32 accumulator registers per lane and block;
//   MR = 16: one v_mfma_f32_16x16x4_f32 per block and k-step (4 k values),
//            4 accumulator registers per lane and block.
//
// k mapping. One MFMA consumes KS = 64 / MR k values: lanes are KS groups of
// MR (group h = lane / MR, position i = lane % MR), and group h supplies
// k-index h (A: lane holds A[i][h]; B: lane holds B[h][i]). Summation order is
// free, so inside a BK-deep k-tile the instruction at k-step s (of KPL =
// BK / KS) takes k = h * KPL + s from group h. A lane then needs k = h * KPL
// .. h * KPL + KPL - 1 of its row across the k-steps: KPL / 4 128-bit LDS
// reads when the tile is stored k-contiguous.
//
// Interleaved blocks. Inside a wave tile, block b of the N direction holds
// columns NB*i + b instead of MR*b + i; likewise rows MB*i + a for the M
// direction. A lane's operands for all NB blocks at one k are then NB
// consecutive floats of an n-contiguous LDS row (one 128-bit read for
// NB = 4), and its results for those blocks are NB consecutive columns of C
// (one 128-bit store), which is the wide-store epilogue of "CuTe-ly writing
// an SM86 SGEMM", section "wide epilogue instructions", obtained here from
// the block assignment alone.
//
// LDS layouts per operand:
//   * mn-contiguous in global memory (A^T stored K x M, or B stored K x N):
//     LDS row = one k, BX floats; lanes read consecutive addresses.
//   * k-contiguous (A stored M x K, or B^T stored N x K): LDS row = one m (or
//     n), BK floats. Rows are placed in "physical" order so that the MR rows
//     read by one instruction are consecutive, and the 16-byte chunks of a
//     row are XOR-swizzled with the bits of the physical row above the rows
//     that share one 256-byte window, so sixteen consecutive rows' chunk c
//     land in sixteen distinct 16-byte slots (the XOR swizzle of "CuTe-ly
//     writing an SM86 SGEMM", section "swizzles & shared memory", at 16-byte
//     granularity).
//
// Loader and pipeline: see sgemm_mfma_kernel below. Every global access goes
// through a buffer resource bounded by the matrix's extent, so no access can
// leave the caller's allocation.
#pragma once

#include "fg_device.h"

namespace fg {
namespace mfma {

// Accumulator block type and MFMA of one block shape.
template <int MR>
struct Mfma;

template <>
struct Mfma<32> {
    using acc_t = f16v;
    static constexpr int kRegs = 16;
    __device__ static acc_t step(float a, float b, acc_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
    }
    // Block row held by accumulator register r of lane group h (the
    // instruction's output layout: rows 8 (r / 4) + 4 h + r % 4).
    __device__ static int row(int r, int h) { return 8 * (r / 4) + 4 * h + (r % 4); }
};

template <>
struct Mfma<16> {
    using acc_t = f4;
    static constexpr int kRegs = 4;
    __device__ static acc_t step(float a, float b, acc_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
    // Output layout of the 16 x 16 instruction: rows 4 h + r.
    __device__ static int row(int r, int h) { return 4 * h + r; }
};

// One operand's share of a k-tile and how this thread loads and reads it
// through registers (2-stage entries, and the partial last k-tile of the
// direct-to-LDS entries).
//   BX: tile extent in M (for A) or N (for B); WX: wave extent; XB: blocks per
//   wave; MN: operand is mn-contiguous in global memory; NT: threads; BK:
//   k-tile depth; MR: block edge.
template <int BX, int WX, int XB, bool MN, int NT, int BK, int MR>
struct Operand {
    static constexpr int kStage = BX * BK;     // floats per LDS buffer
    static constexpr int kVecs = kStage / 4;   // 16-byte vectors per k-tile
    static constexpr int kVPT = (kVecs + NT - 1) / NT;  // vectors per thread
    static constexpr bool kAll = kVecs % NT == 0;        // every thread, every slot
    static constexpr int kKS = 64 / MR;        // k values per instruction
    static constexpr int kKPL = BK / kKS;      // k values per lane per k-tile
    static constexpr int kCH = BK / 4;         // 16-byte chunks per k-contiguous row
    static_assert(BK == 8 || BK == 16 || BK == 32, "k-tile depth 8, 16 or 32");
    static_assert(MR == 16 || MR == 32, "16 x 16 or 32 x 32 blocks");
    static_assert(kKPL == 2 || kKPL % 4 == 0, "k values per lane");
    static_assert(XB == 1 || XB == 2 || XB == 4, "1, 2 or 4 blocks per wave");
    static_assert(WX == MR * XB, "wave extent is XB blocks of MR");

    uint32_t goff[kVPT];  // byte offset inside the k-tile (global)
    int lds[kVPT];        // float offset inside one LDS buffer
    int row[kVPT];        // k row (MN) or m/n row (k-contiguous) within the tile
    int col[kVPT];        // first element along the contiguous direction
    bool act[kVPT];       // this slot exists (kVecs not a multiple of NT)
    f4 reg[kVPT];

    // Physical LDS row of logical tile row x (k-contiguous layout) and back.
    __device__ static int phys_to_logical(int pr) {
        const int w = pr / WX, within = pr % WX;
        const int a = within / MR, i = within % MR;
        return w * WX + i * XB + a;
    }
    // 16-byte chunk swizzle of a k-contiguous row: an ds_read_b128 is served
    // 16 lanes (256 bytes) at a time, a 256-byte window holds 64 / BK rows,
    // and sixteen consecutive physical rows hold chunk c at sixteen distinct
    // 16-byte slots of a window when the chunk index is XORed with the row
    // bits above that (bits 2-3 for BK = 16, 1-3 for 32, bit 3 for 8).
    __device__ static int swz(int pr) { return ((pr * BK) >> 6) & (kCH - 1); }

    __device__ __forceinline__ void init(int tid, int ld) {
#pragma unroll
        for (int q = 0; q < kVPT; ++q) {
            const int v = tid + NT * q;
            act[q] = kAll || v < kVecs;
            if constexpr (MN) {
                const int r = v / (BX / 4), c = v % (BX / 4);
                row[q] = r;
                col[q] = 4 * c;
                lds[q] = r * BX + 4 * c;
                goff[q] = (uint32_t)(r * ld + 4 * c) * 4u;
            } else {
                const int pr = v / kCH, c = v % kCH;
                const int x = phys_to_logical(pr);
                row[q] = x;
                col[q] = 4 * c;
                lds[q] = pr * BK + 4 * (c ^ swz(pr));
                goff[q] = (uint32_t)(x * ld + 4 * c) * 4u;
            }
        }
    }

    // rows_left: valid tile rows (k rows for MN, m/n rows otherwise);
    // len: valid elements along the contiguous direction.
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, bool fast, bool vec, int rows_left,
                         int len) {
        if (fast) {
#pragma unroll
            for (int q = 0; q < kVPT; ++q)
                if (act[q]) reg[q] = ld4(r, goff[q]);
        } else {
#pragma unroll
            for (int q = 0; q < kVPT; ++q) {
                f4 z = {0.f, 0.f, 0.f, 0.f};
                reg[q] = act[q] && row[q] < rows_left ? ld4_guard(r, goff[q], col[q], len, vec) : z;
            }
        }
    }

    __device__ __forceinline__ void store_lds(float* buf) const {
#pragma unroll
        for (int q = 0; q < kVPT; ++q)
            if (act[q]) *reinterpret_cast<f4*>(buf + lds[q]) = reg[q];
    }

    // Operands of this lane for all KPL k-steps and XB blocks:
    // frag[s][x] = op(X) at k = KPL h + s, block x, lane position i.
    __device__ __forceinline__ static void read_frags(const float* buf, int wbase, int i, int h,
                                      float (&frag)[kKPL][XB]) {
        if constexpr (MN) {
#pragma unroll
            for (int s = 0; s < kKPL; ++s) {
                const float* p = buf + (kKPL * h + s) * BX + wbase + XB * i;
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
                const int pr = wbase + MR * x + i;
                const float* rowp = buf + pr * BK;
                if constexpr (kKPL >= 4) {
#pragma unroll
                    for (int q = 0; q < kKPL / 4; ++q) {
                        const int c = h * (kKPL / 4) + q;
                        f4 v = *reinterpret_cast<const f4*>(rowp + 4 * (c ^ swz(pr)));
#pragma unroll
                        for (int e = 0; e < 4; ++e) frag[4 * q + e][x] = v[e];
                    }
                } else {
                    // two k values: half of chunk h / 2
                    const int c = h >> 1;
                    f2 v = *reinterpret_cast<const f2*>(rowp + 4 * (c ^ swz(pr)) + 2 * (h & 1));
                    frag[0][x] = v[0];
                    frag[1][x] = v[1];
                }
            }
        }
    }

    // LDS read instructions read_frags() issues per k-tile.
    static constexpr int kReads = MN ? kKPL : XB * (kKPL >= 4 ? kKPL / 4 : 1);
};

// One operand's k-tile filled by direct-to-LDS buffer loads. A
// buffer_load_dwordx4 ... lds writes 64 lanes x 16 bytes to 1 KiB of
// consecutive LDS (lane L at base + 16 L); buffer_load_dword ... lds writes
// 64 x 4 bytes (lane L at base + 4 L). Instruction j of a stage therefore
// covers LDS floats [j * 64 * W, (j + 1) * 64 * W) for W = BYTES / 4 floats per
// lane, and each lane fetches the global element(s) that belong at its slot
// of the layout read_frags() expects. The 4-byte form needs no alignment of
// the matrix rows. This is the gfx950 counterpart of the asynchronous
// global-to-shared copy of "Matmul II", section 7 (t3) and "CuTe-ly writing
// an SM86 SGEMM", section "mainloop": the data bypasses registers and the
// wave keeps issuing MFMAs.
template <int BX, int WX, int XB, bool MN, int NW, int BYTES, int BK, int MR>
struct DmaOperand {
    using Op = Operand<BX, WX, XB, MN, 64 * NW, BK, MR>;
    static constexpr int kW = BYTES / 4;                    // floats per lane
    static constexpr int kInst = Op::kStage / (64 * kW);    // instructions per stage
    static constexpr int kPerWave = kInst / NW;
    static_assert(BYTES == 4 || BYTES == 16, "dword or dwordx4");
    static_assert(kInst % NW == 0 && kPerWave > 0, "stage must split evenly over the waves");

    uint32_t voff[kPerWave];

    __device__ __forceinline__ void init(int wave, int lane, int ld) {
#pragma unroll
        for (int q = 0; q < kPerWave; ++q) {
            const int j = wave + NW * q;
            const int pos = j * 64 * kW + kW * lane;  // float offset inside the stage
            if constexpr (MN) {
                const int k = pos / BX, col = pos % BX;
                voff[q] = (uint32_t)(k * ld + col) * 4u;
            } else {
                const int pr = pos / BK, slot = (pos % BK) / 4, e = pos % 4;
                const int c = slot ^ Op::swz(pr);
                const int x = Op::phys_to_logical(pr);
                voff[q] = (uint32_t)(x * ld + 4 * c + e) * 4u;
            }
        }
    }

    __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t r, float* stage, int wave) const {
        // Device pass only: in clang's host pass the LDS address-space cast
        // makes it drop the launch stubs of later template instances.
#if defined(__HIP_DEVICE_COMPILE__)
#pragma unroll
        for (int q = 0; q < kPerWave; ++q) {
            const int j = wave + NW * q;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                r, (__attribute__((address_space(3))) void*)(stage + j * 64 * kW), BYTES, voff[q],
                0, 0, 0);
        }
#else
        (void)r, (void)stage, (void)wave;
#endif
    }
};

// s_waitcnt that waits until at most VM vector-memory operations of this wave
// are outstanding and all of its LDS operations have completed (gfx9
// encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4 left at its maximum,
// lgkmcnt 11:8 = 0).
template <int VM>
__device__ __forceinline__ void wait_vm_lds() {
    static_assert(VM >= 0 && VM < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((VM & 0xF) | ((VM >> 4) << 14) | (0x7 << 4));
}

// Orders one wave's LDS accesses across its own lanes (a value one lane wrote
// and another lane of the same wave reads, or the reverse): all of the wave's
// LDS operations have completed, and the "memory" clobber keeps the compiler
// from moving any access across this point. No other wave takes part.
__device__ __forceinline__ void wave_lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Single-element store with the non-temporal hint, like the wide stores of C.
__device__ __forceinline__ void st1_nt(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, float v) {
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, byte_off, 0, 2);
}

// Workgroup barrier without the memory fence of __syncthreads(): the fence
// would make the compiler wait for every outstanding direct-to-LDS load,
// including the ones meant to stay in flight across the barrier. The caller
// orders memory itself with wait_vm_lds<>() first; the "memory" clobber keeps
// the compiler from moving LDS accesses across the barrier.
__device__ __forceinline__ void barrier_no_fence() { asm volatile("s_barrier" ::: "memory"); }

template <int MR, int MB, int NB, int KPL>
__device__ __forceinline__ void mfma_kstep(typename Mfma<MR>::acc_t (&acc)[MB][NB],
                                           const float (&fa)[KPL][MB],
                                           const float (&fb)[KPL][NB], int s) {
#pragma unroll
    for (int a = 0; a < MB; ++a)
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[a][b] = Mfma<MR>::step(fa[s][a], fb[s][b], acc[a][b]);
}

template <int MR, int MB, int NB, int KPL>
__device__ __forceinline__ void mfma_ktile(typename Mfma<MR>::acc_t (&acc)[MB][NB],
                                           const float (&fa)[KPL][MB],
                                           const float (&fb)[KPL][NB]) {
#pragma unroll
    for (int s = 0; s < KPL; ++s) mfma_kstep<MR, MB, NB, KPL>(acc, fa, fb, s);
}

// STAGES == 2: register-staged loop (any alignment, any edges): while the
// MFMAs of k-tile t run from LDS buffer t%2, the registers already hold
// k-tile t+1 loaded from global memory; they are written to buffer (t+1)%2
// after the MFMAs are issued and the loads for k-tile t+2 are started.
// Buffer (t+1)%2 was last read in iteration t-1, which the barrier closing
// that iteration protects.
// STAGES >= 3: direct-to-LDS loop over a STAGES-deep ring, with the next
// k-tile's fragments read during the current k-tile's MFMAs. DMAB = 16 needs
// the rows of A and B to start 16-byte aligned (the dispatcher checks);
// DMAB = 4 takes any rows. Tiles that cross M or N take the same loop: a row
// of op(A) past M (a column of op(B) past N) only feeds elements of C that
// are never stored, and the bounded buffer resources return 0 past the end
// of each matrix. A partial last k-tile (K not a multiple of BK) must read as
// exact zeros past K, so it goes through the guarded register path once
// after the loop.
// OCC: waves per SIMD the register allocation must allow (1 lets a wave use
// all 512 registers of a lane; 2 caps it at 256 so two workgroups share a CU).
template <int BM, int BN, int WAVES_M, int WAVES_N, int BK, int MR, int TA, int TB, int STAGES,
          int DMAB, int OCC>
__global__ void __launch_bounds__(64 * WAVES_M * WAVES_N, OCC)
sgemm_mfma_kernel(GemmParams p) {
    constexpr int NW = WAVES_M * WAVES_N;
    constexpr int NT = 64 * NW;
    constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
    constexpr int MB = WM / MR, NB = WN / MR;
    constexpr bool A_MN = (TA == 1);  // A stored K x M
    constexpr bool B_MN = (TB == 0);  // B stored K x N
    constexpr int NS = STAGES < 2 ? 2 : STAGES;
    using OpA = Operand<BM, WM, MB, A_MN, NT, BK, MR>;
    using OpB = Operand<BN, WN, NB, B_MN, NT, BK, MR>;
    using acc_t = typename Mfma<MR>::acc_t;
    constexpr int KPL = OpA::kKPL;
    constexpr int NREG = Mfma<MR>::kRegs;
    // The quantised second output (FLAG_QUANT) is compiled in only where the
    // accumulators leave room for it: with 256 accumulator registers per
    // lane its store loops pushed the accumulators to scratch memory. The
    // host sends quantised calls to other entries (fg_api.cpp).
    constexpr bool kQuant = MB * NB * NREG <= 128;
    // The same limit for the epilogue that stages C through LDS when C's rows
    // are unaligned (with 256 accumulators its registers spilled).
    constexpr bool kStageC = NB >= 2 && MB * NB * NREG <= 128;
    // The fused and quantised epilogue's staged copy (twelve specialisations,
    // each fully inlined) only where the accumulators are at most 32 per
    // lane: with 64 it doubled the library's build time, with 128 one
    // instance took over half an hour to compile.
    constexpr bool kStageFused = kStageC && MB * NB * NREG <= 32;

    __shared__ f4 smem[NS * (OpA::kStage + OpB::kStage) / 4];
    float* sA = reinterpret_cast<float*>(smem);
    float* sB = sA + NS * OpA::kStage;

    int tm, tn;
    const int tile_id = map_tile(blockIdx.x, gridDim.x, p, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keep in SGPRs
    const int wave_m = wave / WAVES_N, wave_n = wave % WAVES_N;
    const int li = lane % MR, lh = lane / MR;

    const bool vec_a = p.flags & FLAG_VEC_A, vec_b = p.flags & FLAG_VEC_B;
    const bool a_rows_in = m0 + BM <= p.M, b_rows_in = n0 + BN <= p.N;

    // This workgroup's k range: k-tiles [kt0, kt0 + kt_per_split) of K, i.e.
    // Kp elements of k starting at kt0 * BK (all of K without split-K).
    const int kt0 = (int)blockIdx.y * p.kt_per_split;
    const int Kp = min(p.K - kt0 * BK, p.kt_per_split * BK);

    // Element offset of the tile origin (row m0 / column n0, first k of the
    // range) and of one k-tile step, per operand.
    const int64_t a_kstep = A_MN ? (int64_t)BK * p.lda : (int64_t)BK;
    const int64_t b_kstep = B_MN ? (int64_t)BK * p.ldb : (int64_t)BK;
    const int64_t a_org = (A_MN ? (int64_t)m0 : (int64_t)m0 * p.lda) + kt0 * a_kstep;
    const int64_t b_org = (B_MN ? (int64_t)n0 : (int64_t)n0 * p.ldb) + kt0 * b_kstep;

    acc_t acc[MB][NB];
#pragma unroll
    for (int a = 0; a < MB; ++a)
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int r = 0; r < NREG; ++r) acc[a][b][r] = 0.f;

    // Guarded register-path load of k-tile kt of the range (zero past M, N
    // and the end of the range).
    auto load_tiles = [&](OpA& opa, OpB& opb, int kt) {
        const int k0 = kt * BK;
        const int64_t ao = a_org + kt * a_kstep, bo = b_org + kt * b_kstep;
        const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.A + ao, p.a_extent - ao);
        const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.B + bo, p.b_extent - bo);
        const bool k_in = k0 + BK <= Kp;
        const int k_left = Kp - k0;
        if constexpr (A_MN)
            opa.load(ra, vec_a && k_in && a_rows_in, vec_a, k_left, p.M - m0);
        else
            opa.load(ra, vec_a && k_in && a_rows_in, vec_a, p.M - m0, k_left);
        if constexpr (B_MN)
            opb.load(rb, vec_b && k_in && b_rows_in, vec_b, k_left, p.N - n0);
        else
            opb.load(rb, vec_b && k_in && b_rows_in, vec_b, p.N - n0, k_left);
    };

    if constexpr (STAGES >= 3) {
        using DA = DmaOperand<BM, WM, MB, A_MN, NW, DMAB, BK, MR>;
        using DB = DmaOperand<BN, WN, NB, B_MN, NW, DMAB, BK, MR>;
        constexpr int NI = DA::kPerWave + DB::kPerWave;  // DMA ops per wave per k-tile
        static_assert((NS - 3) * NI < 64, "loads left in flight must fit the vmcnt field");
        // With both operands stored k-major by rows (A as K x M, B as K x N),
        // a partial last k-tile goes through the ring like the others: its
        // rows at and past K lie beyond the end of each matrix, where the
        // buffer loads read zeros (a partial k-tile only ever ends at K).
        // Otherwise the last k elements of a row would be followed by the
        // next row's, so the partial k-tile takes the guarded path below.
        constexpr bool kTailInRing = A_MN && B_MN;
        const int nk = kTailInRing ? (Kp + BK - 1) / BK : Kp / BK;  // k-tiles in the ring
        DA da;
        DB db;
        da.init(wave, lane, p.lda);
        db.init(wave, lane, p.ldb);
        // DMA of k-tile kt into buffer kt % NS. A k-tile past the last one
        // (kt >= nk) gets an empty buffer resource: its loads read nothing
        // from memory and write zeros into a buffer no one reads, which keeps
        // the loop below free of branches.
        auto issue = [&](int kt) {
            const int st = kt % NS;
            const bool live = kt < nk;
            const int64_t ao = a_org + kt * a_kstep, bo = b_org + kt * b_kstep;
            da.issue(make_rsrc(p.A + ao, live ? p.a_extent - ao : 0), sA + st * OpA::kStage, wave);
            db.issue(make_rsrc(p.B + bo, live ? p.b_extent - bo : 0), sB + st * OpB::kStage, wave);
        };
        // Prologue: k-tiles 0 .. NS-2 in flight; tiles 0 and 1 must have
        // landed before the first iteration (it reads tile 1's fragments).
#pragma unroll
        for (int j = 0; j < NS - 1; ++j) issue(j);
        wait_vm_lds<(NS - 3) * NI>();
        barrier_no_fence();

        float f0a[KPL][MB], f0b[KPL][NB], f1a[KPL][MB], f1b[KPL][NB];
        OpA::read_frags(sA, wave_m * WM, li, lh, f0a);
        OpB::read_frags(sB, wave_n * WN, li, lh, f0b);

        // k-tile t, branch free: its MFMAs run from registers; after the first
        // k-step the DMA of k-tile t+NS-1 goes into buffer (t+NS-1)%NS, and
        // after the second the fragments of k-tile t+1 are read. Buffer
        // (t+NS-1)%NS last held k-tile t-1, whose fragments were read in
        // iteration t-2: the barriers closing iterations t-2 and t-1 separate
        // those reads from this DMA. The closing wait leaves k-tile t+NS-1's
        // DMA in flight (none when NS = 3) and completes k-tile t+2 (read in
        // iteration t+1).
        auto step = [&](int t, float (&ca)[KPL][MB], float (&cb)[KPL][NB],
                        float (&na)[KPL][MB], float (&nb)[KPL][NB]) {
            const int st = (t + 1) % NS;
            mfma_kstep<MR, MB, NB, KPL>(acc, ca, cb, 0);
            issue(t + NS - 1);
            mfma_kstep<MR, MB, NB, KPL>(acc, ca, cb, 1);
            OpA::read_frags(sA + st * OpA::kStage, wave_m * WM, li, lh, na);
            OpB::read_frags(sB + st * OpB::kStage, wave_n * WN, li, lh, nb);
#pragma unroll
            for (int s = 2; s < KPL; ++s) mfma_kstep<MR, MB, NB, KPL>(acc, ca, cb, s);
            // Issue order for the scheduler: the DMA loads spread over the
            // first MFMAs, then the fragment reads one per MFMA, then the rest
            // of the MFMAs, so that the reads have landed long before the
            // closing wait and the matrix core never waits on memory. Where
            // a k-tile has fewer MFMAs than memory instructions the
            // compiler's order stands.
            constexpr int kMfma = KPL * MB * NB;
            constexpr int kReads = OpA::kReads + OpB::kReads;
            if constexpr (NI + kReads <= kMfma) {
#pragma unroll
                for (int i = 0; i < NI; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
                    __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);  // VMEM (DMA)
                }
#pragma unroll
                for (int i = 0; i < kReads; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
                }
                if constexpr (kMfma > NI + kReads)
                    __builtin_amdgcn_sched_group_barrier(0x008, kMfma - NI - kReads, 0);
            }
            wait_vm_lds<(NS - 3) * NI>();
            barrier_no_fence();
        };
        int t = 0;
        for (; t + 1 < nk; t += 2) {
            step(t, f0a, f0b, f1a, f1b);
            step(t + 1, f1a, f1b, f0a, f0b);
        }
        if (t < nk) step(t, f0a, f0b, f1a, f1b);
        wait_vm_lds<0>();  // no DMA (not even an empty one) outlives the loop

        if (!kTailInRing && Kp % BK) {
            // Partial last k-tile: every wave has finished its DMA and LDS reads
            // (waited above); the barrier makes that true for all of them
            // before buffer 0 is rewritten.
            __syncthreads();
            OpA opa;
            OpB opb;
            opa.init(tid, p.lda);
            opb.init(tid, p.ldb);
            load_tiles(opa, opb, nk);
            opa.store_lds(sA);
            opb.store_lds(sB);
            __syncthreads();
            OpA::read_frags(sA, wave_m * WM, li, lh, f0a);
            OpB::read_frags(sB, wave_n * WN, li, lh, f0b);
            mfma_ktile<MR, MB, NB, KPL>(acc, f0a, f0b);
        }
    } else {
        const int nk = (Kp + BK - 1) / BK;
        OpA opa;
        OpB opb;
        opa.init(tid, p.lda);
        opb.init(tid, p.ldb);

        if (nk > 0) {
            load_tiles(opa, opb, 0);
            opa.store_lds(sA);
            opb.store_lds(sB);
            if (nk > 1) load_tiles(opa, opb, 1);
            __syncthreads();
        }

        for (int kt = 0; kt < nk; ++kt) {
            const int cur = kt & 1;
            float fa[KPL][MB], fb[KPL][NB];
            OpA::read_frags(sA + cur * OpA::kStage, wave_m * WM, li, lh, fa);
            OpB::read_frags(sB + cur * OpB::kStage, wave_n * WN, li, lh, fb);
            mfma_ktile<MR, MB, NB, KPL>(acc, fa, fb);
            if (kt + 1 < nk) {
                opa.store_lds(sA + (cur ^ 1) * OpA::kStage);
                opb.store_lds(sB + (cur ^ 1) * OpB::kStage);
                if (kt + 2 < nk) load_tiles(opa, opb, kt + 2);
            }
            __syncthreads();
        }
    }

    // Epilogue: C = alpha * acc + beta * C, 128-bit where possible, or with
    // FLAG_EPI C = act(alpha * r_i * c_j * acc + beta * C + u_i + w_j) (and,
    // with FLAG_QUANT, Q = quantize(C) beside it). Wide
    // stores carry the non-temporal hint: C is written once (16384^2 x 256,
    // which writes 1 GiB of C: 1.122 -> 1.079 ms).
    // Accumulator register r of a block, lane (i = lane % MR, h = lane / MR),
    // holds block row Mfma<MR>::row(r, h) and block column i.
    // Lane position again from the hardware lane id (v_mbcnt): keeping the
    // earlier values live across the main loop cost a register spill.
    const int elane = (int)__lane_id();
    const int eli = elane % MR, elh = elane / MR;
    // C, this split's slice of C, or (FLAG_TILE_WS) this tile's and split's
    // own BM x BN slot, addressed tile-locally with ldc = BN.
    const bool tile_ws = p.flags & FLAG_TILE_WS;
    const int64_t c_org = tile_ws ? 0 : (int64_t)m0 * p.ldc + n0;
    float* const Cs =
        tile_ws ? p.C + ((int64_t)(tile_id - p.tile_base) * gridDim.y + blockIdx.y) * (BM * BN)
                : p.C + (int64_t)blockIdx.y * p.c_split_stride;
    const __amdgpu_buffer_rsrc_t rc =
        make_rsrc(Cs + c_org, tile_ws ? (int64_t)BM * BN : p.c_extent - c_org);
    const bool beta0 = p.flags & FLAG_BETA0;
    // A lane's NB columns are one 128-bit (NB = 4) or 64-bit (NB = 2) access
    // when C's rows are aligned for it and all NB columns are inside N.
    const bool vec_c = NB == 4 ? (p.flags & FLAG_VEC_C) != 0
                               : (NB == 2 ? (p.flags & FLAG_VEC2_C) != 0 : false);
    const float alpha = p.alpha, beta = p.beta;
    const int col0 = wave_n * WN + NB * eli;  // first of this lane's NB columns
    const int cols_left = p.N - n0 - col0;
    const bool full_vec = vec_c && cols_left >= NB;
    // The epilogue works in chunks of CH accumulator registers of one block
    // row (8 values per lane).
    constexpr int CH = NB >= 8 ? 1 : (8 / NB < NREG ? 8 / NB : NREG);
    constexpr int NQ = MB * (NREG / CH);  // chunks
    static_assert(NREG % CH == 0, "whole chunks");
    // Rows of C not aligned for a lane's NB adjacent columns to be one access
    // (odd ldc or a misaligned base): NB single stores per row would each
    // scatter over the row with a stride of NB elements. Instead each chunk
    // passes through a slice of the idle operand ring that belongs to the
    // wave (the results staged in shared memory before they are stored, as
    // in "Optimising fp32 GEMM on A100", Kernel 6, there for wider stores):
    // the lanes write their accumulators there, then read it back so that
    // lane l holds element l + 64 j of the chunk (local row e / WN, column
    // e % WN), and one single-element store (or old C read) covers 64
    // consecutive elements of a row of C (WN = 32: two rows of 32). Compiled
    // where the accumulators leave room for it (kStageC).
    constexpr int HR = 64 / MR;  // lane groups = rows per register
    constexpr int V = CH * NB;   // elements per lane per chunk
    const bool stage_c = kStageC && !vec_c;
    const int nrow = p.M - m0, ncol = p.N - n0 - wave_n * WN;
    // Elements past M or N get a byte offset past the end of a resource that
    // spans at most 2^31 bytes from the tile origin (every element of a tile
    // lies below that: at most 255 rows of at most 2^21 elements), so that
    // their loads read 0 and their stores are dropped with no branch: a
    // branch around each access made the compiler wait for every earlier
    // store before each use of the old C.
    constexpr uint32_t kOut = 0xFFFFFFF0u;
    constexpr int64_t kSpan = int64_t(1) << 29;  // elements (2^31 bytes)
    const int64_t c_ext = tile_ws ? (int64_t)BM * BN : p.c_extent - c_org;
    const __amdgpu_buffer_rsrc_t rt = make_rsrc(Cs + c_org, c_ext < kSpan ? c_ext : kSpan);
    // Tile row and wave column of element j of chunk q: with WN >= 64 the row
    // is the same for the whole wave (a scalar) and the column is the lane's
    // plus a constant; with WN = 32 the two halves of the wave take two
    // consecutive local rows.
    const int lsub = WN >= 64 ? 0 : elane / WN, lcol = WN >= 64 ? elane : elane % WN;
    auto elem_rc = [&](int q, int j, int& row, int& col) __attribute__((always_inline)) {
        const int a = q / (NREG / CH), r0 = (q % (NREG / CH)) * CH;
        const int lr = WN >= 64 ? (64 * j) / WN : (64 / WN) * j + lsub;
        col = WN >= 64 ? lcol + (64 * j) % WN : lcol;
        row = wave_m * WM + MB * Mfma<MR>::row(r0 + lr / HR, lr % HR) + a;
    };
    auto c_off = [&](int row, int col) __attribute__((always_inline)) -> uint32_t {
        return row < nrow && col < ncol ? (uint32_t)(row * p.ldc + wave_n * WN + col) * 4u
                                        : kOut;
    };
    auto load_cs = [&](int q, float (&cin)[V]) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < V; ++j) {
            int row, col;
            elem_rc(q, j, row, col);
            cin[j] = ld1(rt, c_off(row, col));
        }
    };
    // Chunk q of this lane's accumulators into the wave's slice, and back in
    // the row order: sv[j] = element j of the chunk.
    auto stage_chunk = [&](float* slice, int q, float (&sv)[V]) __attribute__((always_inline)) {
        const int a = q / (NREG / CH), r0 = (q % (NREG / CH)) * CH;
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            float* const d = slice + (i * HR + elh) * WN + NB * eli;
            if constexpr (NB == 4) {
                *reinterpret_cast<f4*>(d) = f4{acc[a][0][r0 + i], acc[a][1][r0 + i],
                                               acc[a][2][r0 + i], acc[a][3][r0 + i]};
            } else if constexpr (NB == 2) {
                *reinterpret_cast<f2*>(d) = f2{acc[a][0][r0 + i], acc[a][1][r0 + i]};
            } else {
#pragma unroll
                for (int b = 0; b < NB; ++b) d[b] = acc[a][b][r0 + i];
            }
        }
        wave_lds_sync();
#pragma unroll
        for (int j = 0; j < V; ++j) sv[j] = slice[elane + 64 * j];
        wave_lds_sync();  // read before the next chunk rewrites the slice
    };
    // Two copies of the store loop, chosen by a uniform branch: the plain
    // one and the fused epilogue. One loop holding both grew past what the
    // compiler fully unrolls, and the accumulators then went to scratch
    // memory for the whole kernel.
    const bool epi = p.flags & FLAG_EPI;
    if (!epi) {
        // With beta != 0 the old C is read in chunks of 8 values per lane
        // (CH accumulator registers of one block row; two chunks in registers
        // at a time, which keeps every entry at its occupancy), each in full
        // before any of it is stored and the next chunk's reads issued before
        // this one's stores: loads and stores share one counter and no load
        // may pass an earlier store to the same buffer, so reading element by
        // element between the stores would cost a memory round trip per row.
        if (stage_c) {
            static_assert(!kStageC || NW * 64 * V <= NS * (OpA::kStage + OpB::kStage),
                          "slices fit in LDS");
            float* const slice = sA + wave * (64 * V);
            auto store_cs = [&](int q, const float (&cin)[V], bool with_c) {
                float sv[V];
                stage_chunk(slice, q, sv);
#pragma unroll
                for (int j = 0; j < V; ++j) {
                    int row, col;
                    elem_rc(q, j, row, col);
                    float v = alpha * sv[j];
                    if (with_c) v += beta * cin[j];
                    st1_nt(rt, c_off(row, col), v);
                }
            };
            lds_barrier();  // every wave is done reading the operand ring
            float s0[V] = {}, s1[V] = {};
            if (beta0) {
#pragma unroll
                for (int q = 0; q < NQ; ++q) store_cs(q, s0, false);
            } else {
                load_cs(0, s0);
#pragma unroll
                for (int q = 0; q < NQ; q += 2) {
                    if (q + 1 < NQ) load_cs(q + 1, s1);
                    store_cs(q, s0, true);
                    if (q + 1 < NQ) {
                        if (q + 2 < NQ) load_cs(q + 2, s0);
                        store_cs(q + 1, s1, true);
                    }
                }
            }
            return;
        }
        auto load_c = [&](int q, float (&cin)[CH][NB]) {
            const int a = q / (NREG / CH), r0 = (q % (NREG / CH)) * CH;
#pragma unroll
            for (int i = 0; i < CH; ++i) {
                const int row = wave_m * WM + MB * Mfma<MR>::row(r0 + i, elh) + a;
#pragma unroll
                for (int b = 0; b < NB; ++b) cin[i][b] = 0.f;
                if (m0 + row >= p.M) continue;
                const uint32_t off = (uint32_t)(row * p.ldc + col0) * 4u;
                if constexpr (NB == 4) {
                    if (full_vec) {
                        const f4 c4 = ld4(rc, off);
#pragma unroll
                        for (int b = 0; b < 4; ++b) cin[i][b] = c4[b];
                        continue;
                    }
                } else if constexpr (NB == 2) {
                    if (full_vec) {
                        const f2 c2 = ld2(rc, off);
                        cin[i][0] = c2[0];
                        cin[i][1] = c2[1];
                        continue;
                    }
                }
#pragma unroll
                for (int b = 0; b < NB; ++b)
                    if (b < cols_left) cin[i][b] = ld1(rc, off + 4 * b);
            }
        };
        auto store_c = [&](int q, const float (&cin)[CH][NB], bool with_c) {
            const int a = q / (NREG / CH), r0 = (q % (NREG / CH)) * CH;
#pragma unroll
            for (int i = 0; i < CH; ++i) {
                const int row = wave_m * WM + MB * Mfma<MR>::row(r0 + i, elh) + a;
                if (m0 + row >= p.M) continue;
                const uint32_t off = (uint32_t)(row * p.ldc + col0) * 4u;
                float v[NB];
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    v[b] = alpha * acc[a][b][r0 + i];
                    if (with_c) v[b] += beta * cin[i][b];
                }
                if constexpr (NB == 4) {
                    if (full_vec) {
                        st4_nt(rc, off, f4{v[0], v[1], v[2], v[3]});
                        continue;
                    }
                } else if constexpr (NB == 2) {
                    if (full_vec) {
                        st2_nt(rc, off, f2{v[0], v[1]});
                        continue;
                    }
                }
#pragma unroll
                for (int b = 0; b < NB; ++b)
                    if (b < cols_left) st1(rc, off + 4 * b, v[b]);
            }
        };
        float c0[CH][NB] = {}, c1[CH][NB] = {};
        if (beta0) {
#pragma unroll
            for (int q = 0; q < NQ; ++q) store_c(q, c0, false);
        } else {
            load_c(0, c0);
#pragma unroll
            for (int q = 0; q < NQ; q += 2) {
                if (q + 1 < NQ) load_c(q + 1, c1);
                store_c(q, c0, true);
                if (q + 1 < NQ) {
                    if (q + 2 < NQ) load_c(q + 2, c0);
                    store_c(q + 1, c1, true);
                }
            }
        }
    } else {
        // The tile's slices of r, u (BM each) and c, w (BN each) are staged in
        // the now idle operand ring, so that the per-row values come from LDS:
        // global loads would share the vector-memory counter with the stores
        // and every row would wait for the previous row's stores. Each
        // element gets one inlined activation; the old C is read (and the
        // result stored) as one vector when the lane's columns allow, else
        // element by element.
        static_assert(3 * BM + 2 * BN <= NS * (OpA::kStage + OpB::kStage), "vectors fit in LDS");
        // r: BM, then u: BM, then c: BN, then w: BN, then the quantiser's row
        // factors s: BM
        float* const vr = sA;
        __syncthreads();                // every wave is done with the operand ring
        const int etid = wave * 64 + elane;
        const bool quant = kQuant && (p.flags & FLAG_QUANT);
        const bool int8q = quant && p.qkind == QUANT_INT8_ROW;
        for (int t = etid; t < BM; t += NT) {
            const int64_t i = (int64_t)m0 + t;
            const bool in = i < p.M;
            vr[t] = (p.row_scale && in) ? p.row_scale[i] : 1.f;
            vr[BM + t] = (p.row_bias && in) ? p.row_bias[i] : 0.f;
            vr[2 * BM + 2 * BN + t] = (int8q && in) ? p.qscale[i] : 1.f;
        }
        for (int t = etid; t < BN; t += NT) {
            const int64_t j = (int64_t)n0 + t;
            const bool in = j < p.N;
            vr[2 * BM + t] = (p.col_scale && in) ? p.col_scale[j] : 1.f;
            vr[2 * BM + BN + t] = (p.col_bias && in) ? p.col_bias[j] : 0.f;
        }
        __syncthreads();
        float csc[NB], cbi[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            csc[b] = vr[2 * BM + col0 + b];
            cbi[b] = vr[2 * BM + BN + col0 + b];
        }
        // Q of this tile: a buffer from the tile origin to the end of Q;
        // element (row, col) of the tile at byte (row * ldq + col) * esize.
        // A lane's NB codes are one store when Q's rows are aligned to 4
        // elements (FLAG_VEC_Q; col0 is a multiple of NB) and all NB columns
        // are inside N.
        const int qes = p.qkind == QUANT_BF16 ? 2 : 1;
        const int64_t q_org = (int64_t)m0 * p.ldq + n0;
        const __amdgpu_buffer_rsrc_t rq =
            make_rsrc_bytes(static_cast<char*>(p.qout) + (quant ? q_org * qes : 0),
                            quant ? (p.q_extent - q_org) * qes : 0);
        const bool vec_q = (p.flags & FLAG_VEC_Q) && cols_left >= NB;
        auto store_q = [&](auto qtag, int row, const float (&v)[NB]) __attribute__((always_inline)) {
            constexpr int QK = decltype(qtag)::value;
            const float qs = vr[2 * BM + 2 * BN + row];
            const uint32_t qoff = (uint32_t)(row * p.ldq + col0) * (uint32_t)qes;
            uint32_t code[NB];
#pragma unroll
            for (int b = 0; b < NB; ++b)
                code[b] = QK == QUANT_BF16 ? bf16_code(v[b]) : int8_code(v[b], qs);
            if constexpr (NB > 1) {
                if (vec_q) {
                    if constexpr (QK == QUANT_BF16) {
                        if constexpr (NB == 4) {
                            f2 w2 = {__builtin_bit_cast(float, code[0] | (code[1] << 16)),
                                     __builtin_bit_cast(float, code[2] | (code[3] << 16))};
                            st2(rq, qoff, w2);
                        } else {
                            __builtin_amdgcn_raw_buffer_store_b32(code[0] | (code[1] << 16), rq,
                                                                  qoff, 0, 0);
                        }
                    } else {
                        if constexpr (NB == 4)
                            __builtin_amdgcn_raw_buffer_store_b32(
                                code[0] | (code[1] << 8) | (code[2] << 16) | (code[3] << 24), rq,
                                qoff, 0, 0);
                        else
                            __builtin_amdgcn_raw_buffer_store_b16(
                                (uint16_t)(code[0] | (code[1] << 8)), rq, qoff, 0, 0);
                    }
                    return;
                }
            }
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                if (b >= cols_left) continue;
                if constexpr (QK == QUANT_BF16)
                    __builtin_amdgcn_raw_buffer_store_b16((uint16_t)code[b], rq, qoff + 2 * b, 0, 0);
                else
                    __builtin_amdgcn_raw_buffer_store_b8((uint8_t)code[b], rq, qoff + b, 0, 0);
            }
        };
        // One copy of the store loop per activation, picked once (a per-element
        // choice cost a chain of branches around every element).
        auto store_tile = [&](auto tag, auto qtag) {
            constexpr int ACT = decltype(tag)::value;
            constexpr int QK = decltype(qtag)::value;
#pragma unroll
            for (int a = 0; a < MB; ++a) {
#pragma unroll
                for (int r = 0; r < NREG; ++r) {
                    const int brow = Mfma<MR>::row(r, elh);
                    const int row = wave_m * WM + MB * brow + a;
                    if (m0 + row >= p.M) continue;
                    const uint32_t off = (uint32_t)(row * p.ldc + col0) * 4u;
                    const float sr = alpha * vr[row];
                    const float rbi = vr[BM + row];
                    float v[NB];
#pragma unroll
                    for (int b = 0; b < NB; ++b) v[b] = (sr * csc[b]) * acc[a][b][r];
                    if (!beta0) {
                        float cin[NB];
                        if constexpr (NB == 4) {
                            if (full_vec) {
                                const f4 c4 = ld4(rc, off);
#pragma unroll
                                for (int b = 0; b < 4; ++b) cin[b] = c4[b];
                            } else {
#pragma unroll
                                for (int b = 0; b < 4; ++b) cin[b] = b < cols_left ? ld1(rc, off + 4 * b) : 0.f;
                            }
                        } else {
#pragma unroll
                            for (int b = 0; b < NB; ++b) cin[b] = b < cols_left ? ld1(rc, off + 4 * b) : 0.f;
                        }
#pragma unroll
                        for (int b = 0; b < NB; ++b) v[b] += beta * cin[b];
                    }
#pragma unroll
                    for (int b = 0; b < NB; ++b) v[b] = activate_t<ACT>((v[b] + rbi) + cbi[b]);
                    if constexpr (QK != QUANT_NONE) store_q(qtag, row, v);
                    if constexpr (NB == 4) {
                        if (full_vec) {
                            st4_nt(rc, off, f4{v[0], v[1], v[2], v[3]});
                            continue;
                        }
                    }
#pragma unroll
                    for (int b = 0; b < NB; ++b)
                        if (b < cols_left) st1(rc, off + 4 * b, v[b]);
                }
            }
        };
        // The same element order on staged rows (rows of C not aligned; see
        // stage_chunk): element j of chunk q at tile row `row` and wave column
        // `col`, its slice after the vectors above; Q's codes one element at
        // a time, past-the-end offsets for elements outside C as for C.
        constexpr int kVec = (3 * BM + 2 * BN + 3) / 4 * 4;  // floats of the vectors
        static_assert(!kStageFused || kVec + NW * 64 * V <= NS * (OpA::kStage + OpB::kStage),
                      "vectors and slices fit in LDS");
        const int64_t q_bytes = quant ? (p.q_extent - q_org) * qes : 0;
        const __amdgpu_buffer_rsrc_t rqt =
            make_rsrc_bytes(static_cast<char*>(p.qout) + (quant ? q_org * qes : 0),
                            q_bytes < 4 * kSpan ? q_bytes : 4 * kSpan);
        auto store_tile_staged = [&](auto tag, auto qtag) __attribute__((always_inline)) {
            constexpr int ACT = decltype(tag)::value;
            constexpr int QK = decltype(qtag)::value;
            float* const slice = vr + kVec + wave * (64 * V);
            auto store_cs = [&](int q, const float (&cin)[V], bool with_c) __attribute__((always_inline)) {
                float sv[V];
                stage_chunk(slice, q, sv);
#pragma unroll
                for (int j = 0; j < V; ++j) {
                    int row, col;
                    elem_rc(q, j, row, col);
                    const int tcol = wave_n * WN + col;
                    const float sr = alpha * vr[row];
                    float v = (sr * vr[2 * BM + tcol]) * sv[j];
                    if (with_c) v += beta * cin[j];
                    v = activate_t<ACT>((v + vr[BM + row]) + vr[2 * BM + BN + tcol]);
                    const bool in = row < nrow && col < ncol;
                    if constexpr (QK == QUANT_BF16)
                        __builtin_amdgcn_raw_buffer_store_b16(
                            (uint16_t)bf16_code(v), rqt,
                            in ? (uint32_t)(row * p.ldq + tcol) * 2u : kOut, 0, 0);
                    else if constexpr (QK == QUANT_INT8_ROW)
                        __builtin_amdgcn_raw_buffer_store_b8(
                            (uint8_t)int8_code(v, vr[2 * BM + 2 * BN + row]), rqt,
                            in ? (uint32_t)(row * p.ldq + tcol) : kOut, 0, 0);
                    st1_nt(rt, c_off(row, col), v);
                }
            };
            float s0[V] = {}, s1[V] = {};
            if (beta0) {
#pragma unroll
                for (int q = 0; q < NQ; ++q) store_cs(q, s0, false);
            } else {
                load_cs(0, s0);
#pragma unroll
                for (int q = 0; q < NQ; q += 2) {
                    if (q + 1 < NQ) load_cs(q + 1, s1);
                    store_cs(q, s0, true);
                    if (q + 1 < NQ) {
                        if (q + 2 < NQ) load_cs(q + 2, s0);
                        store_cs(q + 1, s1, true);
                    }
                }
            }
        };
        // One copy of the store loop per activation and quantised format,
        // chosen by plain switches (through a further generic lambda the
        // compiler kept the accumulators in scratch memory).
#define FG_STORE_BY_ACT(F, QK)                                                            \
    switch (p.act) {                                                                     \
        case ACT_RELU: F(ActTag<ACT_RELU>{}, ActTag<QK>{}); break;                       \
        case ACT_GELU: F(ActTag<ACT_GELU>{}, ActTag<QK>{}); break;                       \
        case ACT_SILU: F(ActTag<ACT_SILU>{}, ActTag<QK>{}); break;                       \
        default: F(ActTag<ACT_NONE>{}, ActTag<QK>{}); break;                             \
    }
#define FG_STORE_BY_QUANT(F)                                                              \
    if constexpr (kQuant) {                                                              \
        if (!quant) {                                                                    \
            FG_STORE_BY_ACT(F, QUANT_NONE)                                               \
        } else if (p.qkind == QUANT_BF16) {                                              \
            FG_STORE_BY_ACT(F, QUANT_BF16)                                               \
        } else {                                                                         \
            FG_STORE_BY_ACT(F, QUANT_INT8_ROW)                                           \
        }                                                                                \
    } else {                                                                             \
        FG_STORE_BY_ACT(F, QUANT_NONE)                                                   \
    }
        if constexpr (kStageFused) {
            if (stage_c) {
                FG_STORE_BY_QUANT(store_tile_staged)
            } else {
                FG_STORE_BY_QUANT(store_tile)
            }
        } else {
            FG_STORE_BY_QUANT(store_tile)
        }
#undef FG_STORE_BY_QUANT
#undef FG_STORE_BY_ACT
    }
}

// Launch of one instance for one operand layout. Grid: x = tiles (all of
// them unless given), y = split-K slices.
template <int BM, int BN, int WAVES_M, int WAVES_N, int BK, int MR, int STAGES, int DMAB, int OCC,
          int TA, int TB>
hipError_t launch_layout(const GemmParams& p, hipStream_t s, int32_t tiles, int32_t splits) {
    const dim3 grid(tiles >= 0 ? tiles : p.tiles_m * p.tiles_n,
                    splits >= 0 ? splits
                                : (p.K + BK * p.kt_per_split - 1) / (BK * p.kt_per_split)),
        block(64 * WAVES_M * WAVES_N);
    hipLaunchKernelGGL(
        (sgemm_mfma_kernel<BM, BN, WAVES_M, WAVES_N, BK, MR, TA, TB, STAGES, DMAB, OCC>), grid,
        block, 0, s, p);
    return hipGetLastError();
}

}  // namespace mfma
}  // namespace fg
