// Host side of the C ABI declared in include/fp32gemm.h: argument
// validation, BLAS quick returns, the tile-configuration table and its
// per-shape selection, and kernel launch on the caller's stream.
//
// The argument list and its meaning follow the BLAS-style routine of
// "CuTe-ly writing an SM86 SGEMM", section "host-side setup" (row-major
// here, with transpose flags); the per-shape choice of tile follows "Matmul
// II: register blocking, warp tiling, tensor cores", section 8 (a library
// ships a family of tile variants and chooses among them for each shape).
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <mutex>

#include "../../include/fp32gemm.h"
#include "../../include/fp32gemm_probe.h"
#include "../../include/fp32gemm_tune.h"
#include "fg_kernels.h"

// The instance list and the fitted efficiencies; a tuner builds a search
// library from other lists by defining these.
#ifndef FG_INSTANCES_INC
#define FG_INSTANCES_INC "fg_mfma_instances.inc"
#endif
#ifndef FG_TUNED_INC
#define FG_TUNED_INC "fg_tuned.inc"
#endif
#ifndef FG_MODEL_INC
#define FG_MODEL_INC "fg_model.inc"
#endif

namespace {

thread_local int32_t t_bad_arg = 0;
thread_local char t_error[256] = "";

fg_status fail(fg_status s, int32_t bad_arg, const char* fmt, ...) {
    t_bad_arg = bad_arg;
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(t_error, sizeof t_error, fmt, ap);
    va_end(ap);
    return s;
}

void clear_error() {
    t_bad_arg = 0;
    t_error[0] = '\0';
}

// ---------------------------------------------------------------------------
// Tile-configuration table.
//
// Matrix-core rows come from the instance list (fg_mfma_instances.inc, one
// compiled kernel instance per row): workgroup tile bm x bn, k-tile bk, wave
// tile wm x wn built from mr x mr accumulator blocks. `wps` is how many waves
// of that kernel one SIMD holds at once (a 128 x 128 wave tile keeps 256
// accumulators plus its operands, which fills the 512 registers a SIMD lane
// has, so one). The vector-ALU and few-row rows are listed here.
struct Entry {
    fg_config cfg;
    int variant;   // index inside the kernel family's launcher (the table id
                   // for matrix-core entries)
    int wps;       // resident waves per SIMD
    int fallback;  // entry used instead when A or B rows are not 16-byte
                   // aligned (entries with 16-byte direct-to-LDS loads only;
                   // -1 = any alignment is fine)
    bool quant;    // writes the quantised second output of fg_sgemm_quant
                   // (matrix-core kernels with at most 128 accumulators per
                   // lane, as sgemm_mfma.h compiles it, and the few-row one)
};

constexpr int kNumCUs = 256;
constexpr int kSimdsPerCU = 4;

Entry make_entry(int id, fg_kind kind, int variant, int bm, int bn, int bk, int wm, int wn,
                 int threads, int stages, int wps, const char* name, int fallback = -1,
                 int mr = 0) {
    Entry e;
    memset(&e, 0, sizeof e);
    e.cfg.id = id;
    e.cfg.kind = kind;
    e.cfg.bm = bm;
    e.cfg.bn = bn;
    e.cfg.bk = bk;
    e.cfg.wm = wm;
    e.cfg.wn = wn;
    e.cfg.threads = threads;
    e.cfg.stages = stages;
    e.cfg.mr = mr;
    e.cfg.lds_bytes = kind == FG_KIND_SKINNY ? 4 * bm * 32 * 4 : stages * (bm + bn) * bk * 4;
    snprintf(e.cfg.name, sizeof e.cfg.name, "%s", name);
    e.variant = variant;
    e.wps = wps;
    e.fallback = fallback;
    e.quant = kind == FG_KIND_SKINNY || (kind == FG_KIND_MFMA && wm * wn / 64 <= 128);
    return e;
}

// Name of a matrix-core entry: tile, k-tile depth, wave grid, then the
// ring depth (direct-to-LDS entries), "_dw" for 4-byte direct-to-LDS loads
// and "_m16" for 16 x 16 blocks.
Entry mfma_entry(int id, int bm, int bn, int waves_m, int waves_n, int bk, int mr, int stages,
                 int dmab, int wps, int fallback) {
    char name[40];
    int n = snprintf(name, sizeof name, "mfma_%dx%dx%d_w%dx%d", bm, bn, bk, waves_m, waves_n);
    if (stages > 2) n += snprintf(name + n, sizeof name - n, "_s%d", stages);
    if (stages > 2 && dmab == 4) n += snprintf(name + n, sizeof name - n, "_dw");
    if (mr == 16) snprintf(name + n, sizeof name - n, "_m16");
    return make_entry(id, FG_KIND_MFMA, id, bm, bn, bk, bm / waves_m, bn / waves_n,
                      64 * waves_m * waves_n, stages, wps, name, fallback, mr);
}

struct Table {
    Entry* rows = nullptr;
    int n = 0;
};

// Number of matrix-core rows in the instance list; they take ids 0 .. n-1
// and the vector-ALU and few-row rows follow them.
#define FG_MFMA_ENTRY(...) +1
constexpr int kNumMfma = 0
#include FG_INSTANCES_INC
    ;
#undef FG_MFMA_ENTRY
constexpr int kIdValu128 = kNumMfma;      // valu_128x128x8_t8x8
constexpr int kIdValu64 = kNumMfma + 1;   // valu_64x64x8_t4x4
constexpr int kIdSkinny = kNumMfma + 2;   // few_rows
// (fg_tuned.inc names the few-row row by this)
#define FG_ID_SKINNY kIdSkinny

const Table& table_rows() {
    static const Table t = [] {
        static Entry mfma[] = {
#define FG_MFMA_ENTRY(id, bm, bn, wm, wn, bk, mr, st, dmab, occ, wps, fb) \
    mfma_entry(id, bm, bn, wm, wn, bk, mr, st, dmab, wps, fb),
#include FG_INSTANCES_INC
#undef FG_MFMA_ENTRY
        };
        static Entry fixed[] = {
            // VALU rows: wm x wn is the per-thread tile; never auto-selected.
            make_entry(kIdValu128, FG_KIND_VALU, 0, 128, 128, 8, 8, 8, 256, 2, 2,
                       "valu_128x128x8_t8x8"),
            make_entry(kIdValu64, FG_KIND_VALU, 1, 64, 64, 8, 4, 4, 256, 2, 4, "valu_64x64x8_t4x4"),
            // Few-row kernel: bm = rows per block (up to 8), bn = columns per
            // workgroup for B stored K x N; memory-bound, costed separately.
            make_entry(kIdSkinny, FG_KIND_SKINNY, 0, 8, 32, 0, 8, 4, 256, 0, 2, "few_rows"),
        };
        constexpr int nf = sizeof fixed / sizeof fixed[0];
        static Entry all[kNumMfma + nf];
        Table t;
        t.rows = all;
        t.n = kNumMfma + nf;
        // Place every row at its id; the ids must be exactly 0 .. n-1.
        bool seen[kNumMfma + nf] = {};
        auto place = [&](const Entry& e) {
            if (e.cfg.id < 0 || e.cfg.id >= t.n || seen[e.cfg.id]) {
                fprintf(stderr, "fp32gemm: table id %d duplicated or out of range\n", e.cfg.id);
                abort();
            }
            seen[e.cfg.id] = true;
            all[e.cfg.id] = e;
        };
        for (int i = 0; i < kNumMfma; ++i) place(mfma[i]);
        for (int i = 0; i < nf; ++i) place(fixed[i]);
        return t;
    }();
    return t;
}

const Entry* table() { return table_rows().rows; }
int num_entries() { return table_rows().n; }

// Cost-model efficiencies, one pair per entry: from the generated table
// (fg_tuned.inc) where it has the entry, else a neutral default, and
// replaceable at run time by a tuner (fg_set_efficiency). Atomics: a tuner
// may set them while other threads plan calls.
struct Efficiency {
    std::atomic<double> eff{0.8}, eff1{0.8};
};
constexpr int kMaxEntries = 256;
static_assert(kNumMfma + 3 <= kMaxEntries, "table larger than the efficiency array");

Efficiency* efficiencies() {
    static Efficiency e[kMaxEntries];
    static std::once_flag once;
    std::call_once(once, [] {
        struct Tuned {
            int id;
            double eff, eff1;
        };
        static const Tuned tuned[] = {
            {-1, 0.0, 0.0},  // (a table may have no rows)
#include FG_TUNED_INC
        };
        for (const Tuned& t : tuned) {
            if (t.id < 0 || t.id >= num_entries()) continue;
            e[t.id].eff.store(t.eff);
            e[t.id].eff1.store(t.eff1);
        }
    });
    return e;
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Estimated time in seconds of the call with MFMA entry e and `splits`
// split-K slices: the rounds of resident waves the grid needs, plus, with
// split-K, the partial slices written, read back and reduced at HBM speed.
constexpr double kSimdFlops = 157.3e12 / (kNumCUs * kSimdsPerCU);  // fp32 MFMA per SIMD

// Constants shared by the entries' cost models (fg_model_constant): the
// defaults below are first estimates from measurements on one MI355X; the
// values fitted by the tuner to the tile search's timings (fg_model.inc)
// replace them; a tuner may set them at run time (fg_set_model_constant).
struct ModelConstants {
    std::atomic<double> v[FG_MODEL_COUNT];
};
ModelConstants& model_constants() {
    static ModelConstants m;
    static std::once_flag once;
    std::call_once(once, [] {
        const double defaults[FG_MODEL_COUNT] = {
            3e-6,    // FG_MODEL_LAUNCH: one more kernel
            6.4e12,  // FG_MODEL_STORE_BW: C tiles leaving the CUs (non-temporal stores)
            0.25,    // FG_MODEL_STORE_EXPOSED: share of those stores not hidden by another
                     //   workgroup's main loop when several share a SIMD
            6.3e12,  // FG_MODEL_STREAM_BW: a stream of the operands, compulsory bytes
            5.0e12,  // FG_MODEL_SPLIT_BW: split-K partial slices, sustained
            5e-6,    // FG_MODEL_FEW_FIXED: launch and reduction of the few-row entry
            0.5,     // FG_MODEL_FEW_MFMA: matrix-core efficiency of the few-row kernel
        };
        for (int i = 0; i < FG_MODEL_COUNT; ++i) m.v[i].store(defaults[i]);
#define FG_MODEL(which, value) m.v[which].store(value);
#include FG_MODEL_INC
#undef FG_MODEL
    });
    return m;
}
double mc(int which) { return model_constants().v[which].load(std::memory_order_relaxed); }

int64_t effective_splits(int64_t K, int64_t bk, int64_t splits, int64_t* kt_per_split) {
    const int64_t kt_total = cdiv(K, bk);
    if (splits < 1) splits = 1;
    if (splits > kt_total) splits = kt_total;
    const int64_t kps = cdiv(kt_total, splits);
    *kt_per_split = kps;
    return cdiv(kt_total, kps);
}

// Time of `workgroups` workgroups of entry e, each summing kps k-tiles, placed
// in rounds of resident workgroups: a workgroup's waves share one CU, and a
// CU holds up to `slots` workgroups (wps waves per SIMD); the last round may
// leave CUs idle. A SIMD shared by `share` waves finishes them after
// share * wave_flops at an efficiency that grows from eff1 (one wave: little
// latency hiding) to eff (wps waves).
double rounds_time(const Entry& e, int64_t workgroups, int64_t kps) {
    const double wave_flops = 2.0 * e.cfg.wm * e.cfg.wn * (double)kps * e.cfg.bk;
    const int64_t w = e.cfg.threads / 64;
    const int64_t slots = std::max<int64_t>(1, (int64_t)e.wps * kSimdsPerCU / w);
    const double full = efficiencies()[e.cfg.id].eff.load(std::memory_order_relaxed);
    const double one = efficiencies()[e.cfg.id].eff1.load(std::memory_order_relaxed);
    double t = 0.0;
    for (int64_t left = workgroups; left > 0;) {
        const int64_t per_cu = std::min<int64_t>(cdiv(left, kNumCUs), slots);
        const int64_t share = std::max<int64_t>(1, cdiv(per_cu * w, kSimdsPerCU));
        const double eff = e.wps > 1 ? one + (full - one) * (double)(share - 1) / (e.wps - 1) : full;
        t += wave_flops * (double)share / (eff * kSimdFlops);
        left -= per_cu * kNumCUs;
    }
    return t;
}

// Time the workgroups' C tiles take to leave the CUs: every round ends with
// each CU writing its tiles (BM x BN floats each). Unless several workgroups
// share each SIMD, the SIMDs of a storing workgroup idle meanwhile; when they
// do, one workgroup's stores overlap another's main loop (counted at a
// quarter).
double store_time(const Entry& e, int64_t workgroups) {
    const int64_t w = e.cfg.threads / 64;
    const int64_t slots = std::max<int64_t>(1, (int64_t)e.wps * kSimdsPerCU / w);
    const double tile_bytes = 4.0 * e.cfg.bm * e.cfg.bn;
    const int64_t per_simd = slots * std::min<int64_t>(w, kSimdsPerCU) / kSimdsPerCU;
    const double exposed = per_simd > 1 ? mc(FG_MODEL_STORE_EXPOSED) : 1.0;
    double t = 0.0;
    for (int64_t left = workgroups; left > 0; left -= (int64_t)kNumCUs * slots)
        t += exposed * (double)std::min<int64_t>(left, (int64_t)kNumCUs * slots) * tile_bytes /
             mc(FG_MODEL_STORE_BW);
    return t;
}

double cost(const Entry& e, int64_t M, int64_t N, int64_t K, int64_t splits, bool beta0) {
    int64_t kps = 0;
    const int64_t s = effective_splits(K, e.cfg.bk, splits, &kps);
    const int64_t tiles = cdiv(M, e.cfg.bm) * cdiv(N, e.cfg.bn);
    const double launch = mc(FG_MODEL_LAUNCH);
    double t = launch + rounds_time(e, tiles * s, kps) + store_time(e, tiles * s);
    // Every operand byte crosses HBM at least once (what bounds few-row
    // shapes whatever the tile).
    const double compulsory =
        4.0 * ((double)M * K + (double)K * N + (double)M * N * (beta0 ? 1 : 2));
    t = std::max(t, launch + compulsory / mc(FG_MODEL_STREAM_BW));
    if (s > 1)
        t += ((double)(2 * s + (beta0 ? 1 : 2)) * M * N * 4.0) / mc(FG_MODEL_SPLIT_BW) + launch;
    return t;
}

// Few-row entry, modelled from measurements on one MI355X: one pass over
// op(B) per block of up to 64 rows, bound by the stream of op(B) (scaled down
// when the grid has fewer than one workgroup per CU) or by the matrix cores,
// which see the rows padded to 16, 32 or 64 and reach a fraction
// FG_MODEL_FEW_MFMA of their peak (about half: 32 x 8192 x 8192 takes 58.6 us,
// 64 rows 99.5). With B stored N x K and at most 4 rows the vector-ALU kernel
// runs instead, at the same stream rate. The entry's efficiency (fitted by
// the tuner) divides the matrix-core term. The fixed cost covers the launch
// and the final reduction.
constexpr int64_t kFewRowsMax = 512;  // rows up to which the entry competes
double skinny_cost(int64_t M, int64_t N, int64_t K, bool beta0, double eff) {
    const double bytes_c = 4.0 * ((double)M * K + (double)M * N * (beta0 ? 1 : 2));
    const int64_t rows = M <= 16 ? 16 : (M <= 32 ? 32 : 64);  // padded rows per pass
    const double passes = (double)cdiv(M, rows);
    const double wgs = passes * (double)cdiv(N, N >= 32 * kNumCUs ? 32 : 16);
    const double fill = std::min(1.0, wgs / kNumCUs);
    const double t_mem = (4.0 * (double)K * N * passes + bytes_c) / (mc(FG_MODEL_STREAM_BW) * fill);
    const double t_mfma = 2.0 * (double)rows * N * K * passes / (157.3e12 * mc(FG_MODEL_FEW_MFMA));
    return mc(FG_MODEL_FEW_FIXED) + std::max(t_mem, t_mfma / eff);
}

// Best MFMA or few-row entry (and split count, at most max_splits). With
// mfma_only (the caller asked for a split), only the MFMA kernels compete.
// A later candidate must beat the best so far by 1%: estimates that close
// are within the model's error (the efficiencies are fitted in steps of
// 0.01), and the earlier table entry -- the tile search keeps entries in the
// order they were chosen, the most widely useful first -- stays the pick, so
// refitted efficiencies do not flip the choice between equivalent kernels.
// (Simulated on the tile search's 27 shapes: the pick runs at 0.998 of the
// fastest instance on geometric mean with a 1% margin, 0.995 with 2%.)
constexpr double kPickMargin = 0.99;
int select_entry(int64_t M, int64_t N, int64_t K, bool ab_aligned, int64_t max_splits,
                 bool beta0, int64_t* best_splits, bool mfma_only = false,
                 bool need_quant = false) {
    static const int64_t kSplits[] = {1, 2, 3, 4, 6, 8, 12, 16, 24, 32, 48, 64};
    int best = -1;
    double best_cost = 0;
    *best_splits = 1;
    for (int i = 0; i < num_entries(); ++i) {
        const Entry& e = table()[i];
        if (need_quant && !e.quant) continue;
        if (e.cfg.kind == FG_KIND_SKINNY) {
            // The few-row model (one pass of op(B) per 64 rows) is fitted on
            // at most 512 rows; past that the matrix-core tiles win on every
            // measured shape.
            if (mfma_only || M > kFewRowsMax) continue;
            const double c = skinny_cost(M, N, K, beta0, efficiencies()[i].eff.load());
            if (best < 0 || c < kPickMargin * best_cost) {
                best = i;
                best_cost = c;
                *best_splits = 1;
            }
            continue;
        }
        if (e.cfg.kind != FG_KIND_MFMA) continue;
        if (e.fallback >= 0 && !ab_aligned) continue;
        for (int64_t sp : kSplits) {
            if (sp > max_splits) break;
            const double c = cost(e, M, N, K, sp, beta0);
            if (best < 0 || c < kPickMargin * best_cost) {
                best = i;
                best_cost = c;
                *best_splits = sp;
            }
        }
    }
    return best;
}

// Raster order of the matrix-core kernels (fg_set_raster in fp32gemm_tune.h;
// for measurements): band height in tile rows, and whether workgroup ids are
// renumbered so each XCD gets a contiguous run of tiles. The default band
// depends on how B is stored; HBM reads per 8192^3 launch, bands of 4 / 8
// tile rows: NN 3.22 / 3.66 GB, TN 3.22 / 3.22, TT 3.49 / 3.22, NT 11.5 / 6.6,
// at equal speed.
constexpr int kGroupMKxN = 4, kGroupMNxK = 8;
std::atomic<int> g_group_m{0};  // 0: the default of the layout
int group_m_for(fg_op transB) {
    const int g = g_group_m.load(std::memory_order_relaxed);
    return g ? g : (transB == FG_OP_T ? kGroupMNxK : kGroupMKxN);
}
// Workgroup size of the few-row kernel's K x N form (fg_set_few_row_threads;
// 0 = automatic).
std::atomic<int> g_few_row_threads{0};
// Few-row kernel family (fg_set_few_row_kernel; 0 = automatic).
std::atomic<int> g_few_row_kernel{0};
std::atomic<int> g_xcd_remap{1};

// ---------------------------------------------------------------------------
// Device check: the kernels are built for gfx950 only.
constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_ok[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other

fg_status check_device() {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return fail(FG_ERR_HIP, 0, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(FG_ERR_UNSUPPORTED, 0, "device index %d out of range", dev);
    int st = g_arch_ok[dev].load(std::memory_order_relaxed);
    if (st == 0) {
        hipDeviceProp_t prop;
        e = hipGetDeviceProperties(&prop, dev);
        if (e != hipSuccess)
            return fail(FG_ERR_HIP, 0, "hipGetDeviceProperties: %s", hipGetErrorString(e));
        st = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
        g_arch_ok[dev].store(st, std::memory_order_relaxed);
    }
    if (st != 1)
        return fail(FG_ERR_UNSUPPORTED, 0, "device %d is not gfx950", dev);
    return FG_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Validation shared by fg_sgemm_ex and fg_select_config.
fg_status validate(fg_op ta, fg_op tb, int64_t M, int64_t N, int64_t K, float alpha,
                   const float* A, int64_t lda, const float* B, int64_t ldb,
                   const float* C, int64_t ldc, bool check_ptrs) {
    if (ta != FG_OP_N && ta != FG_OP_T) return fail(FG_ERR_INVALID_ARG, 1, "transA must be N or T");
    if (tb != FG_OP_N && tb != FG_OP_T) return fail(FG_ERR_INVALID_ARG, 2, "transB must be N or T");
    if (M < 0) return fail(FG_ERR_INVALID_ARG, 3, "M < 0");
    if (N < 0) return fail(FG_ERR_INVALID_ARG, 4, "N < 0");
    if (K < 0) return fail(FG_ERR_INVALID_ARG, 5, "K < 0");
    const int64_t min_lda = ta == FG_OP_N ? K : M;
    const int64_t min_ldb = tb == FG_OP_N ? N : K;
    if (lda < (min_lda > 1 ? min_lda : 1))
        return fail(FG_ERR_INVALID_ARG, 8, "lda=%lld < %lld", (long long)lda, (long long)min_lda);
    if (ldb < (min_ldb > 1 ? min_ldb : 1))
        return fail(FG_ERR_INVALID_ARG, 10, "ldb=%lld < %lld", (long long)ldb, (long long)min_ldb);
    if (ldc < (N > 1 ? N : 1))
        return fail(FG_ERR_INVALID_ARG, 13, "ldc=%lld < N=%lld", (long long)ldc, (long long)N);
    if (check_ptrs) {
        const bool reads_ab = M > 0 && N > 0 && K > 0 && alpha != 0.0f;
        if (reads_ab && !A) return fail(FG_ERR_INVALID_ARG, 7, "A is NULL");
        if (reads_ab && !B) return fail(FG_ERR_INVALID_ARG, 9, "B is NULL");
        if (M > 0 && N > 0 && !C) return fail(FG_ERR_INVALID_ARG, 12, "C is NULL");
    }
    // Limits of this implementation (valid BLAS arguments it cannot run).
    const int64_t kMaxDim = 0x3FFFFFFF;
    if (M > kMaxDim || N > kMaxDim || K > kMaxDim)
        return fail(FG_ERR_UNSUPPORTED, 0, "dimension above %lld", (long long)kMaxDim);
    if (lda > FG_MAX_LD || ldb > FG_MAX_LD || ldc > FG_MAX_LD)
        return fail(FG_ERR_UNSUPPORTED, 0, "leading dimension above %d", FG_MAX_LD);
    return FG_OK;
}

// Stream-K plan for a call: the table entry fg_sgemm would run, its tiles in
// full rounds of resident workgroups (data-parallel), and the tiles of the
// last, partial round (the tail), each split along K into `splits` slices so
// that the tail's tiles x splits workgroups fill one round. Worth it only when
// the tail round is at most three quarters full; otherwise (and whenever the
// workspace holds fewer than two slices per tail tile) the plain call runs.
struct StreamPlan {
    int idx = -1;           // table entry (after the alignment fallback)
    int64_t tiles = 0, full = 0, tail = 0, splits = 1, kps = 0;
    size_t ws_bytes = 0;    // workspace the tail needs
};

// fg_set_streamk_policy: 0 = split the tail when the model expects a gain,
// 1 = whenever the tail round is at most three quarters full.
std::atomic<int> g_streamk_policy{0};

bool plan_streamk(int64_t M, int64_t N, int64_t K, bool ab_aligned, bool beta0, size_t ws_avail,
                  StreamPlan* out) {
    int64_t sp = 1;
    int idx = select_entry(M, N, K, ab_aligned, 1, beta0, &sp);
    if (idx < 0) return false;
    if (table()[idx].fallback >= 0 && !ab_aligned) idx = table()[idx].fallback;
    const Entry& e = table()[idx];
    out->idx = idx;
    if (e.cfg.kind != FG_KIND_MFMA || K <= 0) return false;
    const int64_t waves = e.cfg.threads / 64;
    const int64_t slots = std::max<int64_t>(1, (int64_t)e.wps * kSimdsPerCU / waves);
    const int64_t round = (int64_t)kNumCUs * slots;
    const int64_t tiles = cdiv(M, e.cfg.bm) * cdiv(N, e.cfg.bn);
    const int64_t full = tiles / round * round, tail = tiles - full;
    if (tail == 0 || 4 * tail > 3 * round) return false;
    const int64_t slot_bytes = (int64_t)e.cfg.bm * e.cfg.bn * 4;
    int64_t want = round / tail;
    const int64_t fit = (int64_t)std::min<size_t>(ws_avail / (size_t)(tail * slot_bytes),
                                                  (size_t)1 << 30);
    if (want > fit) want = fit;
    int64_t kps = 0;
    const int64_t splits = effective_splits(K, e.cfg.bk, want, &kps);
    if (splits < 2) return false;
    // Only when the model expects a gain: full rounds + the split tail + the
    // slot traffic of the reduction against the plain call.
    const int64_t kt_total = cdiv(K, e.cfg.bk);
    const double t_split = 3 * mc(FG_MODEL_LAUNCH) + rounds_time(e, full, kt_total) + store_time(e, full) +
                           rounds_time(e, tail * splits, kps) + store_time(e, tail * splits) +
                           (double)tail * (splits + (beta0 ? 1 : 2)) * slot_bytes / mc(FG_MODEL_SPLIT_BW);
    if (g_streamk_policy.load() == 0 && t_split > 0.97 * cost(e, M, N, K, 1, beta0)) return false;
    out->tiles = tiles;
    out->full = full;
    out->tail = tail;
    out->splits = splits;
    out->kps = kps;
    out->ws_bytes = (size_t)(tail * splits * slot_bytes);
    return true;
}

int32_t build_flags(const float* A, int64_t lda, const float* B, int64_t ldb, const float* C,
                    int64_t ldc, float beta) {
    int32_t f = g_xcd_remap.load(std::memory_order_relaxed) ? fg::FLAG_XCD_REMAP : 0;
    if (aligned16(A) && lda % 4 == 0) f |= fg::FLAG_VEC_A;
    if (aligned16(B) && ldb % 4 == 0) f |= fg::FLAG_VEC_B;
    if (aligned16(C) && ldc % 4 == 0) f |= fg::FLAG_VEC_C;
    if (((uintptr_t)C & 7u) == 0 && ldc % 2 == 0) f |= fg::FLAG_VEC2_C;
    if (beta == 0.0f) f |= fg::FLAG_BETA0;
    return f;
}

}  // namespace

extern "C" {

int32_t fg_abi_version(void) { return 2; }

int32_t fg_last_bad_arg(void) { return t_bad_arg; }

const char* fg_last_error(void) { return t_error; }

const char* fg_status_string(fg_status s) {
    switch (s) {
        case FG_OK: return "FG_OK";
        case FG_ERR_INVALID_ARG: return "FG_ERR_INVALID_ARG";
        case FG_ERR_HIP: return "FG_ERR_HIP";
        case FG_ERR_UNSUPPORTED: return "FG_ERR_UNSUPPORTED";
        default: return "FG_UNKNOWN_STATUS";
    }
}

int32_t fg_num_configs(void) { return num_entries(); }

fg_status fg_get_config(int32_t id, fg_config* out) {
    clear_error();
    if (id < 0 || id >= num_entries()) return fail(FG_ERR_INVALID_ARG, 1, "config id %d out of range", id);
    if (!out) return fail(FG_ERR_INVALID_ARG, 2, "out is NULL");
    *out = table()[id].cfg;
    return FG_OK;
}

fg_status fg_select_config(fg_op transA, fg_op transB, int64_t M, int64_t N, int64_t K,
                           const float* A, int64_t lda, const float* B, int64_t ldb,
                           const float* C, int64_t ldc, fg_config* out) {
    clear_error();
    fg_status s = validate(transA, transB, M, N, K, 1.0f, A, lda, B, ldb, C, ldc, false);
    if (s != FG_OK) return s;
    if (!out) return fail(FG_ERR_INVALID_ARG, 12, "out is NULL");
    const int32_t f = build_flags(A, lda, B, ldb, C, ldc, 0.0f);
    const bool ab_aligned = (f & fg::FLAG_VEC_A) && (f & fg::FLAG_VEC_B);
    int64_t splits = 1;
    *out = table()[select_entry(M, N, K, ab_aligned, 1, true, &splits)].cfg;
    return FG_OK;
}

fg_status fg_select_config_quant(fg_op transA, fg_op transB, int64_t M, int64_t N, int64_t K,
                                 const float* A, int64_t lda, const float* B, int64_t ldb,
                                 const float* C, int64_t ldc, int32_t quant_kind,
                                 fg_config* out) {
    clear_error();
    fg_status s = validate(transA, transB, M, N, K, 1.0f, A, lda, B, ldb, C, ldc, false);
    if (s != FG_OK) return s;
    if (quant_kind != FG_QUANT_NONE && quant_kind != FG_QUANT_BF16 &&
        quant_kind != FG_QUANT_INT8_ROW)
        return fail(FG_ERR_INVALID_ARG, 12, "unknown quantised format %d", quant_kind);
    if (!out) return fail(FG_ERR_INVALID_ARG, 13, "out is NULL");
    const int32_t f = build_flags(A, lda, B, ldb, C, ldc, 0.0f);
    const bool ab_aligned = (f & fg::FLAG_VEC_A) && (f & fg::FLAG_VEC_B);
    int64_t splits = 1;
    const int idx = select_entry(M, N, K, ab_aligned, 1, true, &splits, false,
                                 quant_kind != FG_QUANT_NONE);
    if (idx < 0) return fail(FG_ERR_UNSUPPORTED, 0, "no table entry fits this call");
    *out = table()[idx].cfg;
    return FG_OK;
}

}  // extern "C"

namespace {

// The table entry and split-K slice count of a call (the part of run_gemm
// that fg_select_config_ex reports, so the query and the call cannot
// disagree). splits: 1 = no split-K, 0 = choose (bounded by the workspace),
// > 1 = requested; have_ws: a workspace of ws_bytes is given. config_id >= 0
// forces an entry (argument config_arg); ws_arg numbers the workspace size
// in the caller's argument list.
struct Choice {
    int idx = -1;
    int64_t nsplit = 1;  // slices after effective_splits
    int64_t kps = 0;     // k-tiles per slice
};

fg_status choose_entry(int64_t M, int64_t N, int64_t K, bool ab_aligned, float beta,
                       int64_t splits, bool have_ws, size_t ws_bytes, bool quant_on,
                       int32_t config_id, int config_arg, int ws_arg, Choice* out) {
    const int64_t slice = M * N;  // floats per split-K partial
    // One slice needs no workspace, so at least one is always possible.
    int64_t max_splits =
        have_ws && slice > 0 ? (int64_t)(ws_bytes / (sizeof(float) * (size_t)slice)) : 1;
    if (max_splits < 1) max_splits = 1;
    int64_t want = splits;
    int idx;
    if (config_id >= 0) {
        idx = config_id;
        if (want == 0) want = 1;
        if (quant_on && !table()[idx].quant)
            return fail(FG_ERR_INVALID_ARG, config_arg,
                        "entry %s has no quantised output (another entry, or -1)",
                        table()[idx].cfg.name);
    } else {
        int64_t auto_splits = 1;
        idx = select_entry(M, N, K, ab_aligned, want == 0 ? max_splits : want, beta == 0.0f,
                           &auto_splits, want > 1, quant_on);
        if (want == 0) want = auto_splits;
    }
    if (idx < 0 || idx >= num_entries())
        return fail(FG_ERR_UNSUPPORTED, 0, "no table entry fits this call");
    if (table()[idx].fallback >= 0 && !ab_aligned) idx = table()[idx].fallback;
    const Entry& en = table()[idx];
    if (quant_on && !en.quant)
        return fail(FG_ERR_INVALID_ARG, config_arg, "entry %s has no quantised output",
                    en.cfg.name);
    if (en.cfg.kind != FG_KIND_MFMA) want = 1;  // split-K runs on the MFMA kernels
    // The few-row kernels put their blocks of rows (8 on the vector ALU, at
    // least 16 on the matrix cores) on the grid's y dimension (at most 65535).
    if (en.cfg.kind == FG_KIND_SKINNY && cdiv(M, 8) > 65535)
        return fail(FG_ERR_UNSUPPORTED, 0, "the few-row entry takes at most %d rows", 65535 * 8);

    int64_t kps = 0;
    // k-tile depth of the MFMA kernels; the other kinds ignore the split.
    const int64_t split_bk = en.cfg.kind == FG_KIND_MFMA ? en.cfg.bk : 16;
    const int64_t nsplit = effective_splits(K, split_bk, want, &kps);
    if (nsplit > 1 && nsplit > max_splits)
        return fail(FG_ERR_INVALID_ARG, ws_arg,
                    "workspace of %zu bytes holds %lld splits, need %lld", ws_bytes,
                    (long long)max_splits, (long long)nsplit);
    out->idx = idx;
    out->nsplit = nsplit;
    out->kps = kps;
    return FG_OK;
}

// Shared body of fg_sgemm_ex and fg_sgemm_splitk. splits: 1 = no split-K,
// 0 = choose (bounded by the workspace), > 1 = requested.
fg_status run_gemm(fg_op transA, fg_op transB, int64_t M, int64_t N, int64_t K, float alpha,
                   const float* A, int64_t lda, const float* B, int64_t ldb, float beta,
                   float* C, int64_t ldc, hipStream_t stream, int32_t config_id,
                   int64_t splits, float* ws, size_t ws_bytes,
                   const fg_epilogue* epi = nullptr, int config_arg = 15, bool streamk = false,
                   const fg_quant* quant = nullptr) {
    clear_error();
    fg_status s = validate(transA, transB, M, N, K, alpha, A, lda, B, ldb, C, ldc, true);
    if (s != FG_OK) return s;
    if (config_id < -1 || config_id >= num_entries())
        return fail(FG_ERR_INVALID_ARG, config_arg, "config id %d out of range", config_id);
    const bool quant_on = quant && quant->kind != FG_QUANT_NONE;
    const bool epi_on = quant_on || (epi && (epi->row_scale || epi->col_scale || epi->row_bias ||
                                             epi->col_bias || epi->activation != FG_ACT_NONE));

    // Quick returns.
    if (M == 0 || N == 0) return FG_OK;
    const bool no_product = (K == 0 || alpha == 0.0f);
    if (no_product && beta == 1.0f && !epi_on) return FG_OK;

    fg::GemmParams p;
    memset(&p, 0, sizeof p);
    p.A = A;
    p.B = B;
    p.C = C;
    p.M = (int32_t)M;
    p.N = (int32_t)N;
    p.K = (int32_t)K;
    p.lda = (int32_t)lda;
    p.ldb = (int32_t)ldb;
    p.ldc = (int32_t)ldc;
    p.alpha = alpha;
    p.beta = beta;
    // Extent of each stored matrix: rows * ld, minus the unused tail of the last row.
    const int64_t a_rows = transA == FG_OP_N ? M : K, a_cols = transA == FG_OP_N ? K : M;
    const int64_t b_rows = transB == FG_OP_N ? K : N, b_cols = transB == FG_OP_N ? N : K;
    p.a_extent = a_rows > 0 && a_cols > 0 ? (a_rows - 1) * lda + a_cols : 0;
    p.b_extent = b_rows > 0 && b_cols > 0 ? (b_rows - 1) * ldb + b_cols : 0;
    p.c_extent = (M - 1) * ldc + N;
    p.flags = build_flags(A, lda, B, ldb, C, ldc, beta);
    if (epi_on) {
        p.flags |= fg::FLAG_EPI;
        if (epi) {
            p.row_scale = epi->row_scale;
            p.col_scale = epi->col_scale;
            p.row_bias = epi->row_bias;
            p.col_bias = epi->col_bias;
            p.act = epi->activation;
        }
    }
    if (quant_on) {
        const int esize = quant->kind == FG_QUANT_BF16 ? 2 : 1;
        p.flags |= fg::FLAG_QUANT;
        p.qout = quant->out;
        p.ldq = (int32_t)quant->ldq;
        p.qkind = quant->kind == FG_QUANT_BF16 ? fg::QUANT_BF16 : fg::QUANT_INT8_ROW;
        p.qscale = quant->row_factor;
        p.q_extent = (M - 1) * quant->ldq + N;
        if (quant->ldq % 4 == 0 && ((uintptr_t)quant->out % (uintptr_t)(4 * esize)) == 0)
            p.flags |= fg::FLAG_VEC_Q;
    }

    if (no_product) {
        s = check_device();
        if (s != FG_OK) return s;
        const hipError_t e = fg::launch_scale(p, stream);
        if (e != hipSuccess) return fail(FG_ERR_HIP, 0, "kernel launch: %s", hipGetErrorString(e));
        return FG_OK;
    }

    const bool ab_aligned = (p.flags & fg::FLAG_VEC_A) && (p.flags & fg::FLAG_VEC_B);

    StreamPlan plan;
    if (streamk && plan_streamk(M, N, K, ab_aligned, beta == 0.0f, ws ? ws_bytes : 0, &plan)) {
        // Full rounds data-parallel into C, the tail's (tile, split) partials
        // into their workspace slots, then the fixed-order tail reduction.
        const Entry& en = table()[plan.idx];
        s = check_device();
        if (s != FG_OK) return s;
        p.tiles_m = (int32_t)cdiv(M, en.cfg.bm);
        p.tiles_n = (int32_t)cdiv(N, en.cfg.bn);
        p.group_m = std::min(group_m_for(transB), p.tiles_m);
        hipError_t e = hipSuccess;
        if (plan.full > 0) {
            fg::GemmParams d = p;
            d.kt_per_split = (int32_t)cdiv(K, en.cfg.bk);  // tile ids [0, full), all of K
            e = fg::launch_mfma_tiles(en.variant, transA, transB, d, (int32_t)plan.full, 1,
                                      stream);
        }
        if (e == hipSuccess) {
            fg::GemmParams q = p;
            q.C = ws;
            q.ldc = en.cfg.bn;
            q.c_extent = (int64_t)(plan.ws_bytes / sizeof(float));
            q.alpha = 1.0f;
            q.beta = 0.0f;
            q.flags = build_flags(A, lda, B, ldb, ws, en.cfg.bn, 0.0f) | fg::FLAG_TILE_WS;
            q.tile_base = (int32_t)plan.full;
            q.kt_per_split = (int32_t)plan.kps;
            e = fg::launch_mfma_tiles(en.variant, transA, transB, q, (int32_t)plan.tail,
                                      (int32_t)plan.splits, stream);
        }
        if (e == hipSuccess) {
            fg::GemmParams r = p;
            r.tile_base = (int32_t)plan.full;
            e = fg::launch_tile_reduce(ws, (int32_t)plan.splits, (int32_t)plan.tail, en.cfg.bm,
                                       en.cfg.bn, r, stream);
        }
        if (e != hipSuccess) return fail(FG_ERR_HIP, 0, "kernel launch: %s", hipGetErrorString(e));
        return FG_OK;
    }
    Choice ch;
    s = choose_entry(M, N, K, ab_aligned, beta, splits, ws != nullptr, ws_bytes, quant_on,
                     config_id, config_arg, 16, &ch);
    if (s != FG_OK) return s;
    const Entry& en = table()[ch.idx];
    const int64_t slice = M * N;  // floats per split-K partial
    const int64_t nsplit = ch.nsplit, kps = ch.kps;

    s = check_device();
    if (s != FG_OK) return s;

    p.tiles_m = (int32_t)cdiv(M, en.cfg.bm);
    p.tiles_n = (int32_t)cdiv(N, en.cfg.bn);
    const int64_t nblocks = (int64_t)p.tiles_m * p.tiles_n;
    if (nblocks > 0x7FFFFFFF) return fail(FG_ERR_UNSUPPORTED, 0, "too many tiles");
    p.group_m = std::min(group_m_for(transB), p.tiles_m);
    p.kt_per_split = (int32_t)kps;
    p.c_split_stride = 0;

    hipError_t e;
    if (nsplit > 1) {
        // Partial products (alpha = 1, beta = 0) into dense M x N slices of
        // the workspace, then C = alpha * sum + beta * C.
        fg::GemmParams q = p;
        q.C = ws;
        q.ldc = (int32_t)N;
        q.c_extent = slice;
        q.c_split_stride = slice;
        q.alpha = 1.0f;
        q.beta = 0.0f;
        q.flags = build_flags(A, lda, B, ldb, ws, N, 0.0f);
        e = fg::launch_mfma(en.variant, transA, transB, q, stream);
        if (e == hipSuccess) e = fg::launch_splitk_reduce(ws, (int32_t)nsplit, p, stream);
    } else if (en.cfg.kind == FG_KIND_MFMA) {
        e = fg::launch_mfma(en.variant, transA, transB, p, stream);
    } else if (en.cfg.kind == FG_KIND_SKINNY) {
        e = fg::launch_skinny(transA, transB, p, stream, g_few_row_threads.load(),
                              g_few_row_kernel.load());
    } else {
        e = fg::launch_valu(en.variant, transA, transB, p, stream);
    }
    if (e != hipSuccess) return fail(FG_ERR_HIP, 0, "kernel launch: %s", hipGetErrorString(e));
    return FG_OK;
}

}  // namespace

extern "C" {

fg_status fg_sgemm_ex(fg_op transA, fg_op transB, int64_t M, int64_t N, int64_t K, float alpha,
                      const float* A, int64_t lda, const float* B, int64_t ldb, float beta,
                      float* C, int64_t ldc, hipStream_t stream, int32_t config_id) {
    return run_gemm(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream,
                    config_id, 1, nullptr, 0);
}

size_t fg_sgemm_splitk_workspace_size(int64_t M, int64_t N, int32_t splits) {
    if (M <= 0 || N <= 0 || splits <= 1) return 0;
    return (size_t)M * (size_t)N * (size_t)splits * sizeof(float);
}

fg_status fg_sgemm_splitk(fg_op transA, fg_op transB, int64_t M, int64_t N, int64_t K,
                          float alpha, const float* A, int64_t lda, const float* B, int64_t ldb,
                          float beta, float* C, int64_t ldc, int32_t splits, void* workspace,
                          size_t workspace_bytes, hipStream_t stream) {
    clear_error();
    if (splits < 0) return fail(FG_ERR_INVALID_ARG, 14, "splits < 0");
    if (splits > 1 && !workspace) return fail(FG_ERR_INVALID_ARG, 15, "workspace is NULL");
    if (workspace && ((uintptr_t)workspace & 3u))
        return fail(FG_ERR_INVALID_ARG, 15, "workspace is not 4-byte aligned");
    return run_gemm(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream, -1,
                    splits, (float*)workspace, workspace ? workspace_bytes : 0);
}

fg_status fg_select_config_ex(fg_op transA, fg_op transB, int64_t M, int64_t N, int64_t K,
                              const float* A, int64_t lda, const float* B, int64_t ldb,
                              float beta, const float* C, int64_t ldc, int32_t splits,
                              size_t workspace_bytes, int32_t quant_kind, fg_config* out,
                              int32_t* splits_out) {
    clear_error();
    fg_status s = validate(transA, transB, M, N, K, 1.0f, A, lda, B, ldb, C, ldc, false);
    if (s != FG_OK) return s;
    if (splits < 0) return fail(FG_ERR_INVALID_ARG, 13, "splits < 0");
    if (quant_kind != FG_QUANT_NONE && quant_kind != FG_QUANT_BF16 &&
        quant_kind != FG_QUANT_INT8_ROW)
        return fail(FG_ERR_INVALID_ARG, 15, "unknown quantised format %d", quant_kind);
    if (!out) return fail(FG_ERR_INVALID_ARG, 16, "out is NULL");
    const int32_t f = build_flags(A, lda, B, ldb, C, ldc, beta);
    const bool ab_aligned = (f & fg::FLAG_VEC_A) && (f & fg::FLAG_VEC_B);
    Choice ch;
    s = choose_entry(M, N, K, ab_aligned, beta, splits, workspace_bytes > 0, workspace_bytes,
                     quant_kind != FG_QUANT_NONE, -1, 0, 14, &ch);
    if (s != FG_OK) return s;
    *out = table()[ch.idx].cfg;
    if (splits_out) *splits_out = (int32_t)ch.nsplit;
    return FG_OK;
}

fg_status fg_sgemm_splitk_noalloc(fg_op transA, fg_op transB, int64_t M, int64_t N, int64_t K,
                                  float alpha, const float* A, int64_t lda, const float* B,
                                  int64_t ldb, float beta, float* C, int64_t ldc, int32_t splits,
                                  hipStream_t stream) {
    clear_error();
    if (splits < 0) return fail(FG_ERR_INVALID_ARG, 14, "splits < 0");
    // Requests that cannot fit are refused before any device call.
    const size_t cap = FG_NOALLOC_SCRATCH_MAX;
    if (splits > 1 && M > 0 && N > 0 &&
        (double)M * (double)N * (double)splits * sizeof(float) > (double)cap)
        return fail(FG_ERR_INVALID_ARG, 14,
                    "%d slices of %lld x %lld floats need %.0f bytes of scratch; at most %zu",
                    splits, (long long)M, (long long)N,
                    (double)M * (double)N * (double)splits * sizeof(float), cap);
    fg_status s = validate(transA, transB, M, N, K, alpha, A, lda, B, ldb, C, ldc, true);
    if (s != FG_OK) return s;
    if (splits == 1 || M == 0 || N == 0 || K == 0 || alpha == 0.0f)
        return run_gemm(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream, -1,
                        1, nullptr, 0);
    s = check_device();
    if (s != FG_OK) return s;
    void* ws = nullptr;
    size_t ws_bytes = 0;
    const hipError_t e = fg::noalloc_scratch(&ws, &ws_bytes);
    if (e != hipSuccess)
        return fail(FG_ERR_HIP, 0, "scratch address: %s", hipGetErrorString(e));
    return run_gemm(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream, -1,
                    splits, (float*)ws, ws_bytes);
}

size_t fg_sgemm_splitk_noalloc_max_bytes(void) { return FG_NOALLOC_SCRATCH_MAX; }

size_t fg_sgemm_streamk_workspace_size(fg_op transA, fg_op transB, int64_t M, int64_t N,
                                       int64_t K, const float* A, int64_t lda, const float* B,
                                       int64_t ldb) {
    if (validate(transA, transB, M, N, K, 1.0f, A, lda, B, ldb, nullptr, std::max<int64_t>(1, N),
                 false) != FG_OK)
        return 0;
    if (M == 0 || N == 0 || K == 0) return 0;
    const int32_t f = build_flags(A, lda, B, ldb, nullptr, N, 0.0f);
    const bool ab_aligned = (f & fg::FLAG_VEC_A) && (f & fg::FLAG_VEC_B);
    StreamPlan plan;
    // beta does not change the plan (only the cost of the plain choice)
    if (!plan_streamk(M, N, K, ab_aligned, true, (size_t)-1, &plan)) return 0;
    return plan.ws_bytes;
}

fg_status fg_sgemm_streamk(fg_op transA, fg_op transB, int64_t M, int64_t N, int64_t K,
                           float alpha, const float* A, int64_t lda, const float* B, int64_t ldb,
                           float beta, float* C, int64_t ldc, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
    clear_error();
    if (workspace && ((uintptr_t)workspace & 15u))
        return fail(FG_ERR_INVALID_ARG, 14, "workspace is not 16-byte aligned");
    return run_gemm(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream, -1, 1,
                    (float*)workspace, workspace ? workspace_bytes : 0, nullptr, 15, true);
}

fg_status fg_sgemm(fg_op transA, fg_op transB, int64_t M, int64_t N, int64_t K, float alpha,
                   const float* A, int64_t lda, const float* B, int64_t ldb, float beta,
                   float* C, int64_t ldc, hipStream_t stream) {
    return fg_sgemm_ex(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream, -1);
}

fg_status fg_sgemm_fused(fg_op transA, fg_op transB, int64_t M, int64_t N, int64_t K,
                         float alpha, const float* A, int64_t lda, const float* B, int64_t ldb,
                         float beta, float* C, int64_t ldc, const fg_epilogue* epilogue,
                         hipStream_t stream, int32_t config_id) {
    clear_error();
    if (epilogue && (epilogue->activation < FG_ACT_NONE || epilogue->activation > FG_ACT_SILU))
        return fail(FG_ERR_INVALID_ARG, 14, "activation %d is not an fg_activation",
                    epilogue->activation);
    return run_gemm(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream,
                    config_id, 1, nullptr, 0, epilogue, 16);
}

fg_status fg_sgemm_quant(fg_op transA, fg_op transB, int64_t M, int64_t N, int64_t K,
                         float alpha, const float* A, int64_t lda, const float* B, int64_t ldb,
                         float beta, float* C, int64_t ldc, const fg_epilogue* epilogue,
                         const fg_quant* quant, hipStream_t stream, int32_t config_id) {
    clear_error();
    if (epilogue && (epilogue->activation < FG_ACT_NONE || epilogue->activation > FG_ACT_SILU))
        return fail(FG_ERR_INVALID_ARG, 14, "activation %d is not an fg_activation",
                    epilogue->activation);
    if (quant) {
        if (quant->kind < FG_QUANT_NONE || quant->kind > FG_QUANT_INT8_ROW)
            return fail(FG_ERR_INVALID_ARG, 15, "kind %d is not an fg_quant_kind", quant->kind);
        if (quant->kind != FG_QUANT_NONE) {
            if (quant->ldq < std::max<int64_t>(1, N))
                return fail(FG_ERR_INVALID_ARG, 15, "ldq=%lld < N=%lld", (long long)quant->ldq,
                            (long long)N);
            if (quant->ldq > FG_MAX_LD)
                return fail(FG_ERR_UNSUPPORTED, 0, "ldq above %d", FG_MAX_LD);
            if (M > 0 && N > 0 && !quant->out)
                return fail(FG_ERR_INVALID_ARG, 15, "quantised output is NULL");
            if (M > 0 && N > 0 && quant->kind == FG_QUANT_INT8_ROW && !quant->row_factor)
                return fail(FG_ERR_INVALID_ARG, 15, "row factors are NULL");
        }
    }
    return run_gemm(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream,
                    config_id, 1, nullptr, 0, epilogue, 17, false, quant);
}

double fg_estimate_seconds(int64_t M, int64_t N, int64_t K, int32_t config_id, int32_t splits,
                           int32_t beta_zero) {
    if (M < 0 || N < 0 || K < 0 || config_id < 0 || config_id >= num_entries()) return -1.0;
    const Entry& e = table()[config_id];
    if (e.cfg.kind == FG_KIND_SKINNY)
        return skinny_cost(M, N, K, beta_zero != 0, efficiencies()[config_id].eff.load());
    if (e.cfg.kind != FG_KIND_MFMA) return -1.0;
    return cost(e, M, N, K, splits < 1 ? 1 : splits, beta_zero != 0);
}

fg_status fg_get_efficiency(int32_t config_id, double* eff, double* eff1) {
    clear_error();
    if (config_id < 0 || config_id >= num_entries() || table()[config_id].cfg.kind == FG_KIND_VALU)
        return fail(FG_ERR_INVALID_ARG, 1, "config %d has no modelled efficiency", config_id);
    if (!eff) return fail(FG_ERR_INVALID_ARG, 2, "eff is NULL");
    if (!eff1) return fail(FG_ERR_INVALID_ARG, 3, "eff1 is NULL");
    *eff = efficiencies()[config_id].eff.load();
    *eff1 = efficiencies()[config_id].eff1.load();
    return FG_OK;
}

fg_status fg_set_efficiency(int32_t config_id, double eff, double eff1) {
    clear_error();
    if (config_id < 0 || config_id >= num_entries() || table()[config_id].cfg.kind == FG_KIND_VALU)
        return fail(FG_ERR_INVALID_ARG, 1, "config %d has no modelled efficiency", config_id);
    if (!(eff > 0.0 && eff <= 1.0)) return fail(FG_ERR_INVALID_ARG, 2, "eff outside (0, 1]");
    if (!(eff1 > 0.0 && eff1 <= 1.0)) return fail(FG_ERR_INVALID_ARG, 3, "eff1 outside (0, 1]");
    efficiencies()[config_id].eff.store(eff);
    efficiencies()[config_id].eff1.store(eff1);
    return FG_OK;
}

fg_status fg_set_raster(int32_t group_m, int32_t xcd_remap) {
    clear_error();
    if (group_m < 0 || group_m > 4096)
        return fail(FG_ERR_INVALID_ARG, 1, "group_m %d outside 0..4096", group_m);
    if (xcd_remap != 0 && xcd_remap != 1)
        return fail(FG_ERR_INVALID_ARG, 2, "xcd_remap must be 0 or 1");
    g_group_m.store(group_m);
    g_xcd_remap.store(xcd_remap);
    return FG_OK;
}

fg_status fg_set_few_row_threads(int32_t threads) {
    clear_error();
    if (threads != 0 && threads != 256 && threads != 512 && threads != 1024)
        return fail(FG_ERR_INVALID_ARG, 1, "threads must be 0, 256, 512 or 1024");
    g_few_row_threads.store(threads);
    return FG_OK;
}

fg_status fg_get_model_constant(int32_t which, double* value) {
    clear_error();
    if (which < 0 || which >= FG_MODEL_COUNT)
        return fail(FG_ERR_INVALID_ARG, 1, "model constant %d out of range", which);
    if (!value) return fail(FG_ERR_INVALID_ARG, 2, "value is NULL");
    *value = mc(which);
    return FG_OK;
}

fg_status fg_set_model_constant(int32_t which, double value) {
    clear_error();
    if (which < 0 || which >= FG_MODEL_COUNT)
        return fail(FG_ERR_INVALID_ARG, 1, "model constant %d out of range", which);
    const bool fraction = which == FG_MODEL_STORE_EXPOSED || which == FG_MODEL_FEW_MFMA;
    if (!(value > 0.0) || (fraction && value > 1.0) || !(value < 1e300))
        return fail(FG_ERR_INVALID_ARG, 2, "value %g outside its domain", value);
    model_constants().v[which].store(value);
    return FG_OK;
}

fg_status fg_set_few_row_kernel(int32_t kernel) {
    clear_error();
    if (kernel < 0 || kernel > 2)
        return fail(FG_ERR_INVALID_ARG, 1, "kernel must be 0, 1 or 2");
    g_few_row_kernel.store(kernel);
    return FG_OK;
}

fg_status fg_get_raster(int32_t* group_m, int32_t* xcd_remap) {
    clear_error();
    if (!group_m) return fail(FG_ERR_INVALID_ARG, 1, "group_m is NULL");
    if (!xcd_remap) return fail(FG_ERR_INVALID_ARG, 2, "xcd_remap is NULL");
    *group_m = g_group_m.load();
    *xcd_remap = g_xcd_remap.load();
    return FG_OK;
}

fg_status fg_set_streamk_policy(int32_t policy) {
    clear_error();
    if (policy != 0 && policy != 1) return fail(FG_ERR_INVALID_ARG, 1, "policy must be 0 or 1");
    g_streamk_policy.store(policy);
    return FG_OK;
}

double fg_probe_mfma_flops(int32_t workgroups, int32_t iterations) {
    if (workgroups <= 0 || iterations <= 0) return 0.0;
    return (double)workgroups * 4.0 * (double)iterations * 4.0 * 4096.0;
}

fg_status fg_probe_mfma(int32_t workgroups, int32_t iterations, float* out, hipStream_t stream) {
    clear_error();
    if (workgroups < 1 || workgroups > 65536)
        return fail(FG_ERR_INVALID_ARG, 1, "workgroups %d outside 1..65536", workgroups);
    if (iterations < 1 || iterations > (1 << 24))
        return fail(FG_ERR_INVALID_ARG, 2, "iterations %d outside 1..16777216", iterations);
    if (!out) return fail(FG_ERR_INVALID_ARG, 3, "out is NULL");
    fg_status s = check_device();
    if (s != FG_OK) return s;
    const hipError_t e = fg::launch_probe_mfma(workgroups, iterations, out, stream);
    if (e != hipSuccess) return fail(FG_ERR_HIP, 0, "kernel launch: %s", hipGetErrorString(e));
    return FG_OK;
}

fg_status fg_probe_lds_dma(const float* src, int32_t bytes_per_lane, float* out,
                           hipStream_t stream) {
    clear_error();
    if (!src) return fail(FG_ERR_INVALID_ARG, 1, "src is NULL");
    if (bytes_per_lane != 4 && bytes_per_lane != 16)
        return fail(FG_ERR_INVALID_ARG, 2, "bytes_per_lane must be 4 or 16");
    if (!out) return fail(FG_ERR_INVALID_ARG, 3, "out is NULL");
    fg_status s = check_device();
    if (s != FG_OK) return s;
    const hipError_t e = fg::launch_probe_lds_dma(src, bytes_per_lane, out, stream);
    if (e != hipSuccess) return fail(FG_ERR_HIP, 0, "kernel launch: %s", hipGetErrorString(e));
    return FG_OK;
}

fg_status fg_probe_read(const float* x, int64_t n, int32_t workgroups, float* out,
                        hipStream_t stream) {
    clear_error();
    if (n < 0 || (n & 3)) return fail(FG_ERR_INVALID_ARG, 2, "n=%lld is not a multiple of 4 >= 0",
                                      (long long)n);
    if (n > 0 && !x) return fail(FG_ERR_INVALID_ARG, 1, "x is NULL");
    if ((uintptr_t)x & 15u) return fail(FG_ERR_INVALID_ARG, 1, "x is not 16-byte aligned");
    if (workgroups < 1 || workgroups > 65536)
        return fail(FG_ERR_INVALID_ARG, 3, "workgroups %d outside 1..65536", workgroups);
    if (!out) return fail(FG_ERR_INVALID_ARG, 4, "out is NULL");
    fg_status s = check_device();
    if (s != FG_OK) return s;
    const hipError_t e = fg::launch_probe_read(x, n / 4, workgroups, out, stream);
    if (e != hipSuccess) return fail(FG_ERR_HIP, 0, "kernel launch: %s", hipGetErrorString(e));
    return FG_OK;
}

}  // extern "C"
