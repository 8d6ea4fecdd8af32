// One matrix-core table entry in one operand layout: the launcher of one
// instance of sgemm_mfma_kernel (sgemm_mfma.h). The build compiles this file
// once per line of the instance list and layout, with
//   -DFG_ENTRY_ID=<id> -DFG_ENTRY_TA=<0|1> -DFG_ENTRY_TB=<0|1>
//   -DFG_ENTRY_SHAPE=<BM>,<BN>,<WAVES_M>,<WAVES_N>,<BK>,<MR>,<STAGES>,<DMAB>,<OCC>
// so that every kernel is its own translation unit (they compile in
// parallel; one unit holding the 256 x 256 entry's four layouts took over a
// minute and a half).
//
// A tile-search library leaves out layouts its timing shapes never use:
// -DFG_ENTRY_ID=<id> -DFG_ENTRY_STUBS=<mask> defines, for each layout bit
// 2 * TA + TB set in mask, a launcher that only reports hipErrorNotSupported.
#include "sgemm_mfma.h"

#define FG_CAT5(a, b, c, d, e) a##b##c##d##e
#define FG_NAME(id, ta, tb) FG_CAT5(launch_mfma_e, id, _, ta, tb)

namespace fg {

#if defined(FG_ENTRY_STUBS)

#define FG_STUB(ta, tb)                                                                  \
    hipError_t FG_NAME(FG_ENTRY_ID, ta, tb)(const GemmParams&, int32_t, int32_t,         \
                                            hipStream_t) {                               \
        return hipErrorNotSupported;                                                     \
    }
#if (FG_ENTRY_STUBS) & 1
FG_STUB(0, 0)
#endif
#if (FG_ENTRY_STUBS) & 2
FG_STUB(0, 1)
#endif
#if (FG_ENTRY_STUBS) & 4
FG_STUB(1, 0)
#endif
#if (FG_ENTRY_STUBS) & 8
FG_STUB(1, 1)
#endif

#else

#if !defined(FG_ENTRY_ID) || !defined(FG_ENTRY_SHAPE) || !defined(FG_ENTRY_TA) || \
    !defined(FG_ENTRY_TB)
#error "compile with -DFG_ENTRY_ID, -DFG_ENTRY_TA, -DFG_ENTRY_TB and -DFG_ENTRY_SHAPE"
#endif

hipError_t FG_NAME(FG_ENTRY_ID, FG_ENTRY_TA, FG_ENTRY_TB)(const GemmParams& p, int32_t tiles,
                                                         int32_t splits, hipStream_t s) {
    return mfma::launch_layout<FG_ENTRY_SHAPE, FG_ENTRY_TA, FG_ENTRY_TB>(p, s, tiles, splits);
}

#endif

}  // namespace fg
