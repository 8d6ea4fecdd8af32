// Launch of a matrix-core table entry by id and operand layout: one case per
// line of the instance list, each calling the launchers compiled from that
// line (one per layout).
#include "fg_kernels.h"

#ifndef FG_INSTANCES_INC
#define FG_INSTANCES_INC "fg_mfma_instances.inc"
#endif

namespace fg {

typedef hipError_t (*layout_launcher)(const GemmParams& p, int32_t tiles, int32_t splits,
                                      hipStream_t s);

#define FG_MFMA_ENTRY(id, ...)                                                              \
    hipError_t launch_mfma_e##id##_00(const GemmParams&, int32_t, int32_t, hipStream_t);     \
    hipError_t launch_mfma_e##id##_01(const GemmParams&, int32_t, int32_t, hipStream_t);     \
    hipError_t launch_mfma_e##id##_10(const GemmParams&, int32_t, int32_t, hipStream_t);     \
    hipError_t launch_mfma_e##id##_11(const GemmParams&, int32_t, int32_t, hipStream_t);
#include FG_INSTANCES_INC
#undef FG_MFMA_ENTRY

hipError_t launch_mfma_tiles(int id, int ta, int tb, const GemmParams& p, int32_t tiles,
                             int32_t splits, hipStream_t s) {
    layout_launcher f[4] = {nullptr, nullptr, nullptr, nullptr};
    switch (id) {
#define FG_MFMA_ENTRY(id, ...)         \
    case id:                           \
        f[0] = launch_mfma_e##id##_00; \
        f[1] = launch_mfma_e##id##_01; \
        f[2] = launch_mfma_e##id##_10; \
        f[3] = launch_mfma_e##id##_11; \
        break;
#include FG_INSTANCES_INC
#undef FG_MFMA_ENTRY
        default:
            return hipErrorInvalidValue;
    }
    return f[2 * (ta != 0) + (tb != 0)](p, tiles, splits, s);
}

hipError_t launch_mfma(int id, int ta, int tb, const GemmParams& p, hipStream_t s) {
    return launch_mfma_tiles(id, ta, tb, p, -1, -1, s);
}

}  // namespace fg
