// Device-resident scratch for fg_sgemm_splitk_noalloc: the split-K partial
// slices of callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops). The array is part of the library's code
// object, so every GPU the library runs on holds its own copy from module
// load until the process ends; nothing is allocated per call.
//
// In host code the name `scratch` is only a host-side stand-in for the
// device variable. Its device address is looked up once per device, with
// that device current, and only that address is ever passed to a kernel.
#include <hip/hip_runtime.h>

#include <mutex>

#include "fg_kernels.h"

static __device__ __align__(256) unsigned char scratch[FG_NOALLOC_SCRATCH_MAX];

namespace fg {
namespace {

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

}  // namespace

hipError_t noalloc_scratch(void** ptr, size_t* bytes) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    *bytes = sizeof scratch;
    return hipSuccess;
}

}  // namespace fg
