// Library-owned scratch for the entry point that allocates nothing
// (fa_bwd_noalloc): the backward's row terms (-D and LSE * log2 e, one float
// each per row) live in a file-scope device array instead of a caller
// workspace. Every GPU the library runs on gets its own copy of the array,
// allocated with the code object when the library is loaded there and held
// until the process ends.
//
// In host code `scratch` names a host-side stand-in, not the device array:
// its device address is looked up once per device with hipGetSymbolAddress
// (with that device current) and only that address is ever handed to kernels.

#include <mutex>

#include "fa_launch.h"

namespace fa {

// Two vectors of kNoallocMaxRows floats, each starting on a 256-byte boundary.
constexpr size_t kScratchFloats = 2 * kNoallocMaxRows;
static_assert((kNoallocMaxRows * sizeof(float)) % 256 == 0, "second vector stays 256-byte aligned");

static __device__ __align__(256) float scratch[kScratchFloats];

namespace {

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
float* g_ptr[kMaxDevices];
hipError_t g_err[kMaxDevices];

}  // namespace

hipError_t noalloc_scratch(int device, float** delta, float** lse2) {
    if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
    // `device` is current (the caller checks): the lookup gives this device's copy
    std::call_once(g_once[device], [device] {
        void* p = nullptr;
        g_err[device] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_ptr[device] = g_err[device] == hipSuccess ? static_cast<float*>(p) : nullptr;
    });
    if (g_err[device] != hipSuccess) return g_err[device];
    *delta = g_ptr[device];
    *lse2 = g_ptr[device] + kNoallocMaxRows;
    return hipSuccess;
}

}  // namespace fa
