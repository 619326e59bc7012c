// Shared state of the host-only stand-ins (fa_host_stubs.cpp) and their
// checks (fa_host_check.cpp).
#pragma once

#include "../../exact_io_aware_54_amd/csrc/fa_launch.h"

namespace fa {

constexpr int kMaxPtr = 11;

struct Recorded {
    int calls;
    char name[32];
    int n_ptr;
    const void* ptr[kMaxPtr];
    long long arg[6];
    // fp8 backward: the three code conversions
    int n_conv;
    const void* conv_src[3];
    void* conv_dst[3];
    long long conv_n;
    int scratch_device;
};

extern Recorded g_rec;
extern hipError_t g_launch_result;  // what every stand-in launcher returns
extern hipError_t g_pending;        // error hipGetLastError reports (and clears)
extern int g_device;                // hipGetDevice
extern int g_stream_device;         // hipStreamGetDevice

}  // namespace fa
