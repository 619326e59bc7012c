// Measurement probe: the practical bf16 MFMA rate and the shader clock.
//
// Every wave issues `iters` rounds of four independent 32x32x16 bf16 MFMAs
// (operands in registers, no memory traffic), so the chip runs at its dense
// MFMA rate and at the clock it holds under that load. Lane 0..2 of the first
// wave of each workgroup write, with vector stores, the wave's elapsed shader
// clocks (s_memtime), the elapsed ticks of the constant-rate counter
// (s_memrealtime) and a checksum of the accumulators (so the products are
// not removed). The caller turns these into TFLOP/s (with its own timer) and
// MHz (clocks per tick times the counter's rate).

#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

__global__ void __launch_bounds__(256)
mfma_probe_kernel(unsigned long long* __restrict__ sink, int iters) {
    const int lane = threadIdx.x & 63;
    bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(0.001f * (float)(lane + i));
        b[i] = (__bf16)(0.002f * (float)(lane - i));
    }
    f32x16 c0{}, c1{}, c2{}, c3{};
    const unsigned long long t0 = __builtin_amdgcn_s_memtime();
    const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
        c0 = mfma32(a, b, c0);
        c1 = mfma32(b, a, c1);
        c2 = mfma32(a, a, c2);
        c3 = mfma32(b, b, c3);
    }
    float sum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) sum += c0[r] + c1[r] + c2[r] + c3[r];
    const unsigned long long t1 = __builtin_amdgcn_s_memtime();
    const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
    if (threadIdx.x < 3) {
        const unsigned long long vals[3] = {t1 - t0, r1 - r0,
                                            (unsigned long long)__float_as_uint(sum)};
        sink[3 * blockIdx.x + threadIdx.x] = vals[threadIdx.x];
    }
}

}  // namespace

hipError_t launch_mfma_probe(unsigned long long* sink, int blocks, int iters,
                             hipStream_t stream) {
    hipLaunchKernelGGL(mfma_probe_kernel, dim3(blocks), dim3(256), 0, stream, sink, iters);
    return hipGetLastError();
}

}  // namespace fa
