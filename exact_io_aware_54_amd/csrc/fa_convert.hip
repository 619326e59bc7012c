// OCP E4M3 codes -> bfloat16, elementwise and exact (E4M3 has 3 mantissa
// bits and the exponent range of a subset of bfloat16's), for the fp8
// backward, which runs the 16-bit passes on the codes and folds the
// per-tensor descales into its scalar factors.

#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;

// sixteen codes per thread: one 16-byte load, two 16-byte stores
__global__ void __launch_bounds__(256)
e4m3_to_bf16_kernel(const uint8_t* __restrict__ src, __bf16* __restrict__ dst, size_t n) {
    const size_t i0 = ((size_t)blockIdx.x * 256 + threadIdx.x) * 16;
    if (i0 >= n) return;
    if (i0 + 16 <= n) {
        const i32x4 w = *reinterpret_cast<const i32x4*>(src + i0);
        bf16x8 out[2];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8(w[k], false);
            const f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8(w[k], true);
            out[k / 2][4 * (k % 2) + 0] = (__bf16)a[0];
            out[k / 2][4 * (k % 2) + 1] = (__bf16)a[1];
            out[k / 2][4 * (k % 2) + 2] = (__bf16)b[0];
            out[k / 2][4 * (k % 2) + 3] = (__bf16)b[1];
        }
        *reinterpret_cast<bf16x8*>(dst + i0) = out[0];
        *reinterpret_cast<bf16x8*>(dst + i0 + 8) = out[1];
    } else {
        for (size_t i = i0; i < n; ++i) {
            const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8((int)src[i], false);
            dst[i] = (__bf16)a[0];
        }
    }
}

}  // namespace

hipError_t launch_e4m3_to_bf16(const void* src, void* dst, size_t n, hipStream_t stream) {
    const size_t threads = (n + 15) / 16;
    hipLaunchKernelGGL(e4m3_to_bf16_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                       stream, static_cast<const uint8_t*>(src), static_cast<__bf16*>(dst), n);
    return hipGetLastError();
}

}  // namespace fa
