// Measurement probes (not part of the attention computation).
//
// 1. The practical bf16 MFMA rate and the shader clock.
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

// 2. The memory side of a one-pass backward: in that design the dK/dV pass
// would also form each query block's dQ partial, dS K over its key block, and
// add it into a float32 dQ accumulator with float atomics, one 64 x 128
// (d = 128) partial per (key block, 64-query step) pair. This kernel issues
// exactly that stream of additions with no arithmetic around it: one
// workgroup of eight waves per (head, block of KB keys), stepping over the
// 64-query blocks (causal: from the block holding the first key on); wave w
// adds the 32 x 32 block (query half w / 4, head-dim block w % 4) in the MFMA
// accumulator layout (16 floats per lane, lanes along the head dim). Block
// ids map to (head, key block) as in the dK/dV pass (causal: groups of at most
// two heads per XCD, longest blocks first; otherwise whole heads per XCD), so
// every partial of a head comes from one XCD. MODE 0 uses float atomic adds,
// MODE 1 plain stores of the same addresses (the write bandwidth of the
// pattern). Its time is a lower bound on what the atomics add to a one-pass
// dK/dV pass. (On gfx950 the relaxed float add compiles to the same
// instruction at workgroup and at agent scope, and it is performed past the
// XCD's L2 either way: the sums come out exact even when a head's blocks are
// spread over XCDs, at the same ~1.3 TB/s of payload.)
template <int MODE>
__device__ __forceinline__ void dq_probe_body(float* __restrict__ ws, int N, int nkb, int kb_rows,
                                              int causal) {
    const int BH = gridDim.x / nkb;
    int bh, kb;
    if (causal) {
        causal_block(blockIdx.x, nkb, BH, bh, kb, 2);
        kb = nkb - 1 - kb;
    } else {
        const int L = xcd_remap(blockIdx.x, BH * nkb);
        bh = L / nkb;
        kb = L % nkb;
    }
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int l32 = lane & 31, h = lane >> 5;
    const int qsub = wave >> 2, db = wave & 3;
    float* head = ws + (size_t)bh * N * 128;
    const int i0 = causal ? (kb * kb_rows) / 64 : 0;
    float val = 1.0f + 0.001f * (float)lane;
    for (int ib = i0; ib < N / 64; ++ib) {
        const int q0 = ib * 64 + 32 * qsub;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float* p = head + (size_t)(q0 + acc_row(r, h)) * 128 + 32 * db + l32;
            if (MODE == 0)
                __hip_atomic_fetch_add(p, val, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            else
                *p = val;
        }
        val += 1.0f;
    }
}

// two kernels (not one template) so that profiles tell the modes apart by name
__global__ void __launch_bounds__(512)
dq_atomic_add_probe_kernel(float* __restrict__ ws, int N, int nkb, int kb_rows, int causal) {
    dq_probe_body<0>(ws, N, nkb, kb_rows, causal);
}
__global__ void __launch_bounds__(512)
dq_store_probe_kernel(float* __restrict__ ws, int N, int nkb, int kb_rows, int causal) {
    dq_probe_body<1>(ws, N, nkb, kb_rows, causal);
}

}  // namespace

hipError_t launch_dq_atomic_probe(float* ws, int BH, int N, int key_block, int mode, int causal,
                                  hipStream_t stream) {
    const int nkb = N / key_block;
    if (mode == 0)
        hipLaunchKernelGGL(dq_atomic_add_probe_kernel, dim3(BH * nkb), dim3(512), 0, stream, ws, N,
                           nkb, key_block, causal);
    else
        hipLaunchKernelGGL(dq_store_probe_kernel, dim3(BH * nkb), dim3(512), 0, stream, ws, N,
                           nkb, key_block, causal);
    return hipGetLastError();
}

hipError_t launch_mfma_probe(unsigned long long* sink, int blocks, int iters,
                             hipStream_t stream) {
    hipLaunchKernelGGL(mfma_probe_kernel, dim3(blocks), dim3(256), 0, stream, sink, iters);
    return hipGetLastError();
}

}  // namespace fa
