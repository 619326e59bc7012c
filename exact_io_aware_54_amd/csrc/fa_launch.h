// Host-side launchers of the attention kernels (internal to libfa).
// Arguments are validated by the C ABI layer before these are called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace fa {

// waves: 0 = built-in workgroup shape, 4 or 8 = forced (d = 256 takes 4 only)
hipError_t launch_fwd_mfma(int dtype, int d, bool causal, const void* q, const void* k,
                           const void* v, void* o, float* lse, int BH, int N, float scale,
                           int waves, hipStream_t stream);
hipError_t launch_fwd_f32(int d, bool causal, const float* q, const float* k, const float* v,
                          float* o, float* lse, int BH, int N, float scale, hipStream_t stream);
hipError_t launch_fwd_fp8(int d, bool causal, const void* q8, const void* k8, const void* v8,
                          float qk_scale, float v_descale, void* o, float* lse, int BH, int N,
                          hipStream_t stream);
// Factors of the backward passes: exponent factor c (P = 2^(s c - LSE log2 e)
// for the raw product s of the operands), multipliers of the dK and dQ
// outputs, and of the row terms D. Plain use: {scale log2 e, scale, scale, 1}.
struct BwdScales {
    float c, dk_mul, dq_mul, d_mul;
};
hipError_t launch_bwd_scaled(int dtype, int d, bool causal, const void* q, const void* k,
                             const void* v, const void* o, const float* lse, const void* dO,
                             void* dq, void* dk, void* dv, float* delta, float* lse2, int BH,
                             int N, const BwdScales& sc, int stages, hipStream_t stream);
hipError_t launch_e4m3_to_bf16(const void* src, void* dst, size_t n, hipStream_t stream);
hipError_t launch_mfma_probe(unsigned long long* sink, int blocks, int iters,
                             hipStream_t stream);
hipError_t launch_dq_atomic_probe(float* ws, int BH, int N, int key_block, int mode, int causal,
                                  hipStream_t stream);
hipError_t launch_bwd(int dtype, int d, bool causal, const void* q, const void* k, const void* v,
                      const void* o, const float* lse, const void* dO, void* dq, void* dk,
                      void* dv, float* delta, float* lse2, int BH, int N, float scale,
                      int stages, hipStream_t stream);  // stages: bit 0 pre, 1 dK/dV, 2 dQ
hipError_t launch_fwd_splitkv(int dtype, int d, bool causal, const void* q, const void* k,
                              const void* v, void* o, float* lse, float* o_part, float* lse_part,
                              int BH, int Nq, int Nk, int splits, int kps, float scale,
                              hipStream_t stream);
hipError_t launch_lse_merge(int dtype_out, const float* o_parts, const float* lse_parts, int P,
                            long long rows, int d, void* o, float* lse, hipStream_t stream);
hipError_t launch_fwd_v1(int dtype, int d, bool causal, const void* q, const void* k,
                         const void* v, void* o, float* lse, float* ows, float* mws, float* lws,
                         int BH, int N, float scale, hipStream_t stream);
// Scratch of fa_bwd_noalloc: room for the row terms of this many rows
// (B*H*N), two float vectors, 16 MiB per device in all.
constexpr size_t kNoallocMaxRows = (size_t)1 << 21;
// This device's copy of that scratch (`device` must be the current device):
// -D at *delta, LSE * log2 e at *lse2, kNoallocMaxRows floats each.
hipError_t noalloc_scratch(int device, float** delta, float** lse2);
hipError_t launch_std(int dtype, int d, bool causal, const void* q, const void* k, const void* v,
                      void* o, void* s, int BH, int N, float scale, hipStream_t stream);

}  // namespace fa
