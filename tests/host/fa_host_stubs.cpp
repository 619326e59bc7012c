// Host-only stand-ins for the kernel launchers and the few HIP runtime calls
// of libfa's C ABI layer (csrc/fa_api.cpp), so that layer can be built with
// g++ and AddressSanitizer / UndefinedBehaviorSanitizer and driven without a
// GPU. Every launcher records its arguments (pointers and sizes) for the
// checks in fa_host_check.cpp and returns the error the check selects; no
// device memory is touched.

#include "fa_host_stubs.h"

#include <string.h>

namespace fa {

Recorded g_rec;
hipError_t g_launch_result = hipSuccess;
hipError_t g_pending = hipSuccess;
int g_device = 0;
int g_stream_device = 0;

static void note(const char* name, int n_ptr, const void* const* ptrs, long long a0, long long a1,
                 long long a2, long long a3) {
    g_rec.calls += 1;
    strncpy(g_rec.name, name, sizeof(g_rec.name) - 1);
    g_rec.name[sizeof(g_rec.name) - 1] = 0;
    g_rec.n_ptr = n_ptr;
    for (int i = 0; i < n_ptr && i < kMaxPtr; ++i) g_rec.ptr[i] = ptrs[i];
    g_rec.arg[0] = a0;
    g_rec.arg[1] = a1;
    g_rec.arg[2] = a2;
    g_rec.arg[3] = a3;
}

hipError_t launch_fwd_mfma(int dtype, int d, bool causal, const void* q, const void* k,
                           const void* v, void* o, float* lse, int BH, int N, float, int waves,
                           hipStream_t) {
    const void* p[] = {q, k, v, o, lse};
    note("fwd_mfma", 5, p, BH, N, d, dtype * 100 + waves * 10 + causal);
    return g_launch_result;
}
hipError_t launch_fwd_f32(int d, bool causal, const float* q, const float* k, const float* v,
                          float* o, float* lse, int BH, int N, float, hipStream_t) {
    const void* p[] = {q, k, v, o, lse};
    note("fwd_f32", 5, p, BH, N, d, causal);
    return g_launch_result;
}
hipError_t launch_fwd_fp8(int d, bool causal, const void* q8, const void* k8, const void* v8,
                          float, float, void* o, float* lse, int BH, int N, hipStream_t) {
    const void* p[] = {q8, k8, v8, o, lse};
    note("fwd_fp8", 5, p, BH, N, d, causal);
    return g_launch_result;
}
hipError_t launch_bwd_scaled(int dtype, int d, bool causal, const void* q, const void* k,
                             const void* v, const void* o, const float* lse, const void* dO,
                             void* dq, void* dk, void* dv, float* delta, float* lse2, int BH,
                             int N, const BwdScales&, int stages, hipStream_t) {
    const void* p[] = {q, k, v, o, lse, dO, dq, dk, dv, delta, lse2};
    note("bwd_scaled", 11, p, BH, N, d, dtype * 1000 + stages * 10 + causal);
    return g_launch_result;
}
hipError_t launch_bwd(int dtype, int d, bool causal, const void* q, const void* k, const void* v,
                      const void* o, const float* lse, const void* dO, void* dq, void* dk,
                      void* dv, float* delta, float* lse2, int BH, int N, float, int stages,
                      hipStream_t) {
    const void* p[] = {q, k, v, o, lse, dO, dq, dk, dv, delta, lse2};
    note("bwd", 11, p, BH, N, d, dtype * 1000 + stages * 10 + causal);
    return g_launch_result;
}
hipError_t launch_e4m3_to_bf16(const void* src, void* dst, size_t n, hipStream_t) {
    // called three times per fp8 backward: keep all three destinations
    g_rec.conv_dst[g_rec.n_conv % 3] = dst;
    g_rec.conv_src[g_rec.n_conv % 3] = src;
    g_rec.conv_n = (long long)n;
    g_rec.n_conv += 1;
    return g_launch_result;
}
hipError_t launch_mfma_probe(unsigned long long* sink, int blocks, int iters, hipStream_t) {
    const void* p[] = {sink};
    note("mfma_probe", 1, p, blocks, iters, 0, 0);
    return g_launch_result;
}
hipError_t launch_dq_atomic_probe(float* ws, int BH, int N, int key_block, int mode, int causal,
                                  hipStream_t) {
    const void* p[] = {ws};
    note("dq_probe", 1, p, BH, N, key_block, mode * 10 + causal);
    return g_launch_result;
}
hipError_t launch_fwd_splitkv(int dtype, int d, bool causal, const void* q, const void* k,
                              const void* v, void* o, float* lse, float* o_part, float* lse_part,
                              int BH, int Nq, int Nk, int splits, int kps, float, hipStream_t) {
    const void* p[] = {q, k, v, o, lse, o_part, lse_part};
    note("splitkv", 7, p, BH, Nq, Nk, (long long)splits * 1000000 + kps);
    g_rec.arg[4] = d;
    g_rec.arg[5] = dtype * 10 + causal;
    return g_launch_result;
}
hipError_t launch_lse_merge(int dtype_out, const float* o_parts, const float* lse_parts, int P,
                            long long rows, int d, void* o, float* lse, hipStream_t) {
    const void* p[] = {o_parts, lse_parts, o, lse};
    note("lse_merge", 4, p, P, rows, d, dtype_out);
    return g_launch_result;
}
hipError_t launch_fwd_v1(int dtype, int d, bool causal, const void* q, const void* k,
                         const void* v, void* o, float* lse, float* ows, float* mws, float* lws,
                         int BH, int N, float, hipStream_t) {
    const void* p[] = {q, k, v, o, lse, ows, mws, lws};
    note("fwd_v1", 8, p, BH, N, d, dtype * 10 + causal);
    return g_launch_result;
}
hipError_t noalloc_scratch(int device, float** delta, float** lse2) {
    static float scratch[2][16];  // stand-in addresses only; never dereferenced
    g_rec.scratch_device = device;
    *delta = scratch[0];
    *lse2 = scratch[1];
    return g_launch_result;
}
hipError_t launch_std(int dtype, int d, bool causal, const void* q, const void* k, const void* v,
                      void* o, void* s, int BH, int N, float, hipStream_t) {
    const void* p[] = {q, k, v, o, s};
    note("std", 5, p, BH, N, d, dtype * 10 + causal);
    return g_launch_result;
}

}  // namespace fa

// The HIP runtime calls fa_api.cpp makes outside the launchers.
extern "C" {
hipError_t hipGetLastError(void) {
    const hipError_t e = fa::g_pending;
    fa::g_pending = hipSuccess;
    return e;
}
hipError_t hipGetDevice(int* device) {
    *device = fa::g_device;
    return hipSuccess;
}
hipError_t hipStreamGetDevice(hipStream_t, hipDevice_t* device) {
    *device = fa::g_stream_device;
    return hipSuccess;
}
}
