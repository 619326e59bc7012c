// Forward attention in float32 arithmetic throughout (no reduced-precision
// step), for callers that need fp32 inputs and outputs.
//
// Same method as the MFMA kernel ("11.11 Flash Attention", sections "Flash
// Attention: The Key Insight", "The Tiling Algorithm" and "Flash Attention
// 2": Q blocks outer, K/V tiles inner, running max m and running sum l, one
// division at the end), on the vector ALUs: one thread owns one query row and
// keeps its unnormalised output row in registers; a K/V tile of 16 keys is
// staged in LDS and read by all threads as broadcasts. Exponentials use the
// full-precision expf, so the result is float32-accurate.

#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int F32_BM = 64;  // query rows per workgroup (one wavefront)
constexpr int F32_BN = 16;  // keys per tile

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(64)
fwd_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
               const float* __restrict__ V, float* __restrict__ O, float* __restrict__ LSE,
               int BH, int N, int nqb, float scale) {
    __shared__ float sQ[F32_BM * (D + 1)];
    __shared__ float sK[F32_BN * D];
    __shared__ float sV[F32_BN * D];

    const int bh = blockIdx.x / nqb;
    const int qb = blockIdx.x % nqb;
    const size_t head = (size_t)bh * N * D;
    const int tid = threadIdx.x;
    const int q0 = qb * F32_BM;
    const int qrow = q0 + tid;

    // stage the Q block (rows beyond N are zero and never stored)
    for (int e = tid; e < F32_BM * D; e += F32_BM) {
        const int r = e / D, col = e % D;
        const int row = q0 + r;
        sQ[r * (D + 1) + col] = row < N ? Q[head + (size_t)row * D + col] : 0.f;
    }

    float acc[D];
#pragma unroll
    for (int i = 0; i < D; ++i) acc[i] = 0.f;
    float m = -INFINITY, l = 0.f;

    const int q_last = min(N, q0 + F32_BM) - 1;
    const int kend = CAUSAL ? q_last + 1 : N;
    for (int k0 = 0; k0 < kend; k0 += F32_BN) {
        __syncthreads();
        for (int e = tid; e < F32_BN * D; e += F32_BM) {
            const int r = e / D, col = e % D;
            const int key = k0 + r;
            sK[e] = key < N ? K[head + (size_t)key * D + col] : 0.f;
            sV[e] = key < N ? V[head + (size_t)key * D + col] : 0.f;
        }
        __syncthreads();

        float s[F32_BN];
        float tmax = -INFINITY;
#pragma unroll
        for (int j = 0; j < F32_BN; ++j) {
            float dot = 0.f;
#pragma unroll 16
            for (int i = 0; i < D; ++i) dot = fmaf(sQ[tid * (D + 1) + i], sK[j * D + i], dot);
            const int key = k0 + j;
            const bool vis = key < N && (!CAUSAL || key <= qrow);
            s[j] = vis ? dot * scale : -INFINITY;
            tmax = fmaxf(tmax, s[j]);
        }
        const float m_new = fmaxf(m, tmax);
        if (m_new == -INFINITY) continue;  // no visible key yet for this row
        const float alpha = expf(m - m_new);
        float rs = 0.f;
#pragma unroll
        for (int j = 0; j < F32_BN; ++j) {
            s[j] = expf(s[j] - m_new);
            rs += s[j];
        }
        l = l * alpha + rs;
        m = m_new;
#pragma unroll
        for (int i = 0; i < D; ++i) {
            float a = acc[i] * alpha;
#pragma unroll
            for (int j = 0; j < F32_BN; ++j) a = fmaf(s[j], sV[j * D + i], a);
            acc[i] = a;
        }
    }

    if (qrow < N) {
        const float inv = 1.f / l;
        float* orow = O + head + (size_t)qrow * D;
#pragma unroll
        for (int i = 0; i < D; ++i) orow[i] = acc[i] * inv;
        if (LSE != nullptr) LSE[(size_t)bh * N + qrow] = m + logf(l);
    }
}

template <int D, bool CAUSAL>
hipError_t launch_typed(const float* q, const float* k, const float* v, float* o, float* lse,
                        int BH, int N, float scale, hipStream_t stream) {
    const int nqb = (N + F32_BM - 1) / F32_BM;
    hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL>), dim3(BH * nqb), dim3(F32_BM), 0, stream, q,
                       k, v, o, lse, BH, N, nqb, scale);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(int d, bool causal, const float* q, const float* k, const float* v,
                          float* o, float* lse, int BH, int N, float scale, hipStream_t stream) {
    if (d == 64)
        return causal ? launch_typed<64, true>(q, k, v, o, lse, BH, N, scale, stream)
                      : launch_typed<64, false>(q, k, v, o, lse, BH, N, scale, stream);
    return causal ? launch_typed<128, true>(q, k, v, o, lse, BH, N, scale, stream)
                  : launch_typed<128, false>(q, k, v, o, lse, BH, N, scale, stream);
}

}  // namespace fa
