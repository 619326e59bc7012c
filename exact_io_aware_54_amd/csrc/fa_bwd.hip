// Backward attention by recomputation (bf16 / fp16 in, fp32 accumulate).
//
// "11.11 Flash Attention", section "The Recomputation Trade-off": the forward
// keeps no N x N matrix; the backward recomputes the score tiles from Q, K, V
// and the saved per-row statistics (here LSE = m + ln l, so P = exp(S - LSE)).
// The gradient equations are the chain rule through O = P V and the row
// softmax (the pages give none):
//   D_i = sum_k dO_ik O_ik               (equals sum_j P_ij dP_ij)
//   dV  = P^T dO,  dP = dO V^T,  dS = P * (dP - D),
//   dQ  = scale dS K,  dK = scale dS^T Q.
//
// Three launches on the caller's stream:
//  1. bwd_pre: D_i per row (fp32) and zeroing of the fp32 dQ accumulator.
//  2. bwd_main: one workgroup per (batch*head, block of 128 keys); each of its
//     four wavefronts keeps 32 keys' K and V rows in registers (as MFMA
//     operands) and their dK, dV in MFMA accumulators for the whole kernel,
//     and walks the query blocks of 64 rows (causal: only those at or below
//     the diagonal). Per query block: S = Q K^T and dP = dO V^T (the key index
//     across lanes, the query index in registers), P and dS in registers,
//     dV^T += dO^T P and dK^T += Q^T dS with Q^T and dO^T read from LDS copies
//     stored in the accumulator's row order. dS goes to LDS once, and the
//     block's dQ = dS K is split across the four waves and added to the fp32
//     accumulator with hardware float atomics.
//  3. bwd_dq_convert: dQ accumulator -> dtype.

#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

template <typename T, int D>
struct BwdTile {
    static constexpr int BN = 128;            // keys per workgroup (4 waves x 32)
    static constexpr int BM = 64;             // queries per step
    static constexpr int NT = 256;
    static constexpr int QSTR = D + 8;        // row-layout Q / dO in LDS
    static constexpr int TSTR = BM + 8;       // transposed Q^T / dO^T in LDS
    static constexpr int SSTR = BN + 8;       // dS [BM][BN]
    static constexpr int KTSTR = BN + 8;      // K^T [D][BN]
    static constexpr int KS = D / 16;
    static constexpr int DB = D / 32;
    static constexpr int DCH = D / 8;
    static constexpr int QG = BM * D / 8 / NT;   // rows per thread when staging Q / dO
    static constexpr int KG = BN * D / 8 / NT;   // keys per thread when staging K^T
    static constexpr int NSUB = (BM / 32) * DB;  // 32x32 dQ subtiles per step
};

template <typename T, int N_>
struct VecN;
template <typename T>
struct VecN<T, 2> { typedef __attribute__((__vector_size__(2 * sizeof(T)))) T type; };
template <typename T>
struct VecN<T, 4> { typedef __attribute__((__vector_size__(4 * sizeof(T)))) T type; };
template <typename T>
struct VecN<T, 8> { typedef __attribute__((__vector_size__(8 * sizeof(T)))) T type; };

// ---------------------------------------------------------------- 1. D and zeroing
template <typename T, int D>
__global__ void __launch_bounds__(256)
bwd_pre_kernel(const T* __restrict__ O, const T* __restrict__ dO, float* __restrict__ delta,
               float* __restrict__ dq_acc, int rows) {
    using V8 = typename Vec<T>::x8;
    constexpr int TPR = D / 8;  // threads per row
    const int gid = blockIdx.x * 256 + threadIdx.x;
    const int row = gid / TPR, part = gid % TPR;
    float s = 0.f;
    if (row < rows) {
        const V8 o = *reinterpret_cast<const V8*>(O + (size_t)row * D + part * 8);
        const V8 g = *reinterpret_cast<const V8*>(dO + (size_t)row * D + part * 8);
#pragma unroll
        for (int i = 0; i < 8; ++i) s = fmaf((float)o[i], (float)g[i], s);
        f32x4* z = reinterpret_cast<f32x4*>(dq_acc + (size_t)row * D + part * 8);
        z[0] = f32x4{};
        z[1] = f32x4{};
    }
#pragma unroll
    for (int off = TPR / 2; off > 0; off >>= 1) s += __shfl_xor(s, off, TPR);
    if (row < rows && part == 0) delta[row] = s;
}

// ---------------------------------------------------------------- 2. main
template <typename T, int D, bool CAUSAL>
__global__ void __launch_bounds__(256, 1)
bwd_main_kernel(const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
                const T* __restrict__ dO, const float* __restrict__ LSE,
                const float* __restrict__ delta, float* __restrict__ dq_acc, T* __restrict__ dK,
                T* __restrict__ dV, int BH, int N, int nkb, float scale, float c) {
    using C = BwdTile<T, D>;
    using V8 = typename Vec<T>::x8;
    using V4 = typename Vec<T>::x4;
    using VG = typename VecN<T, C::QG>::type;
    using VK = typename VecN<T, C::KG>::type;
    __shared__ __attribute__((aligned(16))) T sQ[C::BM * C::QSTR];
    __shared__ __attribute__((aligned(16))) T sdO[C::BM * C::QSTR];
    __shared__ __attribute__((aligned(16))) T sQT[D * C::TSTR];
    __shared__ __attribute__((aligned(16))) T sdOT[D * C::TSTR];
    __shared__ __attribute__((aligned(16))) T sdS[C::BM * C::SSTR];
    __shared__ __attribute__((aligned(16))) T sKT[D * C::KTSTR];
    __shared__ float sL[C::BM];
    __shared__ float sDel[C::BM];

    const int L = xcd_remap(blockIdx.x, BH * nkb);
    const int bh = L / nkb;
    const int kb = L % nkb;  // causal: small kb has the most query blocks -> dispatched first
    const size_t head = (size_t)bh * N * D;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, h = lane >> 5;
    const int kbase = kb * C::BN;
    const int key0 = kbase + 32 * wave;  // first key of this wave
    const int key = key0 + l32;          // key held by this lane (accumulator column)

    // resident operands: K and V rows of this lane's key (B side of Q K^T and dO V^T)
    V8 kf[C::KS], vf[C::KS];
    if (key < N) {
        const V8* ks = reinterpret_cast<const V8*>(K + head + (size_t)key * D + 8 * h);
        const V8* vs = reinterpret_cast<const V8*>(V + head + (size_t)key * D + 8 * h);
#pragma unroll
        for (int s = 0; s < C::KS; ++s) {
            kf[s] = ks[2 * s];
            vf[s] = vs[2 * s];
        }
    } else {
#pragma unroll
        for (int s = 0; s < C::KS; ++s) {
            kf[s] = V8{};
            vf[s] = V8{};
        }
    }
    // K^T of the whole key block into LDS (B side of dQ = dS K), natural key order
    {
        const int cc = tid % C::DCH, g = tid / C::DCH;
        V8 kr[C::KG];
#pragma unroll
        for (int i = 0; i < C::KG; ++i) {
            const int kk = kbase + g * C::KG + i;
            kr[i] = kk < N ? *reinterpret_cast<const V8*>(K + head + (size_t)kk * D + cc * 8) : V8{};
        }
#pragma unroll
        for (int dd = 0; dd < 8; ++dd) {
            VK w;
#pragma unroll
            for (int i = 0; i < C::KG; ++i) w[i] = kr[i][dd];
            *reinterpret_cast<VK*>(sKT + (cc * 8 + dd) * C::KTSTR + g * C::KG) = w;
        }
    }

    f32x16 dvacc[C::DB], dkacc[C::DB];
#pragma unroll
    for (int b = 0; b < C::DB; ++b) {
        dvacc[b] = f32x16{};
        dkacc[b] = f32x16{};
    }

    const int nqb = (N + C::BM - 1) / C::BM;
    const int i0 = CAUSAL ? kbase / C::BM : 0;
    for (int ib = i0; ib < nqb; ++ib) {
        const int qbase = ib * C::BM;
        __syncthreads();  // previous step's LDS readers are done
        {
            // stage Q and dO rows [qbase, qbase + BM): row layout and transposed layout
            const int cc = tid % C::DCH, g = tid / C::DCH;
            V8 qr[C::QG], gr[C::QG];
#pragma unroll
            for (int i = 0; i < C::QG; ++i) {
                const int r = g * C::QG + i, row = qbase + r;
                if (row < N) {
                    qr[i] = *reinterpret_cast<const V8*>(Q + head + (size_t)row * D + cc * 8);
                    gr[i] = *reinterpret_cast<const V8*>(dO + head + (size_t)row * D + cc * 8);
                } else {
                    qr[i] = V8{};
                    gr[i] = V8{};
                }
                *reinterpret_cast<V8*>(sQ + r * C::QSTR + cc * 8) = qr[i];
                *reinterpret_cast<V8*>(sdO + r * C::QSTR + cc * 8) = gr[i];
            }
            const int r0 = g * C::QG;
            const int pos = (r0 & ~15) + acc_kperm16(r0 & 15);
#pragma unroll
            for (int dd = 0; dd < 8; ++dd) {
                VG wq, wg;
#pragma unroll
                for (int i = 0; i < C::QG; ++i) {
                    wq[i] = qr[i][dd];
                    wg[i] = gr[i][dd];
                }
                *reinterpret_cast<VG*>(sQT + (cc * 8 + dd) * C::TSTR + pos) = wq;
                *reinterpret_cast<VG*>(sdOT + (cc * 8 + dd) * C::TSTR + pos) = wg;
            }
            if (tid < C::BM) {
                const int row = qbase + tid;
                const size_t ri = (size_t)bh * N + row;
                sL[tid] = row < N ? LSE[ri] * kLog2e : INFINITY;  // +inf -> P = 0 for padding rows
                sDel[tid] = row < N ? delta[ri] : 0.f;
            }
        }
        __syncthreads();

        const bool need_mask = (key0 + 31 >= N) || (CAUSAL && key0 + 31 > qbase);
#pragma unroll
        for (int qs = 0; qs < C::BM / 32; ++qs) {
            f32x16 sacc = f32x16{}, pacc = f32x16{};
#pragma unroll
            for (int s = 0; s < C::KS; ++s) {
                const V8 aq = *reinterpret_cast<const V8*>(sQ + (32 * qs + l32) * C::QSTR + 16 * s + 8 * h);
                const V8 ag = *reinterpret_cast<const V8*>(sdO + (32 * qs + l32) * C::QSTR + 16 * s + 8 * h);
                sacc = mfma32(aq, kf[s], sacc);
                pacc = mfma32(ag, vf[s], pacc);
            }
            // sacc / pacc: lane = key, register r = query 32 qs + acc_row(r, h)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int qi = 32 * qs + acc_row(r, h);
                float p = fast_exp2(fmaf(sacc[r], c, -sL[qi]));
                if (need_mask && (key >= N || (CAUSAL && key > qbase + qi))) p = 0.f;
                sacc[r] = p;
                pacc[r] = p * (pacc[r] - sDel[qi]);
            }
            V8 pf[2], sf[2];
            pf[0] = pack8<T>(sacc, 0);
            pf[1] = pack8<T>(sacc, 8);
            sf[0] = pack8<T>(pacc, 0);
            sf[1] = pack8<T>(pacc, 8);
#pragma unroll
            for (int g2 = 0; g2 < 2; ++g2)
#pragma unroll
                for (int b = 0; b < C::DB; ++b) {
                    const int off = (32 * b + l32) * C::TSTR + 32 * qs + 16 * g2 + 8 * h;
                    const V8 at = *reinterpret_cast<const V8*>(sdOT + off);
                    const V8 aq = *reinterpret_cast<const V8*>(sQT + off);
                    dvacc[b] = mfma32(at, pf[g2], dvacc[b]);
                    dkacc[b] = mfma32(aq, sf[g2], dkacc[b]);
                }
            // dS [q][key] for the dQ product
#pragma unroll
            for (int r = 0; r < 16; ++r)
                sdS[(32 * qs + acc_row(r, h)) * C::SSTR + 32 * wave + l32] = (T)pacc[r];
        }
        __syncthreads();

        // dQ[qbase.., :] += scale * dS K over this block's 128 keys
#pragma unroll
        for (int u = 0; u < C::NSUB / 4; ++u) {
            const int t = wave + 4 * u;
            const int qs = t / C::DB, b = t % C::DB;
            f32x16 acc = f32x16{};
#pragma unroll
            for (int s = 0; s < C::BN / 16; ++s) {
                const V8 a = *reinterpret_cast<const V8*>(sdS + (32 * qs + l32) * C::SSTR + 16 * s + 8 * h);
                const V8 bb = *reinterpret_cast<const V8*>(sKT + (32 * b + l32) * C::KTSTR + 16 * s + 8 * h);
                acc = mfma32(a, bb, acc);
            }
            // acc: lane = head dim 32 b + l32, register r = query 32 qs + acc_row(r, h)
            float* dst = dq_acc + head + 32 * b + l32;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = qbase + 32 * qs + acc_row(r, h);
                if (row < N) unsafeAtomicAdd(dst + (size_t)row * D, acc[r] * scale);
            }
        }
    }

    if (key < N) {
        T* dkr = dK + head + (size_t)key * D;
        T* dvr = dV + head + (size_t)key * D;
#pragma unroll
        for (int b = 0; b < C::DB; ++b)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                V4 wk, wv;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    wk[i] = (T)(dkacc[b][4 * r4 + i] * scale);
                    wv[i] = (T)dvacc[b][4 * r4 + i];
                }
                *reinterpret_cast<V4*>(dkr + 32 * b + 8 * r4 + 4 * h) = wk;
                *reinterpret_cast<V4*>(dvr + 32 * b + 8 * r4 + 4 * h) = wv;
            }
    }
}

// ---------------------------------------------------------------- 3. dQ convert
template <typename T>
__global__ void __launch_bounds__(256)
bwd_dq_convert_kernel(const float* __restrict__ acc, T* __restrict__ dq, size_t n8) {
    using V8 = typename Vec<T>::x8;
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n8) return;
    const f32x4* src = reinterpret_cast<const f32x4*>(acc) + 2 * i;
    const f32x4 a = src[0], b = src[1];
    V8 w;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        w[j] = (T)a[j];
        w[j + 4] = (T)b[j];
    }
    reinterpret_cast<V8*>(dq)[i] = w;
}

template <typename T, int D, bool CAUSAL>
hipError_t launch_typed(const void* q, const void* k, const void* v, const void* o,
                        const float* lse, const void* dO, void* dq, void* dk, void* dv,
                        float* dq_acc, float* delta, int BH, int N, float scale, int stages,
                        hipStream_t stream) {
    using C = BwdTile<T, D>;
    const int rows = BH * N;
    hipError_t e = hipSuccess;
    if (stages & 1) {
        const int pre_threads = rows * (D / 8);
        hipLaunchKernelGGL((bwd_pre_kernel<T, D>), dim3((pre_threads + 255) / 256), dim3(256), 0,
                           stream, static_cast<const T*>(o), static_cast<const T*>(dO), delta,
                           dq_acc, rows);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (stages & 2) {
        const int nkb = (N + C::BN - 1) / C::BN;
        hipLaunchKernelGGL((bwd_main_kernel<T, D, CAUSAL>), dim3(BH * nkb), dim3(C::NT), 0,
                           stream, static_cast<const T*>(q), static_cast<const T*>(k),
                           static_cast<const T*>(v), static_cast<const T*>(dO), lse, delta,
                           dq_acc, static_cast<T*>(dk), static_cast<T*>(dv), BH, N, nkb, scale,
                           scale * kLog2e);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (stages & 4) {
        const size_t n8 = (size_t)rows * D / 8;
        hipLaunchKernelGGL((bwd_dq_convert_kernel<T>), dim3((unsigned)((n8 + 255) / 256)),
                           dim3(256), 0, stream, dq_acc, static_cast<T*>(dq), n8);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return e;
}

template <typename T>
hipError_t launch_d(int d, bool causal, const void* q, const void* k, const void* v,
                    const void* o, const float* lse, const void* dO, void* dq, void* dk, void* dv,
                    float* dq_acc, float* delta, int BH, int N, float scale, int stages,
                    hipStream_t stream) {
    if (d == 64)
        return causal ? launch_typed<T, 64, true>(q, k, v, o, lse, dO, dq, dk, dv, dq_acc, delta,
                                                  BH, N, scale, stages, stream)
                      : launch_typed<T, 64, false>(q, k, v, o, lse, dO, dq, dk, dv, dq_acc,
                                                   delta, BH, N, scale, stages, stream);
    return causal ? launch_typed<T, 128, true>(q, k, v, o, lse, dO, dq, dk, dv, dq_acc, delta, BH,
                                               N, scale, stages, stream)
                  : launch_typed<T, 128, false>(q, k, v, o, lse, dO, dq, dk, dv, dq_acc, delta,
                                                BH, N, scale, stages, stream);
}

}  // namespace

hipError_t launch_bwd(int dtype, int d, bool causal, const void* q, const void* k, const void* v,
                      const void* o, const float* lse, const void* dO, void* dq, void* dk,
                      void* dv, float* dq_acc, float* delta, int BH, int N, float scale,
                      int stages, hipStream_t stream) {
    if (dtype == 2)
        return launch_d<__bf16>(d, causal, q, k, v, o, lse, dO, dq, dk, dv, dq_acc, delta, BH, N,
                                scale, stages, stream);
    return launch_d<_Float16>(d, causal, q, k, v, o, lse, dO, dq, dk, dv, dq_acc, delta, BH, N,
                              scale, stages, stream);
}

}  // namespace fa
