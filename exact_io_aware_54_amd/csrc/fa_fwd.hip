// Forward attention on MFMA matrix cores (bf16 / fp16 in, fp32 accumulate).
//
// Method ("11.11 Flash Attention", algomaster.io): Q is split into blocks of
// BM query rows and K/V into blocks of BN keys; one workgroup owns one query
// block of one (batch, head) and walks the K/V blocks in order (section
// "Flash Attention 2": Q-block outer loop, parallel over batch x heads x query
// blocks). Each K/V tile is staged once in LDS and shared by the four
// wavefronts. Per tile: scores, running row max, exponentials against the new
// max, rescaled running sum and rescaled output (sections "Flash Attention:
// The Key Insight" and "The Tiling Algorithm"). The output stays unnormalised
// and is divided by the row sum once at the end (the reduced non-matmul work
// of section "Flash Attention 2"). The score tile never leaves registers.
//
// gfx950 mapping:
//  * Each wavefront owns 32 queries. It computes S^T = K Q^T with 32x32x16
//    MFMAs: the query index runs across lanes, so a lane holds 16 scores of
//    ONE query per 32-key subtile, and a row max or row sum is an in-register
//    reduction plus one exchange with the other half of the wave
//    (v_permlane32_swap). m and l are one register each.
//  * The probabilities P^T, converted to 16-bit, are fed straight back as the
//    B operand of O^T = V^T P^T; V is transposed into LDS (with the row order
//    of the accumulator layout) when it is staged, so every MFMA operand read
//    is one 16-byte LDS load.
//  * Softmax works in base 2: p = 2^(s * scale * log2 e - m) via v_exp_f32.
//  * K/V tiles are double-buffered: the next tile's global loads are in flight
//    while the current tile is computed, then written to the other buffer.
//  * Causal: tiles past the block's last query are never visited, a wave
//    skips tiles wholly above its own rows, and only tiles that straddle the
//    diagonal (or the ragged end of N) pay for the mask.
//  * Launch order: logical workgroup ids are remapped so each XCD gets whole
//    heads (K/V reuse in its L2); causal blocks run longest-first per head.

#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

template <typename T, int D>
struct FwdTile {
    static constexpr int BM = 128;          // queries per workgroup (4 waves x 32)
    static constexpr int BN = 64;           // keys per K/V tile
    static constexpr int NT = 256;          // threads per workgroup
    static constexpr int KSTR = D + 8;      // LDS row stride of K (elements, +16 B pad)
    static constexpr int VSTR = BN + 8;     // LDS row stride of V^T (elements, +16 B pad)
    static constexpr int KS = D / 16;       // MFMA k-steps over the head dim
    static constexpr int DB = D / 32;       // 32-row blocks of O^T
    static constexpr int KCH = BN * D / 8 / NT;   // 16-byte K chunks per thread
    static constexpr int VKG = BN * D / 8 / NT;   // keys per thread in the V transpose
    static constexpr int DCH = D / 8;             // 16-byte chunks per row
};

template <typename T, int D>
struct KVStage {
    using C = FwdTile<T, D>;
    using V8 = typename Vec<T>::x8;
    V8 k[C::KCH];
    V8 v[C::VKG];

    __device__ __forceinline__ void load(const T* Kh, const T* Vh, int kbase, int N, int tid) {
#pragma unroll
        for (int i = 0; i < C::KCH; ++i) {
            const int id = tid + C::NT * i;
            const int row = id / C::DCH, col = (id % C::DCH) * 8;
            const int key = kbase + row;
            if (key < N) k[i] = *reinterpret_cast<const V8*>(Kh + (size_t)key * D + col);
            else k[i] = V8{};
        }
        const int c = tid % C::DCH, g = tid / C::DCH;
#pragma unroll
        for (int i = 0; i < C::VKG; ++i) {
            const int key = kbase + g * C::VKG + i;
            if (key < N) v[i] = *reinterpret_cast<const V8*>(Vh + (size_t)key * D + c * 8);
            else v[i] = V8{};
        }
    }

    __device__ __forceinline__ void store(T* sK, T* sV, int tid) const {
#pragma unroll
        for (int i = 0; i < C::KCH; ++i) {
            const int id = tid + C::NT * i;
            const int row = id / C::DCH, col = (id % C::DCH) * 8;
            *reinterpret_cast<V8*>(sK + row * C::KSTR + col) = k[i];
        }
        // V^T[d][key]: this thread holds VKG consecutive keys x 8 consecutive d.
        const int c = tid % C::DCH, g = tid / C::DCH;
        const int key0 = g * C::VKG;
        const int pos = (key0 & ~15) + acc_kperm16(key0 & 15);
#pragma unroll
        for (int dd = 0; dd < 8; ++dd) {
            T* dst = sV + (c * 8 + dd) * C::VSTR + pos;
            if constexpr (C::VKG == 4) {
                typename Vec<T>::x4 w;
#pragma unroll
                for (int i = 0; i < 4; ++i) w[i] = v[i][dd];
                *reinterpret_cast<typename Vec<T>::x4*>(dst) = w;
            } else {
                static_assert(C::VKG == 2, "V transpose handles 2 or 4 keys per thread");
                typedef __attribute__((__vector_size__(2 * sizeof(T)))) T x2;
                x2 w;
                w[0] = v[0][dd];
                w[1] = v[1][dd];
                *reinterpret_cast<x2*>(dst) = w;
            }
        }
    }
};

template <typename T, int D, bool CAUSAL>
__global__ void __launch_bounds__(256, 2)
fwd_mfma_kernel(const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
                T* __restrict__ O, float* __restrict__ LSE, int BH, int N, int nqb, float c) {
    using C = FwdTile<T, D>;
    using V8 = typename Vec<T>::x8;
    using V4 = typename Vec<T>::x4;
    __shared__ __attribute__((aligned(16))) T sK[2][C::BN * C::KSTR];
    __shared__ __attribute__((aligned(16))) T sV[2][D * C::VSTR];

    const int L = xcd_remap(blockIdx.x, BH * nqb);
    const int bh = L / nqb;
    const int qb = CAUSAL ? (nqb - 1 - L % nqb) : (L % nqb);
    const size_t head = (size_t)bh * N * D;
    const T* Qh = Q + head;
    const T* Kh = K + head;
    const T* Vh = V + head;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, h = lane >> 5;
    const int q0 = qb * C::BM + wave * 32;  // first query row of this wave
    const int qrow = q0 + l32;              // query held by this lane

    // B operand of S^T = K Q^T: slot (h, j) of k-step s is d = 16 s + 8 h + j.
    V8 qf[C::KS];
    if (qrow < N) {
        const V8* src = reinterpret_cast<const V8*>(Qh + (size_t)qrow * D + 8 * h);
#pragma unroll
        for (int s = 0; s < C::KS; ++s) qf[s] = src[2 * s];
    } else {
#pragma unroll
        for (int s = 0; s < C::KS; ++s) qf[s] = V8{};
    }

    const int q_last = min(N, (qb + 1) * C::BM) - 1;
    const int nkt = CAUSAL ? (q_last / C::BN + 1) : (N + C::BN - 1) / C::BN;

    KVStage<T, D> st;
    st.load(Kh, Vh, 0, N, tid);
    st.store(sK[0], sV[0], tid);
    __syncthreads();

    float m_run = -INFINITY;  // running max of s * c (base-2 units)
    float l_run = 0.f;        // this lane's share of the running sum
    f32x16 oacc[C::DB];
#pragma unroll
    for (int b = 0; b < C::DB; ++b) oacc[b] = f32x16{};

    for (int kt = 0; kt < nkt; ++kt) {
        const int buf = kt & 1;
        const bool more = kt + 1 < nkt;
        const int kbase = kt * C::BN;
        if (more) st.load(Kh, Vh, kbase + C::BN, N, tid);

        const bool active = !CAUSAL || kbase <= q0 + 31;
        if (active) {
            const T* kb = sK[buf];
            f32x16 s[2];
            s[0] = f32x16{};
            s[1] = f32x16{};
#pragma unroll
            for (int ks = 0; ks < C::KS; ++ks) {
#pragma unroll
                for (int c2 = 0; c2 < 2; ++c2) {
                    const V8 a = *reinterpret_cast<const V8*>(kb + (32 * c2 + l32) * C::KSTR + 16 * ks + 8 * h);
                    s[c2] = mfma32(a, qf[ks], s[c2]);
                }
            }
            const bool need_mask = (kbase + C::BN > N) || (CAUSAL && kbase + C::BN - 1 > q0);
            if (need_mask) {
#pragma unroll
                for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = kbase + 32 * c2 + acc_row(r, h);
                        if (key >= N || (CAUSAL && key > qrow)) s[c2][r] = -INFINITY;
                    }
            }
            float mx = s[0][0];
#pragma unroll
            for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[0][r]);
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[1][r]);
            mx = wave_half_max(mx);
            const float m_new = fmaxf(m_run, mx * c);
            const float alpha = fast_exp2(m_run - m_new);
            float rs = 0.f;
#pragma unroll
            for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float p = fast_exp2(fmaf(s[c2][r], c, -m_new));
                    s[c2][r] = p;
                    rs += p;
                }
            l_run = l_run * alpha + rs;
            m_run = m_new;
#pragma unroll
            for (int b = 0; b < C::DB; ++b)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[b][r] *= alpha;

            V8 pf[4];
            pf[0] = pack8<T>(s[0], 0);
            pf[1] = pack8<T>(s[0], 8);
            pf[2] = pack8<T>(s[1], 0);
            pf[3] = pack8<T>(s[1], 8);
            const T* vb = sV[buf];
#pragma unroll
            for (int g = 0; g < 4; ++g) {
#pragma unroll
                for (int b = 0; b < C::DB; ++b) {
                    const V8 a = *reinterpret_cast<const V8*>(vb + (32 * b + l32) * C::VSTR + 16 * g + 8 * h);
                    oacc[b] = mfma32(a, pf[g], oacc[b]);
                }
            }
        }
        if (more) st.store(sK[buf ^ 1], sV[buf ^ 1], tid);
        __syncthreads();
    }

    const float lt = wave_half_sum(l_run);
    if (qrow < N) {
        const float inv = 1.f / lt;
        T* orow = O + head + (size_t)qrow * D;
#pragma unroll
        for (int b = 0; b < C::DB; ++b)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                V4 w;
#pragma unroll
                for (int i = 0; i < 4; ++i) w[i] = (T)(oacc[b][4 * r4 + i] * inv);
                *reinterpret_cast<V4*>(orow + 32 * b + 8 * r4 + 4 * h) = w;
            }
        if (LSE != nullptr && h == 0) LSE[(size_t)bh * N + qrow] = (m_run + log2f(lt)) * kLn2;
    }
}

template <typename T, int D, bool CAUSAL>
hipError_t launch_typed(const void* q, const void* k, const void* v, void* o, float* lse, int BH,
                        int N, float scale, hipStream_t stream) {
    using C = FwdTile<T, D>;
    const int nqb = (N + C::BM - 1) / C::BM;
    const dim3 grid(BH * nqb), block(C::NT);
    hipLaunchKernelGGL((fwd_mfma_kernel<T, D, CAUSAL>), grid, block, 0, stream,
                       static_cast<const T*>(q), static_cast<const T*>(k),
                       static_cast<const T*>(v), static_cast<T*>(o), lse, BH, N, nqb,
                       scale * kLog2e);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_d(int d, bool causal, const void* q, const void* k, const void* v, void* o,
                    float* lse, int BH, int N, float scale, hipStream_t stream) {
    if (d == 64)
        return causal ? launch_typed<T, 64, true>(q, k, v, o, lse, BH, N, scale, stream)
                      : launch_typed<T, 64, false>(q, k, v, o, lse, BH, N, scale, stream);
    return causal ? launch_typed<T, 128, true>(q, k, v, o, lse, BH, N, scale, stream)
                  : launch_typed<T, 128, false>(q, k, v, o, lse, BH, N, scale, stream);
}

}  // namespace

hipError_t launch_fwd_mfma(int dtype, int d, bool causal, const void* q, const void* k,
                           const void* v, void* o, float* lse, int BH, int N, float scale,
                           hipStream_t stream) {
    if (dtype == 2) return launch_d<__bf16>(d, causal, q, k, v, o, lse, BH, N, scale, stream);
    return launch_d<_Float16>(d, causal, q, k, v, o, lse, BH, N, scale, stream);
}

}  // namespace fa
