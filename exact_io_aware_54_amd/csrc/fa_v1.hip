// The first-generation loop order, kept for the loop-order ablation.
//
// "11.11 Flash Attention" (algomaster.io), section "The Tiling Algorithm":
// the outer loop walks the K/V blocks and the inner loop the Q blocks; for
// every (K/V block j, Q block i) the running output O_i and statistics m_i,
// l_i are loaded from HBM, updated -- m_new = max(m_i, rowmax(S_ij)),
// l_new = exp(m_i - m_new) l_i + rowsum(exp(S_ij - m_new)),
// O_i = (exp(m_i - m_new) l_i O_i + exp(S_ij - m_new) V_j) / l_new -- and
// written back. Section "Flash Attention 2" names what the second generation
// changed: parallelism over the sequence (here: one workgroup per (batch,
// head) only, as in the first generation), fewer non-matmul operations (here:
// O is renormalised at every step) and the swapped loop order (here: K/V
// outer, so O, m and l make a round trip through HBM per block pair).
//
// Workgroup: four waves, 32 queries each (a Q block is 128 queries); K_j and
// V_j are staged once per outer step in LDS (direct loads, XOR-swizzled like
// the fused kernels); scores and P V on 32x32x16 MFMAs, O in float32 in a
// workspace. A final pass per workgroup converts O to the output type and
// writes LSE = m + ln l.

#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

template <int D>
struct V1Tile {
    static constexpr int BM = 128;                 // queries per Q block (4 waves x 32)
    static constexpr int BN = 64;                  // keys per K/V block
    static constexpr int NT = 256;
    static constexpr int ROWB = 2 * D;
    static constexpr int TILEB = BN * ROWB;
    static constexpr int NLOAD = TILEB / (NT * 16);
    static constexpr int NSUB = BN / 32;
    static constexpr int NG = BN / 16;
    static constexpr int KS = D / 16;
    static constexpr int DB = D / 32;
    static_assert(NLOAD >= 1 && TILEB % (NT * 16) == 0, "tile must split into whole loads");
};

template <typename T, int D, bool CAUSAL>
struct V1Wave {
    using C = V1Tile<D>;
    using V8 = typename Vec<T>::x8;
    using V4 = typename Vec<T>::x4;
    const T* Qh;
    const T* Kh;
    const T* Vh;
    float* Oh;   // fp32 running output [N][D]
    float* mh;   // running max (log2 units of the scaled scores) [N][2]
    float* lh;   // running sum [N][2]
    // m and l are the same in both halves of the wave; each lane keeps its own
    // copy (index 2 q + h) so that it only ever reads what it wrote itself.
    int N, tid, wave, lane, l32, h;
    float c;
    int ld_row[C::NLOAD], ld_col[C::NLOAD];
    int koff[C::KS];
    int voff[2][C::DB];

    __device__ __forceinline__ void init(const T* Qh_, const T* Kh_, const T* Vh_, float* Oh_,
                                         float* mh_, float* lh_, int N_, float c_) {
        Qh = Qh_;
        Kh = Kh_;
        Vh = Vh_;
        Oh = Oh_;
        mh = mh_;
        lh = lh_;
        N = N_;
        c = c_;
        tid = threadIdx.x;
        lane = tid & 63;
        wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        l32 = lane & 31;
        h = lane >> 5;
#pragma unroll
        for (int i = 0; i < C::NLOAD; ++i) {
            const int byte = i * (C::NT * 16) + tid * 16;
            const int r = byte / C::ROWB, p = (byte % C::ROWB) / 16;
            ld_row[i] = r;
            ld_col[i] = (p ^ tile_swz<D>(r)) * 8;
        }
#pragma unroll
        for (int s = 0; s < C::KS; ++s) koff[s] = tile_off<D>(l32, 16 * s + 8 * h);
        const int src_r = 4 * h + (lane & 15) / 4;
        const int src_d = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
            for (int b = 0; b < C::DB; ++b) voff[hf][b] = tile_off<D>(8 * hf + src_r, 32 * b + src_d);
    }

    __device__ __forceinline__ void load_kv(int kbase, char* sK, char* sV) const {
#pragma unroll
        for (int i = 0; i < C::NLOAD; ++i) {
            const size_t row = (size_t)min(kbase + ld_row[i], N - 1) * D;
            char* kd = sK + i * (C::NT * 16) + wave * 1024;
            char* vd = sV + i * (C::NT * 16) + wave * 1024;
            __builtin_amdgcn_global_load_lds(Kh + row + ld_col[i], kd, 16, 0, 0);
            __builtin_amdgcn_global_load_lds(Vh + row + ld_col[i], vd, 16, 0, 0);
        }
    }

    // One (K/V block, Q block) pair for this wave's 32 queries q0 .. q0 + 31.
    __device__ __forceinline__ void pair(int kbase, int q0, bool first, const char* kb,
                                         const char* vb) {
        if (q0 >= N) return;
        if (CAUSAL && kbase > q0 + 31) return;    // every key follows every query
        const int q = q0 + l32;
        const int qr = min(q, N - 1);
        V8 qf[C::KS];
        const V8* src = reinterpret_cast<const V8*>(Qh + (size_t)qr * D + 8 * h);
#pragma unroll
        for (int s = 0; s < C::KS; ++s) qf[s] = src[2 * s];
        f32x16 s[C::NSUB];
#pragma unroll
        for (int c2 = 0; c2 < C::NSUB; ++c2) s[c2] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
            for (int c2 = 0; c2 < C::NSUB; ++c2) {
                const V8 a = *reinterpret_cast<const V8*>(kb + koff[ks] + c2 * 32 * C::ROWB);
                s[c2] = mfma32(a, qf[ks], s[c2]);
            }
        const bool need_mask = (kbase + C::BN > N) || (CAUSAL && kbase + C::BN - 1 > q0);
        if (need_mask) {
            const int lim = (CAUSAL ? qr : N - 1) - kbase - 4 * h;
#pragma unroll
            for (int c2 = 0; c2 < C::NSUB; ++c2)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (32 * c2 + 8 * (r >> 2) + (r & 3) > lim) s[c2][r] = -INFINITY;
        }
        // running statistics of this query from HBM (nothing yet on the first block)
        const float m_i = first ? -INFINITY : mh[2 * qr + h];
        const float l_i = first ? 0.f : lh[2 * qr + h];
        float mx = s[0][0];
#pragma unroll
        for (int c2 = 0; c2 < C::NSUB; ++c2)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[c2][r]);
        const float m_ij = wave_half_max(mx) * c;
        const float m_new = fmaxf(m_i, m_ij);     // finite: block 0 holds key 0 <= every query
        const float alpha = (m_i == -INFINITY) ? 0.f : fast_exp2(m_i - m_new);
        float rs = 0.f;
#pragma unroll
        for (int c2 = 0; c2 < C::NSUB; ++c2)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float p = fast_exp2(fmaf(s[c2][r], c, -m_new));
                s[c2][r] = p;
                rs += p;
            }
        const float l_new = alpha * l_i + wave_half_sum(rs);
        f32x16 pv[C::DB];
#pragma unroll
        for (int b = 0; b < C::DB; ++b) pv[b] = f32x16{};
#pragma unroll
        for (int g = 0; g < C::NG; ++g) {
            const V8 pf = pack8<T>(s[g / 2], 8 * (g % 2));
#pragma unroll
            for (int b = 0; b < C::DB; ++b) {
                const char* vg = vb + g * 16 * C::ROWB;
                const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vg + voff[0][b]));
                const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vg + voff[1][b]));
                const s16x4 w[2] = {lo, hi};
                V8 a;
                __builtin_memcpy(&a, w, sizeof(a));
                pv[b] = mfma32(a, pf, pv[b]);
            }
        }
        // O_i = (alpha l_i O_i + P V_j) / l_new, read from and written back to HBM
        const float keep = alpha * l_i / l_new, inv = 1.f / l_new;
        if (q < N) {
            float* orow = Oh + (size_t)q * D;
#pragma unroll
            for (int b = 0; b < C::DB; ++b)
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    float* p = orow + 32 * b + 8 * r4 + 4 * h;
                    f32x4 o4 = first ? f32x4{0.f, 0.f, 0.f, 0.f} : *reinterpret_cast<const f32x4*>(p);
#pragma unroll
                    for (int i = 0; i < 4; ++i) o4[i] = keep * o4[i] + inv * pv[b][4 * r4 + i];
                    *reinterpret_cast<f32x4*>(p) = o4;
                }
            mh[2 * q + h] = m_new;
            lh[2 * q + h] = l_new;
        }
    }

    // O (fp32) -> output type; LSE = (m + log2 l) ln 2
    __device__ __forceinline__ void finalize(int q0, T* O, float* lse) const {
        const int q = q0 + l32;
        if (q >= N) return;
        const float* orow = Oh + (size_t)q * D;
        T* out = O + (size_t)q * D;
#pragma unroll
        for (int b = 0; b < C::DB; ++b)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int d0 = 32 * b + 8 * r4 + 4 * h;
                const f32x4 o4 = *reinterpret_cast<const f32x4*>(orow + d0);
                V4 w;
#pragma unroll
                for (int i = 0; i < 4; ++i) w[i] = (T)o4[i];
                *reinterpret_cast<V4*>(out + d0) = w;
            }
        if (lse != nullptr && h == 0) lse[q] = (mh[2 * q] + log2f(lh[2 * q])) * kLn2;
    }
};

template <typename T, int D, bool CAUSAL>
__global__ void __launch_bounds__(256)
fwd_v1_kernel(const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
              T* __restrict__ O, float* __restrict__ LSE, float* __restrict__ Ows,
              float* __restrict__ mws, float* __restrict__ lws, int N, float c) {
    using C = V1Tile<D>;
    __shared__ __attribute__((aligned(1024))) char sK[C::TILEB];
    __shared__ __attribute__((aligned(1024))) char sV[C::TILEB];
    const int bh = blockIdx.x;
    const size_t head = (size_t)bh * N * D;
    V1Wave<T, D, CAUSAL> w;
    w.init(Q + head, K + head, V + head, Ows + head, mws + (size_t)bh * N * 2,
           lws + (size_t)bh * N * 2, N, c);
    const int nkb = (N + C::BN - 1) / C::BN, nqb = (N + C::BM - 1) / C::BM;
    for (int j = 0; j < nkb; ++j) {         // outer: K/V blocks
        __syncthreads();                    // everyone is done with the previous K_j, V_j
        w.load_kv(j * C::BN, sK, sV);
        __builtin_amdgcn_s_waitcnt(kVmcntZero);
        __syncthreads();
        for (int i = 0; i < nqb; ++i)       // inner: Q blocks
            w.pair(j * C::BN, i * C::BM + 32 * w.wave, j == 0, sK, sV);
    }
    // each wave finalises the rows it owns (the same rows it updated)
    for (int i = 0; i < nqb; ++i) w.finalize(i * C::BM + 32 * w.wave, O + head,
                                             LSE == nullptr ? nullptr : LSE + (size_t)bh * N);
}

template <typename T, int D>
hipError_t launch_v1_typed(bool causal, const void* q, const void* k, const void* v, void* o,
                           float* lse, float* ows, float* mws, float* lws, int BH, int N,
                           float scale, hipStream_t stream) {
    if (causal)
        hipLaunchKernelGGL((fwd_v1_kernel<T, D, true>), dim3(BH), dim3(256), 0, stream,
                           static_cast<const T*>(q), static_cast<const T*>(k),
                           static_cast<const T*>(v), static_cast<T*>(o), lse, ows, mws, lws, N,
                           scale * kLog2e);
    else
        hipLaunchKernelGGL((fwd_v1_kernel<T, D, false>), dim3(BH), dim3(256), 0, stream,
                           static_cast<const T*>(q), static_cast<const T*>(k),
                           static_cast<const T*>(v), static_cast<T*>(o), lse, ows, mws, lws, N,
                           scale * kLog2e);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_v1(int dtype, int d, bool causal, const void* q, const void* k,
                         const void* v, void* o, float* lse, float* ows, float* mws, float* lws,
                         int BH, int N, float scale, hipStream_t stream) {
    if (dtype == 2)
        return d == 64 ? launch_v1_typed<__bf16, 64>(causal, q, k, v, o, lse, ows, mws, lws, BH, N, scale, stream)
                       : launch_v1_typed<__bf16, 128>(causal, q, k, v, o, lse, ows, mws, lws, BH, N, scale, stream);
    return d == 64 ? launch_v1_typed<_Float16, 64>(causal, q, k, v, o, lse, ows, mws, lws, BH, N, scale, stream)
                   : launch_v1_typed<_Float16, 128>(causal, q, k, v, o, lse, ows, mws, lws, BH, N, scale, stream);
}

}  // namespace fa
