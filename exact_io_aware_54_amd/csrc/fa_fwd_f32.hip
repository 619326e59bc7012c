// Forward attention in float32 arithmetic throughout (no reduced-precision
// step), for callers that need fp32 inputs and outputs.
//
// Same method as the 16-bit kernel ("11.11 Flash Attention", sections "Flash
// Attention: The Key Insight", "The Tiling Algorithm" and "Flash Attention
// 2": Q blocks outer, K/V tiles inner, running max m and running sum l, one
// division at the end), on the fp32 matrix cores.

#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

// gfx950 mapping (v_mfma_f32_32x32x2_f32: fp32 operands, fp32
// accumulation), laid out like the 16-bit forward: four or eight waves per
// workgroup; each wave owns 32 queries and computes S^T = K Q^T for a
// 32-key tile (key across the accumulator rows, query across lanes), the
// online softmax in registers, and O^T += V^T P^T with P^T taken straight
// from the score registers.
//  * k-steps of the score product: lane half h contracts head dim h D/2 + s
//    at step s, so a lane reads its K row's half as contiguous 16-byte
//    pieces and keeps its query's half of Q (D/2 floats) in registers.
//  * P V: step t contracts key acc_row(t, h) in half h, which is exactly the
//    key held in score register t of that lane; the V^T operand is one float
//    of that key's row (head dim 32 b + lane % 32).
//  * K and V tiles (32 keys of D floats) go HBM -> LDS with global_load_lds,
//    double-buffered. K rows use the chunk swizzle of the 16-bit tiles (row
//    reads by 32 lanes of 32 different rows); V rows swap 128-byte halves in
//    rows whose bit 2 is set, so the two lane halves (rows 4 apart) of a
//    one-float column read fall on different banks.
// The exponentials are v_exp_f32 (base 2, 1 ulp), like the 16-bit kernels.

__device__ __forceinline__ f32x16 mfma32_f32(float a, float b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

template <int D, int NW_>
struct F32Tile {
    static constexpr int NW = NW_;                  // waves per workgroup
    static constexpr int BM = 32 * NW;              // queries per workgroup
    static constexpr int BN = 32;                   // keys per K/V tile
    static constexpr int NT = 64 * NW;
    static constexpr int ROWB = 4 * D;              // bytes per K/V row
    static constexpr int TILEB = BN * ROWB;
    static constexpr int NLOAD = TILEB / (NT * 16);  // direct loads per thread per tile
    static constexpr int HALF = D / 2;              // score k-steps (head dims per lane half)
    static constexpr int DB = D / 32;               // 32-row blocks of O^T
    static_assert(NLOAD >= 1 && TILEB % (NT * 16) == 0, "tile must split into whole loads");
};

constexpr float kF32RescaleThreshold = 8.f;  // log2 units: refresh m when it grows by > 2^8

template <int D, bool CAUSAL, int NW>
struct F32Wave {
    using C = F32Tile<D, NW>;
    const float* Kh;
    const float* Vh;
    int N, nkt, tid, wave, lane, h, l32, q0, qrow, kswz;
    float c;
    float qv[C::HALF];              // B operand: Q[qrow][h D/2 + s]
    int ld_row[C::NLOAD];
    unsigned ld_k[C::NLOAD], ld_v[C::NLOAD];  // byte offsets of this thread's 16 bytes within a row
    int voff[C::DB];                // V^T read offsets (key rows 4 h; + row of step t)
    float m_run, l_run;
    f32x16 oacc[C::DB];

    __device__ __forceinline__ void init(const float* Qh, const float* Kh_, const float* Vh_,
                                         int N_, int qb, float c_) {
        Kh = Kh_;
        Vh = Vh_;
        N = N_;
        c = c_;
        tid = threadIdx.x;
        lane = tid & 63;
        wave = tid >> 6;
        l32 = lane & 31;
        h = lane >> 5;
        q0 = qb * C::BM + 32 * wave;
        qrow = q0 + l32;
        const f32x4* src = reinterpret_cast<const f32x4*>(Qh + (size_t)min(qrow, N - 1) * D + h * C::HALF);
#pragma unroll
        for (int j = 0; j < C::HALF / 4; ++j) {
            const f32x4 x = src[j];
#pragma unroll
            for (int t = 0; t < 4; ++t) qv[4 * j + t] = x[t];
        }
        const int q_last = min(N, (qb + 1) * C::BM) - 1;
        nkt = CAUSAL ? (q_last / C::BN + 1) : (N + C::BN - 1) / C::BN;
        // load i of this thread fills LDS bytes [i * NT * 16 + tid * 16, +16) of a
        // tile: row r, chunk position p; K takes global chunk p ^ tile_swz(r),
        // V chunk p ^ 8 ((r / 4) % 2)
#pragma unroll
        for (int i = 0; i < C::NLOAD; ++i) {
            const int byte = i * (C::NT * 16) + tid * 16;
            const int r = byte / C::ROWB, p = (byte % C::ROWB) / 16;
            ld_row[i] = r;
            ld_k[i] = (unsigned)(p ^ tile_swz<2 * D>(r)) * 16u;
            ld_v[i] = (unsigned)(p ^ (8 * ((r >> 2) & 1))) * 16u;
        }
        kswz = tile_swz<2 * D>(l32);
#pragma unroll
        for (int b = 0; b < C::DB; ++b) voff[b] = 4 * h * C::ROWB + 128 * (b ^ h) + 4 * l32;
        m_run = -INFINITY;
        l_run = 0.f;
#pragma unroll
        for (int b = 0; b < C::DB; ++b) oacc[b] = f32x16{};
    }

    __device__ __forceinline__ void issue_tile(int kbase, char* sKd, char* sVd) const {
        const char* kb = reinterpret_cast<const char*>(Kh);
        const char* vb = reinterpret_cast<const char*>(Vh);
#pragma unroll
        for (int i = 0; i < C::NLOAD; ++i) {
            const size_t row = (size_t)min(kbase + ld_row[i], N - 1) * C::ROWB;
            char* kd = sKd + i * (C::NT * 16) + wave * 1024;
            char* vd = sVd + i * (C::NT * 16) + wave * 1024;
            __builtin_amdgcn_global_load_lds(kb + row + ld_k[i], kd, 16, 0, 0);
            __builtin_amdgcn_global_load_lds(vb + row + ld_v[i], vd, 16, 0, 0);
        }
    }

    __device__ __forceinline__ void step(int kt, const char* kb, const char* vb, char* kn,
                                         char* vn) {
        const int kbase = kt * C::BN;
        __builtin_amdgcn_s_waitcnt(kVmcntZero);
        __syncthreads();
        if (!kSerialStaging && kt + 1 < nkt) issue_tile(kbase + C::BN, kn, vn);
        if (CAUSAL && kbase > q0 + 31) return;

        // S^T = K Q^T: two accumulators (even / odd 4-step groups)
        f32x16 sa = f32x16{}, sb = f32x16{};
        const char* krow = kb + l32 * C::ROWB;
#pragma unroll
        for (int j = 0; j < C::HALF / 4; ++j) {
            const f32x4 a = *reinterpret_cast<const f32x4*>(krow + 16 * ((h * (D / 8) + j) ^ kswz));
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                if (j & 1) sb = mfma32_f32(a[t], qv[4 * j + t], sb);
                else sa = mfma32_f32(a[t], qv[4 * j + t], sa);
            }
        }
        f32x16 s;
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = sa[r] + sb[r];
        // key kbase + acc_row(r, h) is visible iff it is <= lim + 4 h + kbase
        const bool need_mask = (kbase + C::BN > N) || (CAUSAL && kbase + C::BN - 1 > q0);
        if (need_mask) {
            const int lim = (CAUSAL ? min(qrow, N - 1) : N - 1) - kbase - 4 * h;
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (8 * (r >> 2) + (r & 3) > lim) s[r] = -INFINITY;
        }
        float mx = s[0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
        mx = wave_half_max(mx) * c;
        if (__builtin_amdgcn_ballot_w64(mx > m_run + kF32RescaleThreshold) != 0) {
            const float m_new = fmaxf(m_run, mx);
            const float alpha = fast_exp2(m_run - m_new);
            m_run = m_new;
            l_run *= alpha;
#pragma unroll
            for (int b = 0; b < C::DB; ++b)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[b][r] *= alpha;
        }
        float rs = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float p = fast_exp2(fmaf(s[r], c, -m_run));
            s[r] = p;
            rs += p;
        }
        l_run += rs;
        // O^T += V^T P^T: step t contracts key acc_row(t, h) = score register t
#pragma unroll
        for (int t = 0; t < 16; ++t)
#pragma unroll
            for (int b = 0; b < C::DB; ++b) {
                const float a = *reinterpret_cast<const float*>(
                    vb + (8 * (t >> 2) + (t & 3)) * C::ROWB + voff[b]);
                oacc[b] = mfma32_f32(a, s[t], oacc[b]);
            }
    }

    __device__ __forceinline__ void finish(float* Oh, float* lse_h) {
        const float lt = wave_half_sum(l_run);
        if (qrow >= N) return;
        const float inv = 1.f / lt;
        float* orow = Oh + (size_t)qrow * D;
#pragma unroll
        for (int b = 0; b < C::DB; ++b)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4)
                *reinterpret_cast<f32x4*>(orow + 32 * b + 8 * r4 + 4 * h) =
                    f32x4{oacc[b][4 * r4] * inv, oacc[b][4 * r4 + 1] * inv,
                          oacc[b][4 * r4 + 2] * inv, oacc[b][4 * r4 + 3] * inv};
        if (lse_h != nullptr && h == 0) lse_h[qrow] = (m_run + log2f(lt)) * kLn2;
    }
};

template <int D, bool CAUSAL, int NW>
__global__ void __launch_bounds__(64 * NW, 8 / NW)
fwd_f32_mfma_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                    const float* __restrict__ V, float* __restrict__ O, float* __restrict__ LSE,
                    int BH, int N, int nqb, float c) {
    using C = F32Tile<D, NW>;
    __shared__ __attribute__((aligned(1024))) char sK0[C::TILEB];
    __shared__ __attribute__((aligned(1024))) char sK1[C::TILEB];
    __shared__ __attribute__((aligned(1024))) char sV0[C::TILEB];
    __shared__ __attribute__((aligned(1024))) char sV1[C::TILEB];
    int bh, qb;
    if (CAUSAL) {
        causal_block(blockIdx.x, nqb, BH, bh, qb);
    } else {
        const int L = xcd_remap(blockIdx.x, BH * nqb);
        bh = L / nqb;
        qb = L % nqb;
    }
    const size_t head = (size_t)bh * N * D;
    F32Wave<D, CAUSAL, NW> w;
    w.init(Q + head, K + head, V + head, N, qb, c);
    w.issue_tile(0, sK0, sV0);
    if constexpr (kSerialStaging) {
        for (int kt = 0; kt < w.nkt; ++kt) {
            w.step(kt, sK0, sV0, sK0, sV0);
            __syncthreads();
            if (kt + 1 < w.nkt) w.issue_tile((kt + 1) * C::BN, sK0, sV0);
        }
    } else {
        for (int kt = 0; kt < w.nkt; kt += 2) {
            w.step(kt, sK0, sV0, sK1, sV1);
            if (kt + 1 < w.nkt) w.step(kt + 1, sK1, sV1, sK0, sV0);
        }
    }
    w.finish(O + head, LSE == nullptr ? nullptr : LSE + (size_t)bh * N);
}

template <int D, bool CAUSAL, int NW>
hipError_t launch_nw(const float* q, const float* k, const float* v, float* o, float* lse,
                     int BH, int N, float scale, hipStream_t stream) {
    using C = F32Tile<D, NW>;
    const int nqb = (N + C::BM - 1) / C::BM;
    hipLaunchKernelGGL((fwd_f32_mfma_kernel<D, CAUSAL, NW>), dim3(BH * nqb), dim3(C::NT), 0,
                       stream, q, k, v, o, lse, BH, N, nqb, scale * kLog2e);
    return hipGetLastError();
}

// Eight waves (256 queries, K/V tiles shared by all eight, one workgroup per
// CU) once the launch has a workgroup per CU: B1 H32 N4096 d128 causal 1.15
// -> 1.05 ms, non-causal 2.04 -> 2.00 ms; four waves (two workgroups per CU)
// below that (the 128-query workload: 0.023 against 0.029 ms).
template <int D, bool CAUSAL>
hipError_t launch_mfma(const float* q, const float* k, const float* v, float* o, float* lse,
                       int BH, int N, float scale, hipStream_t stream) {
    if ((int64_t)BH * ((N + 255) / 256) >= 256)
        return launch_nw<D, CAUSAL, 8>(q, k, v, o, lse, BH, N, scale, stream);
    return launch_nw<D, CAUSAL, 4>(q, k, v, o, lse, BH, N, scale, stream);
}

}  // namespace

hipError_t launch_fwd_f32(int d, bool causal, const float* q, const float* k, const float* v,
                          float* o, float* lse, int BH, int N, float scale, hipStream_t stream) {
    if (d == 64)
        return causal ? launch_mfma<64, true>(q, k, v, o, lse, BH, N, scale, stream)
                      : launch_mfma<64, false>(q, k, v, o, lse, BH, N, scale, stream);
    return causal ? launch_mfma<128, true>(q, k, v, o, lse, BH, N, scale, stream)
                  : launch_mfma<128, false>(q, k, v, o, lse, BH, N, scale, stream);
}

}  // namespace fa
