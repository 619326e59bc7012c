// Split-KV forward (few queries over many keys, e.g. decoding) and the merge
// of partial attention results.
//
// "11.11 Flash Attention" (algomaster.io), section "Flash Attention: The Key
// Insight": a softmax over a row can be built from pieces, each kept as a
// running max and sum and rescaled by exp(m_old - m_new) when pieces meet.
// Here the pieces are whole ranges of keys: the key sequence is cut into
// `splits` ranges, every (batch*head, block of 32 queries, key range) gets its
// own workgroup, which writes its normalised partial output O_s and
// LSE_s = ln sum_{j in range} exp(S_j), and a second kernel merges the parts:
//   LSE = ln sum_s exp(LSE_s),   O = sum_s exp(LSE_s - LSE) O_s.
// With few queries the square kernel would leave most of the machine idle
// (one workgroup per 128-256 queries); splitting the keys restores the
// parallelism, and the work is bound by reading K and V once from HBM.
//
// Layout: Q, O [B, H, Nq, d]; K, V [B, H, Nk, d]; LSE [B, H, Nq]. Causal
// (a reading, not on the pages): the queries are the last Nq positions of the
// key sequence, so query i sees keys 0 .. Nk - Nq + i.
//
// gfx950 mapping of the split kernel: four waves share each 128-key K/V tile
// (direct loads into LDS, double-buffered, XOR-swizzled as in the square
// kernels); wave w takes keys 32 w .. 32 w + 31 of every tile and computes
// S^T = K Q^T for the block's 32 queries (query across lanes), keeps its own
// running max / sum / output, and the four waves' states are merged through
// LDS at the end with the same formula as the merge kernel.

#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr float kRescaleThreshold = 8.f;  // log2 units: refresh m when it grows by > 2^8

template <int D>
struct SkvTile {
    static constexpr int BQ = 32;                  // queries per workgroup
    static constexpr int BN = 128;                 // keys per K/V tile (4 waves x 32)
    static constexpr int NT = 256;
    static constexpr int ROWB = 2 * D;
    static constexpr int TILEB = BN * ROWB;
    static constexpr int NLOAD = TILEB / (NT * 16);
    static constexpr int KS = D / 16;
    static constexpr int DB = D / 32;
    static constexpr int ORS = D * 4 + 16;         // LDS row stride of the fp32 output merge
    static_assert(NLOAD >= 1 && TILEB % (NT * 16) == 0, "tile must split into whole loads");
    static_assert(BQ * ORS <= TILEB, "a wave's output must fit one tile buffer");
};

template <typename T, int D, bool CAUSAL>
struct SkvWave {
    using C = SkvTile<D>;
    using V8 = typename Vec<T>::x8;
    const T* Kh;
    const T* Vh;
    int Nq, Nk, tid, wave, lane, l32, h, q, q0, kend, off;
    float c;
    V8 qf[C::KS];
    int ld_row[C::NLOAD], ld_col[C::NLOAD];
    int koff[C::KS];
    int voff[2][C::DB];
    float m_run, l_run;
    f32x16 oacc[C::DB];

    __device__ __forceinline__ void init(const T* Qh, const T* Kh_, const T* Vh_, int Nq_, int Nk_,
                                         int qb, int kend_, float c_) {
        Kh = Kh_;
        Vh = Vh_;
        Nq = Nq_;
        Nk = Nk_;
        kend = kend_;
        c = c_;
        off = Nk - Nq;  // causal: query i sees keys <= i + off
        tid = threadIdx.x;
        lane = tid & 63;
        wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        l32 = lane & 31;
        h = lane >> 5;
        q0 = qb * C::BQ;
        q = q0 + l32;
        const V8* src = reinterpret_cast<const V8*>(Qh + (size_t)min(q, Nq - 1) * D + 8 * h);
#pragma unroll
        for (int s = 0; s < C::KS; ++s) qf[s] = src[2 * s];
#pragma unroll
        for (int i = 0; i < C::NLOAD; ++i) {
            const int byte = i * (C::NT * 16) + tid * 16;
            const int r = byte / C::ROWB, p = (byte % C::ROWB) / 16;
            ld_row[i] = r;
            ld_col[i] = (p ^ tile_swz<D>(r)) * 8;
        }
#pragma unroll
        for (int s = 0; s < C::KS; ++s) koff[s] = tile_off<D>(32 * wave + l32, 16 * s + 8 * h);
        // V^T via transposing reads, key order of the score registers (see the
        // square forward kernel): key group g of this wave is rows 32 wave + 16 g.
        const int src_r = 32 * wave + 4 * h + (lane & 15) / 4;
        const int src_d = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
            for (int b = 0; b < C::DB; ++b) voff[hf][b] = tile_off<D>(src_r + 8 * hf, 32 * b + src_d);
        m_run = -INFINITY;
        l_run = 0.f;
#pragma unroll
        for (int b = 0; b < C::DB; ++b) oacc[b] = f32x16{};
    }

    __device__ __forceinline__ void issue(int kbase, char* sKd, char* sVd) const {
#pragma unroll
        for (int i = 0; i < C::NLOAD; ++i) {
            const size_t row = (size_t)min(kbase + ld_row[i], Nk - 1) * D;
            char* kd = sKd + i * (C::NT * 16) + wave * 1024;
            char* vd = sVd + i * (C::NT * 16) + wave * 1024;
            __builtin_amdgcn_global_load_lds(Kh + row + ld_col[i], kd, 16, 0, 0);
            __builtin_amdgcn_global_load_lds(Vh + row + ld_col[i], vd, 16, 0, 0);
        }
    }

    // keys kbase + 32 wave .. + 31 of this tile
    __device__ __forceinline__ void step(int kbase, const char* kb, const char* vb) {
        const int k0 = kbase + 32 * wave;
        if (k0 >= kend) return;                                   // past the range
        if (CAUSAL && k0 > min(q0 + C::BQ - 1, Nq - 1) + off) return;  // above every query
        f32x16 s[1] = {f32x16{}};
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
            const V8 a = *reinterpret_cast<const V8*>(kb + koff[ks]);
            s[0] = mfma32(a, qf[ks], s[0]);
        }
        // key k0 + acc_row(r, h) is visible iff it is < kend and (causal) <= q + off
        const bool need_mask = k0 + 32 > kend || (CAUSAL && k0 + 31 > q0 + off);
        if (need_mask) {
            const int lim_end = kend - k0 - 4 * h;                  // row < lim_end
            const int lim_c = CAUSAL ? (min(q, Nq - 1) + off - k0 - 4 * h) : 1 << 30;  // row <= lim_c
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int rr = 8 * (r >> 2) + (r & 3);
                if (rr >= lim_end || rr > lim_c) s[0][r] = -INFINITY;
            }
        }
        float mx = s[0][0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[0][r]);
        mx = wave_half_max(mx) * c;                               // -inf if nothing visible
        if (__builtin_amdgcn_ballot_w64(mx > m_run + kRescaleThreshold) != 0) {
            const float m_new = fmaxf(m_run, mx);
            const float alpha = (m_run == -INFINITY) ? 0.f : fast_exp2(m_run - m_new);
            m_run = m_new;
            l_run *= alpha;
#pragma unroll
            for (int b = 0; b < C::DB; ++b)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[b][r] *= alpha;
        }
        // a query that has seen no key yet keeps m = -inf; its scores are all -inf
        const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
        float rs = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float p = fast_exp2(fmaf(s[0][r], c, -m_use));
            s[0][r] = p;
            rs += p;
        }
        l_run += rs;
        V8 pf[2];
        pf[0] = pack8<T>(s[0], 0);
        pf[1] = pack8<T>(s[0], 8);
#pragma unroll
        for (int g = 0; g < 2; ++g)
#pragma unroll
            for (int b = 0; b < C::DB; ++b) {
                const char* vg = vb + g * 16 * C::ROWB;
                const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vg + voff[0][b]));
                const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vg + voff[1][b]));
                const s16x4 w[2] = {lo, hi};
                V8 a;
                __builtin_memcpy(&a, w, sizeof(a));
                oacc[b] = mfma32(a, pf[g], oacc[b]);
            }
    }

    // Merge the four waves' (m, l, O) through LDS and write this workgroup's
    // normalised partial O (fp32) and LSE (natural log; -inf if no key of the
    // range is visible to the query). Statistics go through `stat`, the
    // output through two buffers `bufA`, `bufB` of 32 rows of D floats:
    // waves 2 and 3 park their scaled outputs there, waves 0 and 1 add them,
    // wave 1 hands its sum to wave 0, which writes the result.
    __device__ __forceinline__ void put_o(char* buf) const {
#pragma unroll
        for (int b = 0; b < C::DB; ++b)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const f32x4 w4 = {oacc[b][4 * r4], oacc[b][4 * r4 + 1], oacc[b][4 * r4 + 2],
                                  oacc[b][4 * r4 + 3]};
                *reinterpret_cast<f32x4*>(buf + l32 * C::ORS + 4 * (32 * b + 8 * r4 + 4 * h)) = w4;
            }
    }
    __device__ __forceinline__ void add_o(const char* buf) {
#pragma unroll
        for (int b = 0; b < C::DB; ++b)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const f32x4 x = *reinterpret_cast<const f32x4*>(buf + l32 * C::ORS +
                                                                4 * (32 * b + 8 * r4 + 4 * h));
#pragma unroll
                for (int i = 0; i < 4; ++i) oacc[b][4 * r4 + i] += x[i];
            }
    }

    __device__ __forceinline__ void finish(char* stat, char* bufA, char* bufB, float* o_part,
                                           float* lse_part) {
        float* sm = reinterpret_cast<float*>(stat);               // [4][32] running max
        float* sl = sm + 4 * C::BQ;                               // [4][32] row sums
        const float lt = wave_half_sum(l_run);
        if (h == 0) {
            sm[wave * C::BQ + l32] = m_run;
            sl[wave * C::BQ + l32] = lt;
        }
        __syncthreads();
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < 4; ++w) M = fmaxf(M, sm[w * C::BQ + l32]);
        float L = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float mw = sm[w * C::BQ + l32];
            if (mw != -INFINITY) L += sl[w * C::BQ + l32] * fast_exp2(mw - M);
        }
        const float f = (L > 0.f && m_run != -INFINITY) ? fast_exp2(m_run - M) / L : 0.f;
#pragma unroll
        for (int b = 0; b < C::DB; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[b][r] *= f;
        if (wave == 2) put_o(bufA);
        if (wave == 3) put_o(bufB);
        __syncthreads();
        if (wave == 0) add_o(bufA);
        if (wave == 1) add_o(bufB);
        __syncthreads();
        if (wave == 1) put_o(bufA);
        __syncthreads();
        if (wave != 0) return;
        add_o(bufA);
        if (q >= Nq) return;
        if (h == 0) lse_part[q] = (L > 0.f) ? (M + log2f(L)) * kLn2 : -INFINITY;
        float* orow = o_part + (size_t)q * D;
#pragma unroll
        for (int b = 0; b < C::DB; ++b)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4)
                *reinterpret_cast<f32x4*>(orow + 32 * b + 8 * r4 + 4 * h) =
                    f32x4{oacc[b][4 * r4], oacc[b][4 * r4 + 1], oacc[b][4 * r4 + 2],
                          oacc[b][4 * r4 + 3]};
    }
};

template <typename T, int D, bool CAUSAL>
__global__ void __launch_bounds__(256)
splitkv_kernel(const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
               float* __restrict__ o_part, float* __restrict__ lse_part, int BH, int Nq, int Nk,
               int nqb, int splits, int kps, float c) {
    using C = SkvTile<D>;
    __shared__ __attribute__((aligned(1024))) char sK0[C::TILEB];
    __shared__ __attribute__((aligned(1024))) char sK1[C::TILEB];
    __shared__ __attribute__((aligned(1024))) char sV0[C::TILEB];
    __shared__ __attribute__((aligned(1024))) char sV1[C::TILEB];
    const int G = BH * nqb * splits;
    const int L = xcd_remap(blockIdx.x, G);
    const int sp = L % splits, qb = (L / splits) % nqb, bh = L / (splits * nqb);
    const int kbeg = sp * kps, kend = min(Nk, kbeg + kps);
    SkvWave<T, D, CAUSAL> w;
    w.init(Q + (size_t)bh * Nq * D, K + (size_t)bh * Nk * D, V + (size_t)bh * Nk * D, Nq, Nk, qb,
           kend, c);
    // causal: keys past the block's last query are never visible
    const int kstop = CAUSAL ? min(kend, min(qb * C::BQ + C::BQ, Nq) - 1 + (Nk - Nq) + 1) : kend;
    const int nkt = kstop > kbeg ? (kstop - kbeg + C::BN - 1) / C::BN : 0;
    if (nkt > 0) w.issue(kbeg, sK0, sV0);
    if constexpr (kSerialStaging) {
        for (int kt = 0; kt < nkt; ++kt) {
            __builtin_amdgcn_s_waitcnt(kVmcntZero);
            __syncthreads();
            w.step(kbeg + kt * C::BN, sK0, sV0);
            __syncthreads();
            if (kt + 1 < nkt) w.issue(kbeg + (kt + 1) * C::BN, sK0, sV0);
        }
    } else {
        for (int kt = 0; kt < nkt; kt += 2) {
            __builtin_amdgcn_s_waitcnt(kVmcntZero);
            __syncthreads();
            if (kt + 1 < nkt) w.issue(kbeg + (kt + 1) * C::BN, sK1, sV1);
            w.step(kbeg + kt * C::BN, sK0, sV0);
            if (kt + 1 < nkt) {
                __builtin_amdgcn_s_waitcnt(kVmcntZero);
                __syncthreads();
                if (kt + 2 < nkt) w.issue(kbeg + (kt + 2) * C::BN, sK0, sV0);
                w.step(kbeg + (kt + 1) * C::BN, sK1, sV1);
            }
        }
    }
    __syncthreads();  // the tile buffers are reused for the merge
    const size_t part = (size_t)sp * BH + bh;
    w.finish(sV0, sK0, sK1, o_part + part * Nq * D, lse_part + part * Nq);
}

// ------------------------------------------------------------- merge of parts
// One thread per four consecutive elements of a row: the parts' LSE values are
// reduced relative to their max, O accumulated in fp32.
template <typename TO>
__global__ void __launch_bounds__(256)
lse_merge_kernel(const float* __restrict__ o_parts, const float* __restrict__ lse_parts, int P,
                 long long rows, int d, TO* __restrict__ o, float* __restrict__ lse) {
    const int per_row = d / 4;
    const long long e = (long long)blockIdx.x * 256 + threadIdx.x;
    if (e >= rows * per_row) return;
    const long long row = e / per_row;
    const int col = 4 * (int)(e % per_row);
    float M = -INFINITY;
    for (int p = 0; p < P; ++p) M = fmaxf(M, lse_parts[(size_t)p * rows + row]);
    float L = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (M != -INFINITY) {
        for (int p = 0; p < P; ++p) {
            const float lp = lse_parts[(size_t)p * rows + row];
            if (lp == -INFINITY) continue;  // an empty part's O is never read
            const float wgt = fast_exp2((lp - M) * kLog2e);
            L += wgt;
            const f32x4 x = *reinterpret_cast<const f32x4*>(o_parts + ((size_t)p * rows + row) * d + col);
            acc += x * wgt;
        }
        acc *= 1.f / L;
    }
    TO* dst = o + (size_t)row * d + col;
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[i] = (TO)acc[i];
    if (lse != nullptr && col == 0) lse[row] = (M == -INFINITY) ? -INFINITY : M + logf(L);
}

template <typename T, int D, bool CAUSAL>
hipError_t launch_split(const void* q, const void* k, const void* v, float* o_part,
                        float* lse_part, int BH, int Nq, int Nk, int splits, int kps, float scale,
                        hipStream_t stream) {
    const int nqb = (Nq + SkvTile<D>::BQ - 1) / SkvTile<D>::BQ;
    hipLaunchKernelGGL((splitkv_kernel<T, D, CAUSAL>), dim3(BH * nqb * splits), dim3(256), 0,
                       stream, static_cast<const T*>(q), static_cast<const T*>(k),
                       static_cast<const T*>(v), o_part, lse_part, BH, Nq, Nk, nqb, splits, kps,
                       scale * kLog2e);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_split_d(int d, bool causal, const void* q, const void* k, const void* v,
                          float* o_part, float* lse_part, int BH, int Nq, int Nk, int splits,
                          int kps, float scale, hipStream_t stream) {
    if (d == 64)
        return causal ? launch_split<T, 64, true>(q, k, v, o_part, lse_part, BH, Nq, Nk, splits, kps, scale, stream)
                      : launch_split<T, 64, false>(q, k, v, o_part, lse_part, BH, Nq, Nk, splits, kps, scale, stream);
    return causal ? launch_split<T, 128, true>(q, k, v, o_part, lse_part, BH, Nq, Nk, splits, kps, scale, stream)
                  : launch_split<T, 128, false>(q, k, v, o_part, lse_part, BH, Nq, Nk, splits, kps, scale, stream);
}

}  // namespace

hipError_t launch_lse_merge(int dtype_out, const float* o_parts, const float* lse_parts, int P,
                            long long rows, int d, void* o, float* lse, hipStream_t stream) {
    const long long threads = rows * (d / 4);
    const dim3 grid((unsigned)((threads + 255) / 256)), block(256);
    if (dtype_out == 2)
        hipLaunchKernelGGL((lse_merge_kernel<__bf16>), grid, block, 0, stream, o_parts, lse_parts,
                           P, rows, d, static_cast<__bf16*>(o), lse);
    else if (dtype_out == 1)
        hipLaunchKernelGGL((lse_merge_kernel<_Float16>), grid, block, 0, stream, o_parts,
                           lse_parts, P, rows, d, static_cast<_Float16*>(o), lse);
    else
        hipLaunchKernelGGL((lse_merge_kernel<float>), grid, block, 0, stream, o_parts, lse_parts,
                           P, rows, d, static_cast<float*>(o), lse);
    return hipGetLastError();
}

hipError_t launch_fwd_splitkv(int dtype, int d, bool causal, const void* q, const void* k,
                              const void* v, void* o, float* lse, float* o_part, float* lse_part,
                              int BH, int Nq, int Nk, int splits, int kps, float scale,
                              hipStream_t stream) {
    const hipError_t e =
        dtype == 2 ? launch_split_d<__bf16>(d, causal, q, k, v, o_part, lse_part, BH, Nq, Nk,
                                            splits, kps, scale, stream)
                   : launch_split_d<_Float16>(d, causal, q, k, v, o_part, lse_part, BH, Nq, Nk,
                                              splits, kps, scale, stream);
    if (e != hipSuccess) return e;
    return launch_lse_merge(dtype, o_part, lse_part, splits, (long long)BH * Nq, d, o, lse,
                            stream);
}

}  // namespace fa
