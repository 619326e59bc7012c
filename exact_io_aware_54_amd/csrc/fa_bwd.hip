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
//  1. bwd_pre: per row, -D_i (fp32) and LSE_i * log2(e) into the workspace.
//  2. bwd_dkdv: one workgroup of eight wavefronts per (batch*head, block of
//     128 keys), walking the query blocks of 64 rows (causal: from the
//     diagonal on). K and V of the block stay in LDS; each wave owns 32 keys x
//     32 queries of every block and keeps partial dK^T, dV^T in MFMA
//     accumulators. Per block: S = Q K^T and dP = dO V^T with the key index
//     across lanes and the query index in registers, P and dS in registers,
//     then dV^T += dO^T P and dK^T += Q^T dS with dO^T and Q^T read straight
//     out of the row-major Q / dO tiles by transposing LDS reads. The two
//     waves sharing a key group sum their partials through LDS at the end.
//  3. bwd_dq: one workgroup per (batch*head, block of 256 queries, eight
//     wavefronts; 128 queries and four wavefronts when a launch would have
//     fewer than 256 such workgroups, and at head dim 256), shaped like the
//     forward: Q and dO rows of the wave's 32 queries stay in
//     registers, K/V tiles stream through LDS; per tile S^T = K Q^T,
//     dP^T = V dO^T, P^T and dS^T with the query across lanes, and
//     dQ^T += K^T dS^T with K^T read transposed out of the K tile and dS^T
//     used straight from registers.
// dQ is computed by its own pass instead of float atomics from the dK/dV
// pass: two more contractions (7 instead of 5) but no read-modify-write
// traffic through memory, and every output is deterministic. (Float atomic
// adds are performed past the XCD's L2, at ~1.3 TB/s of payload: the dQ
// partials of a one-pass design alone took longer than this whole pass on
// B8 H16 N4096 d128 causal, 1.7 ms with 256-key blocks against 0.75 ms.)
// Q, dO, K and V tiles go HBM -> LDS with global_load_lds_dwordx4 into
// double-buffered, XOR-swizzled (tile_swz) row-major buffers.

#include "fa_device.h"
#include "fa_launch.h"

// Head dim 256 runs one wave per SIMD: no partner wave covers the LDS
// latency, so its operand reads run kPf256 MFMA units ahead (B1 H32 N8192:
// dQ -9 %, causal dK/dV -7 %, non-causal dK/dV -1 % against the compiler's own
// order; one ahead was slower than the compiler's order)
constexpr int kPf256 = 4;

namespace fa {
namespace {

typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

template <typename V8>
__device__ __forceinline__ V8 tr_read8(const char* base, int off_lo, int off_hi) {
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + off_lo));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + off_hi));
    const s16x4 w[2] = {lo, hi};
    V8 a;
    __builtin_memcpy(&a, w, sizeof(a));
    return a;
}

// ---------------------------------------------------------------- 1. D and LSE2
template <typename T, int D>
__global__ void __launch_bounds__(256)
bwd_pre_kernel(const T* __restrict__ O, const T* __restrict__ dO, const float* __restrict__ lse,
               float* __restrict__ delta, float* __restrict__ lse2, int rows, float d_mul) {
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
    }
#pragma unroll
    for (int off = TPR / 2; off > 0; off >>= 1) s += __shfl_xor(s, off, TPR);
    if (row < rows && part == 0) {
        delta[row] = -(s * d_mul);  // stored negated: it seeds the dP accumulators
        lse2[row] = lse[row] * kLog2e;
    }
}

// ---------------------------------------------------------------- 2. dK, dV
// Eight wavefronts per workgroup, two per SIMD: wave w owns key group
// kg = w % 4 (32 keys) and query subtile qs = w / 4 (32 of the block's 64
// queries). K and V of the block's 128 keys sit in LDS for the whole kernel
// and are read as MFMA B operands; each wave keeps partial dK^T, dV^T for its
// keys over its half of the queries, and the two halves are summed through
// LDS at the end.
template <int D>
struct DkdvTile {
    static constexpr int BN = 128;               // keys per workgroup (4 key groups x 32)
    static constexpr int BM = 64;                // queries per step (2 subtiles x 32)
    static constexpr int NT = 512;               // 8 waves
    static constexpr int ROWB = 2 * D;
    static constexpr int QTILEB = BM * ROWB;     // bytes of one Q (or dO) tile
    static constexpr int KTILEB = BN * ROWB;     // bytes of the K (or V) block
    static constexpr int NLOADQ = QTILEB / (NT * 16);
    static constexpr int NLOADK = KTILEB / (NT * 16);
    static constexpr int KS = D / 16;
    static constexpr int DB = D / 32;
    static constexpr int PARTB = 32 * D * 4;     // bytes of one key group's fp32 partial
};

template <typename T, int D, bool CAUSAL>
struct DkdvWave {
    using C = DkdvTile<D>;
    using V8 = typename Vec<T>::x8;
    using V4 = typename Vec<T>::x4;

    const T* Qh;
    const T* dOh;
    const float* lse2h;
    const float* delh;
    int N, tid, lane, wave, l32, h, kg, qs, key0, key;
    float c;
    int ldq_row[C::NLOADQ], ldq_col[C::NLOADQ];
    unsigned ldq_off[C::NLOADQ];     // byte offset of this thread's 16 bytes within a full tile
    int roff[C::KS];                 // 16-byte row reads of Q / dO rows 32 qs + l32
    int koff[C::KS];                 // 16-byte row reads of K / V rows 32 kg + l32 (B operands)
    int toff[2][C::DB];              // transposing reads [half][b] (query group 0; +16 rows for g2 = 1)
    f32x16 dkacc[C::DB], dvacc[C::DB];  // partial dK^T, dV^T: head dim in registers, key = lane

    __device__ __forceinline__ void init(const T* Qh_, const T* dOh_, const float* lse2h_,
                                         const float* delh_, int N_, int kb, float c_) {
        Qh = Qh_;
        dOh = dOh_;
        lse2h = lse2h_;
        delh = delh_;
        N = N_;
        c = c_;
        tid = threadIdx.x;
        lane = tid & 63;
        wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches below
        l32 = lane & 31;
        h = lane >> 5;
        kg = wave & 3;
        qs = wave >> 2;
        key0 = kb * C::BN + 32 * kg;
        key = key0 + l32;
#pragma unroll
        for (int i = 0; i < C::NLOADQ; ++i) {
            const int byte = i * (C::NT * 16) + tid * 16;
            const int r = byte / C::ROWB, p = (byte % C::ROWB) / 16;
            ldq_row[i] = r;
            ldq_col[i] = (p ^ tile_swz<D>(r)) * 8;
            ldq_off[i] = (unsigned)(r * D + ldq_col[i]) * 2u;
        }
#pragma unroll
        for (int s = 0; s < C::KS; ++s) {
            roff[s] = tile_off<D>(32 * qs + l32, 16 * s + 8 * h);
            koff[s] = tile_off<D>(32 * kg + l32, 16 * s + 8 * h);
        }
        // transposing reads: this lane supplies row 32 qs + 16 g2 + 8 half + 4 h +
        // (lane % 16) / 4 and head dims 32 b + 16 ((lane / 16) % 2) + 4 (lane % 4);
        // it receives head dim 32 b + lane % 32 at queries 32 qs + 16 g2 + 8 half
        // + 4 h + 0..3, the order of registers 8 g2 + 4 half + 0..3 of the
        // score accumulator.
        const int src_r = 4 * h + (lane & 15) / 4;
        const int src_d = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
            for (int b = 0; b < C::DB; ++b)
                toff[hf][b] = tile_off<D>(32 * qs + 8 * hf + src_r, 32 * b + src_d);
#pragma unroll
        for (int b = 0; b < C::DB; ++b) {
            dkacc[b] = f32x16{};
            dvacc[b] = f32x16{};
        }
    }

    // All rows of the key block into the K / V tiles (rows past N re-read N-1).
    __device__ __forceinline__ void issue_kv(const T* Kh, const T* Vh, int kbase, char* sK,
                                             char* sV) const {
#pragma unroll
        for (int i = 0; i < C::NLOADK; ++i) {
            const int byte = i * (C::NT * 16) + tid * 16;
            const int r = byte / C::ROWB, p = (byte % C::ROWB) / 16;
            const size_t row = (size_t)min(kbase + r, N - 1) * D + (p ^ tile_swz<D>(r)) * 8;
            const int o = i * (C::NT * 16) + wave * 1024;
            __builtin_amdgcn_global_load_lds(Kh + row, sK + o, 16, 0, 0);
            __builtin_amdgcn_global_load_lds(Vh + row, sV + o, 16, 0, 0);
        }
    }

    // Q and dO rows [qbase, qbase + BM) and their LSE2 / D into one buffer set.
    __device__ __forceinline__ void issue(int qbase, char* sQd, char* sGd, float* sLd,
                                          float* sDd) const {
        if (qbase + C::BM <= N) {  // whole tile in range: one add per 16-byte load pair
            const unsigned base = (unsigned)qbase * (D * 2u);
            const char* qb = reinterpret_cast<const char*>(Qh);
            const char* gb = reinterpret_cast<const char*>(dOh);
#pragma unroll
            for (int i = 0; i < C::NLOADQ; ++i) {
                const unsigned off = base + ldq_off[i];
                const int o = i * (C::NT * 16) + wave * 1024;
                __builtin_amdgcn_global_load_lds(qb + off, sQd + o, 16, 0, 0);
                __builtin_amdgcn_global_load_lds(gb + off, sGd + o, 16, 0, 0);
            }
            if (wave == 0) __builtin_amdgcn_global_load_lds(lse2h + qbase + lane, sLd, 4, 0, 0);
            if (wave == 1) __builtin_amdgcn_global_load_lds(delh + qbase + lane, sDd, 4, 0, 0);
            return;
        }
#pragma unroll
        for (int i = 0; i < C::NLOADQ; ++i) {
            const size_t row = (size_t)min(qbase + ldq_row[i], N - 1) * D;
            const int o = i * (C::NT * 16) + wave * 1024;
            __builtin_amdgcn_global_load_lds(Qh + row + ldq_col[i], sQd + o, 16, 0, 0);
            __builtin_amdgcn_global_load_lds(dOh + row + ldq_col[i], sGd + o, 16, 0, 0);
        }
        const int r = min(qbase + lane, N - 1);
        if (wave == 0) __builtin_amdgcn_global_load_lds(lse2h + r, sLd, 4, 0, 0);
        if (wave == 1) __builtin_amdgcn_global_load_lds(delh + r, sDd, 4, 0, 0);
    }

    // P = 2^(s c - LSE2), dS = P (dP - D) with pacc already holding dP - D;
    // masked entries get P = 0
    template <bool MASK>
    __device__ __forceinline__ void softmax(f32x16& sacc, f32x16& pacc, const float* sL,
                                            int qb0) const {
        const int lo = key - qb0 - 4 * h;   // causal-visible iff const(r) >= lo
        const int hi = N - qb0 - 4 * h;     // query < N iff const(r) < hi
        const bool kvalid = key < N;
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            const f32x4 lq = *reinterpret_cast<const f32x4*>(sL + 32 * qs + 8 * r4 + 4 * h);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 4 * r4 + i;
                float l2 = lq[i];
                if (MASK) {
                    const int cr = 8 * r4 + i;
                    const bool vis = kvalid && cr < hi && (!CAUSAL || cr >= lo);
                    if (!vis) l2 = INFINITY;
                }
                const float p = fast_exp2(fmaf(sacc[r], c, -l2));
                sacc[r] = p;
                pacc[r] = p * pacc[r];
            }
        }
    }

    __device__ __forceinline__ void step(int ib, int nqb, const char* sK, const char* sV,
                                         const char* sQ, const char* sG, const float* sL,
                                         const float* sD, char* nQ, char* nG, float* nL,
                                         float* nD) {
        const int qbase = ib * C::BM;
        __builtin_amdgcn_s_waitcnt(kVmcntZero);
        __syncthreads();
        if (!kSerialStaging && ib + 1 < nqb) issue(qbase + C::BM, nQ, nG, nL, nD);
        const int qb0 = qbase + 32 * qs;  // first query of this wave's subtile
        if (CAUSAL && key0 > qb0 + 31) return;  // every query of the subtile precedes every key

        // S = Q K^T and dP - D = dO V^T - D (lane = key, register r = query
        // qb0 + acc_row(r, h)); the dP accumulators start from -D of their query
        f32x16 sacc = f32x16{}, pacc;
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            const f32x4 nd = *reinterpret_cast<const f32x4*>(sD + 32 * qs + 8 * r4 + 4 * h);
#pragma unroll
            for (int i = 0; i < 4; ++i) pacc[4 * r4 + i] = nd[i];
        }
        // operand reads run PF k-steps ahead of their MFMAs (rotating registers,
        // order kept by scheduling fences) to cover the LDS latency; two ahead
        // measured 3 % faster than the compiler's own order on the causal
        // 4K and non-causal 8K shapes, three ahead slower
        constexpr int PF = 2;
        V8 oq[PF], ok[PF], og[PF], ov[PF];
#pragma unroll
        for (int s = 0; s < PF; ++s) {
            oq[s] = *reinterpret_cast<const V8*>(sQ + roff[s]);
            ok[s] = *reinterpret_cast<const V8*>(sK + koff[s]);
            og[s] = *reinterpret_cast<const V8*>(sG + roff[s]);
            ov[s] = *reinterpret_cast<const V8*>(sV + koff[s]);
        }
#pragma unroll
        for (int s = 0; s < C::KS; ++s) {
            const int bf = s % PF;
            sacc = mfma32(oq[bf], ok[bf], sacc);
            pacc = mfma32(og[bf], ov[bf], pacc);
            if (s + PF < C::KS) {
                oq[bf] = *reinterpret_cast<const V8*>(sQ + roff[s + PF]);
                ok[bf] = *reinterpret_cast<const V8*>(sK + koff[s + PF]);
                og[bf] = *reinterpret_cast<const V8*>(sG + roff[s + PF]);
                ov[bf] = *reinterpret_cast<const V8*>(sV + koff[s + PF]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        const bool need_mask = key0 + 31 >= N || qb0 + 31 >= N || (CAUSAL && key0 + 31 > qb0);
        // wave-uniform: only the diagonal and ragged-edge steps pay for the
        // per-element mask
        if (need_mask)
            softmax<true>(sacc, pacc, sL, qb0);
        else
            softmax<false>(sacc, pacc, sL, qb0);
        V8 pf[2], sf[2];
        pf[0] = pack8<T>(sacc, 0);
        pf[1] = pack8<T>(sacc, 8);
        sf[0] = pack8<T>(pacc, 0);
        sf[1] = pack8<T>(pacc, 8);
        // dV^T += dO^T P and dK^T += Q^T dS (unit u: g2 = u / DB, b = u % DB),
        // the transposed operands read PT units ahead
        constexpr int NC = 2 * C::DB, PT = 2;
        V8 ta[PT], tq[PT];
        auto tr_unit = [&](int u, V8& at, V8& aq) {
            const int g2 = u / C::DB, b = u % C::DB;
            const int o0 = toff[0][b] + g2 * 16 * C::ROWB, o1 = toff[1][b] + g2 * 16 * C::ROWB;
            at = tr_read8<V8>(sG, o0, o1);
            aq = tr_read8<V8>(sQ, o0, o1);
        };
#pragma unroll
        for (int u = 0; u < PT; ++u) tr_unit(u, ta[u], tq[u]);
#pragma unroll
        for (int u = 0; u < NC; ++u) {
            const int g2 = u / C::DB, b = u % C::DB, bf = u % PT;
            dvacc[b] = mfma32(ta[bf], pf[g2], dvacc[b]);
            dkacc[b] = mfma32(tq[bf], sf[g2], dkacc[b]);
            if (u + PT < NC) tr_unit(u + PT, ta[bf], tq[bf]);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // Partials of query subtile 1 -> LDS (dK into pk, dV into pv, one region per key group).
    __device__ __forceinline__ void put_partials(char* pk, char* pv) const {
#pragma unroll
        for (int b = 0; b < C::DB; ++b)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int o = ((b * 4 + r4) * 64 + lane) * 16;
                *reinterpret_cast<f32x4*>(pk + o) =
                    f32x4{dkacc[b][4 * r4], dkacc[b][4 * r4 + 1], dkacc[b][4 * r4 + 2], dkacc[b][4 * r4 + 3]};
                *reinterpret_cast<f32x4*>(pv + o) =
                    f32x4{dvacc[b][4 * r4], dvacc[b][4 * r4 + 1], dvacc[b][4 * r4 + 2], dvacc[b][4 * r4 + 3]};
            }
    }

    __device__ __forceinline__ void add_partials(const char* pk, const char* pv) {
#pragma unroll
        for (int b = 0; b < C::DB; ++b)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int o = ((b * 4 + r4) * 64 + lane) * 16;
                const f32x4 a = *reinterpret_cast<const f32x4*>(pk + o);
                const f32x4 v = *reinterpret_cast<const f32x4*>(pv + o);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    dkacc[b][4 * r4 + i] += a[i];
                    dvacc[b][4 * r4 + i] += v[i];
                }
            }
    }

    __device__ __forceinline__ void finish(T* dKh, T* dVh, float scale) {
        if (key >= N) return;
        T* dkr = dKh + (size_t)key * D;
        T* dvr = dVh + (size_t)key * D;
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
};

template <typename T, int D, bool CAUSAL>
__global__ void __launch_bounds__(512, 1)
bwd_dkdv_kernel(const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
                const T* __restrict__ dO, const float* __restrict__ lse2,
                const float* __restrict__ delta, T* __restrict__ dK, T* __restrict__ dV, int BH,
                int N, int nkb, float scale, float c) {
    using C = DkdvTile<D>;
    // The Q / dO tiles (more strictly aligned, so the compiler places them
    // first) sit below 64 KiB of LDS: the per-step reads then carry the
    // buffer base in the instruction's immediate offset instead of a VALU add.
    __shared__ __attribute__((aligned(4096))) char sQG0[2 * C::QTILEB];
    __shared__ __attribute__((aligned(4096))) char sQG1[2 * C::QTILEB];
    __shared__ __attribute__((aligned(1024))) char sK[C::KTILEB];
    __shared__ __attribute__((aligned(1024))) char sV[C::KTILEB];
    char* const sQ0 = sQG0;
    char* const sG0 = sQG0 + C::QTILEB;
    char* const sQ1 = sQG1;
    char* const sG1 = sQG1 + C::QTILEB;
    __shared__ __attribute__((aligned(256))) float sL0[C::BM];
    __shared__ __attribute__((aligned(256))) float sL1[C::BM];
    __shared__ __attribute__((aligned(256))) float sD0[C::BM];
    __shared__ __attribute__((aligned(256))) float sD1[C::BM];
    static_assert(2 * C::PARTB <= C::KTILEB && C::PARTB <= C::QTILEB,
                  "partial sums must fit the K/V and Q/dO tiles");

    int bh, kb;
    if (CAUSAL) {
        // groups of at most two heads per XCD: the bytes fetched past L2 drop
        // from 1.7x to 1.0x the algorithmic bytes on B8 H16 N4096 at equal time
        // (four heads' K, V and Q, dO tiles overflow the XCD's L2)
        causal_block(blockIdx.x, nkb, BH, bh, kb, 2);
        kb = nkb - 1 - kb;  // small kb has the most query blocks
    } else {
        const int L = xcd_remap(blockIdx.x, BH * nkb);
        bh = L / nkb;
        kb = L % nkb;
    }
    const size_t head = (size_t)bh * N * D;
    const size_t rowbase = (size_t)bh * N;

    DkdvWave<T, D, CAUSAL> w;
    w.init(Q + head, dO + head, lse2 + rowbase, delta + rowbase, N, kb, c);
    const int nqb = (N + C::BM - 1) / C::BM;
    const int i0 = CAUSAL ? (kb * C::BN) / C::BM : 0;
    w.issue_kv(K + head, V + head, kb * C::BN, sK, sV);
    w.issue(i0 * C::BM, sQ0, sG0, sL0, sD0);
    if constexpr (kSerialStaging) {
        for (int ib = i0; ib < nqb; ++ib) {
            w.step(ib, nqb, sK, sV, sQ0, sG0, sL0, sD0, sQ0, sG0, sL0, sD0);
            __syncthreads();
            if (ib + 1 < nqb) w.issue((ib + 1) * C::BM, sQ0, sG0, sL0, sD0);
        }
    } else {
        for (int ib = i0; ib < nqb; ib += 2) {
            w.step(ib, nqb, sK, sV, sQ0, sG0, sL0, sD0, sQ1, sG1, sL1, sD1);
            if (ib + 1 < nqb)
                w.step(ib + 1, nqb, sK, sV, sQ1, sG1, sL1, sD1, sQ0, sG0, sL0, sD0);
        }
    }
    // sum the two query halves: subtile-1 waves park their partials in LDS
    __syncthreads();
    char* pk = (w.kg < 2 ? sK : sV) + (w.kg & 1) * C::PARTB;
    char* pv = w.kg == 0 ? sQ0 : w.kg == 1 ? sQ1 : w.kg == 2 ? sG0 : sG1;
    if (w.qs == 1) w.put_partials(pk, pv);
    __syncthreads();
    if (w.qs == 0) {
        w.add_partials(pk, pv);
        w.finish(dK + head, dV + head, scale);
    }
}

// ---------------------------------------------------------------- 2b. dK or dV, d = 256
// At head dim 256 the eight-wave pass does not fit: its dK and dV
// accumulators alone would take every register of a wave. Here four waves,
// one per SIMD, each own 32 keys of a 128-key block with their K (and V) rows
// in registers and walk the query blocks 32 rows at a time; one launch
// accumulates dV = P^T dO, a second one dK = scale dS^T Q (recomputing S and
// computing dP), so a wave holds one accumulator of 32 keys x 256 dims.
template <int D>
struct Dkdv1Tile {
    static constexpr int BN = 128;               // keys per workgroup (4 waves x 32)
    static constexpr int BM = 32;                // queries per step
    static constexpr int NT = 256;
    static constexpr int ROWB = 2 * D;
    static constexpr int QTILEB = BM * ROWB;     // bytes of one Q (or dO) tile
    static constexpr int NLOADQ = QTILEB / (NT * 16);
    static constexpr int KS = D / 16;
    static constexpr int DB = D / 32;
    static_assert(NLOADQ >= 1 && QTILEB % (NT * 16) == 0, "tile must split into whole loads");
};

template <typename T, int D, bool CAUSAL, bool DK>
struct Dkdv1Wave {
    using C = Dkdv1Tile<D>;
    using V8 = typename Vec<T>::x8;
    using V4 = typename Vec<T>::x4;

    const T* Qh;
    const T* dOh;
    const float* lse2h;
    const float* delh;
    int N, tid, lane, wave, l32, h, key0, key;
    float c;
    V8 kf[C::KS], vf[DK ? C::KS : 1];   // B operands: K (and V) rows of this lane's key
    int ld_row[C::NLOADQ];
    unsigned ld_cb[C::NLOADQ];          // byte offset of this thread's 16 bytes within a row
    f32x16 acc[C::DB];                  // dK^T or dV^T: head dim in registers, key = lane

    __device__ __forceinline__ void init(const T* Qh_, const T* Kh, const T* Vh, const T* dOh_,
                                         const float* lse2h_, const float* delh_, int N_, int kb,
                                         float c_) {
        Qh = Qh_;
        dOh = dOh_;
        lse2h = lse2h_;
        delh = delh_;
        N = N_;
        c = c_;
        tid = threadIdx.x;
        lane = tid & 63;
        wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        l32 = lane & 31;
        h = lane >> 5;
        key0 = kb * C::BN + 32 * wave;
        key = key0 + l32;
        const int kr = min(key, N - 1);
        const V8* ks = reinterpret_cast<const V8*>(Kh + (size_t)kr * D + 8 * h);
#pragma unroll
        for (int s = 0; s < C::KS; ++s) kf[s] = ks[2 * s];
        if (DK) {
            const V8* vs = reinterpret_cast<const V8*>(Vh + (size_t)kr * D + 8 * h);
#pragma unroll
            for (int s = 0; s < C::KS; ++s) vf[s] = vs[2 * s];
        }
#pragma unroll
        for (int i = 0; i < C::NLOADQ; ++i) {
            const int byte = i * (C::NT * 16) + tid * 16;
            const int r = byte / C::ROWB, p = (byte % C::ROWB) / 16;
            ld_row[i] = r;
            ld_cb[i] = (unsigned)(p ^ tile_swz<D>(r)) * 16u;
        }
#pragma unroll
        for (int b = 0; b < C::DB; ++b) acc[b] = f32x16{};
    }

    // Q and dO rows [qbase, qbase + BM) and their LSE2 / D into one buffer set
    // (the 4-byte loads fill 64 entries; rows past the block read clamped rows).
    __device__ __forceinline__ void issue(int qbase, char* sQd, char* sGd, float* sLd,
                                          float* sDd) const {
        // 32-bit byte offsets from the head's base (a head holds < 2^31
        // elements): no 64-bit address per load
        const char* qb = reinterpret_cast<const char*>(Qh);
        const char* gb = reinterpret_cast<const char*>(dOh);
#pragma unroll
        for (int i = 0; i < C::NLOADQ; ++i) {
            const unsigned off = (unsigned)min(qbase + ld_row[i], N - 1) * (D * 2u) + ld_cb[i];
            const int o = i * (C::NT * 16) + wave * 1024;
            __builtin_amdgcn_global_load_lds(qb + off, sQd + o, 16, 0, 0);
            __builtin_amdgcn_global_load_lds(gb + off, sGd + o, 16, 0, 0);
        }
        const int r = min(qbase + lane, N - 1);
        if (wave == 0) __builtin_amdgcn_global_load_lds(lse2h + r, sLd, 4, 0, 0);
        if (DK && wave == 1) __builtin_amdgcn_global_load_lds(delh + r, sDd, 4, 0, 0);
    }

    // P = 2^(s c - LSE2) into sacc, or dS = P (dP - D) into pacc (which holds
    // dP - D); masked entries get P = 0. MODE 0: no mask, 1: mask, 2: mask
    // if `masked` (one code path, no branch).
    template <int MODE>
    __device__ __forceinline__ void softmax(f32x16& sacc, f32x16& pacc, const float* sL,
                                            int qbase, bool masked) const {
        const int lo = key - qbase - 4 * h;   // causal-visible iff const(r) >= lo
        const int hi = N - qbase - 4 * h;     // query < N iff const(r) < hi
        const bool kvalid = key < N;
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            const f32x4 lq = *reinterpret_cast<const f32x4*>(sL + 8 * r4 + 4 * h);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 4 * r4 + i;
                float l2 = lq[i];
                if (MODE == 1 || (MODE == 2 && masked)) {
                    const int cr = 8 * r4 + i;
                    const bool vis = kvalid && cr < hi && (!CAUSAL || cr >= lo);
                    if (!vis) l2 = INFINITY;
                }
                const float p = fast_exp2(fmaf(sacc[r], c, -l2));
                if (DK) pacc[r] = p * pacc[r];
                else sacc[r] = p;
            }
        }
    }

    __device__ __forceinline__ void step(int ib, int nqb, const char* sQ, const char* sG,
                                         const float* sL, const float* sD, char* nQ, char* nG,
                                         float* nL, float* nD) {
        const int qbase = ib * C::BM;
        __builtin_amdgcn_s_waitcnt(kVmcntZero);
        __syncthreads();
        if (!kSerialStaging && ib + 1 < nqb) issue(qbase + C::BM, nQ, nG, nL, nD);
        if (CAUSAL && key0 > qbase + C::BM - 1) return;  // every query of the block precedes every key

        // S = Q K^T (and dP - D = dO V^T - D, the dP accumulators starting from
        // -D of their query): lane = key, register r = query qbase + acc_row(r, h)
        f32x16 sacc = f32x16{}, pacc = f32x16{};
        if (DK) {
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const f32x4 nd = *reinterpret_cast<const f32x4*>(sD + 8 * r4 + 4 * h);
#pragma unroll
                for (int i = 0; i < 4; ++i) pacc[4 * r4 + i] = nd[i];
            }
        }
        // one wave per SIMD: the Q (and dO) row operands are read PF k-steps
        // ahead of their MFMAs, order kept by scheduling fences
        constexpr int PF = kPf256;
        V8 oq[PF], og[PF];
        auto rows = [&](int s, V8& aq, V8& ag) {
            const int ro = tile_off<D>(l32, 16 * s + 8 * h);
            aq = *reinterpret_cast<const V8*>(sQ + ro);
            if (DK) ag = *reinterpret_cast<const V8*>(sG + ro);
        };
#pragma unroll
        for (int s = 0; s < PF; ++s) rows(s, oq[s], og[s]);
#pragma unroll
        for (int s = 0; s < C::KS; ++s) {
            sacc = mfma32(oq[s % PF], kf[s], sacc);
            if (DK) pacc = mfma32(og[s % PF], vf[DK ? s : 0], pacc);
            if (s + PF < C::KS) rows(s + PF, oq[s % PF], og[s % PF]);
            __builtin_amdgcn_sched_barrier(0);
        }
        // causal: a wave-uniform branch, so only diagonal and ragged-edge steps
        // pay for the mask; non-causal keeps one path (a second one makes the
        // dK launch spill)
        const bool need_mask = key0 + 31 >= N || qbase + 31 >= N || (CAUSAL && key0 + 31 > qbase);
        if (!CAUSAL)
            softmax<2>(sacc, pacc, sL, qbase, need_mask);
        else if (need_mask)
            softmax<1>(sacc, pacc, sL, qbase, true);
        else
            softmax<0>(sacc, pacc, sL, qbase, false);
        V8 op[2];
        op[0] = pack8<T>(DK ? pacc : sacc, 0);
        op[1] = pack8<T>(DK ? pacc : sacc, 8);
        // dV^T += dO^T P or dK^T += Q^T dS, dO^T / Q^T read transposed: this lane
        // supplies row 16 g2 + 8 half + 4 h + (lane % 16) / 4, head dims 32 b +
        // 16 ((lane / 16) % 2) + 4 (lane % 4); it receives head dim 32 b + lane %
        // 32 at queries 16 g2 + 8 half + 4 h + 0..3 (registers 8 g2 + 4 half + 0..3)
        const char* src = DK ? sQ : sG;
        const int src_r = 4 * h + (lane & 15) / 4;
        const int src_d = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
        auto tr = [&](int u) {  // unit u: g2 = u / DB, b = u % DB
            const int g2 = u / C::DB, b = u % C::DB;
            return tr_read8<V8>(src, tile_off<D>(16 * g2 + src_r, 32 * b + src_d),
                                tile_off<D>(16 * g2 + 8 + src_r, 32 * b + src_d));
        };
        constexpr int NC = 2 * C::DB;
        V8 ta[PF];
#pragma unroll
        for (int u = 0; u < PF; ++u) ta[u] = tr(u);
#pragma unroll
        for (int u = 0; u < NC; ++u) {
            acc[u % C::DB] = mfma32(ta[u % PF], op[u / C::DB], acc[u % C::DB]);
            if (u + PF < NC) ta[u % PF] = tr(u + PF);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    __device__ __forceinline__ void finish(T* outh, float mul) const {
        if (key >= N) return;
        T* row = outh + (size_t)key * D;
#pragma unroll
        for (int b = 0; b < C::DB; ++b)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                V4 w;
#pragma unroll
                for (int i = 0; i < 4; ++i) w[i] = (T)(acc[b][4 * r4 + i] * mul);
                *reinterpret_cast<V4*>(row + 32 * b + 8 * r4 + 4 * h) = w;
            }
    }
};

template <typename T, int D, bool CAUSAL, bool DK>
__global__ void __launch_bounds__(256, 1)
bwd_dkdv1_kernel(const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
                 const T* __restrict__ dO, const float* __restrict__ lse2,
                 const float* __restrict__ delta, T* __restrict__ out, int BH, int N, int nkb,
                 float scale, float c) {
    using C = Dkdv1Tile<D>;
    __shared__ __attribute__((aligned(1024))) char sQ0[C::QTILEB];
    __shared__ __attribute__((aligned(1024))) char sQ1[C::QTILEB];
    __shared__ __attribute__((aligned(1024))) char sG0[C::QTILEB];
    __shared__ __attribute__((aligned(1024))) char sG1[C::QTILEB];
    __shared__ __attribute__((aligned(256))) float sL0[64];
    __shared__ __attribute__((aligned(256))) float sL1[64];
    __shared__ __attribute__((aligned(256))) float sD0[64];
    __shared__ __attribute__((aligned(256))) float sD1[64];

    int bh, kb;
    if (CAUSAL) {
        causal_block(blockIdx.x, nkb, BH, bh, kb);
        kb = nkb - 1 - kb;  // small kb has the most query blocks
    } else {
        const int L = xcd_remap(blockIdx.x, BH * nkb);
        bh = L / nkb;
        kb = L % nkb;
    }
    const size_t head = (size_t)bh * N * D;
    const size_t rowbase = (size_t)bh * N;

    Dkdv1Wave<T, D, CAUSAL, DK> w;
    w.init(Q + head, K + head, V + head, dO + head, lse2 + rowbase, delta + rowbase, N, kb, c);
    const int nqb = (N + C::BM - 1) / C::BM;
    const int i0 = CAUSAL ? (kb * C::BN) / C::BM : 0;
    w.issue(i0 * C::BM, sQ0, sG0, sL0, sD0);
    if constexpr (kSerialStaging) {
        for (int ib = i0; ib < nqb; ++ib) {
            w.step(ib, nqb, sQ0, sG0, sL0, sD0, sQ0, sG0, sL0, sD0);
            __syncthreads();
            if (ib + 1 < nqb) w.issue((ib + 1) * C::BM, sQ0, sG0, sL0, sD0);
        }
    } else {
        for (int ib = i0; ib < nqb; ib += 2) {
            w.step(ib, nqb, sQ0, sG0, sL0, sD0, sQ1, sG1, sL1, sD1);
            if (ib + 1 < nqb) w.step(ib + 1, nqb, sQ1, sG1, sL1, sD1, sQ0, sG0, sL0, sD0);
        }
    }
    w.finish(out + head, DK ? scale : 1.f);
}

// ---------------------------------------------------------------- 3. dQ
template <int D, int NW>
struct DqTile {
    static constexpr int BM = 32 * NW;           // queries per workgroup (NW waves x 32)
    static constexpr int BN = 64;                // keys per tile
    static constexpr int NT = 64 * NW;
    static constexpr int ROWB = 2 * D;
    static constexpr int TILEB = BN * ROWB;
    static constexpr int NLOAD = TILEB / (NT * 16);
    static constexpr int KS = D / 16;
    static constexpr int DB = D / 32;
};

template <typename T, int D, bool CAUSAL, int NW>
struct DqWave {
    using C = DqTile<D, NW>;
    using V8 = typename Vec<T>::x8;
    using V4 = typename Vec<T>::x4;

    const T* Kh;
    const T* Vh;
    int N, nkt, tid, lane, wave, l32, h, q0, qrow;
    float c, lse2, del;             // del: -D of this lane's query
    V8 qf[C::KS], gf[C::KS];        // B operands: Q and dO rows of this lane's query
    int ld_row[C::NLOAD];
    unsigned ld_off[C::NLOAD];      // byte offset of this thread's 16 bytes within a full tile
    int roff[C::KS];                // 16-byte row reads of K / V (key l32; +32 rows for c2 = 1)
    int toff[2][C::DB];             // transposing reads of K [half][b] (g = 0; +16 g rows)
    f32x16 dqacc[C::DB];            // dQ^T: head dim in registers, query = lane
    // -D of this lane's query in every register, the seed of the dP^T
    // accumulators (saves the subtraction per element); kept where its 16
    // registers fit without spilling
    static constexpr bool SEED = D <= 64 || (D == 128 && NW == 8);
    f32x16 dinit;

    __device__ __forceinline__ void init(const T* Qh, const T* Kh_, const T* Vh_, const T* dOh,
                                         const float* lse2h, const float* delh, int N_, int qb,
                                         float c_) {
        Kh = Kh_;
        Vh = Vh_;
        N = N_;
        c = c_;
        tid = threadIdx.x;
        lane = tid & 63;
        wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        l32 = lane & 31;
        h = lane >> 5;
        q0 = qb * C::BM + 32 * wave;
        qrow = q0 + l32;
        const int qr = min(qrow, N - 1);
        const V8* qs = reinterpret_cast<const V8*>(Qh + (size_t)qr * D + 8 * h);
        const V8* gs = reinterpret_cast<const V8*>(dOh + (size_t)qr * D + 8 * h);
#pragma unroll
        for (int s = 0; s < C::KS; ++s) {
            qf[s] = qs[2 * s];
            gf[s] = gs[2 * s];
        }
        lse2 = lse2h[qr];
        del = delh[qr];
        const int q_last = min(N, (qb + 1) * C::BM) - 1;
        nkt = CAUSAL ? (q_last / C::BN + 1) : (N + C::BN - 1) / C::BN;
#pragma unroll
        for (int i = 0; i < C::NLOAD; ++i) {
            const int byte = i * (C::NT * 16) + tid * 16;
            const int r = byte / C::ROWB, p = (byte % C::ROWB) / 16;
            ld_row[i] = r;
            ld_off[i] = (unsigned)(r * D + (p ^ tile_swz<D>(r)) * 8) * 2u;
        }
#pragma unroll
        for (int s = 0; s < C::KS; ++s) roff[s] = tile_off<D>(l32, 16 * s + 8 * h);
        // transposing reads of K: this lane supplies key 16 g + 8 half + 4 h +
        // (lane % 16) / 4, head dims 32 b + 16 ((lane / 16) % 2) + 4 (lane % 4);
        // it receives head dim 32 b + lane % 32 at keys 16 g + 8 half + 4 h + 0..3,
        // the key order of registers 8 (g % 2) + 4 half + 0..3 of dS^T subtile g / 2.
        const int src_r = 4 * h + (lane & 15) / 4;
        const int src_d = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
// the swizzle repeats every 16 rows: rows + 16 g are toff + 16 g rows
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
            for (int b = 0; b < C::DB; ++b)
                toff[hf][b] = tile_off<D>(8 * hf + src_r, 32 * b + src_d);
#pragma unroll
        for (int b = 0; b < C::DB; ++b) dqacc[b] = f32x16{};
#pragma unroll
        for (int r = 0; r < 16; ++r) dinit[r] = SEED ? del : 0.f;
    }

    __device__ __forceinline__ void issue(int kbase, char* sKd, char* sVd) const {
        if (kbase + C::BN <= N) {  // whole tile in range: one add per 16-byte load pair
            const unsigned base = (unsigned)kbase * (D * 2u);
            const char* kb = reinterpret_cast<const char*>(Kh);
            const char* vb = reinterpret_cast<const char*>(Vh);
#pragma unroll
            for (int i = 0; i < C::NLOAD; ++i) {
                const unsigned off = base + ld_off[i];
                const int o = i * (C::NT * 16) + wave * 1024;
                __builtin_amdgcn_global_load_lds(kb + off, sKd + o, 16, 0, 0);
                __builtin_amdgcn_global_load_lds(vb + off, sVd + o, 16, 0, 0);
            }
            return;
        }
        const char* kb = reinterpret_cast<const char*>(Kh);
        const char* vb = reinterpret_cast<const char*>(Vh);
#pragma unroll
        for (int i = 0; i < C::NLOAD; ++i) {
            // rows past N re-read row N - 1 (32-bit byte offsets, as above)
            const unsigned off = (unsigned)min(kbase + ld_row[i], N - 1) * (D * 2u) +
                                 (ld_off[i] - (unsigned)ld_row[i] * (D * 2u));
            const int o = i * (C::NT * 16) + wave * 1024;
            __builtin_amdgcn_global_load_lds(kb + off, sKd + o, 16, 0, 0);
            __builtin_amdgcn_global_load_lds(vb + off, sVd + o, 16, 0, 0);
        }
    }

    __device__ __forceinline__ void step(int kt, const char* kb, const char* vb, char* kn,
                                         char* vn) {
        const int kbase = kt * C::BN;
        __builtin_amdgcn_s_waitcnt(kVmcntZero);
        __syncthreads();
        if (!kSerialStaging && kt + 1 < nkt) issue(kbase + C::BN, kn, vn);
        if (CAUSAL && kbase > q0 + 31) return;
        if constexpr (D > 128 && !CAUSAL) {
            step_halves(kbase, kb, vb);
            return;
        }

        f32x16 s[2], dp[2];
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
            s[c2] = f32x16{};
            dp[c2] = dinit;
        }
        // K / V operand reads run PF units ahead of their MFMAs (unit t:
        // k-step t / 2, subtile t % 2), order kept by scheduling fences; one
        // ahead with the fences measured 1-2 % faster than the compiler's own
        // order, two ahead another 0.6-1.5 % (B8 H16 N4096 causal, B2 H32
        // N8192, d = 64; the eight-wave shape then needs all 256 registers,
        // without spilling)
        constexpr int NU = 2 * C::KS, PF = D > 128 ? kPf256 : 2;
        V8 ok[PF], ov[PF];
        auto kv_unit = [&](int t, V8& ak, V8& av) {
            const int o = roff[t >> 1] + (t & 1) * 32 * C::ROWB;
            ak = *reinterpret_cast<const V8*>(kb + o);
            av = *reinterpret_cast<const V8*>(vb + o);
        };
#pragma unroll
        for (int t = 0; t < PF; ++t) kv_unit(t, ok[t], ov[t]);
#pragma unroll
        for (int t = 0; t < NU; ++t) {
            const int ks = t >> 1, c2 = t & 1, bf = t % PF;
            s[c2] = mfma32(ok[bf], qf[ks], s[c2]);
            dp[c2] = mfma32(ov[bf], gf[ks], dp[c2]);
            if (t + PF < NU) kv_unit(t + PF, ok[bf], ov[bf]);
            __builtin_amdgcn_sched_barrier(0);
        }
        const bool need_mask = (kbase + C::BN > N) || (CAUSAL && kbase + C::BN - 1 > q0);
        if (need_mask) {
            const int lim = (CAUSAL ? min(qrow, N - 1) : N - 1) - kbase - 4 * h;
#pragma unroll
            for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (32 * c2 + 8 * (r >> 2) + (r & 3) > lim) s[c2][r] = -INFINITY;
        }
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float p = fast_exp2(fmaf(s[c2][r], c, -lse2));
                dp[c2][r] = SEED ? p * dp[c2][r] : p * (dp[c2][r] + del);  // dP - D; del holds -D
            }
        V8 sf[4];
        sf[0] = pack8<T>(dp[0], 0);
        sf[1] = pack8<T>(dp[0], 8);
        sf[2] = pack8<T>(dp[1], 0);
        sf[3] = pack8<T>(dp[1], 8);
        // dQ^T += K^T dS^T (unit u: key group g = u / DB, b = u % DB), the
        // transposed K operands read PT units ahead (two at d <= 128: 1.6-2.2 %
        // faster than one on B8 H16 N4096 causal and B2 H32 N8192, same
        // registers, bit-identical)
        constexpr int NC = 4 * C::DB, PT = D > 128 ? kPf256 : 2;
        V8 ta[PT];
#pragma unroll
        for (int u = 0; u < PT; ++u)
            ta[u] = tr_read8<V8>(kb + (u / C::DB) * 16 * C::ROWB, toff[0][u % C::DB],
                                 toff[1][u % C::DB]);
#pragma unroll
        for (int u = 0; u < NC; ++u) {
            const int g = u / C::DB, b = u % C::DB, bf = u % PT;
            dqacc[b] = mfma32(ta[bf], sf[g], dqacc[b]);
            if (u + PT < NC)
                ta[bf] = tr_read8<V8>(kb + ((u + PT) / C::DB) * 16 * C::ROWB,
                                      toff[0][(u + PT) % C::DB], toff[1][(u + PT) % C::DB]);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // Head dim 256 without the causal mask: the tile's two 32-key halves one
    // after the other, so that only one half's S^T / dP^T accumulators are
    // live beside the Q and dO operands and the dQ accumulators (384 of the
    // wave's 512 registers). Both halves at once spilled 208 bytes per lane
    // there (B1 H32 N8192: 6.4 ms, this order 3.7 ms); the causal kernel fits
    // either way and is 5 % faster with both halves at once.
    __device__ __forceinline__ void step_halves(int kbase, const char* kb, const char* vb) {
        const bool need_mask = (kbase + C::BN > N) || (CAUSAL && kbase + C::BN - 1 > q0);
        const int lim = (CAUSAL ? min(qrow, N - 1) : N - 1) - kbase - 4 * h;
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
            if (CAUSAL && kbase + 32 * c2 > q0 + 31) break;  // the half lies past every query
            f32x16 s = f32x16{}, dp = dinit;
            constexpr int PF = kPf256;  // operand reads PF k-steps ahead
            V8 ok[PF], ov[PF];
#pragma unroll
            for (int ks = 0; ks < PF; ++ks) {
                ok[ks] = *reinterpret_cast<const V8*>(kb + roff[ks] + c2 * 32 * C::ROWB);
                ov[ks] = *reinterpret_cast<const V8*>(vb + roff[ks] + c2 * 32 * C::ROWB);
            }
#pragma unroll
            for (int ks = 0; ks < C::KS; ++ks) {
                s = mfma32(ok[ks % PF], qf[ks], s);
                dp = mfma32(ov[ks % PF], gf[ks], dp);
                if (ks + PF < C::KS) {
                    ok[ks % PF] = *reinterpret_cast<const V8*>(kb + roff[ks + PF] + c2 * 32 * C::ROWB);
                    ov[ks % PF] = *reinterpret_cast<const V8*>(vb + roff[ks + PF] + c2 * 32 * C::ROWB);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            if (need_mask) {
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (32 * c2 + 8 * (r >> 2) + (r & 3) > lim) s[r] = -INFINITY;
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float p = fast_exp2(fmaf(s[r], c, -lse2));
                dp[r] = SEED ? p * dp[r] : p * (dp[r] + del);  // dP - D; del holds -D
            }
            const V8 sf0 = pack8<T>(dp, 0), sf1 = pack8<T>(dp, 8);
            auto tr = [&](int u) {  // unit u: g = u / DB, b = u % DB
                return tr_read8<V8>(kb + (2 * c2 + u / C::DB) * 16 * C::ROWB,
                                    toff[0][u % C::DB], toff[1][u % C::DB]);
            };
            V8 ta[PF];
#pragma unroll
            for (int u = 0; u < PF; ++u) ta[u] = tr(u);
#pragma unroll
            for (int u = 0; u < 2 * C::DB; ++u) {
                dqacc[u % C::DB] = mfma32(ta[u % PF], u < C::DB ? sf0 : sf1, dqacc[u % C::DB]);
                if (u + PF < 2 * C::DB) ta[u % PF] = tr(u + PF);
                __builtin_amdgcn_sched_barrier(0);
            }
            __builtin_amdgcn_sched_barrier(0);  // keep the halves apart
        }
    }

    __device__ __forceinline__ void finish(T* dQh, float scale) {
        if (qrow >= N) return;
        T* dst = dQh + (size_t)qrow * D;
#pragma unroll
        for (int b = 0; b < C::DB; ++b)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                V4 w;
#pragma unroll
                for (int i = 0; i < 4; ++i) w[i] = (T)(dqacc[b][4 * r4 + i] * scale);
                *reinterpret_cast<V4*>(dst + 32 * b + 8 * r4 + 4 * h) = w;
            }
    }
};

template <typename T, int D, bool CAUSAL, int NW>
__global__ void __launch_bounds__(64 * NW, (D > 128 || NW == 8) ? 1 : 2)
bwd_dq_kernel(const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
              const T* __restrict__ dO, const float* __restrict__ lse2,
              const float* __restrict__ delta, T* __restrict__ dQ, int BH, int N, int nqb,
              float scale, float c) {
    using C = DqTile<D, NW>;
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
    const size_t rowbase = (size_t)bh * N;

    DqWave<T, D, CAUSAL, NW> w;
    w.init(Q + head, K + head, V + head, dO + head, lse2 + rowbase, delta + rowbase, N, qb, c);
    w.issue(0, sK0, sV0);
    if constexpr (kSerialStaging) {
        for (int kt = 0; kt < w.nkt; ++kt) {
            w.step(kt, sK0, sV0, sK0, sV0);
            __syncthreads();
            if (kt + 1 < w.nkt) w.issue((kt + 1) * C::BN, sK0, sV0);
        }
    } else {
        for (int kt = 0; kt < w.nkt; kt += 2) {
            w.step(kt, sK0, sV0, sK1, sV1);
            if (kt + 1 < w.nkt) w.step(kt + 1, sK1, sV1, sK0, sV0);
        }
    }
    w.finish(dQ + head, scale);
}

template <typename T, int D, bool CAUSAL>
hipError_t launch_typed(const void* q, const void* k, const void* v, const void* o,
                        const float* lse, const void* dO, void* dq, void* dk, void* dv,
                        float* delta, float* lse2, int BH, int N, const BwdScales& sc, int stages,
                        hipStream_t stream) {
    const int rows = BH * N;
    const float c = sc.c;
    auto tq = static_cast<const T*>(q);
    auto tk = static_cast<const T*>(k);
    auto tv = static_cast<const T*>(v);
    auto tdo = static_cast<const T*>(dO);
    hipError_t e = hipSuccess;
    if (stages & 1) {
        const int threads = rows * (D / 8);
        hipLaunchKernelGGL((bwd_pre_kernel<T, D>), dim3((threads + 255) / 256), dim3(256), 0,
                           stream, static_cast<const T*>(o), tdo, lse, delta, lse2, rows, sc.d_mul);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (stages & 2) {
        if constexpr (D > 128) {
            const int nkb = (N + Dkdv1Tile<D>::BN - 1) / Dkdv1Tile<D>::BN;
            hipLaunchKernelGGL((bwd_dkdv1_kernel<T, D, CAUSAL, false>), dim3(BH * nkb), dim3(256),
                               0, stream, tq, tk, tv, tdo, lse2, delta, static_cast<T*>(dv), BH,
                               N, nkb, sc.dk_mul, c);
            if ((e = hipGetLastError()) != hipSuccess) return e;
            hipLaunchKernelGGL((bwd_dkdv1_kernel<T, D, CAUSAL, true>), dim3(BH * nkb), dim3(256),
                               0, stream, tq, tk, tv, tdo, lse2, delta, static_cast<T*>(dk), BH,
                               N, nkb, sc.dk_mul, c);
        } else {
            const int nkb = (N + DkdvTile<D>::BN - 1) / DkdvTile<D>::BN;
            hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, CAUSAL>), dim3(BH * nkb),
                               dim3(DkdvTile<D>::NT), 0, stream, tq, tk, tv, tdo, lse2, delta,
                               static_cast<T*>(dk), static_cast<T*>(dv), BH, N, nkb, sc.dk_mul,
                               c);
        }
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (stages & 4) {
        // eight waves (256 queries, K/V tiles shared by twice as many waves)
        // once the launch has at least one such workgroup per CU; four below
        // that, and always at d = 256 (one wave per SIMD)
        constexpr int NW8 = D > 128 ? 4 : 8;
        const int nqb8 = (N + DqTile<D, NW8>::BM - 1) / DqTile<D, NW8>::BM;
        if (D <= 128 && (int64_t)BH * nqb8 >= 256) {
            hipLaunchKernelGGL((bwd_dq_kernel<T, D, CAUSAL, NW8>), dim3(BH * nqb8),
                               dim3(DqTile<D, NW8>::NT), 0, stream, tq, tk, tv, tdo, lse2, delta,
                               static_cast<T*>(dq), BH, N, nqb8, sc.dq_mul, c);
        } else {
            const int nqb = (N + DqTile<D, 4>::BM - 1) / DqTile<D, 4>::BM;
            hipLaunchKernelGGL((bwd_dq_kernel<T, D, CAUSAL, 4>), dim3(BH * nqb),
                               dim3(DqTile<D, 4>::NT), 0, stream, tq, tk, tv, tdo, lse2, delta,
                               static_cast<T*>(dq), BH, N, nqb, sc.dq_mul, c);
        }
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return e;
}

template <typename T>
hipError_t launch_d(int d, bool causal, const void* q, const void* k, const void* v,
                    const void* o, const float* lse, const void* dO, void* dq, void* dk, void* dv,
                    float* delta, float* lse2, int BH, int N, const BwdScales& sc, int stages,
                    hipStream_t stream) {
    if (d == 64)
        return causal ? launch_typed<T, 64, true>(q, k, v, o, lse, dO, dq, dk, dv, delta, lse2,
                                                  BH, N, sc, stages, stream)
                      : launch_typed<T, 64, false>(q, k, v, o, lse, dO, dq, dk, dv, delta, lse2,
                                                   BH, N, sc, stages, stream);
    if (d == 256)
        return causal ? launch_typed<T, 256, true>(q, k, v, o, lse, dO, dq, dk, dv, delta, lse2,
                                                   BH, N, sc, stages, stream)
                      : launch_typed<T, 256, false>(q, k, v, o, lse, dO, dq, dk, dv, delta,
                                                    lse2, BH, N, sc, stages, stream);
    return causal ? launch_typed<T, 128, true>(q, k, v, o, lse, dO, dq, dk, dv, delta, lse2, BH,
                                               N, sc, stages, stream)
                  : launch_typed<T, 128, false>(q, k, v, o, lse, dO, dq, dk, dv, delta, lse2, BH,
                                                N, sc, stages, stream);
}

}  // namespace

hipError_t launch_bwd_scaled(int dtype, int d, bool causal, const void* q, const void* k,
                             const void* v, const void* o, const float* lse, const void* dO,
                             void* dq, void* dk, void* dv, float* delta, float* lse2, int BH,
                             int N, const BwdScales& sc, int stages, hipStream_t stream) {
    if (dtype == 2)
        return launch_d<__bf16>(d, causal, q, k, v, o, lse, dO, dq, dk, dv, delta, lse2, BH, N,
                                sc, stages, stream);
    return launch_d<_Float16>(d, causal, q, k, v, o, lse, dO, dq, dk, dv, delta, lse2, BH, N,
                              sc, stages, stream);
}

hipError_t launch_bwd(int dtype, int d, bool causal, const void* q, const void* k, const void* v,
                      const void* o, const float* lse, const void* dO, void* dq, void* dk,
                      void* dv, float* delta, float* lse2, int BH, int N, float scale,
                      int stages, hipStream_t stream) {
    const BwdScales sc{scale * kLog2e, scale, scale, 1.f};
    return launch_bwd_scaled(dtype, d, causal, q, k, v, o, lse, dO, dq, dk, dv, delta, lse2, BH,
                             N, sc, stages, stream);
}

}  // namespace fa
