// Forward attention on MFMA matrix cores (bf16 / fp16 in, fp32 accumulate).
//
// Method ("11.11 Flash Attention", algomaster.io): Q is split into blocks of
// BM query rows and K/V into blocks of BN keys; one workgroup owns one query
// block of one (batch, head) and walks the K/V blocks in order (section
// "Flash Attention 2": Q-block outer loop, parallel over batch x heads x query
// blocks). Each K/V tile is staged once in LDS and shared by the workgroup's
// four or eight wavefronts. Per tile: scores, running row max, exponentials against the
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
//    B operand of O^T = V^T P^T.
//  * K and V tiles go HBM -> LDS with global_load_lds_dwordx4 (no VGPR
//    staging, no VALU), double-buffered: the next tile's loads are issued
//    before the current tile is computed. Both are stored row-major with an
//    XOR swizzle of the 16-byte chunks (tile_swz) so that the MFMA operand
//    reads are free of bank conflicts. K is read as 16-byte rows; V^T with
//    ds_read_b64_tr_b16, which transposes 4x4 blocks of 16-bit elements
//    across lanes on the way out of LDS.
//  * Softmax works in base 2: p = 2^(s * scale * log2 e - m) via v_exp_f32.
//    The running max is refreshed only when a row's max grows by more than
//    2^8 (then O and l are rescaled); otherwise p stays <= 2^8 against the
//    stale max. This is exact: m, l and O always use the same reference.
//    At head dim 64 the row max is not even taken: the exponentials against
//    the current reference come first, and a lane sum above 2^8 (the only
//    way a refresh can be due, and always the case on the first tile) sends
//    the tile back through scores, max and refresh.
//  * Causal: tiles past the block's last query are never visited, a wave
//    skips tiles wholly above its own rows, and only tiles that straddle the
//    diagonal (or the ragged end of N) pay for the mask.
//  * Launch order: logical workgroup ids are remapped so each XCD gets whole
//    heads (K/V reuse in its L2); causal blocks run longest-first per head.

#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// NW wavefronts of 32 queries per workgroup share each K/V tile of BN keys.
template <int D, int NW_>
struct FwdTile {
    static constexpr int NW = NW_;
    static constexpr int BM = 32 * NW;             // queries per workgroup
    static constexpr int BN = 64;                  // keys per K/V tile
    static constexpr int NT = 64 * NW;             // threads per workgroup
    static constexpr int NSUB = BN / 32;           // 32-key score subtiles per tile
    static constexpr int NG = BN / 16;             // 16-key groups (P V MFMAs per head-dim block)
    static constexpr int ROWB = D * 2;             // bytes per K/V row
    static constexpr int TILEB = BN * ROWB;        // bytes per K (or V) tile
    static constexpr int NLOAD = TILEB / (NT * 16);  // direct loads per thread per tile
    static constexpr int KS = D / 16;              // MFMA k-steps over the head dim
    static constexpr int DB = D / 32;              // 32-row blocks of O^T
    static_assert(NLOAD >= 1 && TILEB % (NT * 16) == 0, "tile must split into whole direct loads");
};

constexpr float kRescaleThreshold = 8.f;  // log2 units: refresh m when it grows by > 2^8
constexpr float kRescaleSum = 256.f;      // 2^8: a lane's tile sum up to this needs no refresh

// Per-wavefront state of the forward kernel and its steps.
template <typename T, int D, bool CAUSAL, int NW>
struct FwdWave {
    using C = FwdTile<D, NW>;
    using V8 = typename Vec<T>::x8;
    using V4 = typename Vec<T>::x4;

    const T* Kh;
    const T* Vh;
    int N, nkt, tid, wave, lane, h, l32, q0, qrow;
    float c;
    V8 qf[C::KS];               // B operand of S^T = K Q^T (d = 16 s + 8 h + j)
    int ld_row[C::NLOAD], ld_col[C::NLOAD];
    unsigned ld_off[C::NLOAD];  // byte offset of this thread's 16 bytes within a full tile
    int koff[C::KS];            // LDS byte offsets of the K operand reads (rows l32; +32 rows per subtile)
    int voff[2][C::DB];         // LDS byte offsets of the V^T transposing reads (key group 0; +16 rows per group)
    float m_run, l_run;         // running (reference) max of s * c and this lane's sum
    f32x16 oacc[C::DB];         // O^T accumulators (head dim 32 b + row, query = lane)
    // operand reads ahead of their MFMAs: 0 is the compiler's own order,
    // which measured best with two waves per SIMD (d <= 128); at d = 256 (one
    // wave per SIMD) six ahead measured 20 % faster than it (B1 H32 N8192,
    // causal 1.61 -> 1.29 ms, non-causal 3.16 -> 2.50 ms; 2 and 4 ahead in
    // between, 8 no better)
    static constexpr int PF = D > 128 ? 6 : 0;
    // Skip the per-tile row max (tile_skip_max): measured 2-5 % faster at head
    // dim 64 (B4 H16 N2048, causal B4 H16 N4096); at 128 and 256 no faster,
    // the P V MFMAs there waiting for the whole tile's exponentials cost what
    // the max saves.
    static constexpr bool kSkipMax = D == 64;

    __device__ __forceinline__ void init(const T* Qh, const T* Kh_, const T* Vh_, int N_,
                                         int qb, float c_) {
        Kh = Kh_;
        Vh = Vh_;
        N = N_;
        c = c_;
        tid = threadIdx.x;
        lane = tid & 63;
        // wave-uniform (scalar branches and LDS bases) at d = 64 without the
        // causal mask: 2 % faster there, 2 % slower with it and at d = 128
        wave = (D == 64 && !CAUSAL) ? __builtin_amdgcn_readfirstlane(tid >> 6) : tid >> 6;
        l32 = lane & 31;
        h = lane >> 5;
        q0 = qb * C::BM + wave * 32;
        qrow = q0 + l32;
        const V8* src = reinterpret_cast<const V8*>(Qh + (size_t)min(qrow, N - 1) * D + 8 * h);
#pragma unroll
        for (int s = 0; s < C::KS; ++s) qf[s] = src[2 * s];
        const int q_last = min(N, (qb + 1) * C::BM) - 1;
        nkt = CAUSAL ? (q_last / C::BN + 1) : (N + C::BN - 1) / C::BN;

        // Direct-load map: load i of this thread fills LDS bytes [i*4096 +
        // tid*16, +16) of a tile, i.e. row r, stored chunk position p; it
        // fetches global chunk p ^ tile_swz(r) of that row (rows past N re-read
        // row N-1; their scores are masked).
#pragma unroll
        for (int i = 0; i < C::NLOAD; ++i) {
            const int byte = i * (C::NT * 16) + tid * 16;
            const int r = byte / C::ROWB, p = (byte % C::ROWB) / 16;
            ld_row[i] = r;
            ld_col[i] = (p ^ tile_swz<D>(r)) * 8;
            ld_off[i] = (unsigned)(r * D + ld_col[i]) * 2u;
        }
        // K (A side of S^T): key 32 c2 + l32, chunk 2 s + h. The swizzle repeats
        // every 16 rows, so subtile c2 is koff + 32 c2 rows.
#pragma unroll
        for (int s = 0; s < C::KS; ++s) koff[s] = tile_off<D>(l32, 16 * s + 8 * h);
        // V^T (A side of O^T = V^T P^T) via transposing reads. Read `half` of
        // key group g, head-dim block b: this lane supplies row 16 g + 8 half +
        // 4 h + (lane % 16) / 4, columns 32 b + 16 ((lane / 16) % 2) + 4 (lane %
        // 4) .. +3; it receives head dim 32 b + lane % 32 at keys 16 g + 8 half
        // + 4 h + 0..3 -- the key order of its probabilities in P^T.
        const int src_r = 4 * h + (lane & 15) / 4;
        const int src_d = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
            for (int b = 0; b < C::DB; ++b) voff[hf][b] = tile_off<D>(8 * hf + src_r, 32 * b + src_d);
        m_run = -INFINITY;
        l_run = 0.f;
#pragma unroll
        for (int b = 0; b < C::DB; ++b) oacc[b] = f32x16{};
    }

    __device__ __forceinline__ void issue_tile(int kbase, char* sKd, char* sVd) const {
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
        if constexpr (D == 128) {
            // 64-bit addresses here: at head dim 128 the 32-bit offsets below
            // leave the kernel 174 registers instead of 222 and it measured 5 %
            // slower (B8 H16 N4096 causal and B2 H32 N8192); at 64 and 256 they
            // are 5 % and 1 % faster
#pragma unroll
            for (int i = 0; i < C::NLOAD; ++i) {
                const size_t row = (size_t)min(kbase + ld_row[i], N - 1) * D;
                char* kdst = sKd + i * (C::NT * 16) + wave * 1024;
                char* vdst = sVd + i * (C::NT * 16) + wave * 1024;  // this wave's 1 KiB of load i
                __builtin_amdgcn_global_load_lds(Kh + row + ld_col[i], kdst, 16, 0, 0);
                __builtin_amdgcn_global_load_lds(Vh + row + ld_col[i], vdst, 16, 0, 0);
            }
        } else {
            const char* kb = reinterpret_cast<const char*>(Kh);
            const char* vb = reinterpret_cast<const char*>(Vh);
#pragma unroll
            for (int i = 0; i < C::NLOAD; ++i) {
                // 32-bit byte offsets from the head's base (a head holds < 2^31
                // elements)
                const unsigned off = (unsigned)min(kbase + ld_row[i], N - 1) * (D * 2u) +
                                     (ld_off[i] - (unsigned)ld_row[i] * (D * 2u));
                char* kdst = sKd + i * (C::NT * 16) + wave * 1024;
                char* vdst = sVd + i * (C::NT * 16) + wave * 1024;
                __builtin_amdgcn_global_load_lds(kb + off, kdst, 16, 0, 0);
                __builtin_amdgcn_global_load_lds(vb + off, vdst, 16, 0, 0);
            }
        }
    }

    // S^T = K Q^T for one tile (K read from LDS), masked.
    __device__ __forceinline__ void skip_scores(const char* kb, int kbase,
                                                f32x16 (&s)[C::NSUB]) const {
#pragma unroll
        for (int c2 = 0; c2 < C::NSUB; ++c2) {
            s[c2] = f32x16{};
#pragma unroll
            for (int ks = 0; ks < C::KS; ++ks) {
                const V8 a = *reinterpret_cast<const V8*>(kb + koff[ks] + c2 * 32 * C::ROWB);
                s[c2] = mfma32(a, qf[ks], s[c2]);
            }
        }
        // key kbase + 32 c2 + acc_row(r, h) is visible iff it is <= lim + 4 h + kbase
        if ((kbase + C::BN > N) || (CAUSAL && kbase + C::BN - 1 > q0)) {
            const int lim = (CAUSAL ? min(qrow, N - 1) : N - 1) - kbase - 4 * h;
#pragma unroll
            for (int c2 = 0; c2 < C::NSUB; ++c2)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (32 * c2 + 8 * (r >> 2) + (r & 3) > lim) s[c2][r] = -INFINITY;
        }
    }

    // p = 2^(s c - m) in place; returns this lane's sum of them, as four
    // interleaved partial sums so that it is ready soon after the last p.
    __device__ __forceinline__ float skip_exps(f32x16 (&s)[C::NSUB]) const {
        float rs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c2 = 0; c2 < C::NSUB; ++c2)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float p = fast_exp2(fmaf(s[c2][r], c, -m_run));
                s[c2][r] = p;
                rs[r & 3] += p;
            }
        return (rs[0] + rs[1]) + (rs[2] + rs[3]);
    }

    // A tile without the up-front row max. The probabilities are taken
    // against the current reference first. A lane sum <= 2^8 bounds each of
    // its p by 2^8, so no refresh is due (a refresh needs a row max more than
    // 2^8 above the reference) and the result is the one the max would have
    // given. Otherwise (always on the first tile, where the reference is -inf
    // and the sums are inf or NaN) the scores are formed again from the K tile
    // still in LDS, the row max refreshes the reference as in step, and the
    // exponentials are taken again.
    __device__ __forceinline__ void tile_skip_max(int kbase, const char* kb, const char* vb) {
        static_assert(PF == 0, "operand reads ahead are not used with this path");
        auto vread = [&](int g, int b) {
            const char* vg = vb + g * 16 * C::ROWB;
            const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vg + voff[0][b]));
            const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vg + voff[1][b]));
            const s16x4 w[2] = {lo, hi};
            V8 a;
            __builtin_memcpy(&a, w, sizeof(a));
            return a;
        };
        f32x16 s[C::NSUB];
        skip_scores(kb, kbase, s);
        // the first key group's V^T operands do not depend on P: read them
        // now, so that they have landed when P is ready
        V8 ov[C::DB];
#pragma unroll
        for (int b = 0; b < C::DB; ++b) ov[b] = vread(0, b);
        float rs = skip_exps(s);
        if (__builtin_amdgcn_ballot_w64(!(rs <= kRescaleSum)) != 0) {
            // read K again rather than keep the first pass's operands live
            asm volatile("" ::: "memory");
            skip_scores(kb, kbase, s);
            float mx = fmaxf(s[0][0], s[0][1]);
#pragma unroll
            for (int r = 2; r < 16; ++r) mx = fmaxf(mx, s[0][r]);
#pragma unroll
            for (int c2 = 1; c2 < C::NSUB; ++c2)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[c2][r]);
            mx = wave_half_max(mx) * c;
            if (__builtin_amdgcn_ballot_w64(mx > m_run + kRescaleThreshold) != 0) {
                const float m_new = fmaxf(m_run, mx);
                const float alpha = fast_exp2(m_run - m_new);
                m_run = m_new;
                l_run *= alpha;
#pragma unroll
                for (int b = 0; b < C::DB; ++b)
#pragma unroll
                    for (int r = 0; r < 16; ++r) oacc[b][r] *= alpha;
            }
            rs = skip_exps(s);
        }
        l_run += rs;
        V8 pf[C::NG];
#pragma unroll
        for (int g = 0; g < C::NG; ++g) pf[g] = pack8<T>(s[g / 2], 8 * (g % 2));
#pragma unroll
        for (int g = 0; g < C::NG; ++g)
#pragma unroll
            for (int b = 0; b < C::DB; ++b)
                oacc[b] = mfma32(g == 0 ? ov[b] : vread(g, b), pf[g], oacc[b]);
    }

    // One K/V tile: wait for it, start the next one into the other buffers,
    // then scores, online softmax and P V on this one.
    __device__ __forceinline__ void step(int kt, const char* kb, const char* vb, char* kn,
                                         char* vn) {
        const int kbase = kt * C::BN;
        // tile kt has landed in LDS (this thread's direct loads done, then the
        // barrier for everyone's), and the other buffers are no longer read
        __builtin_amdgcn_s_waitcnt(kVmcntZero);
        __syncthreads();
        if (!kSerialStaging && kt + 1 < nkt) issue_tile(kbase + C::BN, kn, vn);

        const bool active = !CAUSAL || kbase <= q0 + 31;
        if (!active) return;
        if constexpr (kSkipMax) {
            tile_skip_max(kbase, kb, vb);
            return;
        }
        f32x16 s[C::NSUB];
#pragma unroll
        for (int c2 = 0; c2 < C::NSUB; ++c2) s[c2] = f32x16{};
        if constexpr (PF > 0) {
            // one wave per SIMD (head dim 256): no partner wave covers the LDS
            // latency, so the K operand reads run PF units ahead of their MFMAs
            // (unit t: k-step t / NSUB, subtile t % NSUB), order kept by
            // scheduling fences
            constexpr int NU = C::KS * C::NSUB;
            V8 ok[PF];
            auto kread = [&](int t) {
                return *reinterpret_cast<const V8*>(kb + koff[t / C::NSUB] + (t % C::NSUB) * 32 * C::ROWB);
            };
#pragma unroll
            for (int t = 0; t < PF; ++t) ok[t] = kread(t);
#pragma unroll
            for (int t = 0; t < NU; ++t) {
                s[t % C::NSUB] = mfma32(ok[t % PF], qf[t / C::NSUB], s[t % C::NSUB]);
                if (t + PF < NU) ok[t % PF] = kread(t + PF);
                __builtin_amdgcn_sched_barrier(0);
            }
        } else {
            // one subtile's k-steps after the other (same accumulation order
            // as k-steps outside, bit-identical): 1-1.5 % faster at d = 64 and
            // 128 than alternating the two subtiles
#pragma unroll
            for (int c2 = 0; c2 < C::NSUB; ++c2)
#pragma unroll
                for (int ks = 0; ks < C::KS; ++ks) {
                    const V8 a = *reinterpret_cast<const V8*>(kb + koff[ks] + c2 * 32 * C::ROWB);
                    s[c2] = mfma32(a, qf[ks], s[c2]);
                }
        }
        // mask: key kbase + 32 c2 + acc_row(r, h) is visible iff it is <= lim + 4 h + kbase
        const bool need_mask = (kbase + C::BN > N) || (CAUSAL && kbase + C::BN - 1 > q0);
        if (need_mask) {
            const int lim = (CAUSAL ? min(qrow, N - 1) : N - 1) - kbase - 4 * h;
#pragma unroll
            for (int c2 = 0; c2 < C::NSUB; ++c2)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (32 * c2 + 8 * (r >> 2) + (r & 3) > lim) s[c2][r] = -INFINITY;
        }
        float mx = fmaxf(s[0][0], s[0][1]);
#pragma unroll
        for (int r = 2; r < 16; ++r) mx = fmaxf(mx, s[0][r]);
#pragma unroll
        for (int c2 = 1; c2 < C::NSUB; ++c2)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[c2][r]);
        mx = wave_half_max(mx) * c;
        if (__builtin_amdgcn_ballot_w64(mx > m_run + kRescaleThreshold) != 0) {
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
        for (int c2 = 0; c2 < C::NSUB; ++c2)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float p = fast_exp2(fmaf(s[c2][r], c, -m_run));
                s[c2][r] = p;
                rs += p;
            }
        l_run += rs;

        V8 pf[C::NG];
#pragma unroll
        for (int g = 0; g < C::NG; ++g) pf[g] = pack8<T>(s[g / 2], 8 * (g % 2));
        auto vread = [&](int g, int b) {
            const char* vg = vb + g * 16 * C::ROWB;
            const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vg + voff[0][b]));
            const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vg + voff[1][b]));
            const s16x4 w[2] = {lo, hi};
            V8 a;
            __builtin_memcpy(&a, w, sizeof(a));
            return a;
        };
        if constexpr (PF > 0) {
            // V^T operands PF units ahead as well (unit u: g = u / DB, b = u % DB)
            constexpr int NC = C::NG * C::DB;
            V8 ov[PF];
#pragma unroll
            for (int u = 0; u < PF; ++u) ov[u] = vread(u / C::DB, u % C::DB);
#pragma unroll
            for (int u = 0; u < NC; ++u) {
                oacc[u % C::DB] = mfma32(ov[u % PF], pf[u / C::DB], oacc[u % C::DB]);
                if (u + PF < NC) ov[u % PF] = vread((u + PF) / C::DB, (u + PF) % C::DB);
                __builtin_amdgcn_sched_barrier(0);
            }
        } else {
#pragma unroll
            for (int g = 0; g < C::NG; ++g)
#pragma unroll
                for (int b = 0; b < C::DB; ++b) oacc[b] = mfma32(vread(g, b), pf[g], oacc[b]);
        }
    }

    __device__ __forceinline__ void finish(T* Oh, float* lse_h) {
        const float lt = wave_half_sum(l_run);
        if (qrow < N) {
            const float inv = 1.f / lt;
            T* orow = Oh + (size_t)qrow * D;
#pragma unroll
            for (int b = 0; b < C::DB; ++b)
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    V4 w;
#pragma unroll
                    for (int i = 0; i < 4; ++i) w[i] = (T)(oacc[b][4 * r4 + i] * inv);
                    *reinterpret_cast<V4*>(orow + 32 * b + 8 * r4 + 4 * h) = w;
                }
            if (lse_h != nullptr && h == 0) lse_h[qrow] = (m_run + log2f(lt)) * kLn2;
        }
    }
};

template <typename T, int D, bool CAUSAL, int NW>
__global__ void __launch_bounds__(64 * NW, D > 128 ? 1 : 2)
fwd_mfma_kernel(const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
                T* __restrict__ O, float* __restrict__ LSE, int BH, int N, int nqb, float c) {
    using C = FwdTile<D, NW>;
    // Two buffers per tensor as four separate LDS objects: the compiler can
    // then tell that the loads in flight into one buffer never alias the
    // reads of the other, and does not wait for them before every read.
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

    FwdWave<T, D, CAUSAL, NW> w;
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

template <typename T, int D, bool CAUSAL, int NW>
hipError_t launch_nw(const void* q, const void* k, const void* v, void* o, float* lse, int BH,
                     int N, float scale, hipStream_t stream) {
    using C = FwdTile<D, NW>;
    const int nqb = (N + C::BM - 1) / C::BM;
    const dim3 grid(BH * nqb), block(C::NT);
    hipLaunchKernelGGL((fwd_mfma_kernel<T, D, CAUSAL, NW>), grid, block, 0, stream,
                       static_cast<const T*>(q), static_cast<const T*>(k),
                       static_cast<const T*>(v), static_cast<T*>(o), lse, BH, N, nqb,
                       scale * kLog2e);
    return hipGetLastError();
}

// Workgroup shape (waves = 0): eight waves (256 queries, one workgroup per
// CU, K/V tiles shared by all eight) measured 1-5 % faster than four on every
// bf16 workload with the causal block order of causal_block; four waves (128
// queries, two workgroups per CU) when a launch would have fewer eight-wave
// workgroups than CUs. waves = 4 or 8 forces the shape.
template <typename T, int D, bool CAUSAL>
hipError_t launch_typed(const void* q, const void* k, const void* v, void* o, float* lse, int BH,
                        int N, float scale, int waves, hipStream_t stream) {
    if (waves == 0) waves = (int64_t)BH * ((N + 255) / 256) >= 256 ? 8 : 4;
    if (waves == 4) return launch_nw<T, D, CAUSAL, 4>(q, k, v, o, lse, BH, N, scale, stream);
    return launch_nw<T, D, CAUSAL, 8>(q, k, v, o, lse, BH, N, scale, stream);
}

// Head dim 256: the Q operand and the output accumulators need about 470
// registers per wave, so one wave per SIMD (four per workgroup), with the
// accumulators in AGPRs.
template <typename T>
hipError_t launch_d(int d, bool causal, const void* q, const void* k, const void* v, void* o,
                    float* lse, int BH, int N, float scale, int waves, hipStream_t stream) {
    if (d == 64)
        return causal ? launch_typed<T, 64, true>(q, k, v, o, lse, BH, N, scale, waves, stream)
                      : launch_typed<T, 64, false>(q, k, v, o, lse, BH, N, scale, waves, stream);
    if (d == 256)
        return causal ? launch_nw<T, 256, true, 4>(q, k, v, o, lse, BH, N, scale, stream)
                      : launch_nw<T, 256, false, 4>(q, k, v, o, lse, BH, N, scale, stream);
    return causal ? launch_typed<T, 128, true>(q, k, v, o, lse, BH, N, scale, waves, stream)
                  : launch_typed<T, 128, false>(q, k, v, o, lse, BH, N, scale, waves, stream);
}

}  // namespace

hipError_t launch_fwd_mfma(int dtype, int d, bool causal, const void* q, const void* k,
                           const void* v, void* o, float* lse, int BH, int N, float scale,
                           int waves, hipStream_t stream) {
    if (dtype == 2)
        return launch_d<__bf16>(d, causal, q, k, v, o, lse, BH, N, scale, waves, stream);
    return launch_d<_Float16>(d, causal, q, k, v, o, lse, BH, N, scale, waves, stream);
}

}  // namespace fa
