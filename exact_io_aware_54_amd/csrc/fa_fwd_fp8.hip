// Forward attention with OCP FP8 (E4M3) Q, K, V and bf16 output.
//
// "11.11 Flash Attention", section "Flash Attention 3": FP8 attention on
// matrix units with twice the 16-bit throughput. Same tiling and online
// softmax as the 16-bit kernel (sections "The Tiling Algorithm" and "Flash
// Attention 2"); what changes:
//  * S^T = K8 Q8^T runs on the gfx950 32x32x64 f8f6f4 MFMA (E4M3 x E4M3,
//    fp32 accumulate). The per-tensor descales and the softmax scale fold
//    into one factor c = scale * q_descale * k_descale * log2(e).
//  * p = 2^(s c - m) lies in (0, 1]; it is multiplied by 2^8 and rounded to
//    E4M3 (v_cvt_pk_fp8_f32: round to nearest even, saturating), which keeps
//    probabilities down to 2^-17 out of the E4M3 subnormal range. The row sum
//    l accumulates the unrounded p in fp32.
//  * O^T = V8^T P8^T is one 32x32x64 MFMA per 64-key tile and 32 head dims;
//    the epilogue multiplies by v_descale / (2^8 l) and writes bf16.
// One 64-key tile is exactly one K = 64 step of the PV MFMA: a lane of half h
// holds the 16 + 16 probabilities of its query from the two 32-key score
// subtiles, which become its 32 operand bytes in register order; V is
// transposed into LDS in the matching key order.

#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int F8_D = 128;
constexpr int F8_BM = 128;               // queries per workgroup (4 waves x 32)
constexpr int F8_BN = 64;                // keys per tile
constexpr int F8_NT = 256;
constexpr int F8_KSTR = F8_D + 16;       // bytes per K row in LDS
constexpr int F8_VSTR = F8_BN + 16;      // bytes per V^T row in LDS
constexpr float F8_PSCALE = 256.f;       // P is stored as E4M3(p * 2^8)

// LDS position (0..63) of key kk of a 64-key tile in a V^T row, so that lane
// half h reads its 32 operand bytes at offset 32 h in the order of its score
// registers: subtile c = kk / 32 contributes register r = acc-row index.
__device__ __forceinline__ int f8_vpos(int kk) {
    const int c = kk >> 5, w = kk & 31;
    const int r = ((w >> 3) << 2) | (w & 3);
    const int h = (w >> 2) & 1;
    return 32 * h + 16 * c + r;
}

__device__ __forceinline__ uint32_t byte_of(uint32_t w, int b) { return (w >> (8 * b)) & 0xffu; }

template <bool CAUSAL>
__global__ void __launch_bounds__(256, 2)
fwd_fp8_kernel(const uint8_t* __restrict__ Q, const uint8_t* __restrict__ K,
               const uint8_t* __restrict__ V, __bf16* __restrict__ O, float* __restrict__ LSE,
               int BH, int N, int nqb, float c, float out_scale) {
    __shared__ __attribute__((aligned(16))) uint8_t sK[2][F8_BN * F8_KSTR];
    __shared__ __attribute__((aligned(16))) uint8_t sV[2][F8_D * F8_VSTR];

    int bh, qb;
    if (CAUSAL) {
        causal_block(blockIdx.x, nqb, BH, bh, qb);
    } else {
        const int L = xcd_remap(blockIdx.x, BH * nqb);
        bh = L / nqb;
        qb = L % nqb;
    }
    const size_t head = (size_t)bh * N * F8_D;
    const uint8_t* Qh = Q + head;
    const uint8_t* Kh = K + head;
    const uint8_t* Vh = V + head;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, h = lane >> 5;
    const int q0 = qb * F8_BM + wave * 32;
    const int qrow = q0 + l32;

    // B operand of S^T: k-step s, slot (h, j) holds d = 64 s + 32 h + j.
    i32x8 qf[2];
    if (qrow < N) {
        const i32x4* src = reinterpret_cast<const i32x4*>(Qh + (size_t)qrow * F8_D + 32 * h);
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const i32x4 lo = src[4 * s], hi = src[4 * s + 1];
            qf[s] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
    } else {
        qf[0] = i32x8{};
        qf[1] = i32x8{};
    }

    const int q_last = min(N, (qb + 1) * F8_BM) - 1;
    const int nkt = CAUSAL ? (q_last / F8_BN + 1) : (N + F8_BN - 1) / F8_BN;

    // staging: K as 2 x 16 B per thread; V as 4 keys x 8 bytes per thread
    i32x4 kreg[2];
    i32x2 vreg[4];
    auto load = [&](int kbase) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int id = tid + F8_NT * i;
            const int row = id >> 3, col = (id & 7) * 16;
            const int key = kbase + row;
            kreg[i] = key < N ? *reinterpret_cast<const i32x4*>(Kh + (size_t)key * F8_D + col) : i32x4{};
        }
        const int cc = tid & 15, g = tid >> 4;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int key = kbase + 4 * g + i;
            vreg[i] = key < N ? *reinterpret_cast<const i32x2*>(Vh + (size_t)key * F8_D + cc * 8) : i32x2{};
        }
    };
    auto store = [&](uint8_t* dK, uint8_t* dV) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int id = tid + F8_NT * i;
            const int row = id >> 3, col = (id & 7) * 16;
            *reinterpret_cast<i32x4*>(dK + row * F8_KSTR + col) = kreg[i];
        }
        const int cc = tid & 15, g = tid >> 4;
        const int pos = f8_vpos(4 * g);  // the 4 keys of the group are contiguous
#pragma unroll
        for (int dd = 0; dd < 8; ++dd) {
            const int wsel = dd >> 2, b = dd & 3;
            const uint32_t w = byte_of((uint32_t)vreg[0][wsel], b) | (byte_of((uint32_t)vreg[1][wsel], b) << 8) |
                               (byte_of((uint32_t)vreg[2][wsel], b) << 16) |
                               (byte_of((uint32_t)vreg[3][wsel], b) << 24);
            *reinterpret_cast<uint32_t*>(dV + (cc * 8 + dd) * F8_VSTR + pos) = w;
        }
    };

    load(0);
    store(sK[0], sV[0]);
    __syncthreads();

    float m_run = -INFINITY, l_run = 0.f;
    f32x16 oacc[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) oacc[b] = f32x16{};

    for (int kt = 0; kt < nkt; ++kt) {
        const int buf = kt & 1;
        const bool more = kt + 1 < nkt;
        const int kbase = kt * F8_BN;
        if (more) load(kbase + F8_BN);

        const bool active = !CAUSAL || kbase <= q0 + 31;
        if (active) {
            const uint8_t* kb = sK[buf];
            f32x16 s[2];
            s[0] = f32x16{};
            s[1] = f32x16{};
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int c2 = 0; c2 < 2; ++c2) {
                    const i32x4* p = reinterpret_cast<const i32x4*>(kb + (32 * c2 + l32) * F8_KSTR + 64 * ks + 32 * h);
                    const i32x4 lo = p[0], hi = p[1];
                    const i32x8 a{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                    s[c2] = mfma32_fp8(a, qf[ks], s[c2]);
                }
            const bool need_mask = (kbase + F8_BN > N) || (CAUSAL && kbase + F8_BN - 1 > q0);
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
            i32x8 pf;
#pragma unroll
            for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
                for (int r = 0; r < 16; r += 4) {
                    float p[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        p[i] = fast_exp2(fmaf(s[c2][r + i], c, -m_new));
                        rs += p[i];
                    }
                    int w = 0;
                    w = __builtin_amdgcn_cvt_pk_fp8_f32(p[0] * F8_PSCALE, p[1] * F8_PSCALE, w, false);
                    w = __builtin_amdgcn_cvt_pk_fp8_f32(p[2] * F8_PSCALE, p[3] * F8_PSCALE, w, true);
                    pf[4 * c2 + r / 4] = w;
                }
            l_run = l_run * alpha + rs;
            m_run = m_new;
#pragma unroll
            for (int b = 0; b < 4; ++b)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[b][r] *= alpha;

            const uint8_t* vb = sV[buf];
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const i32x4* p = reinterpret_cast<const i32x4*>(vb + (32 * b + l32) * F8_VSTR + 32 * h);
                const i32x4 lo = p[0], hi = p[1];
                const i32x8 a{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                oacc[b] = mfma32_fp8(a, pf, oacc[b]);
            }
        }
        if (more) store(sK[buf ^ 1], sV[buf ^ 1]);
        __syncthreads();
    }

    const float lt = wave_half_sum(l_run);
    if (qrow < N) {
        const float inv = out_scale / (F8_PSCALE * lt);
        __bf16* orow = O + head + (size_t)qrow * F8_D;
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                bf16x4 w;
#pragma unroll
                for (int i = 0; i < 4; ++i) w[i] = (__bf16)(oacc[b][4 * r4 + i] * inv);
                *reinterpret_cast<bf16x4*>(orow + 32 * b + 8 * r4 + 4 * h) = w;
            }
        if (LSE != nullptr && h == 0) LSE[(size_t)bh * N + qrow] = (m_run + log2f(lt)) * kLn2;
    }
}

}  // namespace

hipError_t launch_fwd_fp8(int d, bool causal, const void* q8, const void* k8, const void* v8,
                          float qk_scale, float v_descale, void* o, float* lse, int BH, int N,
                          hipStream_t stream) {
    (void)d;  // validated to be 128
    const int nqb = (N + F8_BM - 1) / F8_BM;
    const dim3 grid(BH * nqb), block(F8_NT);
    const float c = qk_scale * kLog2e;
    auto q = static_cast<const uint8_t*>(q8);
    auto k = static_cast<const uint8_t*>(k8);
    auto v = static_cast<const uint8_t*>(v8);
    auto out = static_cast<__bf16*>(o);
    if (causal)
        hipLaunchKernelGGL((fwd_fp8_kernel<true>), grid, block, 0, stream, q, k, v, out, lse, BH, N,
                           nqb, c, v_descale);
    else
        hipLaunchKernelGGL((fwd_fp8_kernel<false>), grid, block, 0, stream, q, k, v, out, lse, BH,
                           N, nqb, c, v_descale);
    return hipGetLastError();
}

}  // namespace fa
