// Forward attention in float32 arithmetic throughout (no reduced-precision
// step), for callers that need fp32 inputs and outputs.
//
// Same method as the MFMA kernel ("11.11 Flash Attention", sections "Flash
// Attention: The Key Insight", "The Tiling Algorithm" and "Flash Attention
// 2": Q blocks outer, K/V tiles inner, running max m and running sum l, one
// division at the end), on the vector ALUs: a lane owns one query row and
// keeps its unnormalised output row in registers; K/V tiles of 16 keys are
// staged in LDS and read by all lanes as broadcasts. Exponentials use the
// full-precision expf, so the result is float32-accurate.

#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int F32_BM = 64;  // query rows per workgroup (one per lane of each wave)
constexpr int F32_BN = 16;  // keys per tile
constexpr int F32_NW = 4;   // waves per workgroup, splitting the key tiles

// Four waves share a block of 64 queries; in round r wave w takes key tile
// F32_NW r + w (each wave a different quarter of the keys, with its own
// running max, sum and output row per query), so a short sequence still
// keeps four waves busy per query block. At the end the four partial
// states (m_w, l_w, O_w) of each query are merged exactly as the online
// softmax merges tiles: m = max_w m_w, l = sum_w e^(m_w - m) l_w and
// O = sum_w e^(m_w - m) O_w / l.
template <int D, bool CAUSAL>
__global__ void __launch_bounds__(64 * F32_NW)
fwd_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
               const float* __restrict__ V, float* __restrict__ O, float* __restrict__ LSE,
               int BH, int N, int nqb, float scale) {
    constexpr int TILE = F32_BN * D;                       // floats per K (or V) tile
    constexpr int MERGE = (F32_NW - 1) * F32_BM * (D + 2);  // partial states of waves 1..3
    constexpr int KVF = 2 * F32_NW * TILE;                  // K and V tiles of one round
    __shared__ float sQ[F32_BM * (D + 1)];
    __shared__ float sKV[KVF > MERGE ? KVF : MERGE];

    const int bh = blockIdx.x / nqb;
    const int qb = blockIdx.x % nqb;
    const size_t head = (size_t)bh * N * D;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int q0 = qb * F32_BM;
    const int qrow = q0 + lane;

    // stage the Q block (rows beyond N are zero and never stored)
    for (int e = tid; e < F32_BM * D; e += F32_BM * F32_NW) {
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
    const int ntiles = (kend + F32_BN - 1) / F32_BN;
    for (int t0 = 0; t0 < ntiles; t0 += F32_NW) {
        __syncthreads();
        // all threads stage the round's (up to) four K/V tiles
        for (int e = tid; e < F32_NW * TILE; e += F32_BM * F32_NW) {
            const int w = e / TILE, r = (e % TILE) / D, col = e % D;
            const int key = (t0 + w) * F32_BN + r;
            sKV[e] = key < N ? K[head + (size_t)key * D + col] : 0.f;
            sKV[F32_NW * TILE + e] = key < N ? V[head + (size_t)key * D + col] : 0.f;
        }
        __syncthreads();
        const int k0 = (t0 + wave) * F32_BN;
        if (k0 >= kend) continue;  // this wave has no tile in this round
        const float* sK = sKV + wave * TILE;
        const float* sV = sKV + F32_NW * TILE + wave * TILE;

        float s[F32_BN];
        float tmax = -INFINITY;
#pragma unroll
        for (int j = 0; j < F32_BN; ++j) {
            float dot = 0.f;
#pragma unroll 16
            for (int i = 0; i < D; ++i) dot = fmaf(sQ[lane * (D + 1) + i], sK[j * D + i], dot);
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

    // merge: waves 1..3 park (m, l, O) per query, wave 0 combines and stores
    __syncthreads();
    if (wave > 0) {
        float* st = sKV + ((wave - 1) * F32_BM + lane) * (D + 2);
        st[0] = m;
        st[1] = l;
#pragma unroll
        for (int i = 0; i < D; ++i) st[2 + i] = acc[i];
    }
    __syncthreads();
    if (wave == 0 && qrow < N) {
        float mt = m;
#pragma unroll
        for (int w = 1; w < F32_NW; ++w) mt = fmaxf(mt, sKV[((w - 1) * F32_BM + lane) * (D + 2)]);
        // every row has a visible key (key 0), so mt is finite
        const float a0 = expf(m - mt);
        float lt = l * a0;
#pragma unroll
        for (int i = 0; i < D; ++i) acc[i] *= a0;
#pragma unroll
        for (int w = 1; w < F32_NW; ++w) {
            const float* st = sKV + ((w - 1) * F32_BM + lane) * (D + 2);
            const float aw = expf(st[0] - mt);  // 0 for a wave that saw no key
            lt += st[1] * aw;
#pragma unroll
            for (int i = 0; i < D; ++i) acc[i] = fmaf(st[2 + i], aw, acc[i]);
        }
        const float inv = 1.f / lt;
        float* orow = O + head + (size_t)qrow * D;
#pragma unroll
        for (int i = 0; i < D; ++i) orow[i] = acc[i] * inv;
        if (LSE != nullptr) LSE[(size_t)bh * N + qrow] = mt + logf(lt);
    }
}

template <int D, bool CAUSAL>
hipError_t launch_typed(const float* q, const float* k, const float* v, float* o, float* lse,
                        int BH, int N, float scale, hipStream_t stream) {
    const int nqb = (N + F32_BM - 1) / F32_BM;
    hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL>), dim3(BH * nqb), dim3(F32_BM * F32_NW), 0, stream, q,
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
