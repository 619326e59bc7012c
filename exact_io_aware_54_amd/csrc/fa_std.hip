// Standard (materialising) attention: the baseline the method is measured
// against.
//
// "11.11 Flash Attention" (algomaster.io), section "Standard Attention: Step
// by Step": the score matrix S = Q K^T / sqrt(d) is written to HBM, read back
// for a row softmax whose result P is written to HBM again, and read once more
// for O = P V. These kernels do exactly those three passes, each as a plain
// HBM-to-HBM kernel, so that the HBM round trips the method removes are paid
// in full:
//  1. std_scores: one workgroup per 128 x 128 tile of S (4 waves, 64 x 64
//     each, 32x32x16 MFMAs with Q and K rows loaded straight from global
//     memory); S = scale Q K^T is stored in the input type, the tile passing
//     through LDS so that rows are written in whole 16-byte pieces.
//  2. std_softmax: persistent; one wavefront per row up to 8192 keys, one
//     workgroup per row beyond, the row held in registers (up to 32768 keys;
//     longer or unaligned rows are read twice): the row max and sum of
//     exponentials (online per thread, then across the row's threads), then
//     P = exp(S - max) / sum written over S (causal: keys after the query get
//     P = 0).
//  3. std_pv: one workgroup per 128 queries (4 waves, 32 queries and the full
//     head dim each), walking the keys in tiles of 64: V tiles and the
//     workgroup's 128 x 64 tiles of P staged in LDS by direct loads; V read
//     transposed, P as the other MFMA operand.
// The workspace holds S and then P in place: B * H * N * N 16-bit values.

#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// 16 bytes from global memory straight into LDS (lane t of the wave writes
// lds + 16 t). Kept out of kernel bodies: the host pass of the compiler only
// sees device functions through their declarations.
__device__ __forceinline__ void load16_to_lds(const void* g, char* lds) {
    __builtin_amdgcn_global_load_lds(g, lds, 16, 0, 0);
}

// ---------------------------------------------------------------- 1. scores
// The workgroup's 128 query rows and 128 key rows are brought into LDS with
// whole-row direct loads (16-byte chunks XOR-swizzled by tile_swz, as in the
// fused kernels), the MFMA operands are read from there, and the finished
// tile goes back through the same LDS (rows padded to 272 bytes: the two
// halves of a wave write rows four apart, which then fall on different
// banks) so that every thread stores whole 16-byte pieces of rows.
template <typename T, int D>
__global__ void __launch_bounds__(256)
std_scores_kernel(const T* __restrict__ Q, const T* __restrict__ K, T* __restrict__ S, int N,
                  int ntile, float scale) {
    using V8 = typename Vec<T>::x8;
    constexpr int ROWB = 2 * D, TILEB = 128 * ROWB, NLOAD = TILEB / 4096, RS = 272;
    constexpr int SMEM = 2 * TILEB > 128 * RS ? 2 * TILEB : 128 * RS;
    __shared__ __attribute__((aligned(1024))) char smem[SMEM];
    char* sQ = smem;
    char* sK = smem + TILEB;
    const int bh = blockIdx.y;
    const int qt = blockIdx.x / ntile, kt = blockIdx.x % ntile;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, h = lane >> 5;
    const T* Qh = Q + (size_t)bh * N * D;
    const T* Kh = K + (size_t)bh * N * D;
#pragma unroll
    for (int i = 0; i < NLOAD; ++i) {
        const int byte = i * 4096 + tid * 16;
        const int r = byte / ROWB, c = (byte % ROWB) / 16;
        const int col = (c ^ tile_swz<D>(r)) * 8;
        const int dst = i * 4096 + wave * 1024;
        load16_to_lds(Qh + (size_t)min(qt * 128 + r, N - 1) * D + col, sQ + dst);
        load16_to_lds(Kh + (size_t)min(kt * 128 + r, N - 1) * D + col, sK + dst);
    }
    __builtin_amdgcn_s_waitcnt(kVmcntZero);
    __syncthreads();
    const int r0 = 64 * (wave >> 1), c0 = 64 * (wave & 1);
    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
        V8 a[2], b[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            a[i] = *reinterpret_cast<const V8*>(sQ + tile_off<D>(r0 + 32 * i + l32, 16 * s + 8 * h));
            b[i] = *reinterpret_cast<const V8*>(sK + tile_off<D>(c0 + 32 * i + l32, 16 * s + 8 * h));
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(a[i], b[j], acc[i][j]);
    }
    __syncthreads();  // every wave is done with the Q / K tiles
    // acc[i][j]: lane holds key column c0 + 32 j + l32, register r holds query
    // row r0 + 32 i + acc_row(r, h) of the tile
    char* sS = smem;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = r0 + 32 * i + acc_row(r, h), col = c0 + 32 * j + l32;
                *reinterpret_cast<T*>(sS + row * RS + 2 * col) = (T)(acc[i][j][r] * scale);
            }
    __syncthreads();
    T* Sh = S + (size_t)bh * N * N;
    const bool vec = (N % 8) == 0;
#pragma unroll
    for (int it = 0; it < 8; ++it) {
        const int c = it * 256 + tid;  // 16-byte piece c of the tile
        const int row = c >> 4, col = (c & 15) * 8;
        const int q = qt * 128 + row, key = kt * 128 + col;
        if (q >= N || key >= N) continue;
        const V8 x = *reinterpret_cast<const V8*>(sS + row * RS + 2 * col);
        T* dst = Sh + (size_t)q * N + key;
        if (vec) {
            *reinterpret_cast<V8*>(dst) = x;
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (key + e < N) dst[e] = x[e];
        }
    }
}

// ---------------------------------------------------------------- 2. softmax
__device__ __forceinline__ void online_add(float& m, float& l, float x) {
    if (x > m) {
        l = l * exp2f((m - x) * kLog2e) + 1.f;
        m = x;
    } else {
        l += exp2f((x - m) * kLog2e);
    }
}

constexpr int kSoftmaxChunks = 16;  // 16-byte pieces of a row held per thread

// max and sum across the row's threads (a wave, or the four waves of the
// workgroup through `red`); every thread receives the result
template <int ROWS_PER_WG>
__device__ __forceinline__ float row_reduce(float v, bool is_max, float* red) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const float o = __shfl_xor(v, off);
        v = is_max ? fmaxf(v, o) : v + o;
    }
    if (ROWS_PER_WG == 1) {
        const int tid = threadIdx.x;
        if ((tid & 63) == 0) red[tid >> 6] = v;
        __syncthreads();
        v = is_max ? fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]))
                   : (red[0] + red[1]) + (red[2] + red[3]);
        __syncthreads();  // red is rewritten by the next reduction
    }
    return v;
}

// Row softmax in place. Persistent: `rows` rows (one per wavefront when
// ROWS_PER_WG = 4, one per workgroup when it is 1) are walked with a grid
// stride. A row whose pieces all fit the threads' registers
// (N % 8 == 0 and N <= kSoftmaxChunks * 8 * threads per row) is read once:
// row max, then the sum of 2^((s - max) log2 e), then the same exponentials
// scaled by 1 / sum are written over S. Other rows are read twice (an online
// max and sum, then P).
template <typename T, int ROWS_PER_WG>
__global__ void __launch_bounds__(256)
std_softmax_kernel(T* __restrict__ S, int N, long long rows, int causal) {
    using V8 = typename Vec<T>::x8;
    constexpr int TPR = 256 / ROWS_PER_WG;  // threads per row
    const int tid = threadIdx.x;
    const int t = tid % TPR, slot = tid / TPR;
    const bool in_regs = (N % 8) == 0 && N <= kSoftmaxChunks * 8 * TPR;
    __shared__ float red[4];
    for (long long row = (long long)blockIdx.x * ROWS_PER_WG + slot; row - slot < rows;
         row += (long long)gridDim.x * ROWS_PER_WG) {
        const bool live = row < rows;
        const int qi = live ? (int)(row % N) : 0;
        const int len = live ? (causal ? qi + 1 : N) : 0;  // visible keys
        T* p = S + (live ? row : 0) * (long long)N;
        if (in_regs) {
            V8 x[kSoftmaxChunks];
#pragma unroll
            for (int i = 0; i < kSoftmaxChunks; ++i) {
                const int c = (i * TPR + t) * 8;
                if (c < len) x[i] = *reinterpret_cast<const V8*>(p + c);
            }
            float m = -INFINITY;
#pragma unroll
            for (int i = 0; i < kSoftmaxChunks; ++i) {
                const int c = (i * TPR + t) * 8;
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    if (c + j < len) m = fmaxf(m, (float)x[i][j]);
            }
            const float M = row_reduce<ROWS_PER_WG>(m, true, red);
            const float mc = M * kLog2e;
            // keep the row as packed 16-bit values between the passes (each pass
            // converts again) instead of 128 live floats per thread
#pragma unroll
            for (int i = 0; i < kSoftmaxChunks; ++i) asm volatile("" : "+v"(x[i]));
            float l = 0.f;
#pragma unroll
            for (int i = 0; i < kSoftmaxChunks; ++i) {
                const int c = (i * TPR + t) * 8;
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    if (c + j < len) l += __builtin_amdgcn_exp2f(fmaf((float)x[i][j], kLog2e, -mc));
            }
            const float inv = 1.f / row_reduce<ROWS_PER_WG>(l, false, red);
            if (!live) continue;
#pragma unroll
            for (int i = 0; i < kSoftmaxChunks; ++i) asm volatile("" : "+v"(x[i]));
#pragma unroll
            for (int i = 0; i < kSoftmaxChunks; ++i) {
                const int c = (i * TPR + t) * 8;
                if (c >= N) continue;
                V8 y;
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    y[j] = (c + j < len)
                               ? (T)(__builtin_amdgcn_exp2f(fmaf((float)x[i][j], kLog2e, -mc)) * inv)
                               : (T)0.f;
                *reinterpret_cast<V8*>(p + c) = y;
            }
        } else {
            float m = -INFINITY, l = 0.f;
            for (int c = t; c < len; c += TPR) online_add(m, l, (float)p[c]);
            // combine (m, l) pairs: rescale every partial sum to the row max
            const float M = row_reduce<ROWS_PER_WG>(m, true, red);
            const float ls = (m == -INFINITY) ? 0.f : l * exp2f((m - M) * kLog2e);
            const float inv = 1.f / row_reduce<ROWS_PER_WG>(ls, false, red);
            if (!live) continue;
            for (int c = t; c < N; c += TPR)
                p[c] = (c < len) ? (T)(exp2f(((float)p[c] - M) * kLog2e) * inv) : (T)0.f;
        }
    }
}

// ---------------------------------------------------------------- 3. O = P V
template <int D>
struct PvTile {
    static constexpr int BM = 128;                 // queries per workgroup (4 waves x 32)
    static constexpr int BN = 64;                  // keys per V tile
    static constexpr int ROWB = 2 * D;
    static constexpr int TILEB = BN * ROWB;
    static constexpr int NLOAD = TILEB / (256 * 16);
    static constexpr int DB = D / 32;
    static_assert(NLOAD >= 1 && TILEB % (256 * 16) == 0, "V tile must split into whole loads");
};

// One wavefront: 32 queries, all head dims; O^T = V^T P^T over the key tiles.
// STAGED (N % 8 == 0, rows of P 16-byte aligned): the workgroup's 128 x 64
// tile of P is brought into LDS with whole-row direct loads, 16-byte chunk c
// of row r stored at chunk position c ^ ((r / 2) % 8) so that the operand
// reads (16 rows, one chunk each) hit every bank once; otherwise every lane
// reads its 8 probabilities straight from memory.
template <typename T, int D, bool STAGED>
struct PvWave {
    using C = PvTile<D>;
    using V8 = typename Vec<T>::x8;
    using V4 = typename Vec<T>::x4;
    static constexpr int PTILEB = C::BM * C::BN * 2;   // bytes of one P tile
    static constexpr int NLOADP = PTILEB / 4096;
    const T* Vh;
    const T* Ph;    // first row of the workgroup's queries
    const T* prow;  // this lane's query row
    int N, tid, wave, lane, h, q, q_first;
    int ld_row[C::NLOAD], ld_col[C::NLOAD];
    int lp_row[NLOADP], lp_col[NLOADP];
    int voff[2][C::DB];
    f32x16 oacc[C::DB];

    __device__ __forceinline__ void init(const T* P, const T* V, int N_, int bh, int qb) {
        N = N_;
        tid = threadIdx.x;
        lane = tid & 63;
        wave = tid >> 6;
        h = lane >> 5;
        q_first = qb * C::BM;
        q = q_first + 32 * wave + (lane & 31);
        Vh = V + (size_t)bh * N * D;
        Ph = P + (size_t)bh * N * (size_t)N;
        prow = Ph + (size_t)min(q, N - 1) * N;
#pragma unroll
        for (int i = 0; i < C::NLOAD; ++i) {
            const int byte = i * 4096 + tid * 16;
            const int r = byte / C::ROWB, c = (byte % C::ROWB) / 16;
            ld_row[i] = r;
            ld_col[i] = (c ^ tile_swz<D>(r)) * 8;
        }
#pragma unroll
        for (int i = 0; i < NLOADP; ++i) {
            const int byte = i * 4096 + tid * 16;
            const int r = byte / 128, pos = (byte % 128) / 16;
            lp_row[i] = r;
            lp_col[i] = (pos ^ ((r >> 1) & 7)) * 8;
        }
        // transposing reads of V^T in natural key order: for key group g and
        // half hf this lane supplies row 16 g + 8 h + 4 hf + (lane % 16) / 4 and
        // head dims 32 b + 16 ((lane / 16) % 2) + 4 (lane % 4); it receives head
        // dim 32 b + lane % 32 at keys 16 g + 8 h + 4 hf + 0..3.
        const int src_r = 8 * h + (lane & 15) / 4;
        const int src_d = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
            for (int b = 0; b < C::DB; ++b) voff[hf][b] = tile_off<D>(src_r + 4 * hf, 32 * b + src_d);
#pragma unroll
        for (int b = 0; b < C::DB; ++b) oacc[b] = f32x16{};
    }

    __device__ __forceinline__ void issue(int kbase, char* vdst, char* pdst) const {
#pragma unroll
        for (int i = 0; i < C::NLOAD; ++i) {
            const size_t row = (size_t)min(kbase + ld_row[i], N - 1) * D;
            __builtin_amdgcn_global_load_lds(Vh + row + ld_col[i], vdst + i * 4096 + wave * 1024,
                                             16, 0, 0);
        }
        if (STAGED) {
#pragma unroll
            for (int i = 0; i < NLOADP; ++i) {
                const size_t row = (size_t)min(q_first + lp_row[i], N - 1) * N;
                const int key = kbase + lp_col[i];
                // chunks past the last key read column 0 and are zeroed when used
                __builtin_amdgcn_global_load_lds(Ph + row + (key < N ? key : 0),
                                                 pdst + i * 4096 + wave * 1024, 16, 0, 0);
            }
        }
    }

    __device__ __forceinline__ void tile(int kbase, const char* vb, const char* pb) {
        const int ql = 32 * wave + (lane & 31);  // query row inside the P tile
#pragma unroll
        for (int g = 0; g < C::BN / 16; ++g) {
            const int cc = 2 * g + h;              // this lane's 8-key chunk
            const int k = kbase + 8 * cc;
            V8 pf;
            if (STAGED) {
                pf = *reinterpret_cast<const V8*>(pb + ql * 128 + 16 * (cc ^ ((ql >> 1) & 7)));
                if (k >= N) pf = V8{};
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j) pf[j] = (k + j < N) ? prow[k + j] : (T)0.f;
            }
            const char* vg = vb + g * 16 * C::ROWB;
#pragma unroll
            for (int b = 0; b < C::DB; ++b) {
                const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vg + voff[0][b]));
                const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vg + voff[1][b]));
                const s16x4 w[2] = {lo, hi};
                V8 a;
                __builtin_memcpy(&a, w, sizeof(a));
                oacc[b] = mfma32(a, pf, oacc[b]);
            }
        }
    }

    __device__ __forceinline__ void finish(T* O, int bh) const {
        if (q >= N) return;
        T* orow = O + ((size_t)bh * N + q) * D;
#pragma unroll
        for (int b = 0; b < C::DB; ++b)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                V4 w;
#pragma unroll
                for (int i = 0; i < 4; ++i) w[i] = (T)oacc[b][4 * r4 + i];
                *reinterpret_cast<V4*>(orow + 32 * b + 8 * r4 + 4 * h) = w;
            }
    }
};

template <typename T, int D, bool STAGED>
__global__ void __launch_bounds__(256)
std_pv_kernel(const T* __restrict__ P, const T* __restrict__ V, T* __restrict__ O, int N,
              int nqb) {
    using C = PvTile<D>;
    using W = PvWave<T, D, STAGED>;
    __shared__ __attribute__((aligned(1024))) char sV0[C::TILEB];
    __shared__ __attribute__((aligned(1024))) char sV1[C::TILEB];
    __shared__ __attribute__((aligned(1024))) char sP0[STAGED ? W::PTILEB : 16];
    __shared__ __attribute__((aligned(1024))) char sP1[STAGED ? W::PTILEB : 16];
    const int bh = blockIdx.x / nqb, qb = blockIdx.x % nqb;
    W w;
    w.init(P, V, N, bh, qb);
    const int nkt = (N + C::BN - 1) / C::BN;
    w.issue(0, sV0, sP0);
    if constexpr (kSerialStaging) {
        for (int kt = 0; kt < nkt; ++kt) {
            __builtin_amdgcn_s_waitcnt(kVmcntZero);
            __syncthreads();
            w.tile(kt * C::BN, sV0, sP0);
            __syncthreads();
            if (kt + 1 < nkt) w.issue((kt + 1) * C::BN, sV0, sP0);
        }
    } else {
        for (int kt = 0; kt < nkt; kt += 2) {
            __builtin_amdgcn_s_waitcnt(kVmcntZero);
            __syncthreads();
            if (kt + 1 < nkt) w.issue((kt + 1) * C::BN, sV1, sP1);
            w.tile(kt * C::BN, sV0, sP0);
            if (kt + 1 < nkt) {
                __builtin_amdgcn_s_waitcnt(kVmcntZero);
                __syncthreads();
                if (kt + 2 < nkt) w.issue((kt + 2) * C::BN, sV0, sP0);
                w.tile((kt + 1) * C::BN, sV1, sP1);
            }
        }
    }
    w.finish(O, bh);
}

template <typename T, int D>
hipError_t launch_std_typed(bool causal, const void* q, const void* k, const void* v, void* o,
                            void* s, int BH, int N, float scale, hipStream_t stream) {
    const int ntile = (N + 127) / 128;
    hipLaunchKernelGGL((std_scores_kernel<T, D>), dim3(ntile * ntile, BH), dim3(256), 0, stream,
                       static_cast<const T*>(q), static_cast<const T*>(k), static_cast<T*>(s), N,
                       ntile, scale);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // short rows: one wavefront per row; long rows: one workgroup per row
    const long long rows = (long long)BH * N;
    if (N <= kSoftmaxChunks * 8 * 64) {
        const long long wgs = (rows + 3) / 4;
        hipLaunchKernelGGL((std_softmax_kernel<T, 4>), dim3((unsigned)min(wgs, 256LL * 16)),
                           dim3(256), 0, stream, static_cast<T*>(s), N, rows, causal ? 1 : 0);
    } else {
        hipLaunchKernelGGL((std_softmax_kernel<T, 1>), dim3((unsigned)min(rows, 256LL * 8)),
                           dim3(256), 0, stream, static_cast<T*>(s), N, rows, causal ? 1 : 0);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int nqb = (N + PvTile<D>::BM - 1) / PvTile<D>::BM;
    if (N % 8 == 0)
        hipLaunchKernelGGL((std_pv_kernel<T, D, true>), dim3(BH * nqb), dim3(256), 0, stream,
                           static_cast<const T*>(s), static_cast<const T*>(v),
                           static_cast<T*>(o), N, nqb);
    else
        hipLaunchKernelGGL((std_pv_kernel<T, D, false>), dim3(BH * nqb), dim3(256), 0, stream,
                           static_cast<const T*>(s), static_cast<const T*>(v),
                           static_cast<T*>(o), N, nqb);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_std_d(int d, bool causal, const void* q, const void* k, const void* v, void* o,
                        void* s, int BH, int N, float scale, hipStream_t stream) {
    if (d == 64) return launch_std_typed<T, 64>(causal, q, k, v, o, s, BH, N, scale, stream);
    return launch_std_typed<T, 128>(causal, q, k, v, o, s, BH, N, scale, stream);
}

}  // namespace

hipError_t launch_std(int dtype, int d, bool causal, const void* q, const void* k, const void* v,
                      void* o, void* s, int BH, int N, float scale, hipStream_t stream) {
    if (dtype == 2) return launch_std_d<__bf16>(d, causal, q, k, v, o, s, BH, N, scale, stream);
    return launch_std_d<_Float16>(d, causal, q, k, v, o, s, BH, N, scale, stream);
}

}  // namespace fa
