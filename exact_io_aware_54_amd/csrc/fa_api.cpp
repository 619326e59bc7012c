// C ABI of libfa (declared in include/fa.h): argument validation, dispatch on
// (dtype, head dim, causal) and launch on the caller's stream. Nothing is
// launched when an argument is invalid.

#include "../../include/fa.h"

#include <math.h>
#include <stdint.h>

#include "fa_launch.h"

namespace {

constexpr int kVersion = 100;  // 0.1.0

// Shape checks shared by the entry points; head dims 64 and 128 everywhere,
// 256 only where the caller allows it (the 16-bit forward and backward).
// Every kernel runs a one-dimensional grid of at most 512 work-items per 32
// rows of each head (B*H*ceil(N/32)*512 in the worst case), and HIP refuses a
// grid dimension of 2^32 work-items or more: that bounds B*H*ceil(N/32) below
// 2^23, which matters only for very short sequences (N <= 2 with d = 64
// would otherwise allow B*H up to 2^25).
// a * b * ... < limit for positive int factors, without overflowing (each
// partial product is checked before the next multiplication).
template <typename... I>
bool product_below(int64_t limit, int a, I... rest) {
    int64_t p = a;
    if (p >= limit) return false;
    for (int f : {rest...}) {
        p *= f;  // p < 2^31 and f < 2^31: no overflow
        if (p >= limit) return false;
    }
    return true;
}

int check_shape(int B, int H, int N, int d, bool allow256 = false) {
    if (B < 1 || H < 1 || N < 1) return FA_ERR_SHAPE;
    if (d != 64 && d != 128 && !(allow256 && d == 256)) return FA_ERR_HEADDIM;
    if (!product_below((int64_t)1 << 31, B, H, N, d)) return FA_ERR_SHAPE;
    if ((int64_t)B * H * ((N + 31) / 32) >= ((int64_t)1 << 23)) return FA_ERR_SHAPE;
    return FA_OK;
}

// Launch failures are read back with hipGetLastError after each launch. An
// error left pending by earlier, unrelated HIP calls of this host thread
// would otherwise be reported as this call's: read (and so clear) it once,
// after validation and before the first launch.
void clear_pending_error() { (void)hipGetLastError(); }

bool good_scale(float s) { return isfinite(s) && s > 0.f; }

int status_of(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_HIP; }

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// The kernels move tensors in 16-byte vectors: every [.., N, d] tensor must
// start on a 16-byte boundary, float32 row statistics on a 4-byte one.
template <typename... P>
bool aligned16(const P*... p) {
    return ((((uintptr_t)p & 15) == 0) && ...);
}
bool aligned4(const float* p) { return ((uintptr_t)p & 3) == 0; }

// Key ranges of fa_fwd_splitkv: whole 128-key tiles, as evenly as possible.
// num_splits = 0 picks enough ranges for about two workgroups per CU.
struct SplitPlan {
    int splits;  // ranges actually used
    int kps;     // keys per range (a multiple of 128)
};

int splitkv_shape(int B, int H, int Nq, int Nk, int d, int num_splits) {
    if (B < 1 || H < 1 || Nq < 1 || Nk < 1) return FA_ERR_SHAPE;
    if (d != 64 && d != 128) return FA_ERR_HEADDIM;
    if (!product_below((int64_t)1 << 31, B, H, Nq, d) || !product_below((int64_t)1 << 31, B, H, Nk, d))
        return FA_ERR_SHAPE;
    const int64_t bh = (int64_t)B * H;
    // the merge and split kernels' grids: see check_shape
    if (bh * ((Nq + 31) / 32) >= ((int64_t)1 << 23)) return FA_ERR_SHAPE;
    if (num_splits < 0 || num_splits > 1024) return FA_ERR_ARG;
    return FA_OK;
}

SplitPlan splitkv_plan(int B, int H, int Nq, int Nk, int num_splits) {
    const int tiles = (Nk + 127) / 128;
    const int64_t units = (int64_t)B * H * ((Nq + 31) / 32);
    int want = num_splits;
    if (want == 0) want = (int)((512 + units - 1) / units);
    want = want < 1 ? 1 : (want > tiles ? tiles : want);
    const int tps = (tiles + want - 1) / want;
    return SplitPlan{(tiles + tps - 1) / tps, tps * 128};
}

}  // namespace

extern "C" {

int fa_version(void) { return kVersion; }

int fa_build_flags(void) {
#ifdef FA_SERIAL_STAGING
    return FA_BUILD_SERIAL_STAGING;
#else
    return 0;
#endif
}

const char* fa_status_string(int status) {
    switch (status) {
        case FA_OK: return "ok";
        case FA_ERR_NULL: return "a required pointer is NULL";
        case FA_ERR_SHAPE: return "invalid shape (B, H, N must be >= 1, B*H*N*d < 2^31 and B*H*ceil(N/32) < 2^23)";
        case FA_ERR_DTYPE: return "dtype not supported by this entry point";
        case FA_ERR_HEADDIM: return "head dim not supported";
        case FA_ERR_WORKSPACE: return "workspace too small";
        case FA_ERR_HIP: return "HIP runtime error at launch";
        case FA_ERR_ARG: return "invalid scalar argument (scale, descale, split count) or misaligned pointer";
        case FA_ERR_TOO_LARGE: return "problem larger than the library's fixed scratch (fa_bwd_noalloc: B*H*N above fa_bwd_noalloc_max_rows())";
        default: return "unknown status";
    }
}

int fa_fwd(int dtype, const void* q, const void* k, const void* v, void* o, float* lse, int B,
           int H, int N, int d, float scale, int causal, hipStream_t stream) {
    if (!q || !k || !v || !o) return FA_ERR_NULL;
    if (dtype != FA_F32 && dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_DTYPE;
    const int st = check_shape(B, H, N, d, dtype != FA_F32);
    if (st != FA_OK) return st;
    if (!good_scale(scale)) return FA_ERR_ARG;
    if (!aligned16(q, k, v, o) || !aligned4(lse)) return FA_ERR_ARG;
    const int BH = B * H;
    clear_pending_error();
    if (dtype == FA_F32)
        return status_of(fa::launch_fwd_f32(d, causal != 0, static_cast<const float*>(q),
                                            static_cast<const float*>(k),
                                            static_cast<const float*>(v), static_cast<float*>(o),
                                            lse, BH, N, scale, stream));
    return status_of(
        fa::launch_fwd_mfma(dtype, d, causal != 0, q, k, v, o, lse, BH, N, scale, 0, stream));
}

int fa_fwd_waves(int dtype, const void* q, const void* k, const void* v, void* o, float* lse,
                 int B, int H, int N, int d, float scale, int causal, int waves,
                 hipStream_t stream) {
    if (!q || !k || !v || !o) return FA_ERR_NULL;
    if (dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_DTYPE;
    const int st = check_shape(B, H, N, d, true);
    if (st != FA_OK) return st;
    if (!good_scale(scale)) return FA_ERR_ARG;
    if (!aligned16(q, k, v, o) || !aligned4(lse)) return FA_ERR_ARG;
    if (waves != 0 && waves != 4 && waves != 8) return FA_ERR_ARG;
    if (d == 256 && waves == 8) return FA_ERR_ARG;
    clear_pending_error();
    return status_of(fa::launch_fwd_mfma(dtype, d, causal != 0, q, k, v, o, lse, B * H, N, scale,
                                         waves, stream));
}

int fa_fwd_fp8(const void* q8, const void* k8, const void* v8, float q_descale, float k_descale,
               float v_descale, void* o_bf16, float* lse, int B, int H, int N, int d,
               float scale, int causal, hipStream_t stream) {
    if (!q8 || !k8 || !v8 || !o_bf16) return FA_ERR_NULL;
    const int st = check_shape(B, H, N, d);
    if (st != FA_OK) return st;
    if (d != 128) return FA_ERR_HEADDIM;
    if (!good_scale(scale) || !good_scale(q_descale) || !good_scale(k_descale) ||
        !good_scale(v_descale))
        return FA_ERR_ARG;
    const float qk = scale * q_descale * k_descale;
    if (!good_scale(qk)) return FA_ERR_ARG;
    if (!aligned16(q8, k8, v8, o_bf16) || !aligned4(lse)) return FA_ERR_ARG;
    clear_pending_error();
    return status_of(fa::launch_fwd_fp8(d, causal != 0, q8, k8, v8, qk, v_descale, o_bf16, lse,
                                        B * H, N, stream));
}

size_t fa_bwd_workspace_bytes(int B, int H, int N, int d) {
    if (check_shape(B, H, N, d, true) != FA_OK) return 0;
    const size_t rows = (size_t)B * H * N;
    return 2 * align256(rows * sizeof(float));  // D and LSE * log2(e), one float per row each
}

namespace {
// Validation shared by the backward entry points (everything but
// the workspace).
int bwd_check(int dtype, const void* q, const void* k, const void* v, const void* o,
              const float* lse, const void* dO, void* dq, void* dk, void* dv, int B, int H, int N,
              int d, float scale) {
    if (!q || !k || !v || !o || !lse || !dO || !dq || !dk || !dv) return FA_ERR_NULL;
    if (dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_DTYPE;
    const int st = check_shape(B, H, N, d, true);
    if (st != FA_OK) return st;
    if (!good_scale(scale)) return FA_ERR_ARG;
    if (!aligned16(q, k, v, o, dO, dq, dk, dv) || !aligned4(lse)) return FA_ERR_ARG;
    return FA_OK;
}

int bwd_common(int dtype, const void* q, const void* k, const void* v, const void* o,
               const float* lse, const void* dO, void* dq, void* dk, void* dv, void* workspace,
               size_t workspace_bytes, int B, int H, int N, int d, float scale, int causal,
               int stages, hipStream_t stream) {
    const int st = bwd_check(dtype, q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d, scale);
    if (st != FA_OK) return st;
    if (!workspace) return FA_ERR_NULL;
    if (workspace_bytes < fa_bwd_workspace_bytes(B, H, N, d)) return FA_ERR_WORKSPACE;
    if (((uintptr_t)workspace & 255) != 0) return FA_ERR_WORKSPACE;
    const size_t rows = (size_t)B * H * N;
    float* delta = static_cast<float*>(workspace);
    float* lse2 = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                           align256(rows * sizeof(float)));
    clear_pending_error();
    return status_of(fa::launch_bwd(dtype, d, causal != 0, q, k, v, o, lse, dO, dq, dk, dv,
                                    delta, lse2, B * H, N, scale, stages, stream));
}
}  // namespace

int fa_bwd(int dtype, const void* q, const void* k, const void* v, const void* o,
           const float* lse, const void* dO, void* dq, void* dk, void* dv, void* workspace,
           size_t workspace_bytes, int B, int H, int N, int d, float scale, int causal,
           hipStream_t stream) {
    return bwd_common(dtype, q, k, v, o, lse, dO, dq, dk, dv, workspace, workspace_bytes, B, H, N,
                      d, scale, causal, 7, stream);
}

int fa_bwd_stage(int stage, int dtype, const void* q, const void* k, const void* v,
                 const void* o, const float* lse, const void* dO, void* dq, void* dk, void* dv,
                 void* workspace, size_t workspace_bytes, int B, int H, int N, int d,
                 float scale, int causal, hipStream_t stream) {
    if (stage < 1 || stage > 3) return FA_ERR_ARG;
    return bwd_common(dtype, q, k, v, o, lse, dO, dq, dk, dv, workspace, workspace_bytes, B, H, N,
                      d, scale, causal, 1 << (stage - 1), stream);
}

int fa_bwd_noalloc(int dtype, const void* q, const void* k, const void* v, const void* o,
                   const float* lse, const void* dO, void* dq, void* dk, void* dv, int B, int H,
                   int N, int d, float scale, int causal, hipStream_t stream) {
    const int st = bwd_check(dtype, q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d, scale);
    if (st != FA_OK) return st;
    if ((size_t)B * H * N > fa::kNoallocMaxRows) return FA_ERR_TOO_LARGE;
    // the scratch is per device: the current one, which must own the stream
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return FA_ERR_HIP;
    if (stream != nullptr) {
        hipDevice_t sdev = -1;
        if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return FA_ERR_HIP;
        if (sdev != dev) return FA_ERR_ARG;
    }
    float* delta = nullptr;
    float* lse2 = nullptr;
    if (fa::noalloc_scratch(dev, &delta, &lse2) != hipSuccess) return FA_ERR_HIP;
    clear_pending_error();
    return status_of(fa::launch_bwd(dtype, d, causal != 0, q, k, v, o, lse, dO, dq, dk, dv,
                                    delta, lse2, B * H, N, scale, 7, stream));
}

size_t fa_bwd_noalloc_max_rows(void) { return fa::kNoallocMaxRows; }

size_t fa_bwd_fp8_workspace_bytes(int B, int H, int N, int d) {
    if (check_shape(B, H, N, d, true) != FA_OK) return 0;
    const size_t el = (size_t)B * H * N * d;
    return 3 * align256(el * 2) + fa_bwd_workspace_bytes(B, H, N, d);
}

int fa_bwd_fp8(const void* q8, const void* k8, const void* v8, float q_descale, float k_descale,
               float v_descale, const void* o_bf16, const float* lse, const void* dO_bf16,
               void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes, int B,
               int H, int N, int d, float scale, int causal, hipStream_t stream) {
    if (!q8 || !k8 || !v8 || !o_bf16 || !lse || !dO_bf16 || !dq || !dk || !dv || !workspace)
        return FA_ERR_NULL;
    const int st = check_shape(B, H, N, d, true);
    if (st != FA_OK) return st;
    if (!good_scale(scale) || !good_scale(q_descale) || !good_scale(k_descale) ||
        !good_scale(v_descale))
        return FA_ERR_ARG;
    const float c = scale * q_descale * k_descale * 1.4426950408889634f;
    const float dk_mul = scale * q_descale * v_descale, dq_mul = scale * k_descale * v_descale;
    const float d_mul = 1.f / v_descale;
    if (!good_scale(c) || !good_scale(dk_mul) || !good_scale(dq_mul) || !good_scale(d_mul))
        return FA_ERR_ARG;
    if (!aligned16(q8, k8, v8, o_bf16, dO_bf16, dq, dk, dv) || !aligned4(lse)) return FA_ERR_ARG;
    if (workspace_bytes < fa_bwd_fp8_workspace_bytes(B, H, N, d)) return FA_ERR_WORKSPACE;
    if (((uintptr_t)workspace & 255) != 0) return FA_ERR_WORKSPACE;
    const size_t el = (size_t)B * H * N * d, rows = (size_t)B * H * N;
    char* ws = static_cast<char*>(workspace);
    void* qc = ws;
    void* kc = ws + align256(el * 2);
    void* vc = ws + 2 * align256(el * 2);
    float* delta = reinterpret_cast<float*>(ws + 3 * align256(el * 2));
    float* lse2 = reinterpret_cast<float*>(ws + 3 * align256(el * 2) + align256(rows * 4));
    hipError_t e;
    clear_pending_error();
    if ((e = fa::launch_e4m3_to_bf16(q8, qc, el, stream)) != hipSuccess) return FA_ERR_HIP;
    if ((e = fa::launch_e4m3_to_bf16(k8, kc, el, stream)) != hipSuccess) return FA_ERR_HIP;
    if ((e = fa::launch_e4m3_to_bf16(v8, vc, el, stream)) != hipSuccess) return FA_ERR_HIP;
    const fa::BwdScales sc{c, dk_mul, dq_mul, d_mul};
    return status_of(fa::launch_bwd_scaled(FA_BF16, d, causal != 0, qc, kc, vc, o_bf16, lse,
                                           dO_bf16, dq, dk, dv, delta, lse2, B * H, N, sc, 7,
                                           stream));
}

int fa_probe_mfma(unsigned long long* sink, int blocks, int iters, hipStream_t stream) {
    if (!sink) return FA_ERR_NULL;
    if (blocks < 1 || blocks > 65536 || iters < 1 || iters > (1 << 24)) return FA_ERR_ARG;
    if (((uintptr_t)sink & 7) != 0) return FA_ERR_ARG;
    clear_pending_error();
    return status_of(fa::launch_mfma_probe(sink, blocks, iters, stream));
}

int fa_probe_dq_atomics(float* ws, size_t ws_bytes, int B, int H, int N, int key_block,
                        int mode, int causal, hipStream_t stream) {
    if (!ws) return FA_ERR_NULL;
    if (B < 1 || H < 1 || N < 64 || N % 64 != 0) return FA_ERR_SHAPE;
    if (key_block != 128 && key_block != 256) return FA_ERR_ARG;
    if (N % key_block != 0) return FA_ERR_SHAPE;
    if (mode != 0 && mode != 1) return FA_ERR_ARG;
    if (!product_below((int64_t)1 << 31, B, H, N, 128)) return FA_ERR_SHAPE;
    const int64_t el = (int64_t)B * H * N * 128;
    if ((int64_t)B * H * (N / key_block) * 512 >= ((int64_t)1 << 32)) return FA_ERR_SHAPE;
    if (ws_bytes < (size_t)el * sizeof(float)) return FA_ERR_WORKSPACE;
    if (((uintptr_t)ws & 255) != 0) return FA_ERR_WORKSPACE;
    clear_pending_error();
    return status_of(fa::launch_dq_atomic_probe(ws, B * H, N, key_block, mode, causal != 0,
                                                stream));
}

size_t fa_fwd_splitkv_workspace_bytes(int B, int H, int Nq, int Nk, int d, int num_splits) {
    if (splitkv_shape(B, H, Nq, Nk, d, num_splits) != FA_OK) return 0;
    const SplitPlan pl = splitkv_plan(B, H, Nq, Nk, num_splits);
    const size_t rows = (size_t)pl.splits * B * H * Nq;
    return align256(rows * d * sizeof(float)) + align256(rows * sizeof(float));
}

int fa_fwd_splitkv(int dtype, const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int H, int Nq, int Nk, int d, float scale, int causal, int num_splits,
                   void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (!q || !k || !v || !o || !workspace) return FA_ERR_NULL;
    if (dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_DTYPE;
    const int st = splitkv_shape(B, H, Nq, Nk, d, num_splits);
    if (st != FA_OK) return st;
    if (causal && Nq > Nk) return FA_ERR_SHAPE;
    if (!good_scale(scale)) return FA_ERR_ARG;
    if (!aligned16(q, k, v, o) || !aligned4(lse)) return FA_ERR_ARG;
    if (workspace_bytes < fa_fwd_splitkv_workspace_bytes(B, H, Nq, Nk, d, num_splits))
        return FA_ERR_WORKSPACE;
    if (((uintptr_t)workspace & 255) != 0) return FA_ERR_WORKSPACE;
    const SplitPlan pl = splitkv_plan(B, H, Nq, Nk, num_splits);
    const int BH = B * H;
    // one workgroup of 256 work-items per (batch*head, 32 queries, key range)
    if ((int64_t)BH * ((Nq + 31) / 32) * pl.splits * 256 >= ((int64_t)1 << 32)) return FA_ERR_SHAPE;
    const size_t rows = (size_t)pl.splits * BH * Nq;
    float* o_part = static_cast<float*>(workspace);
    float* lse_part = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                               align256(rows * d * sizeof(float)));
    clear_pending_error();
    return status_of(fa::launch_fwd_splitkv(dtype, d, causal != 0, q, k, v, o, lse, o_part,
                                            lse_part, BH, Nq, Nk, pl.splits, pl.kps, scale,
                                            stream));
}

int fa_lse_merge(int dtype_out, int num_parts, const float* o_parts, const float* lse_parts,
                 void* o, float* lse, int rows, int d, hipStream_t stream) {
    if (!o_parts || !lse_parts || !o) return FA_ERR_NULL;
    if (dtype_out != FA_F32 && dtype_out != FA_F16 && dtype_out != FA_BF16) return FA_ERR_DTYPE;
    if (num_parts < 1 || rows < 1 || d < 4 || d % 4 != 0 || d > 65536) return FA_ERR_SHAPE;
    // one work-item per 4 output elements, in a one-dimensional grid
    if ((int64_t)rows * (d / 4) > ((int64_t)1 << 32) - 256) return FA_ERR_SHAPE;
    if (!aligned16(o_parts) || !aligned4(lse_parts) || !aligned4(lse)) return FA_ERR_ARG;
    if (((uintptr_t)o & (dtype_out == FA_F32 ? 3 : 1)) != 0) return FA_ERR_ARG;
    clear_pending_error();
    return status_of(fa::launch_lse_merge(dtype_out, o_parts, lse_parts, num_parts, rows, d, o, lse,
                                          stream));
}

size_t fa_fwd_v1_workspace_bytes(int B, int H, int N, int d) {
    if (check_shape(B, H, N, d) != FA_OK) return 0;
    const size_t rows = (size_t)B * H * N;
    return align256(rows * d * sizeof(float)) + 2 * align256(rows * 2 * sizeof(float));
}

int fa_fwd_v1(int dtype, const void* q, const void* k, const void* v, void* o, float* lse,
              void* workspace, size_t workspace_bytes, int B, int H, int N, int d, float scale,
              int causal, hipStream_t stream) {
    if (!q || !k || !v || !o || !workspace) return FA_ERR_NULL;
    if (dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_DTYPE;
    const int st = check_shape(B, H, N, d);
    if (st != FA_OK) return st;
    if (!good_scale(scale)) return FA_ERR_ARG;
    if (!aligned16(q, k, v, o) || !aligned4(lse)) return FA_ERR_ARG;
    if (workspace_bytes < fa_fwd_v1_workspace_bytes(B, H, N, d)) return FA_ERR_WORKSPACE;
    if (((uintptr_t)workspace & 255) != 0) return FA_ERR_WORKSPACE;
    const size_t rows = (size_t)B * H * N;
    char* ws = static_cast<char*>(workspace);
    float* ows = reinterpret_cast<float*>(ws);
    float* mws = reinterpret_cast<float*>(ws + align256(rows * d * sizeof(float)));
    float* lws = reinterpret_cast<float*>(ws + align256(rows * d * sizeof(float)) +
                                          align256(rows * 2 * sizeof(float)));
    clear_pending_error();
    return status_of(fa::launch_fwd_v1(dtype, d, causal != 0, q, k, v, o, lse, ows, mws, lws,
                                       B * H, N, scale, stream));
}

size_t fa_std_workspace_bytes(int B, int H, int N, int d) {
    if (check_shape(B, H, N, d) != FA_OK) return 0;
    return (size_t)B * H * N * (size_t)N * 2;  // one 16-bit N x N matrix per head
}

int fa_std_fwd(int dtype, const void* q, const void* k, const void* v, void* o, void* workspace,
               size_t workspace_bytes, int B, int H, int N, int d, float scale, int causal,
               hipStream_t stream) {
    if (!q || !k || !v || !o || !workspace) return FA_ERR_NULL;
    if (dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_DTYPE;
    const int st = check_shape(B, H, N, d);
    if (st != FA_OK) return st;
    if ((int64_t)B * H > 65535) return FA_ERR_SHAPE;
    // the score pass has one 256-work-item workgroup per 128 x 128 tile of a head
    const int64_t ntile = (N + 127) / 128;
    if (ntile * ntile * 256 >= ((int64_t)1 << 32)) return FA_ERR_SHAPE;
    if (!good_scale(scale)) return FA_ERR_ARG;
    if (!aligned16(q, k, v, o)) return FA_ERR_ARG;
    if (workspace_bytes < fa_std_workspace_bytes(B, H, N, d)) return FA_ERR_WORKSPACE;
    if (((uintptr_t)workspace & 255) != 0) return FA_ERR_WORKSPACE;
    clear_pending_error();
    return status_of(
        fa::launch_std(dtype, d, causal != 0, q, k, v, o, workspace, B * H, N, scale, stream));
}

}  // extern "C"
