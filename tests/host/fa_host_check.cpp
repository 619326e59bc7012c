// Drives every entry point of libfa's C ABI layer (csrc/fa_api.cpp) with the
// kernel launchers replaced by recording stand-ins (fa_host_stubs.cpp), built
// with AddressSanitizer and UndefinedBehaviorSanitizer. Checks: the documented
// status for invalid arguments, with nothing launched; the launch arguments of
// valid calls, including that every sub-buffer carved out of a workspace lies
// inside the size the matching *_workspace_bytes function reports and that
// the sub-buffers do not overlap; the error state (a pending error from
// earlier work is not reported as this call's, a launch failure is); and
// extreme sizes, where the sanitizers watch the size arithmetic for signed
// overflow. Prints one line per failed check and exits non-zero if any failed.

#include <limits.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>

#include "../../include/fa.h"
#include "fa_host_stubs.h"

using fa::g_rec;

static int g_checks = 0, g_failed = 0;

#define CHECK(cond)                                                          \
    do {                                                                     \
        ++g_checks;                                                          \
        if (!(cond)) {                                                       \
            ++g_failed;                                                      \
            fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
        }                                                                    \
    } while (0)

// Status of a call that must not launch anything.
#define REJECTS(call, status)                   \
    do {                                        \
        const int before_ = g_rec.calls;        \
        CHECK((call) == (status));              \
        CHECK(g_rec.calls == before_);          \
    } while (0)

static void* P(int i) { return (void*)(uintptr_t)(0x10000000ull * (uint64_t)(i + 1)); }
static float* F(int i) { return (float*)P(i); }
static char* C(void* p) { return (char*)p; }
static size_t a256(size_t x) { return (x + 255) & ~(size_t)255; }
static const hipStream_t kStream = (hipStream_t)(uintptr_t)0x5000;

// [p, p + n) inside [base, base + size)
static bool inside(const void* p, size_t n, const void* base, size_t size) {
    return C((void*)p) >= C((void*)base) && C((void*)p) + n <= C((void*)base) + size;
}
static bool disjoint(const void* a, size_t na, const void* b, size_t nb) {
    return C((void*)a) + na <= C((void*)b) || C((void*)b) + nb <= C((void*)a);
}

static void status_and_version() {
    CHECK(fa_version() >= 100);
    CHECK(fa_build_flags() == 0);
    for (int s = -10; s <= 1; ++s) CHECK(fa_status_string(s) != nullptr && fa_status_string(s)[0]);
}

static void forward() {
    // valid: 16-bit and fp32 paths, arguments passed through
    CHECK(fa_fwd(FA_BF16, P(0), P(1), P(2), P(3), F(4), 2, 3, 100, 128, 0.1f, 1, kStream) == FA_OK);
    CHECK(g_rec.arg[0] == 6 && g_rec.arg[1] == 100 && g_rec.arg[2] == 128);
    CHECK(g_rec.ptr[0] == P(0) && g_rec.ptr[3] == P(3) && g_rec.ptr[4] == P(4));
    CHECK(fa_fwd(FA_F32, P(0), P(1), P(2), P(3), nullptr, 1, 2, 128, 64, 0.1f, 0, kStream) == FA_OK);
    CHECK(g_rec.ptr[4] == nullptr);
    CHECK(fa_fwd(FA_F16, P(0), P(1), P(2), P(3), F(4), 1, 1, 1, 256, 0.1f, 0, kStream) == FA_OK);
    // invalid: nothing launched
    REJECTS(fa_fwd(FA_BF16, nullptr, P(1), P(2), P(3), F(4), 1, 1, 64, 64, 0.1f, 0, kStream), FA_ERR_NULL);
    REJECTS(fa_fwd(FA_BF16, P(0), P(1), P(2), nullptr, F(4), 1, 1, 64, 64, 0.1f, 0, kStream), FA_ERR_NULL);
    REJECTS(fa_fwd(7, P(0), P(1), P(2), P(3), F(4), 1, 1, 64, 64, 0.1f, 0, kStream), FA_ERR_DTYPE);
    REJECTS(fa_fwd(FA_BF16, P(0), P(1), P(2), P(3), F(4), 1, 1, 64, 96, 0.1f, 0, kStream), FA_ERR_HEADDIM);
    REJECTS(fa_fwd(FA_F32, P(0), P(1), P(2), P(3), F(4), 1, 1, 64, 256, 0.1f, 0, kStream), FA_ERR_HEADDIM);
    REJECTS(fa_fwd(FA_BF16, P(0), P(1), P(2), P(3), F(4), 0, 1, 64, 64, 0.1f, 0, kStream), FA_ERR_SHAPE);
    REJECTS(fa_fwd(FA_BF16, P(0), P(1), P(2), P(3), F(4), 1, -3, 64, 64, 0.1f, 0, kStream), FA_ERR_SHAPE);
    REJECTS(fa_fwd(FA_BF16, P(0), P(1), P(2), P(3), F(4), 1 << 14, 1 << 10, 1 << 10, 128, 0.1f, 0, kStream), FA_ERR_SHAPE);
    REJECTS(fa_fwd(FA_BF16, P(0), P(1), P(2), P(3), F(4), INT_MAX, INT_MAX, INT_MAX, 128, 0.1f, 0, kStream), FA_ERR_SHAPE);
    REJECTS(fa_fwd(FA_BF16, P(0), P(1), P(2), P(3), F(4), 1 << 12, 1 << 11, 1, 64, 0.1f, 0, kStream), FA_ERR_SHAPE);
    REJECTS(fa_fwd(FA_BF16, P(0), P(1), P(2), P(3), F(4), 1, 1, 64, 64, 0.f, 0, kStream), FA_ERR_ARG);
    REJECTS(fa_fwd(FA_BF16, P(0), P(1), P(2), P(3), F(4), 1, 1, 64, 64, NAN, 0, kStream), FA_ERR_ARG);
    REJECTS(fa_fwd(FA_BF16, P(0), P(1), P(2), P(3), F(4), 1, 1, 64, 64, INFINITY, 0, kStream), FA_ERR_ARG);
    REJECTS(fa_fwd(FA_BF16, C(P(0)) + 8, P(1), P(2), P(3), F(4), 1, 1, 64, 64, 0.1f, 0, kStream), FA_ERR_ARG);
    REJECTS(fa_fwd(FA_BF16, P(0), P(1), P(2), P(3), (float*)(C(P(4)) + 2), 1, 1, 64, 64, 0.1f, 0, kStream), FA_ERR_ARG);
    // an error left pending by earlier work is not this call's; a failed launch is
    fa::g_pending = hipErrorInvalidValue;
    CHECK(fa_fwd(FA_BF16, P(0), P(1), P(2), P(3), F(4), 1, 1, 64, 64, 0.1f, 0, kStream) == FA_OK);
    CHECK(fa::g_pending == hipSuccess);
    fa::g_launch_result = hipErrorLaunchFailure;
    CHECK(fa_fwd(FA_BF16, P(0), P(1), P(2), P(3), F(4), 1, 1, 64, 64, 0.1f, 0, kStream) == FA_ERR_HIP);
    fa::g_launch_result = hipSuccess;
    // workgroup shapes
    CHECK(fa_fwd_waves(FA_BF16, P(0), P(1), P(2), P(3), F(4), 1, 4, 512, 128, 0.1f, 1, 8, kStream) == FA_OK);
    CHECK(g_rec.arg[3] == FA_BF16 * 100 + 80 + 1);
    CHECK(fa_fwd_waves(FA_F16, P(0), P(1), P(2), P(3), F(4), 1, 4, 512, 256, 0.1f, 0, 4, kStream) == FA_OK);
    REJECTS(fa_fwd_waves(FA_F16, P(0), P(1), P(2), P(3), F(4), 1, 4, 512, 256, 0.1f, 0, 8, kStream), FA_ERR_ARG);
    REJECTS(fa_fwd_waves(FA_F16, P(0), P(1), P(2), P(3), F(4), 1, 4, 512, 128, 0.1f, 0, 5, kStream), FA_ERR_ARG);
    REJECTS(fa_fwd_waves(FA_F32, P(0), P(1), P(2), P(3), F(4), 1, 4, 512, 128, 0.1f, 0, 0, kStream), FA_ERR_DTYPE);
    // fp8
    CHECK(fa_fwd_fp8(P(0), P(1), P(2), 0.5f, 0.25f, 2.f, P(3), F(4), 2, 32, 8192, 128, 0.088f, 0, kStream) == FA_OK);
    CHECK(g_rec.arg[0] == 64 && g_rec.arg[1] == 8192);
    REJECTS(fa_fwd_fp8(P(0), P(1), P(2), 0.5f, 0.25f, 2.f, P(3), F(4), 1, 1, 64, 64, 0.1f, 0, kStream), FA_ERR_HEADDIM);
    REJECTS(fa_fwd_fp8(P(0), P(1), P(2), 0.f, 0.25f, 2.f, P(3), F(4), 1, 1, 64, 128, 0.1f, 0, kStream), FA_ERR_ARG);
    REJECTS(fa_fwd_fp8(P(0), P(1), P(2), 1e30f, 1e30f, 2.f, P(3), F(4), 1, 1, 64, 128, 1e30f, 0, kStream), FA_ERR_ARG);
}

static void backward() {
    const int B = 2, H = 3, N = 1000, d = 128;
    const size_t rows = (size_t)B * H * N;
    const size_t wsb = fa_bwd_workspace_bytes(B, H, N, d);
    CHECK(wsb == 2 * a256(rows * 4));
    CHECK(fa_bwd_workspace_bytes(0, H, N, d) == 0 && fa_bwd_workspace_bytes(B, H, N, 96) == 0);
    void* ws = P(11);
    CHECK(fa_bwd(FA_BF16, P(0), P(1), P(2), P(3), F(4), P(5), P(6), P(7), P(8), ws, wsb, B, H, N, d, 0.1f, 1, kStream) == FA_OK);
    CHECK(g_rec.arg[3] == FA_BF16 * 1000 + 7 * 10 + 1);
    const void* delta = g_rec.ptr[9];
    const void* lse2 = g_rec.ptr[10];
    CHECK(inside(delta, rows * 4, ws, wsb) && inside(lse2, rows * 4, ws, wsb));
    CHECK(disjoint(delta, rows * 4, lse2, rows * 4));
    CHECK(((uintptr_t)delta & 255) == 0 && ((uintptr_t)lse2 & 255) == 0);
    for (int stage = 1; stage <= 3; ++stage) {
        CHECK(fa_bwd_stage(stage, FA_F16, P(0), P(1), P(2), P(3), F(4), P(5), P(6), P(7), P(8), ws, wsb, B, H, N, 64, 0.1f, 0, kStream) == FA_OK);
        CHECK(g_rec.arg[3] == FA_F16 * 1000 + (1 << (stage - 1)) * 10);
    }
    REJECTS(fa_bwd_stage(0, FA_F16, P(0), P(1), P(2), P(3), F(4), P(5), P(6), P(7), P(8), ws, wsb, B, H, N, 64, 0.1f, 0, kStream), FA_ERR_ARG);
    REJECTS(fa_bwd_stage(4, FA_F16, P(0), P(1), P(2), P(3), F(4), P(5), P(6), P(7), P(8), ws, wsb, B, H, N, 64, 0.1f, 0, kStream), FA_ERR_ARG);
    REJECTS(fa_bwd(FA_BF16, P(0), P(1), P(2), P(3), F(4), P(5), P(6), P(7), P(8), ws, wsb - 1, B, H, N, d, 0.1f, 1, kStream), FA_ERR_WORKSPACE);
    REJECTS(fa_bwd(FA_BF16, P(0), P(1), P(2), P(3), F(4), P(5), P(6), P(7), P(8), C(ws) + 16, wsb, B, H, N, d, 0.1f, 1, kStream), FA_ERR_WORKSPACE);
    REJECTS(fa_bwd(FA_BF16, P(0), P(1), P(2), P(3), F(4), P(5), P(6), P(7), P(8), nullptr, wsb, B, H, N, d, 0.1f, 1, kStream), FA_ERR_NULL);
    REJECTS(fa_bwd(FA_BF16, P(0), P(1), P(2), P(3), nullptr, P(5), P(6), P(7), P(8), ws, wsb, B, H, N, d, 0.1f, 1, kStream), FA_ERR_NULL);
    REJECTS(fa_bwd(FA_F32, P(0), P(1), P(2), P(3), F(4), P(5), P(6), P(7), P(8), ws, wsb, B, H, N, d, 0.1f, 1, kStream), FA_ERR_DTYPE);
    REJECTS(fa_bwd(FA_BF16, P(0), P(1), P(2), P(3), F(4), C(P(5)) + 4, P(6), P(7), P(8), ws, wsb, B, H, N, d, 0.1f, 1, kStream), FA_ERR_ARG);

    // allocation-free variant: the current device's scratch, the stream on that device
    fa::g_device = 3;
    fa::g_stream_device = 3;
    CHECK(fa_bwd_noalloc(FA_BF16, P(0), P(1), P(2), P(3), F(4), P(5), P(6), P(7), P(8), B, H, N, d, 0.1f, 1, kStream) == FA_OK);
    CHECK(g_rec.scratch_device == 3 && g_rec.arg[3] == FA_BF16 * 1000 + 71);
    CHECK(fa_bwd_noalloc(FA_BF16, P(0), P(1), P(2), P(3), F(4), P(5), P(6), P(7), P(8), B, H, N, d, 0.1f, 1, nullptr) == FA_OK);
    fa::g_stream_device = 2;
    REJECTS(fa_bwd_noalloc(FA_BF16, P(0), P(1), P(2), P(3), F(4), P(5), P(6), P(7), P(8), B, H, N, d, 0.1f, 1, kStream), FA_ERR_ARG);
    fa::g_device = fa::g_stream_device = 0;
    const size_t maxr = fa_bwd_noalloc_max_rows();
    CHECK(fa_bwd_noalloc(FA_BF16, P(0), P(1), P(2), P(3), F(4), P(5), P(6), P(7), P(8), 1, 1, (int)maxr, 64, 0.1f, 0, kStream) == FA_OK);
    REJECTS(fa_bwd_noalloc(FA_BF16, P(0), P(1), P(2), P(3), F(4), P(5), P(6), P(7), P(8), 1, 1, (int)maxr + 1, 64, 0.1f, 0, kStream), FA_ERR_TOO_LARGE);

    // fp8 backward: three code conversions into the workspace, then the 16-bit passes
    const size_t el = rows * d;
    const size_t wsb8 = fa_bwd_fp8_workspace_bytes(B, H, N, d);
    CHECK(wsb8 == 3 * a256(el * 2) + wsb);
    g_rec.n_conv = 0;
    CHECK(fa_bwd_fp8(P(0), P(1), P(2), 0.5f, 0.25f, 2.f, P(3), F(4), P(5), P(6), P(7), P(8), ws, wsb8, B, H, N, d, 0.1f, 1, kStream) == FA_OK);
    CHECK(g_rec.n_conv == 3 && g_rec.conv_n == (long long)el);
    for (int i = 0; i < 3; ++i) {
        CHECK(g_rec.conv_src[i] == P(i));
        CHECK(inside(g_rec.conv_dst[i], el * 2, ws, wsb8));
        CHECK(g_rec.ptr[i] == g_rec.conv_dst[i]);  // the 16-bit passes read the widened codes
        for (int j = 0; j < i; ++j) CHECK(disjoint(g_rec.conv_dst[i], el * 2, g_rec.conv_dst[j], el * 2));
    }
    CHECK(inside(g_rec.ptr[9], rows * 4, ws, wsb8) && inside(g_rec.ptr[10], rows * 4, ws, wsb8));
    for (int i = 0; i < 3; ++i) {
        CHECK(disjoint(g_rec.conv_dst[i], el * 2, g_rec.ptr[9], rows * 4));
        CHECK(disjoint(g_rec.conv_dst[i], el * 2, g_rec.ptr[10], rows * 4));
    }
    REJECTS(fa_bwd_fp8(P(0), P(1), P(2), 0.5f, 0.25f, 2.f, P(3), F(4), P(5), P(6), P(7), P(8), ws, wsb8 - 1, B, H, N, d, 0.1f, 1, kStream), FA_ERR_WORKSPACE);
    REJECTS(fa_bwd_fp8(P(0), P(1), P(2), 0.5f, 0.25f, 0.f, P(3), F(4), P(5), P(6), P(7), P(8), ws, wsb8, B, H, N, d, 0.1f, 1, kStream), FA_ERR_ARG);
    // the dK factor scale * q_descale * v_descale underflows to 0
    REJECTS(fa_bwd_fp8(P(0), P(1), P(2), 0.5f, 0.25f, 1e-44f, P(3), F(4), P(5), P(6), P(7), P(8), ws, wsb8, B, H, N, d, 0.1f, 1, kStream), FA_ERR_ARG);
    fa::g_launch_result = hipErrorLaunchFailure;  // the first conversion fails: the call says so
    CHECK(fa_bwd_fp8(P(0), P(1), P(2), 0.5f, 0.25f, 2.f, P(3), F(4), P(5), P(6), P(7), P(8), ws, wsb8, B, H, N, d, 0.1f, 1, kStream) == FA_ERR_HIP);
    fa::g_launch_result = hipSuccess;
}

static void splitkv_case(int B, int H, int Nq, int Nk, int d, int causal, int splits_req) {
    const size_t wsb = fa_fwd_splitkv_workspace_bytes(B, H, Nq, Nk, d, splits_req);
    CHECK(wsb > 0);
    void* ws = P(12);
    CHECK(fa_fwd_splitkv(FA_BF16, P(0), P(1), P(2), P(3), F(4), B, H, Nq, Nk, d, 0.1f, causal, splits_req, ws, wsb, kStream) == FA_OK);
    const long long splits = g_rec.arg[3] / 1000000, kps = g_rec.arg[3] % 1000000;
    CHECK(splits >= 1 && kps % 128 == 0 && kps >= 128);
    CHECK(splits * kps >= Nk && (splits - 1) * kps < Nk);  // every key range holds keys
    if (splits_req > 0) CHECK(splits <= splits_req);
    const size_t rows = (size_t)splits * B * H * Nq;
    CHECK(inside(g_rec.ptr[5], rows * d * 4, ws, wsb) && inside(g_rec.ptr[6], rows * 4, ws, wsb));
    CHECK(disjoint(g_rec.ptr[5], rows * d * 4, g_rec.ptr[6], rows * 4));
    REJECTS(fa_fwd_splitkv(FA_BF16, P(0), P(1), P(2), P(3), F(4), B, H, Nq, Nk, d, 0.1f, causal, splits_req, ws, wsb - 1, kStream), FA_ERR_WORKSPACE);
}

static void splitkv_and_merge() {
    splitkv_case(8, 32, 1, 32768, 128, 0, 0);
    splitkv_case(1, 32, 1, 131072, 128, 0, 0);
    splitkv_case(8, 32, 16, 8192, 128, 1, 0);
    splitkv_case(2, 4, 300, 1300, 64, 1, 3);
    splitkv_case(1, 1, 1, 1, 64, 0, 7);
    splitkv_case(1, 1, 5, 129, 128, 0, 1024);
    REJECTS(fa_fwd_splitkv(FA_BF16, P(0), P(1), P(2), P(3), F(4), 1, 1, 10, 5, 128, 0.1f, 1, 0, P(12), 1 << 20, kStream), FA_ERR_SHAPE);
    REJECTS(fa_fwd_splitkv(FA_BF16, P(0), P(1), P(2), P(3), F(4), 1, 1, 10, 50, 128, 0.1f, 0, -1, P(12), 1 << 20, kStream), FA_ERR_ARG);
    REJECTS(fa_fwd_splitkv(FA_BF16, P(0), P(1), P(2), P(3), F(4), 1, 1, 10, 50, 128, 0.1f, 0, 1025, P(12), 1 << 20, kStream), FA_ERR_ARG);
    CHECK(fa_fwd_splitkv_workspace_bytes(1, 1, 10, 50, 128, -1) == 0);

    CHECK(fa_lse_merge(FA_F32, 3, F(0), F(1), P(2), F(3), 333, 128, kStream) == FA_OK);
    CHECK(g_rec.arg[0] == 3 && g_rec.arg[1] == 333 && g_rec.arg[2] == 128);
    CHECK(fa_lse_merge(FA_BF16, 1, F(0), F(1), C(P(2)) + 2, nullptr, 5, 12, kStream) == FA_OK);
    REJECTS(fa_lse_merge(FA_BF16, 1, F(0), F(1), C(P(2)) + 1, nullptr, 5, 12, kStream), FA_ERR_ARG);
    REJECTS(fa_lse_merge(FA_F32, 1, F(0), F(1), C(P(2)) + 2, nullptr, 5, 12, kStream), FA_ERR_ARG);
    REJECTS(fa_lse_merge(FA_F32, 1, F(0), F(1), P(2), nullptr, 5, 6, kStream), FA_ERR_SHAPE);
    REJECTS(fa_lse_merge(FA_F32, 0, F(0), F(1), P(2), nullptr, 5, 8, kStream), FA_ERR_SHAPE);
    REJECTS(fa_lse_merge(FA_F32, 1, F(0), F(1), P(2), nullptr, INT_MAX, 65536, kStream), FA_ERR_SHAPE);
}

static void baselines_and_probes() {
    const int B = 1, H = 2, N = 1000, d = 128;
    const size_t rows = (size_t)B * H * N;
    const size_t wsv = fa_fwd_v1_workspace_bytes(B, H, N, d);
    void* ws = P(13);
    CHECK(fa_fwd_v1(FA_F16, P(0), P(1), P(2), P(3), F(4), ws, wsv, B, H, N, d, 0.1f, 1, kStream) == FA_OK);
    CHECK(inside(g_rec.ptr[5], rows * d * 4, ws, wsv));
    CHECK(inside(g_rec.ptr[6], rows * 2 * 4, ws, wsv) && inside(g_rec.ptr[7], rows * 2 * 4, ws, wsv));
    CHECK(disjoint(g_rec.ptr[5], rows * d * 4, g_rec.ptr[6], rows * 8));
    CHECK(disjoint(g_rec.ptr[6], rows * 8, g_rec.ptr[7], rows * 8));
    REJECTS(fa_fwd_v1(FA_F16, P(0), P(1), P(2), P(3), F(4), ws, wsv - 1, B, H, N, d, 0.1f, 1, kStream), FA_ERR_WORKSPACE);

    const size_t wss = fa_std_workspace_bytes(B, H, N, d);
    CHECK(wss == (size_t)B * H * N * N * 2);
    CHECK(fa_std_fwd(FA_BF16, P(0), P(1), P(2), P(3), ws, wss, B, H, N, d, 0.1f, 0, kStream) == FA_OK);
    CHECK(g_rec.ptr[4] == ws);
    REJECTS(fa_std_fwd(FA_BF16, P(0), P(1), P(2), P(3), ws, wss - 1, B, H, N, d, 0.1f, 0, kStream), FA_ERR_WORKSPACE);
    REJECTS(fa_std_fwd(FA_BF16, P(0), P(1), P(2), P(3), ws, (size_t)-1, 256, 256, 1, 64, 0.1f, 0, kStream), FA_ERR_SHAPE);

    CHECK(fa_probe_mfma((unsigned long long*)P(0), 512, 4096, kStream) == FA_OK);
    REJECTS(fa_probe_mfma((unsigned long long*)P(0), 0, 4096, kStream), FA_ERR_ARG);
    REJECTS(fa_probe_mfma((unsigned long long*)(C(P(0)) + 4), 1, 1, kStream), FA_ERR_ARG);
    CHECK(fa_probe_dq_atomics(F(0), (size_t)8 * 16 * 4096 * 128 * 4, 8, 16, 4096, 128, 0, 1, kStream) == FA_OK);
    REJECTS(fa_probe_dq_atomics(F(0), (size_t)8 * 16 * 4096 * 128 * 4 - 1, 8, 16, 4096, 128, 0, 1, kStream), FA_ERR_WORKSPACE);
    REJECTS(fa_probe_dq_atomics(F(0), (size_t)1 << 40, 8, 16, 4096, 64, 0, 1, kStream), FA_ERR_ARG);
    REJECTS(fa_probe_dq_atomics(F(0), (size_t)1 << 40, 8, 16, 4000, 128, 0, 1, kStream), FA_ERR_SHAPE);
}

// Every size function and entry point over extreme sizes: the sanitizers
// watch the arithmetic; the results must be either a rejection or, for sizes
// that pass, a workspace size of at least the bytes the carving uses.
static void extremes() {
    const int vals[] = {INT_MIN, -1, 0, 1, 2, 31, 33, 1000, 1 << 15, 1 << 20, 1 << 24, INT_MAX};
    const int dims[] = {0, 64, 96, 128, 256, INT_MAX};
    for (int B : vals)
        for (int H : vals)
            for (int N : vals)
                for (int d : dims) {
                    const size_t wb = fa_bwd_workspace_bytes(B, H, N, d);
                    const size_t w8 = fa_bwd_fp8_workspace_bytes(B, H, N, d);
                    const size_t wv = fa_fwd_v1_workspace_bytes(B, H, N, d);
                    const size_t wsd = fa_std_workspace_bytes(B, H, N, d);
                    const size_t wk = fa_fwd_splitkv_workspace_bytes(B, H, N, N, d, 0);
                    if (wb) CHECK(wb >= 2 * (size_t)B * H * N * 4);
                    if (w8) CHECK(w8 >= wb + 3 * (size_t)B * H * N * d * 2);
                    (void)wv;
                    (void)wsd;
                    (void)wk;
                    const int s1 = fa_fwd(FA_BF16, P(0), P(1), P(2), P(3), F(4), B, H, N, d, 0.1f, 1, kStream);
                    const int s2 = fa_bwd(FA_BF16, P(0), P(1), P(2), P(3), F(4), P(5), P(6), P(7), P(8), P(11), (size_t)-1, B, H, N, d, 0.1f, 1, kStream);
                    const int s3 = fa_std_fwd(FA_F16, P(0), P(1), P(2), P(3), P(11), (size_t)-1, B, H, N, d, 0.1f, 0, kStream);
                    const int s4 = fa_fwd_splitkv(FA_BF16, P(0), P(1), P(2), P(3), F(4), B, H, 1, N, d, 0.1f, 0, 0, P(12), (size_t)-1, kStream);
                    CHECK(s1 <= 0 && s2 <= 0 && s3 <= 0 && s4 <= 0);
                    if (B < 1 || H < 1 || N < 1) CHECK(s1 == FA_ERR_SHAPE || s1 == FA_ERR_HEADDIM);
                }
}

int main() {
    status_and_version();
    forward();
    backward();
    splitkv_and_merge();
    baselines_and_probes();
    extremes();
    printf("%d checks, %d failed\n", g_checks, g_failed);
    return g_failed == 0 ? 0 : 1;
}
