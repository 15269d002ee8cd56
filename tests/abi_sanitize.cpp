// Host-side argument validation of every libattn.so entry point, built with
// AddressSanitizer and UndefinedBehaviorSanitizer on the host code (the CPU
// test builds it from the library's sources and runs it). Every call here
// must fail validation, so no device is touched: the pointers are fake. The
// forward and decode sources are built whole (their plan functions are host
// logic the checks use); the backward kernels are replaced by the stubs below.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "attn.h"
#include "attn_kernels.h"

static int failures = 0;

// The backward launchers (their kernels are not built into this program):
// a call that passes validation would reach them, which is a failure here.
namespace attn {
hipError_t launch_bwd(const BwdParams&, int, int, int, int, hipStream_t) {
    std::printf("FAIL: a backward call passed validation\n");
    ++failures;
    return hipErrorInvalidValue;
}
hipError_t launch_bwd_dq(const BwdParams&, int, int, int, hipStream_t) {
    std::printf("FAIL: a dQ call passed validation\n");
    ++failures;
    return hipErrorInvalidValue;
}
}  // namespace attn
#define EXPECT(expr, want)                                                                   \
    do {                                                                                     \
        const int got_ = (int)(expr);                                                        \
        if (got_ != (int)(want)) {                                                           \
            std::printf("FAIL line %d: %s = %d, want %d\n", __LINE__, #expr, got_, (int)(want)); \
            ++failures;                                                                      \
        }                                                                                    \
    } while (0)

static void* const P = reinterpret_cast<void*>(0x10000);
static float* const PF = reinterpret_cast<float*>(0x10000);

static attn_tensor T(long long sb = 1 << 20, long long sh = 1 << 12, long long sn = 64) {
    attn_tensor t;
    t.data = P;
    t.stride_b = sb;
    t.stride_h = sh;
    t.stride_n = sn;
    return t;
}

static attn_problem prob(int N = 64, int d = 64) {
    attn_problem p;
    std::memset(&p, 0, sizeof p);
    p.B = 1; p.Hq = 2; p.Hkv = 1; p.N = N; p.d = d; p.scale = 0.125f;
    p.mask = ATTN_MASK_CAUSAL; p.dtype = ATTN_DTYPE_BF16;
    return p;
}

int main() {
    // status strings, including out-of-range codes
    for (int c = -1; c < 20; ++c) {
        const char* s = attn_status_string((attn_status)c);
        if (!s || !std::strlen(s)) { std::printf("FAIL: empty status string %d\n", c); ++failures; }
    }
    if (std::strlen(attn_last_hip_error()) != 0) { std::printf("FAIL: stale hip error\n"); ++failures; }

    // forward
    EXPECT(attn_fwd(nullptr, P, P, P, PF, 1, 2, 1, 64, 64, 0.125f, 1, nullptr), ATTN_ERR_NULL);
    EXPECT(attn_fwd(P, P, P, P, nullptr, 1, 2, 1, 64, 64, 0.125f, 1, nullptr), ATTN_ERR_NULL);
    EXPECT(attn_fwd(P, P, P, P, PF, 0, 2, 1, 64, 64, 0.125f, 1, nullptr), ATTN_ERR_SHAPE);
    EXPECT(attn_fwd(P, P, P, P, PF, 1, 2, 1, (1 << 24) + 1, 64, 0.125f, 1, nullptr), ATTN_ERR_SHAPE);
    EXPECT(attn_fwd(P, P, P, P, PF, 1 << 30, 1 << 30, 1, 64, 64, 0.125f, 1, nullptr), ATTN_ERR_SHAPE);
    EXPECT(attn_fwd(P, P, P, P, PF, 1, 1 << 15, 1, 1 << 16, 64, 0.125f, 1, nullptr), ATTN_ERR_SHAPE);
    EXPECT(attn_fwd(P, P, P, P, PF, 1, 3, 2, 64, 64, 0.125f, 1, nullptr), ATTN_ERR_GQA);
    EXPECT(attn_fwd(P, P, P, P, PF, 1, 2, 1, 64, 72, 0.125f, 1, nullptr), ATTN_ERR_HEAD_DIM);
    EXPECT(attn_fwd(P, P, P, P, PF, 1, 2, 1, 64, 64, NAN, 1, nullptr), ATTN_ERR_SCALE);
    EXPECT(attn_fwd(P, P, P, P, PF, 1, 2, 1, 64, 64, -1.0f, 1, nullptr), ATTN_ERR_SCALE);
    EXPECT(attn_fwd((char*)P + 2, P, P, P, PF, 1, 2, 1, 64, 64, 0.125f, 1, nullptr), ATTN_ERR_ALIGN);
    EXPECT(attn_fwd_window(P, P, P, P, PF, 1, 2, 1, 64, 64, 0.125f, 0, nullptr), ATTN_ERR_WINDOW);

    // backward, its passes and the no-allocation variant
    const size_t ws = attn_bwd_workspace_bytes(1, 2, 1, 64, 64);
    EXPECT(ws, 2 * 512);
    EXPECT(attn_bwd_workspace_bytes(0, 2, 1, 64, 64), 0);
    EXPECT(attn_bwd(P, P, P, P, PF, P, P, P, P, nullptr, ws, 1, 2, 1, 64, 64, 0.125f, 1, nullptr),
           ATTN_ERR_WORKSPACE);
    EXPECT(attn_bwd(P, P, P, P, PF, P, P, P, P, P, ws - 1, 1, 2, 1, 64, 64, 0.125f, 1, nullptr),
           ATTN_ERR_WORKSPACE);
    EXPECT(attn_bwd(P, P, P, P, PF, P, nullptr, P, P, P, ws, 1, 2, 1, 64, 64, 0.125f, 1, nullptr),
           ATTN_ERR_NULL);
    EXPECT(attn_bwd(P, P, P, P, PF, P, P, P, P, P, ws, 1, 2, 1, 64, 96 + 16, 0.125f, 1, nullptr),
           ATTN_ERR_HEAD_DIM);
    EXPECT(attn_bwd_window(P, P, P, P, PF, P, P, P, P, P, ws, 1, 2, 1, 64, 64, 0.125f, -3, nullptr),
           ATTN_ERR_WINDOW);
    EXPECT(attn_bwd_preprocess(P, P, PF, nullptr, ws, 1, 2, 1, 64, 64, nullptr), ATTN_ERR_WORKSPACE);
    EXPECT(attn_bwd_dkdv(P, P, P, PF, P, P, P, P, ws, 1, 2, 1, 64, 64, 0.0f, 1, 0, nullptr), ATTN_ERR_SCALE);
    EXPECT(attn_bwd_dq(P, P, P, PF, P, P, P, ws, 1, 2, 1, 0, 64, 0.125f, 0, 0, nullptr), ATTN_ERR_SHAPE);
    EXPECT(attn_bwd_noalloc(P, P, P, P, PF, P, P, P, nullptr, 1, 2, 1, 64, 64, 0.125f, 1, nullptr),
           ATTN_ERR_NULL);
    EXPECT(attn_bwd_noalloc(P, P, P, P, PF, P, P, P, P, 1, 32, 1, 65537, 64, 0.125f, 1, nullptr),
           ATTN_ERR_SCRATCH);
    EXPECT(attn_bwd_noalloc_max_rows(), 1 << 21);

    // strided interface
    attn_tensor t = T(), tneg = T(1 << 20, -4096, 64), tmis = T(1 << 20, 1 << 12, 60);
    attn_problem pr = prob();
    EXPECT(attn_fwd_ex(nullptr, &t, &t, &t, &t, PF, nullptr), ATTN_ERR_NULL);
    EXPECT(attn_fwd_ex(&pr, &tneg, &t, &t, &t, PF, nullptr), ATTN_ERR_STRIDE);
    EXPECT(attn_fwd_ex(&pr, &tmis, &t, &t, &t, PF, nullptr), ATTN_ERR_ALIGN);
    pr.dtype = 7;
    EXPECT(attn_fwd_ex(&pr, &t, &t, &t, &t, PF, nullptr), ATTN_ERR_DTYPE);
    pr = prob();
    pr.dropout_p = 1.0f;
    EXPECT(attn_fwd_ex(&pr, &t, &t, &t, &t, PF, nullptr), ATTN_ERR_DROPOUT);
    pr = prob();
    pr.mask = ATTN_MASK_NONE;
    pr.window = 5;
    EXPECT(attn_fwd_ex(&pr, &t, &t, &t, &t, PF, nullptr), ATTN_ERR_WINDOW);
    pr = prob();
    EXPECT(attn_bwd_ex(&pr, &t, &t, &t, &t, PF, &t, &t, &t, &t, P, ws, 0u, nullptr), ATTN_ERR_PASSES);
    EXPECT(attn_bwd_ex(&pr, &t, &t, &t, &t, PF, &t, &t, &t, &t, P, ws, 9u, nullptr), ATTN_ERR_PASSES);
    EXPECT(attn_bwd_ex(&pr, &t, &t, &t, &t, PF, &t, &t, &t, &t, nullptr, ws, ATTN_BWD_ALL, nullptr),
           ATTN_ERR_WORKSPACE);

    // plans and decode
    attn_plan plan;
    EXPECT(attn_fwd_plan(1, 8, 8, 400, 64, 0, nullptr), ATTN_ERR_NULL);
    EXPECT(attn_fwd_plan(1, 8, 8, 400, 64, 0, &plan), ATTN_OK);
    EXPECT(plan.key_splits, 8);
    EXPECT(attn_fwd_plan(1, 64, 8, 8192, 128, 1, &plan), ATTN_OK);
    EXPECT(plan.key_splits, 1);
    EXPECT(attn_fwd_plan(1, 8, 8, 400, 100, 0, &plan), ATTN_ERR_HEAD_DIM);
    attn_decode_problem dp;
    std::memset(&dp, 0, sizeof dp);
    dp.B = 2; dp.Hq = 8; dp.Hkv = 2; dp.Nq = 1; dp.Nk = 4096; dp.d = 128; dp.scale = 0.088f;
    dp.mask = ATTN_MASK_CAUSAL; dp.dtype = ATTN_DTYPE_BF16;
    const size_t dws = attn_decode_workspace_bytes(&dp);
    EXPECT(attn_decode_workspace_bytes(nullptr), 0);
    EXPECT(attn_decode_fwd(&dp, &t, &t, &t, nullptr, &t, PF, nullptr, dws, nullptr),
           dws ? ATTN_ERR_WORKSPACE : ATTN_OK);
    dp.Nq = 0;
    EXPECT(attn_decode_fwd(&dp, &t, &t, &t, nullptr, &t, PF, P, dws, nullptr), ATTN_ERR_SHAPE);

    std::printf("%s: %d failure(s)\n", failures ? "FAILED" : "passed", failures);
    return failures ? 1 : 0;
}
