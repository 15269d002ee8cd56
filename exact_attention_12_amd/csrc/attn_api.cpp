// attn_api.cpp - the C ABI declared in include/attn.h: argument validation,
// tile plans and kernel dispatch. No allocation, no synchronisation: every
// check runs on the host before anything is enqueued.
#include "attn.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "attn_kernels.h"

namespace {

thread_local char g_last_hip_error[256] = "";

constexpr float kLog2eHost = 1.4426950408889634f;

bool head_dim_ok(int d) { return d == 64 || d == 80 || d == 128 || d == 256; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Shape checks shared by every entry point. Head-dimension and grouping are
// checked after the plain sizes so that the most basic error is reported.
attn_status check_shape(int B, int Hq, int Hkv, int N, int d) {
    if (B < 1 || Hq < 1 || Hkv < 1 || N < 1) return ATTN_ERR_SHAPE;
    if (N > ATTN_MAX_SEQ_LEN) return ATTN_ERR_SHAPE;
    // Element counts must fit comfortably in 64-bit offsets, and the
    // workgroup counts of every kernel in a 32-bit grid dimension.
    const long double elems = (long double)B * Hq * N * 256.0L;
    if (elems > 4.0e18L) return ATTN_ERR_SHAPE;
    const long long rows = (long long)B * Hq * ((N + 127) / 128);
    if (rows > 0x7fffffffLL) return ATTN_ERR_SHAPE;
    if ((long long)B * Hq * N / 16 + 1 > 0x7fffffffLL) return ATTN_ERR_SHAPE;
    if (Hq % Hkv != 0) return ATTN_ERR_GQA;
    if (!head_dim_ok(d)) return ATTN_ERR_HEAD_DIM;
    return ATTN_OK;
}

attn_status check_scale(float scale) {
    if (!std::isfinite(scale) || !(scale > 0.0f)) return ATTN_ERR_SCALE;
    return ATTN_OK;
}

attn_status hip_status(hipError_t e) {
    if (e == hipSuccess) return ATTN_OK;
    std::snprintf(g_last_hip_error, sizeof g_last_hip_error, "%s", hipGetErrorString(e));
    return ATTN_ERR_HIP;
}

// Window as the kernels take it: 0 = no band, else W with 1 <= W < N (a band
// of N or more keys is the plain causal mask).
int kernel_window(int window, int N) { return window >= N ? 0 : window; }

int mask_kind(int causal, int kernel_window) {
    if (causal == 0) return attn::kMaskNone;
    return kernel_window > 0 ? attn::kMaskWindow : attn::kMaskCausal;
}

attn_status fwd_common(const void* q, const void* k, const void* v, void* o, float* lse,
                       int B, int Hq, int Hkv, int N, int d, float scale, int causal,
                       int window, void* stream) {
    if (!q || !k || !v || !o || !lse) return ATTN_ERR_NULL;
    attn_status st = check_shape(B, Hq, Hkv, N, d);
    if (st != ATTN_OK) return st;
    st = check_scale(scale);
    if (st != ATTN_OK) return st;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
        return ATTN_ERR_ALIGN;

    attn::FwdPlan plan;
    attn::fwd_plan(B, Hq, N, d, &plan);
    attn::FwdParams p;
    p.q = q;
    p.k = k;
    p.v = v;
    p.o = o;
    p.lse = lse;
    p.N = N;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.G = Hq / Hkv;
    p.BH = B * Hq;
    p.nqb = (N + plan.block_q - 1) / plan.block_q;
    p.window = kernel_window(window, N);
    p.c = scale * kLog2eHost;
    g_last_hip_error[0] = '\0';
    return hip_status(attn::launch_fwd(p, d, mask_kind(causal, p.window), plan,
                                       static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

attn_status attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                     int B, int Hq, int Hkv, int N, int d, float scale, int causal,
                     void* stream) {
    return fwd_common(q, k, v, o, lse, B, Hq, Hkv, N, d, scale, causal, 0, stream);
}

attn_status attn_fwd_window(const void* q, const void* k, const void* v, void* o, float* lse,
                            int B, int Hq, int Hkv, int N, int d, float scale, int window,
                            void* stream) {
    if (window < 1) return ATTN_ERR_WINDOW;
    return fwd_common(q, k, v, o, lse, B, Hq, Hkv, N, d, scale, 1, window, stream);
}

size_t attn_bwd_workspace_bytes(int B, int Hq, int Hkv, int N, int d) {
    if (check_shape(B, Hq, Hkv, N, d) != ATTN_OK) return 0;
    const size_t bytes = (size_t)B * Hq * N * sizeof(float);
    return (bytes + 255) & ~(size_t)255;
}

}  // extern "C"

namespace {

// Shared validation and dispatch of attn_bwd and its three pass entry points.
// Only the pointers the selected passes read or write are checked; the
// others are NULL and never dereferenced.
attn_status bwd_common(const void* q, const void* k, const void* v, const void* o,
                       const float* lse, const void* dout, void* dq, void* dk, void* dv,
                       const void* workspace, size_t workspace_bytes,
                       int B, int Hq, int Hkv, int N, int d, float scale, int causal,
                       int window, void* stream, int passes) {
    const bool pre = passes & attn::kBwdPre, kv = passes & attn::kBwdDkDv, qq = passes & attn::kBwdDq;
    const bool main = kv || qq;
    const void* used[] = {pre ? o : dout, dout, main ? q : dout, main ? k : dout,
                          main ? v : dout, main ? static_cast<const void*>(lse) : dout,
                          qq ? dq : dout, kv ? dk : dout, kv ? dv : dout};
    for (const void* ptr : used)
        if (!ptr) return ATTN_ERR_NULL;
    attn_status st = check_shape(B, Hq, Hkv, N, d);
    if (st != ATTN_OK) return st;
    if (main) {
        st = check_scale(scale);
        if (st != ATTN_OK) return st;
        if (window < 0 || (window > 0 && causal == 0)) return ATTN_ERR_WINDOW;
    }
    if (!workspace || workspace_bytes < attn_bwd_workspace_bytes(B, Hq, Hkv, N, d))
        return ATTN_ERR_WORKSPACE;
    for (const void* ptr : used)
        if (!aligned16(ptr)) return ATTN_ERR_ALIGN;
    if (!aligned16(workspace)) return ATTN_ERR_ALIGN;

    attn::BwdParams p;
    p.q = q;
    p.k = k;
    p.v = v;
    p.o = o;
    p.lse = lse;
    p.dout = dout;
    p.dq = dq;
    p.dk = dk;
    p.dv = dv;
    p.delta = static_cast<float*>(const_cast<void*>(workspace));
    p.N = N;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.G = Hq / Hkv;
    p.B = B;
    p.window = kernel_window(window, N);
    p.scale = scale;
    p.c = scale * kLog2eHost;
    g_last_hip_error[0] = '\0';
    return hip_status(attn::launch_bwd(p, d, mask_kind(causal, p.window), passes,
                                       static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

attn_status attn_bwd(const void* q, const void* k, const void* v, const void* o,
                     const float* lse, const void* dout,
                     void* dq, void* dk, void* dv,
                     void* workspace, size_t workspace_bytes,
                     int B, int Hq, int Hkv, int N, int d, float scale, int causal,
                     void* stream) {
    return bwd_common(q, k, v, o, lse, dout, dq, dk, dv, workspace, workspace_bytes, B, Hq, Hkv, N,
                      d, scale, causal, 0, stream, attn::kBwdAll);
}

attn_status attn_bwd_window(const void* q, const void* k, const void* v, const void* o,
                            const float* lse, const void* dout,
                            void* dq, void* dk, void* dv,
                            void* workspace, size_t workspace_bytes,
                            int B, int Hq, int Hkv, int N, int d, float scale, int window,
                            void* stream) {
    if (window < 1) return ATTN_ERR_WINDOW;
    return bwd_common(q, k, v, o, lse, dout, dq, dk, dv, workspace, workspace_bytes, B, Hq, Hkv, N,
                      d, scale, 1, window, stream, attn::kBwdAll);
}

attn_status attn_bwd_preprocess(const void* o, const void* dout, void* workspace,
                                size_t workspace_bytes, int B, int Hq, int Hkv, int N, int d,
                                void* stream) {
    return bwd_common(nullptr, nullptr, nullptr, o, nullptr, dout, nullptr, nullptr, nullptr,
                      workspace, workspace_bytes, B, Hq, Hkv, N, d, 1.0f, 0, 0, stream, attn::kBwdPre);
}

attn_status attn_bwd_dkdv(const void* q, const void* k, const void* v, const float* lse,
                          const void* dout, void* dk, void* dv,
                          const void* workspace, size_t workspace_bytes,
                          int B, int Hq, int Hkv, int N, int d, float scale, int causal,
                          int window, void* stream) {
    return bwd_common(q, k, v, nullptr, lse, dout, nullptr, dk, dv, workspace, workspace_bytes, B, Hq,
                      Hkv, N, d, scale, causal, window, stream, attn::kBwdDkDv);
}

attn_status attn_bwd_dq(const void* q, const void* k, const void* v, const float* lse,
                        const void* dout, void* dq,
                        const void* workspace, size_t workspace_bytes,
                        int B, int Hq, int Hkv, int N, int d, float scale, int causal,
                        int window, void* stream) {
    return bwd_common(q, k, v, nullptr, lse, dout, dq, nullptr, nullptr, workspace, workspace_bytes, B,
                      Hq, Hkv, N, d, scale, causal, window, stream, attn::kBwdDq);
}

const char* attn_status_string(attn_status status) {
    switch (status) {
        case ATTN_OK: return "ok";
        case ATTN_ERR_NULL: return "a required pointer is NULL";
        case ATTN_ERR_SHAPE: return "B, Hq, Hkv and N must be >= 1 and the sizes must fit the grid";
        case ATTN_ERR_GQA: return "Hq must be a multiple of Hkv";
        case ATTN_ERR_HEAD_DIM: return "unsupported head dimension (supported: 64, 80, 128, 256)";
        case ATTN_ERR_SCALE: return "scale must be finite and > 0";
        case ATTN_ERR_ALIGN: return "device pointers must be 16-byte aligned";
        case ATTN_ERR_WORKSPACE: return "workspace is NULL or smaller than attn_bwd_workspace_bytes()";
        case ATTN_ERR_HIP: return "the HIP runtime refused a launch (see attn_last_hip_error)";
        case ATTN_ERR_WINDOW: return "window must be >= 1 and needs the causal mask";
    }
    return "unknown status";
}

const char* attn_last_hip_error(void) { return g_last_hip_error; }

attn_status attn_fwd_plan(int B, int Hq, int Hkv, int N, int d, int causal, attn_plan* plan) {
    (void)causal;
    if (!plan) return ATTN_ERR_NULL;
    const attn_status st = check_shape(B, Hq, Hkv, N, d);
    if (st != ATTN_OK) return st;
    attn::FwdPlan fp;
    attn::fwd_plan(B, Hq, N, d, &fp);
    plan->rows_per_wave = fp.rows_per_wave;
    plan->block_q = fp.block_q;
    plan->block_kv = fp.block_kv;
    plan->threads = fp.threads;
    plan->workgroups = fp.workgroups;
    plan->lds_bytes = fp.lds_bytes;
    return ATTN_OK;
}

}  // extern "C"
