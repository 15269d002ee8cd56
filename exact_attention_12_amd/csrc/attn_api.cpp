// attn_api.cpp - the C ABI declared in include/attn.h: argument validation,
// tile plans and kernel dispatch. No allocation, no synchronisation: every
// check runs on the host before anything is enqueued.
#include "attn.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "attn_kernels.h"

// Device scratch of the backward entry point that allocates nothing
// (attn_bwd_noalloc): its row terms live in this fixed array, which every GPU
// the library runs on holds from the module's load until the process ends.
// In host code `scratch` names a host-side stand-in, not device memory: its
// device address is looked up once per device (hipGetSymbolAddress, with
// that device current) and only that address is handed to kernels.
static constexpr size_t kScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

thread_local char g_last_hip_error[256] = "";

constexpr float kLog2eHost = 1.4426950408889634f;

bool head_dim_ok(int d) {
    switch (d) {
#define ATTN_HEAD_DIM_OK(D_) case D_:
        ATTN_FOR_EACH_HEAD_DIM(ATTN_HEAD_DIM_OK)
#undef ATTN_HEAD_DIM_OK
        return true;
        default: return false;
    }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Shape checks shared by every entry point. Head-dimension and grouping are
// checked after the plain sizes so that the most basic error is reported.
attn_status check_shape(int B, int Hq, int Hkv, int N, int d) {
    if (B < 1 || Hq < 1 || Hkv < 1 || N < 1) return ATTN_ERR_SHAPE;
    if (N > ATTN_MAX_SEQ_LEN) return ATTN_ERR_SHAPE;
    // Element counts must fit comfortably in 64-bit offsets. A HIP grid
    // holds fewer than 2^32 work-items per dimension; the forward, dQ and
    // dK/dV kernels launch at most two work-items per query (or key) row,
    // rows padded to 256, and the row-term pass loops over its rows, so
    // B * Hq * round_up(N, 256) < 2^31 keeps every launch inside the limit.
    const long double elems = (long double)B * Hq * N * 256.0L;
    if (elems > 4.0e18L) return ATTN_ERR_SHAPE;
    const long double padded_rows = (long double)B * Hq * (long double)(((long long)N + 255) / 256 * 256);
    if (padded_rows >= 2147483648.0L) return ATTN_ERR_SHAPE;
    if (Hq % Hkv != 0) return ATTN_ERR_GQA;
    if (!head_dim_ok(d)) return ATTN_ERR_HEAD_DIM;
    return ATTN_OK;
}

attn_status check_scale(float scale) {
    if (!std::isfinite(scale) || !(scale > 0.0f)) return ATTN_ERR_SCALE;
    return ATTN_OK;
}

// Mask kind and window of a problem; the window is returned in the form the
// kernels take: 0 = no band, else W with 1 <= W < N (a band of N or more keys
// is the plain causal mask).
attn_status check_mask(const attn_problem& pr, int* kernel_mask, int* kernel_window) {
    switch (pr.mask) {
        case ATTN_MASK_NONE:
        case ATTN_MASK_CAUSAL:
            if (pr.window != 0) return ATTN_ERR_WINDOW;
            *kernel_mask = pr.mask == ATTN_MASK_NONE ? attn::kMaskNone : attn::kMaskCausal;
            *kernel_window = 0;
            return ATTN_OK;
        case ATTN_MASK_SLIDING_WINDOW:
            if (pr.window < 1) return ATTN_ERR_WINDOW;
            if (pr.window >= pr.N) {
                *kernel_mask = attn::kMaskCausal;
                *kernel_window = 0;
            } else {
                *kernel_mask = attn::kMaskWindow;
                *kernel_window = pr.window;
            }
            return ATTN_OK;
        default: return ATTN_ERR_WINDOW;
    }
}

attn_status hip_status(hipError_t e) {
    if (e == hipSuccess) return ATTN_OK;
    std::snprintf(g_last_hip_error, sizeof g_last_hip_error, "%s", hipGetErrorString(e));
    return ATTN_ERR_HIP;
}

attn::Strides strides_of(const attn_tensor& t) { return {t.stride_b, t.stride_h, t.stride_n}; }

// Dropout parameters of a problem: threshold floor(p * 2^32) on the 32-bit
// Philox words, and the 1/(1-p) scale of the kept weights.
attn_status make_drop(const attn_problem& pr, attn::DropParams* d) {
    const float pd = pr.dropout_p;
    if (!std::isfinite(pd) || pd < 0.0f || pd >= 1.0f) return ATTN_ERR_DROPOUT;
    // 16-bit threshold: the realised drop probability is thr / 2^16, and the
    // kept weights are scaled by its complement's inverse (unbiased).
    const double t = std::floor((double)pd * 65536.0);
    d->thr = t >= 65535.0 ? 65535u : (uint32_t)t;
    d->scale = (float)(1.0 / (1.0 - d->thr / 65536.0));
    d->seed_lo = (uint32_t)(pr.seed & 0xffffffffull);
    d->seed_hi = (uint32_t)(pr.seed >> 32);
    d->offset = pr.offset;
    return ATTN_OK;
}

// Contiguous BHSD view of a plain pointer.
attn_tensor bhsd(const void* p, int H, int N, int d) {
    attn_tensor t;
    t.data = const_cast<void*>(p);
    t.stride_n = d;
    t.stride_h = (long long)N * d;
    t.stride_b = (long long)H * N * d;
    return t;
}

// Checks of the tensors an entry point uses: presence first (NULL), then
// strides (STRIDE, ALIGN) and data alignment (ALIGN), so that the error
// reported is the same whichever tensor carries it.
attn_status check_null(const attn_tensor* const* ts, int n) {
    for (int i = 0; i < n; ++i)
        if (!ts[i] || !ts[i]->data) return ATTN_ERR_NULL;
    return ATTN_OK;
}
// rows > 0: the kernels address a head's rows through 32-bit byte offsets,
// so (rows - 1) * stride_n + d elements must stay under 2^31.
attn_status check_layout(const attn_tensor* const* ts, int n, int rows = 0, int d = 0) {
    for (int i = 0; i < n; ++i)
        if (ts[i]->stride_b < 0 || ts[i]->stride_h < 0 || ts[i]->stride_n < 0) return ATTN_ERR_STRIDE;
    if (rows > 0)
        for (int i = 0; i < n; ++i)
            if ((double)(rows - 1) * (double)ts[i]->stride_n + d >= 2147483648.0) return ATTN_ERR_STRIDE;
    for (int i = 0; i < n; ++i) {
        const attn_tensor& t = *ts[i];
        if (!aligned16(t.data) || (t.stride_b | t.stride_h | t.stride_n) & 7) return ATTN_ERR_ALIGN;
    }
    return ATTN_OK;
}

attn_status fwd_impl(const attn_problem* pr, const attn_tensor* q, const attn_tensor* k,
                     const attn_tensor* v, const attn_tensor* o, float* lse, hipStream_t stream) {
    if (!pr) return ATTN_ERR_NULL;
    const attn_tensor* ts[] = {q, k, v, o};
    attn_status st = check_null(ts, 4);
    if (st != ATTN_OK) return st;
    if (!lse) return ATTN_ERR_NULL;
    st = check_shape(pr->B, pr->Hq, pr->Hkv, pr->N, pr->d);
    if (st != ATTN_OK) return st;
    st = check_scale(pr->scale);
    if (st != ATTN_OK) return st;
    int mask = 0, window = 0;
    st = check_mask(*pr, &mask, &window);
    if (st != ATTN_OK) return st;
    if (pr->dtype != ATTN_DTYPE_BF16 && pr->dtype != ATTN_DTYPE_FP16) return ATTN_ERR_DTYPE;
    attn::DropParams drop;
    st = make_drop(*pr, &drop);
    if (st != ATTN_OK) return st;
    st = check_layout(ts, 4, pr->N, pr->d);
    if (st != ATTN_OK) return st;
    if (!aligned16(lse)) return ATTN_ERR_ALIGN;

    attn::FwdPlan plan;
    attn::fwd_plan(pr->B, pr->Hq, pr->N, pr->d, mask != attn::kMaskNone, drop.thr != 0, &plan);
    attn::FwdParams p;
    p.q = q->data;
    p.k = k->data;
    p.v = v->data;
    p.o = o->data;
    p.lse = lse;
    p.sq = strides_of(*q);
    p.sk = strides_of(*k);
    p.sv = strides_of(*v);
    p.so = strides_of(*o);
    p.N = pr->N;
    p.Hq = pr->Hq;
    p.Hkv = pr->Hkv;
    p.G = pr->Hq / pr->Hkv;
    p.BH = pr->B * pr->Hq;
    p.nqb = (pr->N + plan.block_q - 1) / plan.block_q;
    p.window = window;
    p.c = pr->scale * kLog2eHost;
    p.drop = drop;
    g_last_hip_error[0] = '\0';
    return hip_status(attn::launch_fwd(p, pr->dtype, pr->d, mask, plan, stream));
}

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mutex;

attn_status scratch_of_current_device(const void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e);
    if (dev < 0 || dev >= kMaxDevices) return hip_status(hipErrorInvalidDevice);
    void* ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!ptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mutex);
        ptr = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (!ptr) {
            e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return hip_status(e);
            if (!ptr || !aligned16(ptr)) return hip_status(hipErrorInvalidSymbol);
            g_scratch_ptr[dev].store(ptr, std::memory_order_release);
        }
    }
    *out = ptr;
    return ATTN_OK;
}

// Two float32 per query row, each array 256-byte aligned: D_i, then
// LSE_i * log2(e).
size_t row_terms_bytes(int B, int Hq, int N) {
    const size_t bytes = (size_t)B * Hq * N * sizeof(float);
    return (bytes + 255) & ~(size_t)255;
}

// fp32 partial dK and dV of the head-split or the query-split dK/dV kernel,
// when a shape can use one (the query split's causal threshold covers the
// unmasked one too).
size_t partial_bytes(int B, int Hq, int Hkv, int N, int d) {
    if (attn::dkdv_wide_split(B, Hq, Hkv, N, d) != 2 && attn::dkdv_query_split(B, Hq, Hkv, N, d, true) != 2)
        return 0;
    return 2 * 2 * (size_t)B * Hkv * N * d * sizeof(float);
}

size_t workspace_bytes_for(int B, int Hq, int Hkv, int N, int d) {
    if (check_shape(B, Hq, Hkv, N, d) != ATTN_OK) return 0;
    return 2 * row_terms_bytes(B, Hq, N) + partial_bytes(B, Hq, Hkv, N, d);
}

// Shared validation and dispatch of every backward entry point. Only the
// tensors the selected passes read or write are checked; the others may be
// NULL and are never dereferenced.
// no_alloc: the workspace arguments are ignored and the row terms go to the
// library's fixed scratch array instead (see attn_bwd_noalloc).
attn_status bwd_impl(const attn_problem* pr, const attn_tensor* q, const attn_tensor* k,
                     const attn_tensor* v, const attn_tensor* o, const float* lse,
                     const attn_tensor* dout, const attn_tensor* dq, const attn_tensor* dk,
                     const attn_tensor* dv, const void* workspace, size_t workspace_bytes,
                     unsigned passes, hipStream_t stream, bool no_alloc = false) {
    if (!pr) return ATTN_ERR_NULL;
    if (passes == 0 || (passes & ~(unsigned)attn::kBwdAll)) return ATTN_ERR_PASSES;
    const bool pre = passes & attn::kBwdPre, kv = passes & attn::kBwdDkDv, qq = passes & attn::kBwdDq;
    const bool main = kv || qq;
    const attn_tensor* ts[8];
    int n = 0;
    ts[n++] = dout;
    if (pre) ts[n++] = o;
    if (main) { ts[n++] = q; ts[n++] = k; ts[n++] = v; }
    if (qq) ts[n++] = dq;
    if (kv) { ts[n++] = dk; ts[n++] = dv; }
    attn_status st = check_null(ts, n);
    if (st != ATTN_OK) return st;
    if (!lse) return ATTN_ERR_NULL;  // every pass reads it (the preprocess rescales it)
    st = check_shape(pr->B, pr->Hq, pr->Hkv, pr->N, pr->d);
    if (st != ATTN_OK) return st;
    int mask = 0, window = 0;
    attn::DropParams drop = {0u, 1.0f, 0u, 0u, 0u};
    if (main) {
        st = check_scale(pr->scale);
        if (st != ATTN_OK) return st;
        st = check_mask(*pr, &mask, &window);
        if (st != ATTN_OK) return st;
    }
    if (pr->dtype != ATTN_DTYPE_BF16 && pr->dtype != ATTN_DTYPE_FP16) return ATTN_ERR_DTYPE;
    if (main) {
        st = make_drop(*pr, &drop);
        if (st != ATTN_OK) return st;
    }
    if (no_alloc) {
        if (2 * row_terms_bytes(pr->B, pr->Hq, pr->N) > kScratchBytes) return ATTN_ERR_SCRATCH;
    } else if (!workspace || workspace_bytes < workspace_bytes_for(pr->B, pr->Hq, pr->Hkv, pr->N, pr->d)) {
        return ATTN_ERR_WORKSPACE;
    }
    st = check_layout(ts, n, pr->N, pr->d);
    if (st != ATTN_OK) return st;
    if (!aligned16(lse) || (!no_alloc && !aligned16(workspace))) return ATTN_ERR_ALIGN;
    if (no_alloc) {
        st = scratch_of_current_device(&workspace);
        if (st != ATTN_OK) return st;
    }

    const attn_tensor none = {nullptr, 0, 0, 0};
    auto or_none = [&](const attn_tensor* t, bool used) -> const attn_tensor& {
        return used ? *t : none;
    };
    attn::BwdParams p;
    p.q = or_none(q, main).data;
    p.k = or_none(k, main).data;
    p.v = or_none(v, main).data;
    p.o = or_none(o, pre).data;
    p.lse = lse;
    p.dout = dout->data;
    p.dq = or_none(dq, qq).data;
    p.dk = or_none(dk, kv).data;
    p.dv = or_none(dv, kv).data;
    p.delta = static_cast<float*>(const_cast<void*>(workspace));
    p.lse2 = reinterpret_cast<float*>(static_cast<char*>(const_cast<void*>(workspace)) +
                                      row_terms_bytes(pr->B, pr->Hq, pr->N));
    // The head-split dK/dV kernel needs fp32 partials in the workspace; the
    // fixed scratch has no room for them, so there the 32-key kernel (the
    // faster of the two others on such grids) takes its place.
    p.dkdv = attn::dkdv_wide_split(pr->B, pr->Hq, pr->Hkv, pr->N, pr->d);
    if (no_alloc && p.dkdv == 2) p.dkdv = 0;
    p.hsplit = p.dkdv == 2 ? 2 : 1;
    // The query split of the 32-key kernel; in the fixed scratch only when
    // its partials fit beside the row terms.
    p.qsplit = 1;
    if (p.dkdv == 0 && attn::dkdv_query_split(pr->B, pr->Hq, pr->Hkv, pr->N, pr->d, mask != attn::kMaskNone) == 2) {
        const size_t need = 2 * row_terms_bytes(pr->B, pr->Hq, pr->N) +
                            2 * 2 * (size_t)pr->B * pr->Hkv * pr->N * pr->d * sizeof(float);
        if (!no_alloc || need <= kScratchBytes) p.qsplit = 2;
    }
    p.part = (p.hsplit == 2 || p.qsplit == 2)
                 ? reinterpret_cast<float*>(static_cast<char*>(const_cast<void*>(workspace)) +
                                            2 * row_terms_bytes(pr->B, pr->Hq, pr->N))
                 : nullptr;
    p.sq = strides_of(or_none(q, main));
    p.sk = strides_of(or_none(k, main));
    p.sv = strides_of(or_none(v, main));
    p.so = strides_of(or_none(o, pre));
    p.sdo = strides_of(*dout);
    p.sdq = strides_of(or_none(dq, qq));
    p.sdk = strides_of(or_none(dk, kv));
    p.sdv = strides_of(or_none(dv, kv));
    p.N = pr->N;
    p.Hq = pr->Hq;
    p.Hkv = pr->Hkv;
    p.G = pr->Hq / pr->Hkv;
    p.B = pr->B;
    p.window = window;
    p.scale = pr->scale;
    p.c = pr->scale * kLog2eHost;
    p.drop = drop;
    g_last_hip_error[0] = '\0';
    return hip_status(attn::launch_bwd(p, pr->dtype, pr->d, mask, (int)passes,
                                       stream));
}

attn_problem plain_problem(int B, int Hq, int Hkv, int N, int d, float scale, int causal,
                           int window) {
    attn_problem pr;
    pr.B = B;
    pr.Hq = Hq;
    pr.Hkv = Hkv;
    pr.N = N;
    pr.d = d;
    pr.scale = scale;
    pr.mask = window > 0 ? ATTN_MASK_SLIDING_WINDOW : (causal ? ATTN_MASK_CAUSAL : ATTN_MASK_NONE);
    pr.window = window;
    pr.dtype = ATTN_DTYPE_BF16;
    pr.dropout_p = 0.0f;
    pr.seed = 0;
    pr.offset = 0;
    return pr;
}

// The plain-pointer backward entry points: contiguous bf16 BHSD views of
// whatever pointers a pass uses (NULL stays NULL).
attn_status bwd_plain(const void* q, const void* k, const void* v, const void* o,
                      const float* lse, const void* dout, void* dq, void* dk, void* dv,
                      const void* workspace, size_t workspace_bytes,
                      int B, int Hq, int Hkv, int N, int d, float scale, int causal, int window,
                      hipStream_t stream, unsigned passes) {
    if (window < 0 || (window > 0 && causal == 0)) {
        if (passes & (attn::kBwdDkDv | attn::kBwdDq)) return ATTN_ERR_WINDOW;
        window = 0;
    }
    const attn_problem pr = plain_problem(B, Hq, Hkv, N, d, scale, causal, window);
    const attn_tensor tq = bhsd(q, Hq, N, d), tk = bhsd(k, Hkv, N, d), tv = bhsd(v, Hkv, N, d),
                      to = bhsd(o, Hq, N, d), tdo = bhsd(dout, Hq, N, d), tdq = bhsd(dq, Hq, N, d),
                      tdk = bhsd(dk, Hkv, N, d), tdv = bhsd(dv, Hkv, N, d);
    return bwd_impl(&pr, &tq, &tk, &tv, &to, lse, &tdo, &tdq, &tdk, &tdv, workspace, workspace_bytes,
                    passes, stream);
}

attn_status check_decode(const attn_decode_problem& pr, attn::DecPlan* plan, int* kernel_mask,
                         int* kernel_window) {
    if (pr.Nq < 1 || pr.Nk < 1 || pr.Nq > ATTN_MAX_SEQ_LEN || pr.Nk > ATTN_MAX_SEQ_LEN)
        return ATTN_ERR_SHAPE;
    attn_status st = check_shape(pr.B, pr.Hq, pr.Hkv, pr.Nq > pr.Nk ? pr.Nq : pr.Nk, pr.d);
    if (st != ATTN_OK) return st;
    st = check_scale(pr.scale);
    if (st != ATTN_OK) return st;
    switch (pr.mask) {
        case ATTN_MASK_NONE:
        case ATTN_MASK_CAUSAL:
            if (pr.window != 0) return ATTN_ERR_WINDOW;
            *kernel_mask = pr.mask == ATTN_MASK_NONE ? attn::kMaskNone : attn::kMaskCausal;
            *kernel_window = 0;
            break;
        case ATTN_MASK_SLIDING_WINDOW:
            if (pr.window < 1) return ATTN_ERR_WINDOW;
            // A band of Nk or more keys reaches back past the start of the cache.
            *kernel_mask = pr.window >= pr.Nk ? attn::kMaskCausal : attn::kMaskWindow;
            *kernel_window = pr.window >= pr.Nk ? 0 : pr.window;
            break;
        default: return ATTN_ERR_WINDOW;
    }
    if (pr.dtype != ATTN_DTYPE_BF16 && pr.dtype != ATTN_DTYPE_FP16) return ATTN_ERR_DTYPE;
    attn::decode_plan(pr.B, pr.Hkv, pr.Hq / pr.Hkv, pr.Nq, pr.Nk, pr.d, plan);
    if (plan->workgroups > 0x7fffffffLL) return ATTN_ERR_SHAPE;
    return ATTN_OK;
}

}  // namespace

extern "C" {

size_t attn_decode_workspace_bytes(const attn_decode_problem* problem) {
    if (!problem) return 0;
    attn::DecPlan plan;
    int mask = 0, window = 0;
    if (check_decode(*problem, &plan, &mask, &window) != ATTN_OK) return 0;
    return plan.workspace_bytes;
}

attn_status attn_decode_fwd(const attn_decode_problem* problem, const attn_tensor* q,
                            const attn_tensor* k_cache, const attn_tensor* v_cache,
                            const int* kv_lens, const attn_tensor* o, float* lse,
                            void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (!problem) return ATTN_ERR_NULL;
    const attn_tensor* ts[] = {q, k_cache, v_cache, o};
    attn_status st = check_null(ts, 4);
    if (st != ATTN_OK) return st;
    if (!lse) return ATTN_ERR_NULL;
    attn::DecPlan plan;
    int mask = 0, window = 0;
    st = check_decode(*problem, &plan, &mask, &window);
    if (st != ATTN_OK) return st;
    if (plan.workspace_bytes > 0 && (!workspace || workspace_bytes < plan.workspace_bytes))
        return ATTN_ERR_WORKSPACE;
    st = check_layout(ts, 4);
    if (st != ATTN_OK) return st;
    if (!aligned16(lse) || (plan.workspace_bytes > 0 && !aligned16(workspace)) ||
        (reinterpret_cast<uintptr_t>(kv_lens) & 3u))
        return ATTN_ERR_ALIGN;

    const attn_decode_problem& pr = *problem;
    attn::DecParams p;
    p.q = q->data;
    p.k = k_cache->data;
    p.v = v_cache->data;
    p.o = o->data;
    p.lse = lse;
    p.kv_lens = kv_lens;
    const size_t rows = (size_t)pr.B * pr.Hkv * plan.R;
    p.part_o = plan.workspace_bytes > 0 ? static_cast<float*>(workspace) : nullptr;
    p.part_lse = plan.workspace_bytes > 0
                     ? reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                                ((rows * plan.S * (size_t)pr.d * 4 + 255) & ~(size_t)255))
                     : nullptr;
    p.sq = strides_of(*q);
    p.sk = strides_of(*k_cache);
    p.sv = strides_of(*v_cache);
    p.so = strides_of(*o);
    p.B = pr.B;
    p.Hq = pr.Hq;
    p.Hkv = pr.Hkv;
    p.G = pr.Hq / pr.Hkv;
    p.Nq = pr.Nq;
    p.Nk = pr.Nk;
    p.R = plan.R;
    p.RT = plan.RT;
    p.S = plan.S;
    p.LC = plan.LC;
    p.window = window;
    p.c = pr.scale * kLog2eHost;
    g_last_hip_error[0] = '\0';
    return hip_status(attn::launch_decode(p, pr.dtype, pr.d, mask, stream));
}

attn_status attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                     int B, int Hq, int Hkv, int N, int d, float scale, int causal,
                     hipStream_t stream) {
    const attn_problem pr = plain_problem(B, Hq, Hkv, N, d, scale, causal, 0);
    const attn_tensor tq = bhsd(q, Hq, N, d), tk = bhsd(k, Hkv, N, d), tv = bhsd(v, Hkv, N, d),
                      to = bhsd(o, Hq, N, d);
    return fwd_impl(&pr, &tq, &tk, &tv, &to, lse, stream);
}

attn_status attn_fwd_window(const void* q, const void* k, const void* v, void* o, float* lse,
                            int B, int Hq, int Hkv, int N, int d, float scale, int window,
                            hipStream_t stream) {
    if (window < 1) return ATTN_ERR_WINDOW;
    const attn_problem pr = plain_problem(B, Hq, Hkv, N, d, scale, 1, window);
    const attn_tensor tq = bhsd(q, Hq, N, d), tk = bhsd(k, Hkv, N, d), tv = bhsd(v, Hkv, N, d),
                      to = bhsd(o, Hq, N, d);
    return fwd_impl(&pr, &tq, &tk, &tv, &to, lse, stream);
}

attn_status attn_fwd_ex(const attn_problem* problem, const attn_tensor* q, const attn_tensor* k,
                        const attn_tensor* v, const attn_tensor* o, float* lse, hipStream_t stream) {
    return fwd_impl(problem, q, k, v, o, lse, stream);
}

size_t attn_bwd_workspace_bytes(int B, int Hq, int Hkv, int N, int d) {
    return workspace_bytes_for(B, Hq, Hkv, N, d);
}

attn_status attn_bwd(const void* q, const void* k, const void* v, const void* o,
                     const float* lse, const void* dout,
                     void* dq, void* dk, void* dv,
                     void* workspace, size_t workspace_bytes,
                     int B, int Hq, int Hkv, int N, int d, float scale, int causal,
                     hipStream_t stream) {
    return bwd_plain(q, k, v, o, lse, dout, dq, dk, dv, workspace, workspace_bytes, B, Hq, Hkv, N, d,
                     scale, causal, 0, stream, attn::kBwdAll);
}

attn_status attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                             const float* lse, const void* dout, void* dq, void* dk, void* dv,
                             int B, int Hq, int Hkv, int N, int d, float scale, int causal,
                             hipStream_t stream) {
    const attn_problem pr = plain_problem(B, Hq, Hkv, N, d, scale, causal, 0);
    const attn_tensor tq = bhsd(q, Hq, N, d), tk = bhsd(k, Hkv, N, d), tv = bhsd(v, Hkv, N, d),
                      to = bhsd(o, Hq, N, d), tdo = bhsd(dout, Hq, N, d), tdq = bhsd(dq, Hq, N, d),
                      tdk = bhsd(dk, Hkv, N, d), tdv = bhsd(dv, Hkv, N, d);
    return bwd_impl(&pr, &tq, &tk, &tv, &to, lse, &tdo, &tdq, &tdk, &tdv, nullptr, 0, attn::kBwdAll,
                    stream, true);
}

size_t attn_bwd_noalloc_max_rows(void) { return kScratchBytes / (2 * sizeof(float)); }

attn_status attn_bwd_window(const void* q, const void* k, const void* v, const void* o,
                            const float* lse, const void* dout,
                            void* dq, void* dk, void* dv,
                            void* workspace, size_t workspace_bytes,
                            int B, int Hq, int Hkv, int N, int d, float scale, int window,
                            hipStream_t stream) {
    if (window < 1) return ATTN_ERR_WINDOW;
    return bwd_plain(q, k, v, o, lse, dout, dq, dk, dv, workspace, workspace_bytes, B, Hq, Hkv, N, d,
                     scale, 1, window, stream, attn::kBwdAll);
}

attn_status attn_bwd_preprocess(const void* o, const void* dout, const float* lse, void* workspace,
                                size_t workspace_bytes, int B, int Hq, int Hkv, int N, int d,
                                hipStream_t stream) {
    return bwd_plain(nullptr, nullptr, nullptr, o, lse, dout, nullptr, nullptr, nullptr, workspace,
                     workspace_bytes, B, Hq, Hkv, N, d, 1.0f, 0, 0, stream, attn::kBwdPre);
}

attn_status attn_bwd_dkdv(const void* q, const void* k, const void* v, const float* lse,
                          const void* dout, void* dk, void* dv,
                          const void* workspace, size_t workspace_bytes,
                          int B, int Hq, int Hkv, int N, int d, float scale, int causal,
                          int window, hipStream_t stream) {
    return bwd_plain(q, k, v, nullptr, lse, dout, nullptr, dk, dv, workspace, workspace_bytes, B, Hq,
                     Hkv, N, d, scale, causal, window, stream, attn::kBwdDkDv);
}

attn_status attn_bwd_dq(const void* q, const void* k, const void* v, const float* lse,
                        const void* dout, void* dq,
                        const void* workspace, size_t workspace_bytes,
                        int B, int Hq, int Hkv, int N, int d, float scale, int causal,
                        int window, hipStream_t stream) {
    return bwd_plain(q, k, v, nullptr, lse, dout, dq, nullptr, nullptr, workspace, workspace_bytes, B,
                     Hq, Hkv, N, d, scale, causal, window, stream, attn::kBwdDq);
}

attn_status attn_bwd_ex(const attn_problem* problem, const attn_tensor* q, const attn_tensor* k,
                        const attn_tensor* v, const attn_tensor* o, const float* lse,
                        const attn_tensor* dout, const attn_tensor* dq, const attn_tensor* dk,
                        const attn_tensor* dv, void* workspace, size_t workspace_bytes,
                        unsigned passes, hipStream_t stream) {
    return bwd_impl(problem, q, k, v, o, lse, dout, dq, dk, dv, workspace, workspace_bytes, passes,
                    stream);
}

const char* attn_status_string(attn_status status) {
    // C callers may pass any int; reading an out-of-range value through the
    // enum type is undefined in C++, so the code is copied out as an int.
    int code;
    std::memcpy(&code, &status, sizeof code);
    switch (code) {
        case ATTN_OK: return "ok";
        case ATTN_ERR_NULL: return "a required pointer is NULL";
        case ATTN_ERR_SHAPE: return "B, Hq, Hkv and N must be >= 1 and the sizes must fit the grid";
        case ATTN_ERR_GQA: return "Hq must be a multiple of Hkv";
        case ATTN_ERR_HEAD_DIM:
            return "unsupported head dimension (supported: 32, 64, 80, 96, 128, 192, 256)";
        case ATTN_ERR_SCALE: return "scale must be finite and > 0";
        case ATTN_ERR_ALIGN:
            return "device pointers must be 16-byte aligned and strides multiples of 8 elements";
        case ATTN_ERR_WORKSPACE: return "workspace is NULL or smaller than attn_bwd_workspace_bytes()";
        case ATTN_ERR_HIP: return "the HIP runtime refused a launch (see attn_last_hip_error)";
        case ATTN_ERR_WINDOW:
            return "unknown mask kind, or a window that is < 1 or comes without the causal mask";
        case ATTN_ERR_STRIDE: return "strides must be >= 0";
        case ATTN_ERR_DTYPE: return "unknown element type (supported: bf16, fp16)";
        case ATTN_ERR_PASSES: return "passes must be a nonzero subset of ATTN_BWD_ALL";
        case ATTN_ERR_DROPOUT: return "dropout_p must be in [0, 1)";
        case ATTN_ERR_SCRATCH:
            return "the problem needs more scratch than the fixed buffer of attn_bwd_noalloc holds "
                   "(more than attn_bwd_noalloc_max_rows() query rows)";
    }
    return "unknown status";
}

const char* attn_last_hip_error(void) { return g_last_hip_error; }

attn_status attn_fwd_plan(int B, int Hq, int Hkv, int N, int d, int causal, attn_plan* plan) {
    if (!plan) return ATTN_ERR_NULL;
    const attn_status st = check_shape(B, Hq, Hkv, N, d);
    if (st != ATTN_OK) return st;
    attn::FwdPlan fp;
    attn::fwd_plan(B, Hq, N, d, causal != 0, false, &fp);
    plan->rows_per_wave = fp.rows_per_wave;
    plan->block_q = fp.block_q;
    plan->block_kv = fp.block_kv;
    plan->threads = fp.threads;
    plan->workgroups = fp.workgroups;
    plan->lds_bytes = fp.lds_bytes;
    plan->key_splits = fp.key_splits;
    plan->key_groups = fp.key_groups;
    plan->products16 = fp.m16;
    return ATTN_OK;
}

}  // extern "C"
