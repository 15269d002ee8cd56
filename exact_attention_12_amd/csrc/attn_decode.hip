// attn_decode.hip - attention of a few new queries against a key/value cache
// (decoding), for gfx950.
//
// What it computes: per sequence b with L_b valid cache rows, query i of
// query head h sits at position p_i = L_b - Nq + i and attends to the cache
// rows j < L_b that its mask allows (all of them; j <= p_i when causal;
// p_i - W < j <= p_i under a sliding window of W), i.e. the last Nq rows of
// self-attention over the cached sequence. The KV cache that GQA shrinks is
// the subject of the yunthe.com GQA page (sections on the MHA KV cache and
// on GQA); the mask modes are those of the CANN FlashAttention page's tuning
// section.
//
// The work is bound by reading the cache once, so the kernels are laid out
// for HBM, not for the matrix cores:
//  * all G query heads of a KV head are processed together (R = G * Nq rows
//    in 32-row tiles), so each cache row is read once per KV head, not G
//    times;
//  * the cache of each (sequence, KV head) is cut into S splits of LC keys
//    so that the grid holds thousands of one-wave workgroups even at batch 1;
//    each wave streams its split through a 32-key LDS tile (the next tile's
//    16-byte global loads are issued before the current tile's math);
//  * S^T = K Q^T and O^T += V^T P^T run on the matrix cores in the forward
//    kernel's orientation (one query row per lane, V^T through the
//    transposing LDS read); the online softmax keeps m, l per lane;
//  * a split writes its normalised partial O and its log2-domain LSE; the
//    merge kernel combines the S partials of a row with the online-softmax
//    identity O = sum_s w_s O_s / sum_s w_s, w_s = 2^(lse_s - max lse).
#include "attn_device.h"
#include "attn_kernels.h"

namespace attn {

namespace {

constexpr int kDecThreads = 64;  // one wave per workgroup
constexpr int kDecBC = 32;       // keys per tile

// Maximum and sum over the 64 lanes of a wave.
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
    return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

}  // namespace

// Two waves per SIMD at D <= 128 (for D = 128 the compiler then spills a few
// registers; the second wave's loads in flight are worth more: 116 -> 109 us
// on a 32 x 8-KV-head x 4096-key bf16 cache).
template <int DT, int D, int MASK>
__global__ __launch_bounds__(kDecThreads) __attribute__((amdgpu_waves_per_eu(D <= 128 ? 2 : 1)))
void decode_split_kernel(DecParams p) {
    constexpr bool CAUSAL = MASK != kMaskNone;
    constexpr bool WINDOW = MASK == kMaskWindow;
    constexpr int BC = kDecBC;
    constexpr int T = kDecThreads;
    constexpr int KS = D / 16;
    constexpr int NDT = (D + 31) / 32;
    constexpr int PVS = BC / 16;
    constexpr int KP = k_pitch(D);
    constexpr int VP = v_pitch(D);
    constexpr int CPR = D / 8;
    constexpr int CHUNKS = BC * CPR;
    constexpr int NCH = (CHUNKS + T - 1) / T;

    __shared__ __attribute__((aligned(16))) e16 smem[BC * (KP + VP)];
    e16* Ks = smem;
    e16* Vs = smem + BC * KP;

    const int lane = threadIdx.x;
    const int l32 = lane & 31;
    const int h = lane >> 5;

    const int bid = blockIdx.x;
    const int s = bid % p.S;
    const int t = (bid / p.S) % p.RT;
    const int bhk = bid / (p.S * p.RT);
    const int b = bhk / p.Hkv;
    const int hkv = bhk - b * p.Hkv;
    int Lb = p.Nk;
    if (p.kv_lens) Lb = min(max(p.kv_lens[b], 0), p.Nk);
    const int k_begin = s * p.LC;
    const int k_end = min(k_begin + p.LC, Lb);

    // This lane's query row: r = t*32 + l32 -> (group member g, position i).
    const int r = t * 32 + l32;
    const bool row_ok = r < p.R;
    const int g = row_ok ? r / p.Nq : 0;
    const int i = row_ok ? r - g * p.Nq : 0;
    const int hq = hkv * p.G + g;
    const int pos = Lb - p.Nq + i;

    if constexpr (NDT * 32 > D) {
        constexpr int PADC = NDT * 32 - D;
        for (int x = lane; x < BC * PADC; x += T) Vs[(x / PADC) * VP + D + x % PADC] = (e16)0;
    }

    e16x8 qf[KS];
    if (row_ok) {
        const e16* qp = static_cast<const e16*>(p.q) + b * p.sq.b + hq * p.sq.h + i * p.sq.n + h * 8;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qf[ks] = *reinterpret_cast<const e16x8*>(qp + ks * 16);
    } else {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qf[ks] = e16x8{};
    }

    // Under a window no row of the tile sees keys before the earliest band
    // start, min_i p_i - W + 1 = L_b - Nq - W + 1: start the split there.
    int kv_first = k_begin;
    if (WINDOW) {
        const int lo = Lb - p.Nq - p.window + 1;
        if (lo > k_begin) kv_first = k_begin + ((lo - k_begin) / BC) * BC;
    }

    const e16* Kh = static_cast<const e16*>(p.k) + b * p.sk.b + hkv * p.sk.h;
    const e16* Vh = static_cast<const e16*>(p.v) + b * p.sv.b + hkv * p.sv.h;
    uint4 kreg[NCH], vreg[NCH];
    auto load_tile = [&](int kv0) {
#pragma unroll
        for (int x = 0; x < NCH; ++x) {
            const int c = lane + x * T;
            if (CHUNKS % T == 0 || c < CHUNKS) {
                const int row = c / CPR;
                const int col = c - row * CPR;
                const int key = kv0 + row;
                if (key < k_end) {
                    kreg[x] = *reinterpret_cast<const uint4*>(Kh + key * p.sk.n + col * 8);
                    vreg[x] = *reinterpret_cast<const uint4*>(Vh + key * p.sv.n + col * 8);
                } else {
                    kreg[x] = zero4();
                    vreg[x] = zero4();
                }
            }
        }
    };
    auto store_tile = [&]() {
#pragma unroll
        for (int x = 0; x < NCH; ++x) {
            const int c = lane + x * T;
            if (CHUNKS % T == 0 || c < CHUNKS) {
                const int row = c / CPR;
                const int col = c - row * CPR;
                *reinterpret_cast<uint4*>(Ks + row * KP + col * 8) = kreg[x];
                *reinterpret_cast<uint4*>(Vs + row * VP + col * 8) = vreg[x];
            }
        }
    };

    f32x16 oacc[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) oacc[dt] = f32x16{};
    float m = -__builtin_huge_valf();
    float l = 0.0f;
    const float c = p.c;
    const int g16 = lane >> 4;
    const int j16 = lane & 15;
    const int tr_row = (g16 >> 1) * 4 + (j16 >> 2);
    const int tr_col = (g16 & 1) * 16 + (j16 & 3) * 4;
    // Allowed keys of this row, relative to kv0 + 4h: [lo_rel, hi_rel].
    const int hi_abs = CAUSAL ? min(k_end - 1, pos) : k_end - 1;
    const int lo_abs = WINDOW ? pos - p.window + 1 : 0;

    if (kv_first < k_end) {
        load_tile(kv_first);
        store_tile();
    }
    __syncthreads();
    for (int kv0 = kv_first; kv0 < k_end; kv0 += BC) {
        const bool has_next = kv0 + BC < k_end;
        if (has_next) load_tile(kv0 + BC);

        f32x16 sc = f32x16{};
        {
            const e16* kp = Ks + l32 * KP + h * 8;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) sc = mfma32<DT>(lds_read8(kp + ks * 16), qf[ks], sc);
        }
        const int hi = hi_abs - kv0 - 4 * h;
        const int lo = lo_abs - kv0 - 4 * h;
        float mx = -__builtin_huge_valf();
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int koff = (e >> 2) * 8 + (e & 3);
            sc[e] = (koff > hi || koff < lo) ? -__builtin_huge_valf() : sc[e] * c;
            mx = fmaxf(mx, sc[e]);
        }
        const float m_new = fmaxf(m, max_across_halves(mx));
        // A row with no allowed key so far keeps m = -inf: exponents use 0.
        const float m_use = (m_new == -__builtin_huge_valf()) ? 0.0f : m_new;
        const float alpha = fast_exp2(m - m_use);
        m = m_new;
        l *= alpha;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) oacc[dt] *= alpha;

        e16x8 pb[PVS];
#pragma unroll
        for (int u = 0; u < PVS; ++u) {
            e16x2 pr[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float a0 = fast_exp2(sc[u * 8 + 2 * e] - m_use);
                const float a1 = fast_exp2(sc[u * 8 + 2 * e + 1] - m_use);
                pr[e] = cvt2<DT>(a0, a1);
                l += a0 + a1;
            }
            pb[u] = cat8(pr[0], pr[1], pr[2], pr[3]);
        }
#pragma unroll
        for (int u = 0; u < PVS; ++u) {
            const e16* vp = Vs + (u * 16 + tr_row) * VP + tr_col;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
                const e16x8 a = join8(lds_read_tr4(vp + dt * 32), lds_read_tr4(vp + 8 * VP + dt * 32));
                oacc[dt] = mfma32<DT>(a, pb[u], oacc[dt]);
            }
        }
        __syncthreads();
        if (has_next) store_tile();
        __syncthreads();
    }

    if (!row_ok) return;
    const float lt = sum_across_halves(l);
    const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
    const float lse2 = lt > 0.0f ? m + __builtin_amdgcn_logf(lt) : -__builtin_huge_valf();
    if (p.S == 1) {
        e16* orow = static_cast<e16*>(p.o) + b * p.so.b + hq * p.so.h + i * p.so.n;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int d = dt * 32 + g4 * 8 + h * 4;
                if (d < D)
                    store4<DT>(orow + d, oacc[dt][g4 * 4 + 0] * inv, oacc[dt][g4 * 4 + 1] * inv,
                               oacc[dt][g4 * 4 + 2] * inv, oacc[dt][g4 * 4 + 3] * inv);
            }
        if (h == 0) p.lse[((size_t)b * p.Hq + hq) * p.Nq + i] = lse2 * kLn2;
        return;
    }
    const size_t prow = (size_t)bhk * p.R + r;
    if (h == 0) p.part_lse[prow * p.S + s] = lse2;
    if (lt > 0.0f) {  // empty splits are skipped by the merge
        float* po = p.part_o + (prow * p.S + s) * D;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int d = dt * 32 + g4 * 8 + h * 4;
                if (d < D)
                    *reinterpret_cast<f32x4*>(po + d) =
                        f32x4{oacc[dt][g4 * 4 + 0] * inv, oacc[dt][g4 * 4 + 1] * inv,
                              oacc[dt][g4 * 4 + 2] * inv, oacc[dt][g4 * 4 + 3] * inv};
            }
    }
}

// One wave per query row: lanes cover d (4 consecutive values each). The
// row index is wave-uniform, so the split LSEs are scalar loads; the maximum
// and the weight sum run across lanes (split s on lane s % 64), and the
// partial outputs are fetched eight splits at a time.
template <int DT, int D>
__global__ __launch_bounds__(256)
void decode_merge_kernel(DecParams p, long long rows) {
    const long long prow =
        (long long)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int lane = threadIdx.x & 63;
    if (prow >= rows) return;
    const int S = p.S;
    const float* pl = p.part_lse + prow * S;
    float mloc = -__builtin_huge_valf();
    for (int s = lane; s < S; s += 64) mloc = fmaxf(mloc, pl[s]);
    const float M = wave_max(mloc);
    const bool any = M != -__builtin_huge_valf();  // some split saw an allowed key
    float wl = 0.0f;
    for (int s = lane; s < S; s += 64) {
        const float ls = pl[s];
        wl += (any && ls != -__builtin_huge_valf()) ? fast_exp2(ls - M) : 0.0f;
    }
    const float wsum = wave_sum(wl);
    const long long bhk = prow / p.R;
    const int r = (int)(prow - bhk * p.R);
    const int b = (int)(bhk / p.Hkv);
    const int hkv = (int)(bhk - (long long)b * p.Hkv);
    const int g = r / p.Nq;
    const int i = r - g * p.Nq;
    const int hq = hkv * p.G + g;
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    const int d0 = lane * 4;
    if (any && d0 < D) {
        const float* po = p.part_o + prow * S * D + d0;
        for (int s0 = 0; s0 < S; s0 += 8) {
            f32x4 x[8];
            float w[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int s = s0 + u;
                const float ls = s < S ? pl[s] : -__builtin_huge_valf();
                w[u] = ls != -__builtin_huge_valf() ? fast_exp2(ls - M) : 0.0f;
                // empty splits wrote no partial O: their slot is read but not used
                x[u] = s < S ? *reinterpret_cast<const f32x4*>(po + (long long)s * D) : f32x4{};
            }
#pragma unroll
            for (int u = 0; u < 8; ++u)
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[e] = fmaf(w[u], w[u] > 0.0f ? x[u][e] : 0.0f, acc[e]);
        }
    }
    const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
    if (d0 < D) {
        e16* orow = static_cast<e16*>(p.o) + b * p.so.b + hq * p.so.h + i * p.so.n;
        store4<DT>(orow + d0, acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
    }
    if (lane == 0)
        p.lse[((size_t)b * p.Hq + hq) * p.Nq + i] =
            wsum > 0.0f ? (M + __builtin_amdgcn_logf(wsum)) * kLn2 : -__builtin_huge_valf();
}

template <int DT, int D, int MASK>
static hipError_t launch_decode_dm(const DecParams& p, hipStream_t stream) {
    const long long wgs = (long long)p.B * p.Hkv * p.RT * p.S;
    hipLaunchKernelGGL((decode_split_kernel<DT, D, MASK>), dim3((unsigned)wgs), dim3(kDecThreads), 0,
                       stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.S == 1) return e;
    const long long rows = (long long)p.B * p.Hkv * p.R;
    hipLaunchKernelGGL((decode_merge_kernel<DT, D>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0,
                       stream, p, rows);
    return hipGetLastError();
}

template <int DT, int D>
static hipError_t launch_decode_d(const DecParams& p, int mask, hipStream_t stream) {
    switch (mask) {
        case kMaskNone: return launch_decode_dm<DT, D, kMaskNone>(p, stream);
        case kMaskCausal: return launch_decode_dm<DT, D, kMaskCausal>(p, stream);
        case kMaskWindow: return launch_decode_dm<DT, D, kMaskWindow>(p, stream);
        default: return hipErrorInvalidValue;
    }
}

template <int DT>
static hipError_t launch_decode_t(const DecParams& p, int d, int mask, hipStream_t stream) {
    switch (d) {
#define ATTN_DEC_CASE(D_) \
        case D_: return launch_decode_d<DT, D_>(p, mask, stream);
        ATTN_FOR_EACH_HEAD_DIM(ATTN_DEC_CASE)
#undef ATTN_DEC_CASE
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_decode(const DecParams& p, int dtype, int d, int mask, hipStream_t stream) {
    switch (dtype) {
        case kBF16: return launch_decode_t<kBF16>(p, d, mask, stream);
        case kFP16: return launch_decode_t<kFP16>(p, d, mask, stream);
        default: return hipErrorInvalidValue;
    }
}

// Split plan: enough one-wave workgroups for 8 per compute unit (2048),
// splits of at least 64 keys, LC a multiple of the 32-key tile.
bool decode_plan(int B, int Hkv, int G, int Nq, int Nk, int d, DecPlan* plan) {
    (void)d;
    const long long R = (long long)G * Nq;
    const long long RT = (R + 31) / 32;
    const long long groups = (long long)B * Hkv * RT;
    long long S = (2048 + groups - 1) / groups;
    const long long max_s = (Nk + 63) / 64;
    if (S > max_s) S = max_s;
    if (S < 1) S = 1;
    long long LC = (Nk + S - 1) / S;
    LC = (LC + 31) / 32 * 32;
    S = (Nk + LC - 1) / LC;
    if (S < 1) S = 1;
    plan->R = (int)R;
    plan->RT = (int)RT;
    plan->S = (int)S;
    plan->LC = (int)LC;
    plan->workgroups = groups * S;
    const size_t rows = (size_t)B * Hkv * R;
    plan->workspace_bytes = S == 1 ? 0 : ((rows * S * (size_t)d * 4 + 255) & ~(size_t)255) +
                                             ((rows * S * 4 + 255) & ~(size_t)255);
    return true;
}

}  // namespace attn
