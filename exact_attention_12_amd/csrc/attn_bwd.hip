// attn_bwd.hip - attention backward with recomputation, for gfx950.
//
// The forward keeps only O and the row log-sum-exp; the backward recomputes
// the scores and probabilities from Q, K, V and that LSE instead of reading
// stored ones (lpnh.cn FlashAttention-2 article, section 2.3). The pages give
// no gradient formulas; these are the plain chain rule of the forward:
//   P_ij  = exp(scale*<q_i,k_j> - LSE_i)            (allowed keys only)
//   dV_j  = sum_i P_ij dO_i
//   dP_ij = <dO_i, v_j>
//   dS_ij = P_ij (dP_ij - D_i),  D_i = <dO_i, O_i> = sum_j P_ij dP_ij
//   dQ_i  = scale * sum_j dS_ij k_j
//   dK_j  = scale * sum_i dS_ij q_i
// with dK, dV summed over the query heads that share a KV head (GQA).
//
// Three kernels on one stream, no atomics (bitwise deterministic):
//  1. bwd_pre: D_i for every query row (memory bound).
//  2. bwd_dkdv: one workgroup per (batch, KV head, 128-key block); each wave
//     owns 32 keys with K and V held as MFMA operands in VGPRs and dK^T,
//     dV^T accumulated in AGPRs, looping over the G query heads of the
//     group and their 64-row query blocks (under the causal mask only the
//     blocks at or after the keys). Per step: S = Q K^T and dP = dO V^T with
//     Q, dO from LDS (one key per lane, 16 queries per lane in registers);
//     dV^T += dO^T P and dK^T += Q^T dS with dO^T, Q^T read from the same
//     row-major LDS tiles by the transposing read.
//  3. bwd_dq: one workgroup per (batch, query head, 128-row query block), the
//     forward's orientation: S^T = K Q^T and dP^T = V dO^T put one query per
//     lane, so LSE_i and D_i are per-lane scalars; dQ^T += K^T dS^T with K^T
//     read transposed from the K tile.
#include <type_traits>

#include "attn_bwd_common.h"

namespace attn {

// ---------------------------------------------------------------- D_i

template <int D>
__global__ __launch_bounds__(256)
void bwd_pre_kernel(const bf16* __restrict__ o, const bf16* __restrict__ dout,
                    float* __restrict__ delta, long long rows) {
    constexpr int CPR = D / 8;
    const long long row = (long long)blockIdx.x * 16 + (threadIdx.x >> 4);
    const int j = threadIdx.x & 15;
    float acc = 0.0f;
    if (row < rows) {
        const bf16* op = o + row * D;
        const bf16* dp = dout + row * D;
        for (int c = j; c < CPR; c += 16) {
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(op + c * 8);
            const bf16x8 g = *reinterpret_cast<const bf16x8*>(dp + c * 8);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc = fmaf((float)a[e], (float)g[e], acc);
        }
    }
    acc += __shfl_xor(acc, 8);
    acc += __shfl_xor(acc, 4);
    acc += __shfl_xor(acc, 2);
    acc += __shfl_xor(acc, 1);
    if (row < rows && j == 0) delta[row] = acc;
}

// ---------------------------------------------------------------- dK, dV

template <int D, int MASK>
__global__ __launch_bounds__(256, 1)
void bwd_dkdv_kernel(BwdParams p) {
    constexpr bool CAUSAL = MASK != kMaskNone;
    constexpr bool WINDOW = MASK == kMaskWindow;
    constexpr int NW = 4;
    constexpr int T = NW * 64;
    constexpr int BK = NW * 32;        // keys per workgroup
    constexpr int BQ = (D <= 128) ? 64 : 32;  // queries per step
    constexpr int NQT = BQ / 32;
    constexpr int PVS = BQ / 16;
    constexpr int KS = D / 16;
    constexpr int NDT = (D + 31) / 32;
    constexpr int QP = sw_pitch(D);    // Q, dO tiles: row reads and transposing reads
    constexpr int TILE = BQ * QP;
    constexpr int BUF = 2 * TILE * 2 + 2 * BQ * 4;  // bytes: Q, dO, lse2, D

    __shared__ __attribute__((aligned(16))) unsigned char smem_raw[2 * BUF];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l32 = lane & 31;
    const int h = lane >> 5;
    const int N = p.N;

    const int BHk = p.B * p.Hkv;
    const int bid = blockIdx.x;
    const int kb = bid / BHk;           // ascending key blocks: heaviest first when causal
    const int bhk = bid - kb * BHk;
    const int b = bhk / p.Hkv;
    const int hkv = bhk - b * p.Hkv;
    const int k0 = kb * BK;
    const int kw0 = k0 + wave * 32;
    const int key = kw0 + l32;

    const size_t kv_off = (size_t)bhk * N * D;
    const bf16* Kh = static_cast<const bf16*>(p.k) + kv_off;
    const bf16* Vh = static_cast<const bf16*>(p.v) + kv_off;

    auto qtile = [&](int bufi) { return reinterpret_cast<bf16*>(smem_raw + bufi * BUF); };
    auto dotile = [&](int bufi) { return reinterpret_cast<bf16*>(smem_raw + bufi * BUF) + TILE; };
    auto lsetile = [&](int bufi) { return reinterpret_cast<float*>(smem_raw + bufi * BUF + 4 * TILE); };
    auto deltile = [&](int bufi) { return reinterpret_cast<float*>(smem_raw + bufi * BUF + 4 * TILE) + BQ; };

    for (int bufi = 0; bufi < 2; ++bufi) {
        zero_pad_cols_sw<D>(qtile(bufi), BQ, QP, tid, T);
        zero_pad_cols_sw<D>(dotile(bufi), BQ, QP, tid, T);
    }

    // K, V as B operands (lane = key, 8 dims per register group).
    bf16x8 kf[KS], vf[KS];
    if (key < N) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            kf[ks] = *reinterpret_cast<const bf16x8*>(Kh + (size_t)key * D + ks * 16 + h * 8);
            vf[ks] = *reinterpret_cast<const bf16x8*>(Vh + (size_t)key * D + ks * 16 + h * 8);
        }
    } else {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) { kf[ks] = bf16x8{}; vf[ks] = bf16x8{}; }
    }

    const int nqb = (N + BQ - 1) / BQ;
    const int qb_start = CAUSAL ? (k0 / BQ) : 0;
    // Sliding window: only queries i <= (last key) + window - 1 see this block.
    const int W = WINDOW ? p.window : 0;
    const int qb_stop = WINDOW ? min(nqb, (k0 + BK - 1 + W - 1) / BQ + 1) : nqb;
    const int nq_iter = qb_stop - qb_start;
    const int total = p.G * nq_iter;

    TileIO<D, BQ, T> qio, doio;
    float lse_r = 0.0f, del_r = 0.0f;
    auto load_step = [&](int it) {
        const int g = it / nq_iter;
        const int qb = qb_start + (it - g * nq_iter);
        const int hq = hkv * p.G + g;
        const size_t q_off = ((size_t)b * p.Hq + hq) * N;
        const int r0 = qb * BQ;
        qio.load(static_cast<const bf16*>(p.q) + q_off * D, r0, N, tid);
        doio.load(static_cast<const bf16*>(p.dout) + q_off * D, r0, N, tid);
        if (tid < BQ) {
            const int r = r0 + tid;
            lse_r = (r < N) ? p.lse[q_off + r] * kLog2e : __builtin_huge_valf();
        } else if (tid < 2 * BQ) {
            const int r = r0 + tid - BQ;
            del_r = (r < N) ? p.delta[q_off + r] : 0.0f;
        }
    };
    auto store_step = [&](int bufi) {
        qio.store_sw(qtile(bufi), QP, tid);
        doio.store_sw(dotile(bufi), QP, tid);
        if (tid < BQ) lsetile(bufi)[tid] = lse_r;
        else if (tid < 2 * BQ) deltile(bufi)[tid - BQ] = del_r;
    };

    f32x16 dkacc[NDT], dvacc[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) { dkacc[dt] = f32x16{}; dvacc[dt] = f32x16{}; }

    const float c = p.c;
    const int g16 = lane >> 4;
    const int j16 = lane & 15;
    const int tr_row = (g16 >> 1) * 4 + (j16 >> 2);
    const int tr_col = (g16 & 1) * 16 + (j16 & 3) * 4;

    if (total > 0) {
        load_step(0);
        store_step(0);
    }
    __syncthreads();

    for (int it = 0; it < total; ++it) {
        const int bufi = it & 1;
        const bool has_next = it + 1 < total;
        if (has_next) load_step(it + 1);

        const int g = it / nq_iter;
        const int q0 = (qb_start + (it - g * nq_iter)) * BQ;
        // Every step runs for every wave (no data-dependent branch in the
        // loop body): a wave whose keys all lie after this query block just
        // contributes zeros through the mask.
        {
            const bf16* Qs = qtile(bufi);
            const bf16* dOs = dotile(bufi);
            const float* Ls = lsetile(bufi);
            const float* Ds = deltile(bufi);
            f32x16 s[NQT], dp[NQT];
#pragma unroll
            for (int qt = 0; qt < NQT; ++qt) {
                s[qt] = f32x16{};
                dp[qt] = f32x16{};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const int off = sw_off(qt * 32 + l32, ks * 16 + h * 8, QP);
                    s[qt] = mfma32(lds_read8(Qs + off), kf[ks], s[qt]);
                    dp[qt] = mfma32(lds_read8(dOs + off), vf[ks], dp[qt]);
                }
            }
            // P = exp2(c*S - LSE2) and dS = P (dP - D), packed to bf16 in the
            // B-operand order of the dV/dK products. Under the causal mask the
            // query of register r (local offset qoff(r) + 4h) is masked for
            // this lane's key when key - q0 - 4h > qoff(r) (one compare with a
            // constant per element), and under a sliding window also when
            // qoff(r) > key - q0 - 4h + W - 1.
            bf16x8 pb[PVS], dsb[PVS];
            {
                const int kq = key - q0 - 4 * h;
                const int kq_w = kq + W - 1;
#pragma unroll
                for (int u = 0; u < PVS; ++u) {
                    const int qt = u >> 1;
                    const int r0 = (u & 1) * 8;
                    bf16x2 pp[4], dd[4];
#pragma unroll
                    for (int e2 = 0; e2 < 4; ++e2) {
                        float pv[2], dv[2];
#pragma unroll
                        for (int w = 0; w < 2; ++w) {
                            const int r = r0 + 2 * e2 + w;
                            const int qoff = qt * 32 + (r >> 2) * 8 + (r & 3);
                            const int ql = qoff + h * 4;
                            float pe = fast_exp2(fmaf(s[qt][r], c, -Ls[ql]));
                            if (CAUSAL && kq > qoff) pe = 0.0f;
                            if (WINDOW && qoff > kq_w) pe = 0.0f;
                            pv[w] = pe;
                            dv[w] = pe * (dp[qt][r] - Ds[ql]);
                        }
                        pp[e2] = to_bf16x2(pv[0], pv[1]);
                        dd[e2] = to_bf16x2(dv[0], dv[1]);
                    }
                    pb[u] = cat8(pp[0], pp[1], pp[2], pp[3]);
                    dsb[u] = cat8(dd[0], dd[1], dd[2], dd[3]);
                }
            }
            // dV^T += dO^T P and dK^T += Q^T dS. The transposed operands of
            // contraction step u+1 are read from LDS before the products of
            // step u are issued, so the reads overlap the matrix work.
            bf16x8 a_do[NDT], a_q[NDT];
            auto read_ops = [&](int u, bf16x8* ado, bf16x8* aq) {
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) {
                    // Rows u*16 + tr_row and +8 share (row & 7) = tr_row.
                    const int o0 = sw_off(u * 16 + tr_row, dt * 32 + tr_col, QP);
                    ado[dt] = join8(lds_read_tr4(dOs + o0), lds_read_tr4(dOs + o0 + 8 * QP));
                    aq[dt] = join8(lds_read_tr4(Qs + o0), lds_read_tr4(Qs + o0 + 8 * QP));
                }
            };
            // (d = 256 has no registers to spare for the look-ahead copy.)
            constexpr bool LOOKAHEAD = NDT <= 4;
            read_ops(0, a_do, a_q);
#pragma unroll
            for (int u = 0; u < PVS; ++u) {
                bf16x8 n_do[NDT], n_q[NDT];
                if (LOOKAHEAD && u + 1 < PVS) read_ops(u + 1, n_do, n_q);
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) {
                    mfma32_agpr(dvacc[dt], a_do[dt], pb[u]);
                    mfma32_agpr(dkacc[dt], a_q[dt], dsb[u]);
                }
                if (!LOOKAHEAD && u + 1 < PVS) read_ops(u + 1, a_do, a_q);
                if (LOOKAHEAD && u + 1 < PVS) {
#pragma unroll
                    for (int dt = 0; dt < NDT; ++dt) { a_do[dt] = n_do[dt]; a_q[dt] = n_q[dt]; }
                }
            }
        }
        if (has_next) store_step(bufi ^ 1);
        __syncthreads();
    }

#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
        agpr_acc_ready(dkacc[dt]);
        agpr_acc_ready(dvacc[dt]);
    }
    if (key < N) {
        bf16* dkrow = static_cast<bf16*>(p.dk) + kv_off + (size_t)key * D;
        bf16* dvrow = static_cast<bf16*>(p.dv) + kv_off + (size_t)key * D;
        const float sc = p.scale;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int d = dt * 32 + g4 * 8 + h * 4;
                if (d < D) {
                    store_bf16x4(dkrow + d, dkacc[dt][g4 * 4 + 0] * sc, dkacc[dt][g4 * 4 + 1] * sc,
                                 dkacc[dt][g4 * 4 + 2] * sc, dkacc[dt][g4 * 4 + 3] * sc);
                    store_bf16x4(dvrow + d, dvacc[dt][g4 * 4 + 0], dvacc[dt][g4 * 4 + 1],
                                 dvacc[dt][g4 * 4 + 2], dvacc[dt][g4 * 4 + 3]);
                }
            }
    }
}

// ---------------------------------------------------------------- launch

template <int D, int MASK>
static hipError_t launch_bwd_dc(const BwdParams& p, int passes, hipStream_t stream) {
    if (passes & kBwdPre) {
        const long long rows = (long long)p.B * p.Hq * p.N;
        hipLaunchKernelGGL((bwd_pre_kernel<D>), dim3((unsigned)((rows + 15) / 16)), dim3(256), 0,
                           stream, static_cast<const bf16*>(p.o), static_cast<const bf16*>(p.dout),
                           p.delta, rows);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (passes & kBwdDkDv) {
        const long long nkb = (p.N + 127) / 128;
        hipLaunchKernelGGL((bwd_dkdv_kernel<D, MASK>), dim3((unsigned)(nkb * p.B * p.Hkv)), dim3(256),
                           0, stream, p);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (passes & kBwdDq) {
        const hipError_t e = launch_bwd_dq(p, D, MASK, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <int D>
static hipError_t launch_bwd_d(const BwdParams& p, int mask, int passes, hipStream_t stream) {
    switch (mask) {
        case kMaskNone: return launch_bwd_dc<D, kMaskNone>(p, passes, stream);
        case kMaskCausal: return launch_bwd_dc<D, kMaskCausal>(p, passes, stream);
        case kMaskWindow: return launch_bwd_dc<D, kMaskWindow>(p, passes, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_bwd(const BwdParams& p, int d, int mask, int passes, hipStream_t stream) {
    switch (d) {
        case 64: return launch_bwd_d<64>(p, mask, passes, stream);
        case 80: return launch_bwd_d<80>(p, mask, passes, stream);
        case 128: return launch_bwd_d<128>(p, mask, passes, stream);
        case 256: return launch_bwd_d<256>(p, mask, passes, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace attn
