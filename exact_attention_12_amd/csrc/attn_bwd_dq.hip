// attn_bwd_dq.hip - dQ pass of the attention backward, for gfx950.
//
// One workgroup per (batch, query head, 128-row query block), in the
// forward's orientation: S^T = K Q^T and dP^T = V dO^T put one query per
// lane, so LSE_i and D_i are per-lane scalars; dQ^T += K^T dS^T with K^T read
// from the (chunk-swizzled) K tile by the transposing LDS read. It is a
// separate translation unit because it is scheduled for occupancy (two waves
// per SIMD), while the dK/dV pass, one wave per SIMD, is scheduled for ILP.
// The formulas are the chain rule written out in attn_bwd.hip.
#include <type_traits>

#include "attn_bwd_common.h"

namespace attn {

// ---------------------------------------------------------------- dQ

template <int DT, int D, int MASK, bool DROP>
__global__ __launch_bounds__(256, (D <= 128 ? 2 : 1))
void bwd_dq_kernel(BwdParams p) {
    constexpr bool CAUSAL = MASK != kMaskNone;
    constexpr bool WINDOW = MASK == kMaskWindow;
    constexpr int NW = 4;
    constexpr int T = NW * 64;
    constexpr int BQ = NW * 32;
    // Keys per step: 64 halves the per-step overhead while two waves per SIMD
    // still fit without spills; dropout (its keep bits) and d > 128 take 32.
    constexpr int BC = (D <= 128 && !DROP) ? 64 : 32;
    constexpr int KS = D / 16;
    constexpr int NDT = (D + 31) / 32;
    constexpr int NKT = BC / 32;
    constexpr int PVS = BC / 16;
    constexpr int KP = sw_pitch(D);    // K tile: row reads and transposing reads
    constexpr int VP = k_pitch(D);     // V tile: row reads only
    constexpr int BUF = BC * (KP + VP);

    __shared__ __attribute__((aligned(16))) e16 smem[2 * BUF];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches and buffer resources
    const int l32 = lane & 31;
    const int h = lane >> 5;
    const int N = p.N;

    const int BH = p.B * p.Hq;
    const int nqb = (N + BQ - 1) / BQ;
    const int bid = blockIdx.x;
    const int bh = xcd_head(bid % BH, BH);
    const int qb = CAUSAL ? (nqb - 1 - bid / BH) : (bid / BH);
    const int b = bh / p.Hq;
    const int hq = bh - b * p.Hq;
    const int hkv = hq / p.G;
    const size_t row_off = (size_t)bh * N;  // LSE, D_i: contiguous [B, Hq, N]
    const e16* Kh = static_cast<const e16*>(p.k) + b * p.sk.b + hkv * p.sk.h;
    const e16* Vh = static_cast<const e16*>(p.v) + b * p.sv.b + hkv * p.sv.h;

    const int q0 = qb * BQ;
    const int qw0 = q0 + wave * 32;
    const int qrow = qw0 + l32;


    e16x8 qf[KS], gf[KS];
    float lse2 = __builtin_huge_valf(), ndel = 0.0f;  // ndel = -D_i, as the preprocess stores it
    if (qrow < N) {
        const e16* qp = static_cast<const e16*>(p.q) + b * p.sq.b + hq * p.sq.h + qrow * p.sq.n + h * 8;
        const e16* gp =
            static_cast<const e16*>(p.dout) + b * p.sdo.b + hq * p.sdo.h + qrow * p.sdo.n + h * 8;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            qf[ks] = *reinterpret_cast<const e16x8*>(qp + ks * 16);
            gf[ks] = *reinterpret_cast<const e16x8*>(gp + ks * 16);
        }
        lse2 = p.lse[row_off + qrow] * kLog2e;
        ndel = p.delta[row_off + qrow];
    } else {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) { qf[ks] = e16x8{}; gf[ks] = e16x8{}; }
    }

    const int nkb = (N + BC - 1) / BC;
    const int kb_end = CAUSAL ? min(nkb, (q0 + BQ - 1) / BC + 1) : nkb;
    // Sliding window: keys before the first row's band are skipped.
    const int W = WINDOW ? p.window : 0;
    const int kb_begin = WINDOW ? max(0, q0 - W + 1) / BC : 0;
    // Key blocks that need no per-element mask form [ku_begin, ku_end): all
    // keys at or before the workgroup's first query (kv0 + BC - 1 <= q0),
    // inside its last query's band (kv0 >= q0 + BQ - W) and before N. Keys
    // past N must stay masked: their zero scores would give exp2(-LSE2),
    // which overflows for rows with a very negative LSE.
    int ku_begin = kb_begin, ku_end = min(kb_end, N / BC);
    if (CAUSAL) ku_end = min(ku_end, (q0 + 1) / BC);
    if (WINDOW) {
        const int t = q0 + BQ - W;
        ku_begin = min(kb_end, max(kb_begin, t > 0 ? (t + BC - 1) / BC : 0));
    }
    ku_end = max(ku_end, ku_begin);

    // K/V tiles go straight from memory to LDS: each 64-lane buffer load
    // with the LDS flag fills 64 consecutive 16-byte chunks; lane i of load j
    // covers chunk 64j + i of the padded tile (row = chunk / pitch-chunks).
    // The K tile is swizzled, so that slot holds logical chunk slot ^
    // sw_swizzle(row). Chunks past d (padding) and rows past N read as zeros; lanes past
    // the end of a tile whose chunk count is not a multiple of 64 are idle.
    constexpr int CKK = KP / 8, CKV = VP / 8;
    constexpr int NLK = (BC * CKK + 63) / 64, NLV = (BC * CKV + 63) / 64;
    constexpr int LPWK = (NLK + NW - 1) / NW, LPWV = (NLV + NW - 1) / NW;
    uint32_t offk[LPWK], offv[LPWV];
    {
        const uint32_t sk2 = (uint32_t)p.sk.n * 2u, sv2 = (uint32_t)p.sv.n * 2u;
#pragma unroll
        for (int i = 0; i < LPWK; ++i) {
            const int chunk = (wave + i * NW) * 64 + lane;
            const int row = chunk / CKK;
            const int lc = (chunk - row * CKK) ^ sw_swizzle(row);
            offk[i] = lc < D / 8 ? (uint32_t)row * sk2 + (uint32_t)lc * 16u : 0xFFFFFFF0u;
        }
#pragma unroll
        for (int i = 0; i < LPWV; ++i) {
            const int chunk = (wave + i * NW) * 64 + lane;
            const int row = chunk / CKV;
            const int lc = chunk - row * CKV;
            offv[i] = lc < D / 8 ? (uint32_t)row * sv2 + (uint32_t)lc * 16u : 0xFFFFFFF0u;
        }
    }
    auto issue_tile = [&](int kv0, int bufi) {
        const uint32_t sk2 = (uint32_t)p.sk.n * 2u, sv2 = (uint32_t)p.sv.n * 2u;
        const auto rk = buf_rsrc(Kh + (long long)kv0 * p.sk.n, (uint32_t)(N - kv0 - 1) * sk2 + D * 2);
        const auto rv = buf_rsrc(Vh + (long long)kv0 * p.sv.n, (uint32_t)(N - kv0 - 1) * sv2 + D * 2);
        char* k_lds = reinterpret_cast<char*>(smem + bufi * BUF);
        char* v_lds = k_lds + BC * KP * 2;
#pragma unroll
        for (int i = 0; i < LPWK; ++i) {
            const int j = wave + i * NW;
            if ((NLK % NW == 0 || j < NLK) && (BC * CKK % 64 == 0 || j * 64 + lane < BC * CKK))
                buf_load16_to_lds(rk, k_lds + j * 1024, offk[i]);
        }
#pragma unroll
        for (int i = 0; i < LPWV; ++i) {
            const int j = wave + i * NW;
            if ((NLV % NW == 0 || j < NLV) && (BC * CKV % 64 == 0 || j * 64 + lane < BC * CKV))
                buf_load16_to_lds(rv, v_lds + j * 1024, offv[i]);
        }
    };
    issue_tile(kb_begin * BC, kb_begin & 1);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    f32x16 dqacc[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) dqacc[dt] = f32x16{};
    const float c = p.c;
    const int g16 = lane >> 4;
    const int j16 = lane & 15;
    const int tr_row = (g16 >> 1) * 4 + (j16 >> 2);
    const int tr_col = (g16 & 1) * 16 + (j16 & 3) * 4;
    // Per-lane offsets into the swizzled K tile; the other row and column
    // blocks are immediate offsets (sw_off repeats every 16 rows and 32
    // columns). Row reads: chunk 2ks + h, ks even / odd. Transposing reads:
    // rows tr_row and tr_row + 8.
    const int krd[2] = {sw_off(l32, h * 8, KP), sw_off(l32, 16 + h * 8, KP)};
    const int ktr0 = sw_off(tr_row, tr_col, KP), ktr1 = sw_off(tr_row + 8, tr_col, KP);

    auto run_step = [&](int kb, auto masked_tag) {
        constexpr bool MASKED = decltype(masked_tag)::value;
        const int bufi = kb & 1;
        // The last step reloads its own tile into the idle buffer (never
        // read again), so the loads need no branch.
        issue_tile(min(kb + 1, kb_end - 1) * BC, bufi ^ 1);
        const int kv0 = kb * BC;
        const e16* Ks = smem + bufi * BUF;
        const e16* Vs = Ks + BC * KP;
        // Branch-free step: in the masked blocks, keys past a wave's last
        // query are masked to zero.
        {
            f32x16 s[NKT], dp[NKT];
            // S^T = K Q^T and dP^T = V dO^T with the K and V row reads kept
            // two products ahead, pinned in order by scheduling barriers.
            constexpr int NS = NKT * KS;
            e16x8 kr[3], vr[3];
            auto rd = [&](int idx) {
                const int kt = idx / KS, ks = idx % KS;
                kr[idx % 3] = lds_read8(Ks + krd[ks & 1] + kt * 32 * KP + (ks >> 1) * 32);
                vr[idx % 3] = lds_read8(Vs + (kt * 32 + l32) * VP + h * 8 + ks * 16);
            };
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt) {
                s[kt] = f32x16{};
                dp[kt] = f32x16{};
            }
            // dS^T = P^T (dP^T - D) with P^T = exp2(c*S^T - LSE2), packed to 16 bits
            // in the B-operand order of dQ^T += K^T dS^T. Key kv0 + koff(r) + 4h
            // is masked when it is >= N, (causal) > qrow or (sliding window)
            // < qrow - W + 1: compares with a constant per element, skipped
            // when the block needs no mask.
            // Dropout: dP of a dropped score is zero and a kept one is
            // scaled by 1/(1-p); P itself (and the row term) are not.
            uint32_t keep[NKT];
            if constexpr (DROP) {
#pragma unroll
                for (int kt = 0; kt < NKT; ++kt) {
                    keep[kt] = 0;
#pragma unroll
                    for (int gp = 0; gp < 2; ++gp)
                        keep[kt] |= keep_bits_query_lane(p.drop, kv0 + kt * 32 + 16 * gp + 4 * h, qrow,
                                                         bh) << (8 * gp);
                }
            }
            const int lim = (CAUSAL ? min(qrow, N - 1) : N - 1) - kv0 - 4 * h;
            const int lo = qrow - W + 1 - kv0 - 4 * h;
            e16x2 dd[PVS][4];
            e16x8 dsb[PVS];
            // dS^T of registers (r, r+1) of contraction step u (key tile u >> 1).
            auto sm_pair = [&](int u, int e2) {
                const int kt = u >> 1;
                const int r0 = (u & 1) * 8;
                float dv[2];
#pragma unroll
                for (int w = 0; w < 2; ++w) {
                    const int r = r0 + 2 * e2 + w;
                    const int koff = kt * 32 + (r >> 2) * 8 + (r & 3);
                    float pe = fast_exp2(fmaf(s[kt][r], c, -lse2));
                    if (MASKED && koff > lim) pe = 0.0f;
                    if (MASKED && WINDOW && koff < lo) pe = 0.0f;
                    float dpe = dp[kt][r];
                    if constexpr (DROP) dpe = ((keep[kt] >> r) & 1u) ? dpe * p.drop.scale : 0.0f;
                    dv[w] = pe * (dpe + ndel);
                }
                dd[u][e2] = cvt2<DT>(dv[0], dv[1]);
            };
            auto pack = [&](int u) { dsb[u] = cat8(dd[u][0], dd[u][1], dd[u][2], dd[u][3]); };
            // K^T operand of contraction step u, 32-row tile dt.
            auto ktr = [&](int u, int dt) {
                const int ob = u * 16 * KP + dt * 32;
                return join8(lds_read_tr4(Ks + ktr0 + ob), lds_read_tr4(Ks + ktr1 + ob));
            };
            if constexpr (NKT == 2) {
                // Software pipeline of one step, pinned in order by
                // scheduling barriers between small chunks:
                //   A0: S^T/dP^T of key tile 0, row reads two products ahead;
                //   A1: those of tile 1, with tile 0's dS^T and the first
                //       transposed K reads in their shadow;
                //   C0: the dQ^T products of contraction steps 0 and 1, with
                //       tile 1's dS^T and the next transposed reads;
                //   C1: those of steps 2 and 3.
                rd(0);
                rd(1);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {  // A0
                    rd(ks + 2);
                    s[0] = mfma32<DT>(kr[ks % 3], qf[ks], s[0]);
                    dp[0] = mfma32<DT>(vr[ks % 3], gf[ks], dp[0]);
                    __builtin_amdgcn_sched_barrier(0);
                }
                e16x8 opA[NDT], opB[NDT];
                constexpr int PRA = (8 + KS - 1) / KS;
                constexpr int TRA = (NDT + KS - 1) / KS;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {  // A1
                    const int idx = KS + ks;
                    if (idx + 2 < NS) rd(idx + 2);
                    s[1] = mfma32<DT>(kr[idx % 3], qf[ks], s[1]);
                    dp[1] = mfma32<DT>(vr[idx % 3], gf[ks], dp[1]);
#pragma unroll
                    for (int j = 0; j < PRA; ++j) {
                        const int pr = ks * PRA + j;
                        if (pr < 8) sm_pair(pr / 4, pr % 4);
                    }
#pragma unroll
                    for (int j = 0; j < TRA; ++j) {
                        const int dt = ks * TRA + j;
                        if (dt < NDT) opA[dt] = ktr(0, dt);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
                pack(0);
                pack(1);
                constexpr int PRC = (8 + 2 * NDT - 1) / (2 * NDT);
#pragma unroll
                for (int k = 0; k < 2 * NDT; ++k) {  // C0: u = 0 (operands A), u = 1 (B)
                    const int dt = k % NDT;
                    if (k < NDT) {
                        dqacc[dt] = mfma32<DT>(opA[dt], dsb[0], dqacc[dt]);
                        opB[dt] = ktr(1, dt);
                    } else {
                        dqacc[dt] = mfma32<DT>(opB[dt], dsb[1], dqacc[dt]);
                        opA[dt] = ktr(2, dt);
                    }
#pragma unroll
                    for (int j = 0; j < PRC; ++j) {
                        const int pr = k * PRC + j;
                        if (pr < 8) sm_pair(2 + pr / 4, pr % 4);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
                pack(2);
                pack(3);
#pragma unroll
                for (int k = 0; k < 2 * NDT; ++k) {  // C1: u = 2 (A), u = 3 (B)
                    const int dt = k % NDT;
                    if (k < NDT) {
                        dqacc[dt] = mfma32<DT>(opA[dt], dsb[2], dqacc[dt]);
                        opB[dt] = ktr(3, dt);
                    } else {
                        dqacc[dt] = mfma32<DT>(opB[dt], dsb[3], dqacc[dt]);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            } else {
                rd(0);
                if (NS > 1) rd(1);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int idx = 0; idx < NS; ++idx) {
                    if (idx + 2 < NS) rd(idx + 2);
                    s[idx / KS] = mfma32<DT>(kr[idx % 3], qf[idx % KS], s[idx / KS]);
                    dp[idx / KS] = mfma32<DT>(vr[idx % 3], gf[idx % KS], dp[idx / KS]);
                    __builtin_amdgcn_sched_barrier(0);
                }
#pragma unroll
                for (int u = 0; u < PVS; ++u) {
#pragma unroll
                    for (int e2 = 0; e2 < 4; ++e2) sm_pair(u, e2);
                    pack(u);
                }
#pragma unroll
                for (int u = 0; u < PVS; ++u)
#pragma unroll
                    for (int dt = 0; dt < NDT; ++dt) dqacc[dt] = mfma32<DT>(ktr(u, dt), dsb[u], dqacc[dt]);
            }
        }
        __builtin_amdgcn_s_waitcnt(0);  // the next tile has landed in LDS
        __syncthreads();
    };
    int kb = kb_begin;
    for (; kb < ku_begin; ++kb) run_step(kb, std::true_type{});
    for (; kb < ku_end; ++kb) run_step(kb, std::false_type{});
    for (; kb < kb_end; ++kb) run_step(kb, std::true_type{});

    if (qrow < N) {
        e16* dqrow = static_cast<e16*>(p.dq) + b * p.sdq.b + hq * p.sdq.h + qrow * p.sdq.n;
        const float sc = p.scale;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int d = dt * 32 + g4 * 8 + h * 4;
                if (d < D)
                    store4<DT>(dqrow + d, dqacc[dt][g4 * 4 + 0] * sc, dqacc[dt][g4 * 4 + 1] * sc,
                                 dqacc[dt][g4 * 4 + 2] * sc, dqacc[dt][g4 * 4 + 3] * sc);
            }
    }
}

template <int DT, int D, int MASK>
static hipError_t launch_dq_dc(const BwdParams& p, hipStream_t stream) {
    const long long nqb = (p.N + 127) / 128;
    const dim3 grid((unsigned)(nqb * p.B * p.Hq)), block(256);
    if (p.drop.thr != 0)
        hipLaunchKernelGGL((bwd_dq_kernel<DT, D, MASK, true>), grid, block, 0, stream, p);
    else
        hipLaunchKernelGGL((bwd_dq_kernel<DT, D, MASK, false>), grid, block, 0, stream, p);
    return hipGetLastError();
}

template <int DT, int D>
static hipError_t launch_dq_d(const BwdParams& p, int mask, hipStream_t stream) {
    switch (mask) {
        case kMaskNone: return launch_dq_dc<DT, D, kMaskNone>(p, stream);
        case kMaskCausal: return launch_dq_dc<DT, D, kMaskCausal>(p, stream);
        case kMaskWindow: return launch_dq_dc<DT, D, kMaskWindow>(p, stream);
        default: return hipErrorInvalidValue;
    }
}

template <int DT>
static hipError_t launch_dq_t(const BwdParams& p, int d, int mask, hipStream_t stream) {
    switch (d) {
#define ATTN_DQ_CASE(D_) \
        case D_: return launch_dq_d<DT, D_>(p, mask, stream);
        ATTN_FOR_EACH_HEAD_DIM(ATTN_DQ_CASE)
#undef ATTN_DQ_CASE
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_bwd_dq(const BwdParams& p, int dtype, int d, int mask, hipStream_t stream) {
    switch (dtype) {
        case kBF16: return launch_dq_t<kBF16>(p, d, mask, stream);
        case kFP16: return launch_dq_t<kFP16>(p, d, mask, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace attn
