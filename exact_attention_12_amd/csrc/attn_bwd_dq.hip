// attn_bwd_dq.hip - dQ pass of the attention backward, for gfx950.
//
// One workgroup per (batch, query head, 128-row query block), in the
// forward's orientation: S^T = K Q^T and dP^T = V dO^T put one query per
// lane, so LSE_i and D_i are per-lane scalars; dQ^T += K^T dS^T with K^T read
// from the (chunk-swizzled) K tile by the transposing LDS read. On grids too
// small to hide the longest block's key loop, one workgroup per 64-row block
// instead, whose two pairs of waves each take half of the block's key tiles
// and add their partial dQ through LDS at the end. It is a
// separate translation unit because it is scheduled for occupancy (two waves
// per SIMD), while the dK/dV pass, one wave per SIMD, is scheduled for ILP.
// The formulas are the chain rule written out in attn_bwd.hip.
#include <type_traits>

#include "attn_bwd_common.h"

namespace attn {

// ---------------------------------------------------------------- dQ

template <int DT, int D, int MASK, bool DROP, int KG>
__global__ __launch_bounds__(256, (D <= 128 && KG == 1 ? 2 : 1))
void bwd_dq_kernel(BwdParams p) {
    constexpr bool CAUSAL = MASK != kMaskNone;
    constexpr bool WINDOW = MASK == kMaskWindow;
    constexpr int NW = 4;
    constexpr int WG = NW / KG;  // waves per key group
    constexpr int BQ = WG * 32;
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
    static_assert(KG == 1 || (KG == 2 && BC == 64), "key groups: d <= 128, no dropout");

    __shared__ __attribute__((aligned(16))) e16 smem[2 * BUF * KG];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches and buffer resources
    const int grp = KG == 1 ? 0 : wave / WG;  // key group
    const int gw = wave - grp * WG;           // wave within the group = its 32-row tile
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
    const int qw0 = q0 + gw * 32;
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
    // A group's tiles are loaded by its own WG waves.
    constexpr int LPWK = (NLK + WG - 1) / WG, LPWV = (NLV + WG - 1) / WG;
    uint32_t offk[LPWK], offv[LPWV];
    {
        const uint32_t sk2 = (uint32_t)p.sk.n * 2u, sv2 = (uint32_t)p.sv.n * 2u;
#pragma unroll
        for (int i = 0; i < LPWK; ++i) {
            const int chunk = (gw + i * WG) * 64 + lane;
            const int row = chunk / CKK;
            const int lc = (chunk - row * CKK) ^ sw_swizzle(row);
            offk[i] = lc < D / 8 ? (uint32_t)row * sk2 + (uint32_t)lc * 16u : 0xFFFFFFF0u;
        }
#pragma unroll
        for (int i = 0; i < LPWV; ++i) {
            const int chunk = (gw + i * WG) * 64 + lane;
            const int row = chunk / CKV;
            const int lc = chunk - row * CKV;
            offv[i] = lc < D / 8 ? (uint32_t)row * sv2 + (uint32_t)lc * 16u : 0xFFFFFFF0u;
        }
    }
    e16* const gsm = smem + grp * 2 * BUF;  // this group's two tile buffers
    auto issue_tile = [&](int kv0, int bufi) {
        const uint32_t sk2 = (uint32_t)p.sk.n * 2u, sv2 = (uint32_t)p.sv.n * 2u;
        const auto rk = buf_rsrc(Kh + (long long)kv0 * p.sk.n, (uint32_t)(N - kv0 - 1) * sk2 + D * 2);
        const auto rv = buf_rsrc(Vh + (long long)kv0 * p.sv.n, (uint32_t)(N - kv0 - 1) * sv2 + D * 2);
        char* k_lds = reinterpret_cast<char*>(gsm + bufi * BUF);
        char* v_lds = k_lds + BC * KP * 2;
#pragma unroll
        for (int i = 0; i < LPWK; ++i) {
            const int j = gw + i * WG;
            if ((NLK % WG == 0 || j < NLK) && (BC * CKK % 64 == 0 || j * 64 + lane < BC * CKK))
                buf_load16_to_lds(rk, k_lds + j * 1024, offk[i]);
        }
#pragma unroll
        for (int i = 0; i < LPWV; ++i) {
            const int j = gw + i * WG;
            if ((NLV % WG == 0 || j < NLV) && (BC * CKV % 64 == 0 || j * 64 + lane < BC * CKV))
                buf_load16_to_lds(rv, v_lds + j * 1024, offv[i]);
        }
    };
    // Key tiles of this group: [gs, ge); with two groups, group 0 takes the
    // first ceil(n/2).
    const int kmid = kb_begin + (kb_end - kb_begin + 1) / 2;
    const int gs = KG == 1 ? kb_begin : (grp == 0 ? kb_begin : kmid);
    const int ge = KG == 1 ? kb_end : (grp == 0 ? kmid : kb_end);
    if (KG == 1)
        issue_tile(kb_begin * BC, kb_begin & 1);
    else if (gs < ge)
        issue_tile(gs * BC, 0);
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

    // One step: tile kb in buffer bufi, the next tile (kb + 1, at most
    // kb_last) loaded into the other buffer. `has` is false only for the
    // idle last step of a key group with fewer tiles.
    auto run_step = [&](int kb, int bufi, int kb_last, bool has, auto masked_tag) {
        constexpr bool MASKED = decltype(masked_tag)::value;
        // The last step reloads its own tile into the idle buffer (never
        // read again), so the loads need no branch.
        if (has) issue_tile(min(kb + 1, kb_last) * BC, bufi ^ 1);
        const int kv0 = kb * BC;
        const e16* Ks = gsm + bufi * BUF;
        const e16* Vs = Ks + BC * KP;
        // Branch-free step: in the masked blocks, keys past a wave's last
        // query are masked to zero.
        if (has) {
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
    if constexpr (KG == 1) {
        int kb = kb_begin;
        for (; kb < ku_begin; ++kb) run_step(kb, kb & 1, kb_end - 1, true, std::true_type{});
        for (; kb < ku_end; ++kb) run_step(kb, kb & 1, kb_end - 1, true, std::false_type{});
        for (; kb < kb_end; ++kb) run_step(kb, kb & 1, kb_end - 1, true, std::true_type{});
    } else {
        // Both groups step together (one barrier per step); group 0 has the
        // same number of tiles as group 1 or one more.
        const int nit = kmid - kb_begin;
        for (int it = 0; it < nit; ++it) {
            const int kb = gs + it;
            const bool has = kb < ge;
            if (has && (kb < ku_begin || kb >= ku_end))
                run_step(kb, it & 1, ge - 1, true, std::true_type{});
            else
                run_step(kb, it & 1, ge - 1, has, std::false_type{});
        }
        // Group 1 adds its partial dQ^T to the wave of group 0 with the same
        // rows, through the tile buffers (every wave has finished with them:
        // each waited for its own loads before the last barrier).
        constexpr int OSZ = WG * NDT * 16 * 64;
        static_assert(OSZ * 4 <= 2 * KG * BUF * 2, "partial dQ must fit the tile buffers");
        float* xs = reinterpret_cast<float*>(smem);
        if (grp == 1) {
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) xs[((gw * NDT + dt) * 16 + r) * 64 + lane] = dqacc[dt][r];
        }
        __syncthreads();
        if (grp == 1) return;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) dqacc[dt][r] += xs[((gw * NDT + dt) * 16 + r) * 64 + lane];
    }

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

// ------------------------------------------------- dQ on 16x16x32 products
//
// d = 128 without dropout, one key group: the same pass on
// v_mfma_f32_16x16x32 products, which the chip sustains at a higher rate
// than 32x32x16 ones on random operands (the rate probe of attn_probe.h),
// in the layout of the forward's fwd_m16_kernel:
//  * a wave holds two 16-query tiles (qt). S^T = K Q^T and dP^T = V dO^T of
//    a 64-key step are 4 key tiles (kt) x 2 query tiles of 16x16; lane l
//    then holds, for query qw0 + 16 qt + l % 16, keys 16 kt + 4 (l / 16) + r
//    (r = 0..3), and its LSE and -D_i are per-lane scalars.
//  * dQ^T += K^T dS^T over the step's two 32-key halves: the lane's dS^T
//    values are already the B operand (key order 4g..4g+3, 16+4g..16+4g+3
//    in 16-lane group g), and K^T is read transposed in the same order.
//  * The K tile is read row-wise (S^T) and transposed (K^T), the V tile
//    row-wise. Both have the forward's 16x16x32 pitch of 144 elements (288
//    bytes), which serves both reads of this layout without bank conflicts
//    (measured with SQ_LDS_BANK_CONFLICT; a 136-element pitch, or this one
//    with its chunks swizzled by bit 3 of the row, doubles the LDS cycles
//    of the row reads).
//  * Each of the two K and two V buffers is its own LDS object, with the
//    buffer known at compile time, so the transposing reads of the current
//    buffer do not wait for the loads in flight into the other one.
//  * A step runs in four regions pinned by scheduling barriers: the S^T and
//    dP^T products of the first key half; those of the second half with the
//    first half's dS^T in their shadow; the first half's dQ^T products with
//    the second half's dS^T; the second half's dQ^T products. Each dS^T value
//    goes through three stages a product pair apart (exponent FMA,
//    exponential with the mask, product with dP^T + (-D_i) and rounding).
template <int DT>
__device__ __forceinline__ f32x4 dq_mfma16(e16x8 a, e16x8 b, f32x4 c) {
    if constexpr (DT == kBF16)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

constexpr int kDq16Pitch = 144;  // elements: 288 bytes, 9 x 32
static_assert((kDq16Pitch * 2 / 32) % 2 == 1 && kDq16Pitch >= 128 + 8, "");

template <int DT, int MASK>
__global__ __launch_bounds__(256, 2)
void bwd_dq_m16_kernel(BwdParams p) {
    constexpr int D = 128;
    constexpr bool CAUSAL = MASK != kMaskNone;
    constexpr bool WINDOW = MASK == kMaskWindow;
    constexpr int NW = 4;
    constexpr int BQ = NW * 32;
    constexpr int BC = 64;
    constexpr int KS = D / 32;     // contraction steps of S^T and dP^T
    constexpr int NDT = D / 16;    // 16-row tiles of dQ^T
    constexpr int KP = kDq16Pitch;
    constexpr int VP = kDq16Pitch;

    __shared__ __attribute__((aligned(16))) e16 sK0[BC * KP];
    __shared__ __attribute__((aligned(16))) e16 sK1[BC * KP];
    __shared__ __attribute__((aligned(16))) e16 sV0[BC * VP];
    __shared__ __attribute__((aligned(16))) e16 sV1[BC * VP];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15;
    const int g = lane >> 4;
    const int N = p.N;

    const int BH = p.B * p.Hq;
    const int nqb = (N + BQ - 1) / BQ;
    const int bid = blockIdx.x;
    const int bh = xcd_head(bid % BH, BH);
    const int qb = CAUSAL ? (nqb - 1 - bid / BH) : (bid / BH);
    const int b = bh / p.Hq;
    const int hq = bh - b * p.Hq;
    const int hkv = hq / p.G;
    const size_t row_off = (size_t)bh * N;
    const e16* Kh = static_cast<const e16*>(p.k) + b * p.sk.b + hkv * p.sk.h;
    const e16* Vh = static_cast<const e16*>(p.v) + b * p.sv.b + hkv * p.sv.h;
    const long long skn = p.sk.n, svn = p.sv.n;

    const int q0 = qb * BQ;
    const int qw0 = q0 + wave * 32;
    const int qrow[2] = {qw0 + l16, qw0 + 16 + l16};

    // Q and dO operands (B of S^T and dP^T): query qrow[qt], dims 32 ks + 8 g .. +7.
    e16x8 qf[2][KS], gf[2][KS];
    float lse2[2], ndel[2];  // ndel = -D_i, as the preprocess stores it
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
        const int qr = qrow[qt];
        if (qr < N) {
            const e16* qp = static_cast<const e16*>(p.q) + b * p.sq.b + hq * p.sq.h + qr * p.sq.n + g * 8;
            const e16* gp = static_cast<const e16*>(p.dout) + b * p.sdo.b + hq * p.sdo.h + qr * p.sdo.n + g * 8;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                qf[qt][ks] = *reinterpret_cast<const e16x8*>(qp + ks * 32);
                gf[qt][ks] = *reinterpret_cast<const e16x8*>(gp + ks * 32);
            }
            lse2[qt] = p.lse[row_off + qr] * kLog2e;
            ndel[qt] = p.delta[row_off + qr];
        } else {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) { qf[qt][ks] = e16x8{}; gf[qt][ks] = e16x8{}; }
            lse2[qt] = __builtin_huge_valf();
            ndel[qt] = 0.0f;
        }
    }

    const int nkb = (N + BC - 1) / BC;
    const int kb_end = CAUSAL ? min(nkb, (q0 + BQ - 1) / BC + 1) : nkb;
    const int W = WINDOW ? p.window : 0;
    const int kb_begin = WINDOW ? max(0, q0 - W + 1) / BC : 0;
    // Blocks needing no per-element mask, as in bwd_dq_kernel (keys past N
    // stay masked: their zero scores would give exp2(-LSE2)).
    int ku_begin = kb_begin, ku_end = min(kb_end, N / BC);
    if (CAUSAL) ku_end = min(ku_end, (q0 + 1) / BC);
    if (WINDOW) {
        const int t = q0 + BQ - W;
        ku_begin = min(kb_end, max(kb_begin, t > 0 ? (t + BC - 1) / BC : 0));
    }
    ku_end = max(ku_end, ku_begin);

    // Tile loads straight to LDS.
    constexpr int CKK = KP / 8, CKV = VP / 8;
    constexpr int NLK = BC * CKK / 64, NLV = BC * CKV / 64;
    constexpr int LPWK = (NLK + NW - 1) / NW, LPWV = (NLV + NW - 1) / NW;
    static_assert(BC * CKK % 64 == 0 && BC * CKV % 64 == 0, "tile must be whole loads");
    uint32_t offk[LPWK], offv[LPWV];
    {
        const uint32_t sk2 = (uint32_t)skn * 2u, sv2 = (uint32_t)svn * 2u;
#pragma unroll
        for (int i = 0; i < LPWK; ++i) {
            const int chunk = (wave + i * NW) * 64 + lane;
            const int row = chunk / CKK;
            const int lc = chunk - row * CKK;
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
    auto issue = [&](int kb, e16* kbuf, e16* vbuf) {
        const int kv0 = kb * BC;
        const auto rk = buf_rsrc(Kh + (long long)kv0 * skn, (uint32_t)(N - kv0 - 1) * (uint32_t)skn * 2u + D * 2);
        const auto rv = buf_rsrc(Vh + (long long)kv0 * svn, (uint32_t)(N - kv0 - 1) * (uint32_t)svn * 2u + D * 2);
#pragma unroll
        for (int i = 0; i < LPWK; ++i) {
            const int j = wave + i * NW;
            if (NLK % NW == 0 || j < NLK) buf_load16_to_lds(rk, reinterpret_cast<char*>(kbuf) + j * 1024, offk[i]);
        }
#pragma unroll
        for (int i = 0; i < LPWV; ++i) {
            const int j = wave + i * NW;
            if (NLV % NW == 0 || j < NLV) buf_load16_to_lds(rv, reinterpret_cast<char*>(vbuf) + j * 1024, offv[i]);
        }
    };

    // Per-lane read offsets (elements); the other tiles are immediate offsets.
    //  K rows (S^T operand): row 16 kt + l16, dims 32 ks + 8 g.
    //  V rows (dP^T operand): row 16 kt + l16, dims 32 ks + 8 g.
    //  K^T (transposing read): lane 4t + s of group g reads key row 4 g + t
    //  (+ 32 jj, + 16 for the second half of the operand), dims 16 dt + 4 s.
    const int krd = l16 * KP + 8 * g;
    const int vrd = l16 * VP + 8 * g;
    const int ktr = (4 * g + (l16 >> 2)) * KP + 4 * (l16 & 3);

    f32x4 dq[NDT][2];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) dq[dt][0] = dq[dt][1] = f32x4{};
    const float c = p.c;

    auto step = [&](int kb, const e16* Ks, const e16* Vs, auto masked_tag) {
        constexpr bool MASKED = decltype(masked_tag)::value;
        const int kv0 = kb * BC;
        // s[kt][qt][r], dp[kt][qt][r]: key kv0 + 16 kt + 4 g + r, query qrow[qt].
        f32x4 s[4][2], dp[4][2];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) s[kt][0] = s[kt][1] = dp[kt][0] = dp[kt][1] = f32x4{};
        // Product pair idx of key half jj: ks = idx / 4, kt = 2 jj + (idx / 2) % 2,
        // S^T (idx even, K operand) or dP^T (idx odd, V operand).
        e16x8 op[3];
        auto rd_row = [&](int jj, int idx) {
            const int ks = idx >> 2, kt = 2 * jj + ((idx >> 1) & 1);
            op[idx % 3] = (idx & 1) ? lds_read8(Vs + vrd + kt * 16 * VP + ks * 32)
                                    : lds_read8(Ks + krd + kt * 16 * KP + ks * 32);
        };
        auto sprod = [&](int jj, int idx) {
            const int ks = idx >> 2, kt = 2 * jj + ((idx >> 1) & 1);
            if (idx + 2 < 16) rd_row(jj, idx + 2);
            if (idx & 1) {
                dp[kt][0] = dq_mfma16<DT>(op[idx % 3], gf[0][ks], dp[kt][0]);
                dp[kt][1] = dq_mfma16<DT>(op[idx % 3], gf[1][ks], dp[kt][1]);
            } else {
                s[kt][0] = dq_mfma16<DT>(op[idx % 3], qf[0][ks], s[kt][0]);
                s[kt][1] = dq_mfma16<DT>(op[idx % 3], qf[1][ks], s[kt][1]);
            }
        };
        // Masks: key offset kt * 16 + r (from kv0 + 4 g) against the query's bounds.
        int hi[2], lo[2];
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
            hi[qt] = (CAUSAL ? min(qrow[qt], N - 1) : N - 1) - kv0 - 4 * g;
            lo[qt] = (WINDOW ? qrow[qt] - W + 1 : 0) - kv0 - 4 * g;
        }
        // dS^T value u (0..31): half jj = u / 16, query tile qt = (u / 8) % 2,
        // i = u % 8: key tile 2 jj + i / 4, register i % 4, i.e. B element i.
        float ta[32], xb[32];
        e16x2 pp[2][8];
        auto stage_a = [&](int u) {
            const int jj = u >> 4, qt = (u >> 3) & 1, i = u & 7;
            ta[u] = fmaf(s[2 * jj + (i >> 2)][qt][i & 3], c, -lse2[qt]);
        };
        auto stage_b = [&](int u) {
            const int jj = u >> 4, qt = (u >> 3) & 1, i = u & 7;
            const int koff = (2 * jj + (i >> 2)) * 16 + (i & 3);
            float x = fast_exp2(ta[u]);
            if (MASKED && (koff > hi[qt] || (WINDOW && koff < lo[qt]))) x = 0.0f;
            xb[u] = x;
        };
        auto stage_c = [&](int u) {
            const int jj = u >> 4, qt = (u >> 3) & 1, i = u & 7;
            const float d = xb[u] * (dp[2 * jj + (i >> 2)][qt][i & 3] + ndel[qt]);
            if (i & 1)
                pp[jj][(u & 15) >> 1] = cvt2<DT>(ta[u - 1], d);
            else
                ta[u] = d;  // the even value waits here for its pair
        };
        auto units = [&](int lo_u, int hi_u, int start, int end) {
            if (lo_u == start) {
                stage_a(start);
                stage_a(start + 1);
                stage_b(start);
            }
#pragma unroll
            for (int u = lo_u + 2; u < hi_u + 2 && u < end; ++u) stage_a(u);
#pragma unroll
            for (int u = lo_u + 1; u < hi_u + 1 && u < end; ++u) stage_b(u);
#pragma unroll
            for (int u = lo_u; u < hi_u; ++u) stage_c(u);
        };
        e16x8 pb[2][2];
        auto pack = [&](int jj, int qt) {
            const e16x2* x = &pp[jj][qt * 4];
            pb[jj][qt] = cat8(x[0], x[1], x[2], x[3]);
        };
        // K^T operand of half jj, dims 16 dt .. +15.
        e16x8 kt_op[3];
        auto rd_tr = [&](int jj, int dt) {
            const e16* kp = Ks + ktr + jj * 32 * KP + dt * 16;
            kt_op[dt % 3] = join8(lds_read_tr4(kp), lds_read_tr4(kp + 16 * KP));
        };
        auto dqprod = [&](int jj, int dt) {
            if (dt + 2 < NDT) rd_tr(jj, dt + 2);
            dq[dt][0] = dq_mfma16<DT>(kt_op[dt % 3], pb[jj][0], dq[dt][0]);
            dq[dt][1] = dq_mfma16<DT>(kt_op[dt % 3], pb[jj][1], dq[dt][1]);
        };

        // R1: S^T and dP^T of the first key half.
        rd_row(0, 0);
        rd_row(0, 1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int idx = 0; idx < 16; ++idx) {
            sprod(0, idx);
            __builtin_amdgcn_sched_barrier(0);
        }
        // R2: those of the second half, with the first half's dS^T.
        rd_row(1, 0);
        rd_row(1, 1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int idx = 0; idx < 16; ++idx) {
            sprod(1, idx);
            units(idx, idx + 1, 0, 16);
            __builtin_amdgcn_sched_barrier(0);
        }
        pack(0, 0);
        pack(0, 1);
        rd_tr(0, 0);
        rd_tr(0, 1);
        __builtin_amdgcn_sched_barrier(0);
        // R3: dQ^T products of the first half, with the second half's dS^T.
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            dqprod(0, dt);
            units(16 + 2 * dt, 18 + 2 * dt, 16, 32);
            __builtin_amdgcn_sched_barrier(0);
        }
        pack(1, 0);
        pack(1, 1);
        rd_tr(1, 0);
        rd_tr(1, 1);
        __builtin_amdgcn_sched_barrier(0);
        // R4: dQ^T products of the second half.
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            dqprod(1, dt);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // Block t's tiles sit in buffer (t - ku_begin) & 1. The mask-free blocks
    // run in pairs whose buffers are known at compile time; the masked
    // blocks before and after them (and a last unpaired mask-free block,
    // for which the masks change nothing) pick their buffers at run time.
    // (loads go through a branch on the buffer, not a select of addresses:
    // each then names its LDS object, which unoptimised builds need)
    auto run_masked = [&](int kb) {
        const bool par = (kb - ku_begin) & 1;
        if (kb + 1 < kb_end) {
            if (par)
                issue(kb + 1, sK0, sV0);
            else
                issue(kb + 1, sK1, sV1);
        }
        step(kb, par ? sK1 : sK0, par ? sV1 : sV0, std::true_type{});
        __builtin_amdgcn_s_waitcnt(0);  // the next tile has landed in LDS
        __syncthreads();
    };
    auto run_pair = [&](int kb) {
        if (kb + 1 < kb_end) issue(kb + 1, sK1, sV1);
        step(kb, sK0, sV0, std::false_type{});
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (kb + 2 < kb_end) issue(kb + 2, sK0, sV0);
        step(kb + 1, sK1, sV1, std::false_type{});
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    };
    if ((kb_begin - ku_begin) & 1)
        issue(kb_begin, sK1, sV1);
    else
        issue(kb_begin, sK0, sV0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    int kb = kb_begin;
    for (; kb < ku_begin; ++kb) run_masked(kb);
    for (; kb + 1 < ku_end; kb += 2) run_pair(kb);
    for (; kb < kb_end; ++kb) run_masked(kb);

    // dQ = scale * sum_j dS_ij k_j; dq[dt][qt][r] is dim 16 dt + 4 g + r of query qrow[qt].
    const float sc = p.scale;
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
        const int qr = qrow[qt];
        if (qr < N) {
            e16* dqrow = static_cast<e16*>(p.dq) + b * p.sdq.b + hq * p.sdq.h + qr * p.sdq.n;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
                store4<DT>(dqrow + dt * 16 + 4 * g, dq[dt][qt][0] * sc, dq[dt][qt][1] * sc,
                           dq[dt][qt][2] * sc, dq[dt][qt][3] * sc);
        }
    }
}

template <int DT, int D, int MASK>
static hipError_t launch_dq_dc(const BwdParams& p, hipStream_t stream) {
    const dim3 block(256);
    if (p.drop.thr != 0) {
        const dim3 grid((unsigned)((p.N + 127) / 128 * p.B * p.Hq));
        hipLaunchKernelGGL((bwd_dq_kernel<DT, D, MASK, true, 1>), grid, block, 0, stream, p);
    } else if (D <= 128 && key_groups_pay(p.B, p.Hq, p.N, MASK != kMaskNone)) {
        if constexpr (D <= 128) {
            const dim3 grid((unsigned)((p.N + 63) / 64 * p.B * p.Hq));
            hipLaunchKernelGGL((bwd_dq_kernel<DT, D, MASK, false, 2>), grid, block, 0, stream, p);
        }
    } else if constexpr (D == 128) {
        const dim3 grid((unsigned)((p.N + 127) / 128 * p.B * p.Hq));
        hipLaunchKernelGGL((bwd_dq_m16_kernel<DT, MASK>), grid, block, 0, stream, p);
    } else {
        const dim3 grid((unsigned)((p.N + 127) / 128 * p.B * p.Hq));
        hipLaunchKernelGGL((bwd_dq_kernel<DT, D, MASK, false, 1>), grid, block, 0, stream, p);
    }
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
