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
//  1. bwd_pre: -D_i (stored negated) and the base-2 LSE for every query row
//     (memory bound).
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

// One 16-lane group per query row; rows are numbered (b * Hq + h) * N + n,
// the layout of the D_i workspace. The grid is capped (kPreMaxBlocks) and
// each group steps through the rows by the grid's row count, so a launch
// stays far below the 2^32 work-items of a grid dimension at any size.
constexpr long long kPreMaxBlocks = 1 << 20;

template <int DT, int D>
__global__ __launch_bounds__(256)
void bwd_pre_kernel(BwdParams p, long long rows) {
    constexpr int CPR = D / 8;
    const int j = threadIdx.x & 15;
    // All 16 lanes of a group share their row, so the loop exit and the
    // shuffles (inside the group) see the group whole.
    for (long long row = (long long)blockIdx.x * 16 + (threadIdx.x >> 4); row < rows;
         row += (long long)gridDim.x * 16) {
        const long long bh = row / p.N;
        const int n = (int)(row - bh * p.N);
        const int b = (int)(bh / p.Hq);
        const int hq = (int)(bh - (long long)b * p.Hq);
        const e16* op = static_cast<const e16*>(p.o) + b * p.so.b + hq * p.so.h + n * p.so.n;
        const e16* dp = static_cast<const e16*>(p.dout) + b * p.sdo.b + hq * p.sdo.h + n * p.sdo.n;
        float acc = 0.0f;
        for (int c = j; c < CPR; c += 16) {
            const e16x8 a = *reinterpret_cast<const e16x8*>(op + c * 8);
            const e16x8 g = *reinterpret_cast<const e16x8*>(dp + c * 8);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc = fmaf(widen<DT>(a[e]), widen<DT>(g[e]), acc);
        }
        acc += __shfl_xor(acc, 8);
        acc += __shfl_xor(acc, 4);
        acc += __shfl_xor(acc, 2);
        acc += __shfl_xor(acc, 1);
        if (j == 0) {
            p.delta[row] = -acc;  // -D_i: the dK/dV pass starts its dP sums from it
            p.lse2[row] = p.lse[row] * kLog2e;  // the dK/dV pass's log2-domain LSE
        }
    }
}

// ---------------------------------------------------------------- dK, dV

template <int DT, int D, int MASK, bool DROP, int QS>
__global__ __launch_bounds__(256, 1)
void bwd_dkdv_kernel(BwdParams p) {
    constexpr bool CAUSAL = MASK != kMaskNone;
    constexpr bool WINDOW = MASK == kMaskWindow;
    constexpr int NW = 4;
    constexpr int T = NW * 64;
    constexpr int BK = NW * 32;        // keys per workgroup
    constexpr int BQ = (D <= 128) ? 64 : 32;  // queries per step
    constexpr int NQT = BQ / 32;
    // d = 32: the compiler sinks part of the P / dS packing past the region
    // gaps, and in the query-split kernels it moves accumulator tiles between
    // AGPRs right before their product: there every dV/dK product carries its
    // own two wait states.
    constexpr bool ACC_GAP = D <= 32 || QS == 2;
    constexpr int PVS = BQ / 16;
    constexpr int KS = D / 16;
    constexpr int NDT = (D + 31) / 32;
    constexpr int QP = sw_pitch(D);    // Q, dO tiles: row reads and transposing reads
    constexpr int TILE = BQ * QP;
    constexpr int BUF = 2 * TILE * 2 + T * 4;  // bytes: Q, dO, lse2, D, spare row terms

    __shared__ __attribute__((aligned(16))) unsigned char smem_raw[2 * BUF];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches and buffer resources
    const int l32 = lane & 31;
    const int h = lane >> 5;
    const int N = p.N;

    // Workgroup index: key block (ascending: heaviest first when causal),
    // then the part of its query range (QS parts), then the KV head, fastest.
    const int BHk = p.B * p.Hkv;
    const int bid = blockIdx.x;
    const int kb = bid / (BHk * QS);
    const int rem = bid - kb * BHk * QS;
    const int part = QS == 1 ? 0 : rem / BHk;
    const int bhk = rem - part * BHk;
    const int b = bhk / p.Hkv;
    const int hkv = bhk - b * p.Hkv;
    const int k0 = kb * BK;
    const int kw0 = k0 + wave * 32;
    const int key = kw0 + l32;

    const e16* Kh = static_cast<const e16*>(p.k) + b * p.sk.b + hkv * p.sk.h;
    const e16* Vh = static_cast<const e16*>(p.v) + b * p.sv.b + hkv * p.sv.h;

    auto qtile = [&](int bufi) { return reinterpret_cast<e16*>(smem_raw + bufi * BUF); };
    auto dotile = [&](int bufi) { return reinterpret_cast<e16*>(smem_raw + bufi * BUF) + TILE; };
    auto lsetile = [&](int bufi) { return reinterpret_cast<float*>(smem_raw + bufi * BUF + 4 * TILE); };
    auto deltile = [&](int bufi) { return reinterpret_cast<float*>(smem_raw + bufi * BUF + 4 * TILE) + BQ; };

    for (int bufi = 0; bufi < 2; ++bufi) {
        zero_pad_cols_sw<D>(qtile(bufi), BQ, QP, tid, T);
        zero_pad_cols_sw<D>(dotile(bufi), BQ, QP, tid, T);
    }

    // K, V as B operands (lane = key, 8 dims per register group).
    e16x8 kf[KS], vf[KS];
    if (key < N) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            kf[ks] = *reinterpret_cast<const e16x8*>(Kh + key * p.sk.n + ks * 16 + h * 8);
            vf[ks] = *reinterpret_cast<const e16x8*>(Vh + key * p.sv.n + ks * 16 + h * 8);
        }
    } else {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) { kf[ks] = e16x8{}; vf[ks] = e16x8{}; }
    }

    const int nqb = (N + BQ - 1) / BQ;
    int qb_start = CAUSAL ? (k0 / BQ) : 0;
    // Sliding window: only queries i <= (last key) + window - 1 see this block.
    const int W = WINDOW ? p.window : 0;
    int qb_stop = WINDOW ? min(nqb, (k0 + BK - 1 + W - 1) / BQ + 1) : nqb;
    // Query blocks that need no per-element mask form [qu_begin, qu_end):
    // every query is at or after every key of the workgroup (q0 >= k0 + BK
    // - 1) and, under a window, every key lies in every query's band
    // (q0 + BQ - 1 < k0 + W). Rows past N need no mask either: their Q, dO
    // and row terms read as zeros, so they add nothing to dK or dV. The
    // masked blocks of all G heads run first, then the unmasked ones, each
    // phase with its own copy of the step.
    int qu_begin = qb_start, qu_end = qb_stop;
    if (CAUSAL) qu_begin = min(qb_stop, max(qb_start, (k0 + BK - 1 + BQ - 1) / BQ));
    if (WINDOW) {
        const int t = k0 + W - BQ;
        qu_end = max(qu_begin, min(qb_stop, t >= 0 ? t / BQ + 1 : 0));
    }
    if constexpr (QS == 2) {
        // This workgroup's part of the query range: the first or the second
        // half of its blocks (the masked ones keep their classification).
        const int mid = qb_start + (qb_stop - qb_start + 1) / 2;
        const int lo = part == 0 ? qb_start : mid, hi = part == 0 ? mid : qb_stop;
        qb_start = lo;
        qb_stop = hi;
        qu_begin = min(max(qu_begin, lo), hi);
        qu_end = min(max(qu_end, qu_begin), hi);
    }
    const int nq_iter = qb_stop - qb_start;
    const int total = p.G * nq_iter;
    const int nu = qu_end - qu_begin;
    const int nmG = p.G * (nq_iter - nu);
    // Step cursor (head g of the group, query block qb), advanced with a few
    // scalar compares instead of dividing the step index every step. Masked
    // phase, per head: qb_start .. qu_begin-1, then qu_end .. qb_stop-1.
    // Unmasked phase, per head: qu_begin .. qu_end-1.
    // The cursor also carries the head's Q and dO base pointers and its
    // offset in the row-term arrays, updated only when the head changes; the
    // row offsets r0 * stride fit in 32 bits (a view's row span is < 2^31).
    struct Step {
        int g, qb;
        const e16* qh;
        const e16* dh;
        size_t rt;
    };
    const int hq0 = hkv * p.G;
    const Step head0{0, 0, static_cast<const e16*>(p.q) + b * p.sq.b + hq0 * p.sq.h,
                     static_cast<const e16*>(p.dout) + b * p.sdo.b + hq0 * p.sdo.h,
                     ((size_t)b * p.Hq + hq0) * N};  // row terms: contiguous [B, Hq, N]
    const int qm_first = qb_start < qu_begin ? qb_start : qu_end;
    auto next_head = [&](Step st, int qb) {
        st.g += 1;
        st.qb = qb;
        st.qh += p.sq.h;
        st.dh += p.sdo.h;
        st.rt += N;
        return st;
    };
    auto next_step = [&](Step st, int it_next) {
        if (it_next >= total) return st;  // the last step reloads its own tiles
        const int qb = st.qb + 1;
        if (it_next < nmG) {
            const int qn = qb == qu_begin ? qu_end : qb;
            if (qn == qb_stop) return next_head(st, qm_first);
            st.qb = qn;
            return st;
        }
        if (it_next == nmG) {
            Step h = head0;
            h.qb = qu_begin;
            return h;
        }
        if (qb == qu_end) return next_head(st, qu_begin);
        st.qb = qb;
        return st;
    };
    Step first = head0;
    first.qb = nmG > 0 ? qm_first : qu_begin;

    // d <= 128: tiles go straight from memory to LDS. Each 64-lane buffer
    // load with the LDS flag fills 64 consecutive 16-byte chunks; lane i of
    // load j covers physical chunk (64j + i) % (QP / 8) of row (64j + i) /
    // (QP / 8), which holds logical chunk (physical ^ sw_swizzle(row)) of the
    // swizzled layout. Chunks past d (padding) and rows past N get offsets
    // beyond the buffer and read as zeros. The row terms (log2-domain LSE
    // and D_i, written by the preprocess) arrive the same way, 4 bytes per
    // lane; past N they read as zeros, which is harmless because those Q
    // and dO rows are zero too.
    constexpr bool DIRECT = BQ == 64;
    constexpr int CKQ = QP / 8;
    constexpr int NLQ = BQ * CKQ / 64;
    constexpr int LPWQ = (NLQ + NW - 1) / NW;
    static_assert(!DIRECT || BQ * CKQ % 64 == 0, "tile must be whole loads");
    uint32_t offq[DIRECT ? LPWQ : 1], offd[DIRECT ? LPWQ : 1];
    if constexpr (DIRECT) {
        const uint32_t sq2 = (uint32_t)p.sq.n * 2u, sd2 = (uint32_t)p.sdo.n * 2u;
#pragma unroll
        for (int i = 0; i < LPWQ; ++i) {
            const int chunk = (wave + i * NW) * 64 + lane;
            const int row = chunk / CKQ;
            const int lc = (chunk - row * CKQ) ^ sw_swizzle(row);
            offq[i] = lc < D / 8 ? (uint32_t)row * sq2 + (uint32_t)lc * 16u : 0xFFFFFFF0u;
            offd[i] = lc < D / 8 ? (uint32_t)row * sd2 + (uint32_t)lc * 16u : 0xFFFFFFF0u;
        }
    }
    // Buffer bases and sizes of a step's loads; the unmasked steps of a head
    // advance them by one query block instead of recomputing them.
    struct Issue {
        const e16* bq;
        const e16* bd;
        const float* br;
        uint32_t nq, nd, nr;
    };
    auto issue_params = [&](const Step& st) {
        const int r0 = st.qb * BQ;
        const uint32_t sq2 = (uint32_t)p.sq.n * 2u, sd2 = (uint32_t)p.sdo.n * 2u;
        Issue x;
        x.bq = st.qh + r0 * (int)p.sq.n;
        x.bd = st.dh + r0 * (int)p.sdo.n;
        x.nq = (uint32_t)(N - r0 - 1) * sq2 + D * 2;
        x.nd = (uint32_t)(N - r0 - 1) * sd2 + D * 2;
        x.br = (wave == 0 ? p.lse2 : p.delta) + st.rt + r0;
        x.nr = (uint32_t)(N - r0) * 4u;
        return x;
    };
    auto issue_loads = [&](const Issue& x, int bufi) {
        const auto rq = buf_rsrc(x.bq, x.nq);
        const auto rd = buf_rsrc(x.bd, x.nd);
        char* qt_lds = reinterpret_cast<char*>(qtile(bufi));
        char* dt_lds = reinterpret_cast<char*>(dotile(bufi));
#pragma unroll
        for (int i = 0; i < LPWQ; ++i) {
            const int j = wave + i * NW;
            if (NLQ % NW == 0 || j < NLQ) {
                buf_load16_to_lds(rq, qt_lds + j * 1024, offq[i]);
                buf_load16_to_lds(rd, dt_lds + j * 1024, offd[i]);
            }
        }
        if (wave < 2)
            buf_load4_to_lds(buf_rsrc(x.br, x.nr), wave == 0 ? lsetile(bufi) : deltile(bufi), (uint32_t)lane * 4u);
    };
    auto issue_step = [&](const Step& st, int bufi) { issue_loads(issue_params(st), bufi); };

    TileIO<D, BQ, T> qio, doio;
    // Row terms of the step: threads 0 .. BQ-1 fetch log2-domain LSE, BQ ..
    // 2BQ-1 the D_i; the others repeat a D_i fetch into a spare LDS slot, so
    // the loop body has no branch.
    float row_r = 0.0f;
    const int rt_kind = tid / BQ;        // 0: LSE, 1: D_i, 2+: spare
    const int rt_row = tid - rt_kind * BQ;
    auto load_step = [&](const Step& st) {
        const size_t row_off = st.rt;
        const int r0 = st.qb * BQ;
        qio.load(st.qh, p.sq.n, r0, N, tid);
        doio.load(st.dh, p.sdo.n, r0, N, tid);
        const int r = r0 + rt_row;
        const size_t rc = row_off + min(r, N - 1);
        const float x = rt_kind == 0 ? p.lse2[rc] : p.delta[rc];
        row_r = rt_kind == 0 ? (r < N ? x : __builtin_huge_valf()) : (r < N ? x : 0.0f);
    };
    auto store_step = [&](int bufi) {
        qio.store_sw(qtile(bufi), QP, tid);
        doio.store_sw(dotile(bufi), QP, tid);
        lsetile(bufi)[tid] = row_r;  // LSE tile, then D_i tile, then the spare slots
    };

    f32x16 dkacc[NDT], dvacc[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) { dkacc[dt] = f32x16{}; dvacc[dt] = f32x16{}; }

    const float c = p.c;
    const int g16 = lane >> 4;
    const int j16 = lane & 15;
    const int tr_row = (g16 >> 1) * 4 + (j16 >> 2);
    const int tr_col = (g16 & 1) * 16 + (j16 & 3) * 4;
    // Per-lane offsets into the swizzled Q and dO tiles; the other row and
    // column blocks are immediate offsets (sw_off repeats every 16 rows and
    // 32 columns). Row reads: chunk 2ks + h, ks even / odd. Transposing
    // reads: rows tr_row and tr_row + 8.
    const int qrd[2] = {sw_off(l32, h * 8, QP), sw_off(l32, 16 + h * 8, QP)};
    const int qtr0 = sw_off(tr_row, tr_col, QP), qtr1 = sw_off(tr_row + 8, tr_col, QP);

    if (total > 0) {
        if constexpr (DIRECT) {
            issue_step(first, 0);
            __builtin_amdgcn_s_waitcnt(0);
        } else {
            load_step(first);
            store_step(0);
        }
    }
    __syncthreads();

    // Step it works on `cur` (whose tiles are in LDS) and moves `cur` on to
    // the next step, whose loads it issues. The last step reloads its own
    // tiles into the idle buffer (never read), so no step tests for being
    // the last one.
    Issue cx = issue_params(first);  // the step whose tiles are in LDS
    auto run_step = [&](int it, Step& cur, auto masked_tag) {
        constexpr bool MASKED = decltype(masked_tag)::value;
        const int bufi = it & 1;
        const int g = cur.g;
        const int q0 = cur.qb * BQ;
        if constexpr (DIRECT) {
            // Unmasked steps move on to the next query block of the same head
            // (a few scalar adds); the others go through the general cursor.
            if (!MASKED && cur.qb + 1 < qu_end) {
                const int sqb = BQ * (int)p.sq.n, sdb = BQ * (int)p.sdo.n;
                cx.bq += sqb;
                cx.bd += sdb;
                cx.br += BQ;
                cx.nq -= (uint32_t)sqb * 2u;
                cx.nd -= (uint32_t)sdb * 2u;
                cx.nr -= BQ * 4u;
                cur.qb += 1;
            } else {
                cur = next_step(cur, it + 1);
                cx = issue_params(cur);
            }
            issue_loads(cx, bufi ^ 1);
        } else {
            cur = next_step(cur, it + 1);
            load_step(cur);
        }

        // Every step runs for every wave (no data-dependent branch in the
        // loop body): a wave whose keys all lie after this query block just
        // contributes zeros through the mask.
        {
            const e16* Qs = qtile(bufi);
            const e16* dOs = dotile(bufi);
            const float* Ls = lsetile(bufi);
            const float* Ds = deltile(bufi);
            f32x16 s[NQT], dp[NQT];
            // Start value of the dP sums of tile qt: -D_i of each register's
            // query (registers 4k .. 4k+3 hold queries 8k + 4h .. +3), so the
            // products leave dP - D_i. Dropout scales dP alone, so it starts
            // from zero and subtracts D_i later.
            auto dp_init = [&](int qt) {
                f32x16 a{};
                if constexpr (!DROP) {
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const f32x4 v = *reinterpret_cast<const f32x4*>(Ds + qt * 32 + 8 * k + 4 * h);
#pragma unroll
                        for (int e = 0; e < 4; ++e) a[4 * k + e] = v[e];
                    }
                }
                return a;
            };
            // S = Q K^T and dP = dO V^T for the 32 queries of tile qt.
            auto mma_sd = [&](int qt) {
                s[qt] = f32x16{};
                dp[qt] = dp_init(qt);
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const int off = qrd[ks & 1] + qt * 32 * QP + (ks >> 1) * 32;
                    s[qt] = mfma32<DT>(lds_read8(Qs + off), kf[ks], s[qt]);
                    dp[qt] = mfma32<DT>(lds_read8(dOs + off), vf[ks], dp[qt]);
                }
            };
            // P = exp2(c*S - LSE2) and dS = P (dP - D), packed to 16 bits in the
            // B-operand order of the dV/dK products. Under the causal mask the
            // query of register r (local offset qoff(r) + 4h) is masked for
            // this lane's key when key - q0 - 4h > qoff(r) (one compare with a
            // constant per element), and under a sliding window also when
            // qoff(r) > key - q0 - 4h + W - 1.
            e16x8 pb[PVS], dsb[PVS];
            e16x2 pp[PVS][4], dd[PVS][4];
            const int kq = key - q0 - 4 * h;
            const int kq_w = kq + W - 1;
            // Dropout: the lane's key meets 4 consecutive queries per
            // register group (bit r of keep[qt] for register r); a Philox
            // block covers them for this key and the neighbouring one, so
            // each lane pair shares its four blocks. dV takes P * M / (1-p);
            // dP is scaled the same way before the softmax step.
            uint32_t keep[NQT];
            if constexpr (DROP) {
                const uint32_t bh = (uint32_t)(b * p.Hq + hkv * p.G + g);
#pragma unroll
                for (int qt = 0; qt < NQT; ++qt)
                    keep[qt] = keep_bits_key_lane(p.drop, (uint32_t)key, (uint32_t)(q0 + qt * 32 + 4 * h) >> 2, bh);
            }
            // One pair of registers (r, r+1) of contraction step u.
            auto softmax_pair = [&](int u, int e2) {
                const int qt = u >> 1;
                const int r0 = (u & 1) * 8;
                float pv[2], dv[2];
#pragma unroll
                for (int w = 0; w < 2; ++w) {
                    const int r = r0 + 2 * e2 + w;
                    const int qoff = qt * 32 + (r >> 2) * 8 + (r & 3);
                    const int ql = qoff + h * 4;
                    float pe = fast_exp2(fmaf(s[qt][r], c, -Ls[ql]));
                    if (MASKED && CAUSAL && kq > qoff) pe = 0.0f;
                    if (MASKED && WINDOW && qoff > kq_w) pe = 0.0f;
                    if constexpr (DROP) {
                        const bool kept = (keep[qt] >> r) & 1u;
                        pv[w] = kept ? pe * p.drop.scale : 0.0f;
                        dv[w] = pe * ((kept ? dp[qt][r] * p.drop.scale : 0.0f) + Ds[ql]);
                    } else {
                        pv[w] = pe;
                        dv[w] = pe * dp[qt][r];  // dp already holds dP - D_i
                    }
                }
                pp[u][e2] = cvt2<DT>(pv[0], pv[1]);
                dd[u][e2] = cvt2<DT>(dv[0], dv[1]);
                // keep the conversions in this chunk (the compiler would sink
                // them all to the pack, outside the products' shadow)
                asm volatile("" : "+v"(pp[u][e2]), "+v"(dd[u][e2]));
            };
            auto pack = [&](int u) {
                pb[u] = cat8(pp[u][0], pp[u][1], pp[u][2], pp[u][3]);
                dsb[u] = cat8(dd[u][0], dd[u][1], dd[u][2], dd[u][3]);
            };
            // dV^T += dO^T P and dK^T += Q^T dS for contraction step u, with
            // dO^T and Q^T read transposed from the row-major tiles.
            auto read_ops = [&](int u, e16x8* ado, e16x8* aq) {
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) {
                    const int ob = u * 16 * QP + dt * 32;
                    ado[dt] = join8(lds_read_tr4(dOs + qtr0 + ob), lds_read_tr4(dOs + qtr1 + ob));
                    aq[dt] = join8(lds_read_tr4(Qs + qtr0 + ob), lds_read_tr4(Qs + qtr1 + ob));
                }
            };
            if constexpr (NQT == 2) {
                // Software pipeline of one step (d <= 128), pinned in order by
                // scheduling barriers between small chunks:
                //   A0: S/dP products of query tile 0, their row reads kept
                //       two steps ahead;
                //   A1: those of tile 1, with the softmax of tile 0 and the
                //       transposed reads of the first dV/dK step in their
                //       shadow;
                //   C0: the first two dV/dK steps, with the softmax of tile 1
                //       and the next transposed reads in their shadow;
                //   C1: the last two dV/dK steps.
                constexpr int NA = 2 * KS;  // row-read pairs of both tiles
                e16x8 ra_q[3], ra_d[3];     // ring of prefetched row operands
                auto rd = [&](int idx) {
                    const int qt = idx / KS, ks = idx % KS;
                    const int off = qrd[ks & 1] + qt * 32 * QP + (ks >> 1) * 32;
                    ra_q[idx % 3] = lds_read8(Qs + off);
                    ra_d[idx % 3] = lds_read8(dOs + off);
                };
                auto mma_step = [&](int idx) {
                    const int qt = idx / KS, ks = idx % KS;
                    s[qt] = mfma32<DT>(ra_q[idx % 3], kf[ks], s[qt]);
                    dp[qt] = mfma32<DT>(ra_d[idx % 3], vf[ks], dp[qt]);
                };
                e16x8 opA_d[NDT], opA_q[NDT], opB_d[NDT], opB_q[NDT];
                auto tr_read_d = [&](int u, int dt, e16x8* ado) {
                    const int ob = u * 16 * QP + dt * 32;
                    ado[dt] = join8(lds_read_tr4(dOs + qtr0 + ob), lds_read_tr4(dOs + qtr1 + ob));
                };
                auto tr_read_q = [&](int u, int dt, e16x8* aq) {
                    const int ob = u * 16 * QP + dt * 32;
                    aq[dt] = join8(lds_read_tr4(Qs + qtr0 + ob), lds_read_tr4(Qs + qtr1 + ob));
                };
                auto tr_read = [&](int u, int dt, e16x8* ado, e16x8* aq) {
                    const int ob = u * 16 * QP + dt * 32;
                    ado[dt] = join8(lds_read_tr4(dOs + qtr0 + ob), lds_read_tr4(dOs + qtr1 + ob));
                    aq[dt] = join8(lds_read_tr4(Qs + qtr0 + ob), lds_read_tr4(Qs + qtr1 + ob));
                };
                s[0] = f32x16{};
                dp[0] = dp_init(0);
                s[1] = f32x16{};
                dp[1] = dp_init(1);
                rd(0);
                rd(1);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {  // A0
                    rd(ks + 2);
                    mma_step(ks);
                    __builtin_amdgcn_sched_barrier(0);
                }
                constexpr int PAIRS_A1 = (8 + KS - 1) / KS;  // softmax pairs per A1 chunk
                constexpr int TR_A1 = (NDT + KS - 1) / KS;   // transposed-read groups per chunk
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {  // A1
                    if (KS + ks + 2 < NA) rd(KS + ks + 2);
                    mma_step(KS + ks);
#pragma unroll
                    for (int j = 0; j < PAIRS_A1; ++j) {
                        const int pr = ks * PAIRS_A1 + j;
                        if (pr < 8) softmax_pair(pr / 4, pr % 4);
                    }
#pragma unroll
                    for (int j = 0; j < TR_A1; ++j) {
                        const int dt = ks * TR_A1 + j;
                        if (dt < NDT) tr_read(0, dt, opA_d, opA_q);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
                pack(0);
                pack(1);
                valu_mfma_gap();
                // C0: dV/dK steps u = 0 (operands A) and u = 1 (operands B);
                // the reads for u = 1 go into B while u = 0 runs, those for
                // u = 2 into A while u = 1 runs.
#pragma unroll
                for (int k = 0; k < 2 * NDT; ++k) {
                    const int u = k / NDT, dt = k % NDT;
                    // dV half: its product, then the dO^T reads of the next
                    // contraction step
                    if (u == 0) {
                        mfma32_agpr<DT, ACC_GAP>(dvacc[dt], opA_d[dt], pb[0]);
                        tr_read_d(1, dt, opB_d);
                    } else {
                        mfma32_agpr<DT, ACC_GAP>(dvacc[dt], opB_d[dt], pb[1]);
                        tr_read_d(2, dt, opA_d);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                    // dK half: its product, the Q^T reads and a share of the softmax
                    if (u == 0) {
                        mfma32_agpr<DT, ACC_GAP>(dkacc[dt], opA_q[dt], dsb[0]);
                        tr_read_q(1, dt, opB_q);
                    } else {
                        mfma32_agpr<DT, ACC_GAP>(dkacc[dt], opB_q[dt], dsb[1]);
                        tr_read_q(2, dt, opA_q);
                    }
#pragma unroll
                    for (int j = 0; j < (8 + 2 * NDT - 1) / (2 * NDT); ++j) {
                        const int pr = k * ((8 + 2 * NDT - 1) / (2 * NDT)) + j;
                        if (pr < 8) softmax_pair(2 + pr / 4, pr % 4);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
                pack(2);
                pack(3);
                valu_mfma_gap();
#pragma unroll
                for (int k = 0; k < 2 * NDT; ++k) {  // C1: u = 2 (A), u = 3 (B)
                    const int u = 2 + k / NDT, dt = k % NDT;
                    if (u == 2) {
                        mfma32_agpr<DT, ACC_GAP>(dvacc[dt], opA_d[dt], pb[2]);
                        tr_read_d(3, dt, opB_d);
                        __builtin_amdgcn_sched_barrier(0);
                        mfma32_agpr<DT, ACC_GAP>(dkacc[dt], opA_q[dt], dsb[2]);
                        tr_read_q(3, dt, opB_q);
                    } else {
                        mfma32_agpr<DT, ACC_GAP>(dvacc[dt], opB_d[dt], pb[3]);
                        mfma32_agpr<DT, ACC_GAP>(dkacc[dt], opB_q[dt], dsb[3]);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            } else {
#pragma unroll
                for (int qt = 0; qt < NQT; ++qt) mma_sd(qt);
#pragma unroll
                for (int u = 0; u < PVS; ++u) {
#pragma unroll
                    for (int e2 = 0; e2 < 4; ++e2) softmax_pair(u, e2);
                    pack(u);
                }
                valu_mfma_gap();
                e16x8 a_do[NDT], a_q[NDT];
#pragma unroll
                for (int u = 0; u < PVS; ++u) {
                    read_ops(u, a_do, a_q);
#pragma unroll
                    for (int dt = 0; dt < NDT; ++dt) {
                        mfma32_agpr<DT, ACC_GAP>(dvacc[dt], a_do[dt], pb[u]);
                        mfma32_agpr<DT, ACC_GAP>(dkacc[dt], a_q[dt], dsb[u]);
                    }
                }
            }
        }
        if constexpr (DIRECT)
            __builtin_amdgcn_s_waitcnt(0);  // the next step's tiles have landed in LDS
        else
            store_step(bufi ^ 1);
        __syncthreads();
    };
    int it = 0;
    Step cur = first;
    for (; it < nmG; ++it) run_step(it, cur, std::true_type{});
    for (; it < total; ++it) run_step(it, cur, std::false_type{});

#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
        agpr_acc_ready(dkacc[dt]);
        agpr_acc_ready(dvacc[dt]);
    }
    if constexpr (QS > 1) {
        // fp32 partial sums [2][QS][B][Hkv][N][D]: dK (scaled), then dV
        if (key < N) {
            const float sc = p.scale;
            const size_t plane = (size_t)QS * BHk * N * D;
            float* pk = p.part + (((size_t)part * BHk + bhk) * N + key) * D;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const int d = dt * 32 + g4 * 8 + h * 4;
                    if (d < D) {
                        *reinterpret_cast<f32x4*>(pk + d) =
                            f32x4{dkacc[dt][g4 * 4 + 0] * sc, dkacc[dt][g4 * 4 + 1] * sc,
                                  dkacc[dt][g4 * 4 + 2] * sc, dkacc[dt][g4 * 4 + 3] * sc};
                        *reinterpret_cast<f32x4*>(pk + plane + d) =
                            f32x4{dvacc[dt][g4 * 4 + 0], dvacc[dt][g4 * 4 + 1], dvacc[dt][g4 * 4 + 2],
                                  dvacc[dt][g4 * 4 + 3]};
                    }
                }
        }
        return;
    }
    if (key < N) {
        e16* dkrow = static_cast<e16*>(p.dk) + b * p.sdk.b + hkv * p.sdk.h + key * p.sdk.n;
        e16* dvrow = static_cast<e16*>(p.dv) + b * p.sdv.b + hkv * p.sdv.h + key * p.sdv.n;
        const float sc = p.scale;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int d = dt * 32 + g4 * 8 + h * 4;
                if (d < D) {
                    store4<DT>(dkrow + d, dkacc[dt][g4 * 4 + 0] * sc, dkacc[dt][g4 * 4 + 1] * sc,
                                 dkacc[dt][g4 * 4 + 2] * sc, dkacc[dt][g4 * 4 + 3] * sc);
                    store4<DT>(dvrow + d, dvacc[dt][g4 * 4 + 0], dvacc[dt][g4 * 4 + 1],
                                 dvacc[dt][g4 * 4 + 2], dvacc[dt][g4 * 4 + 3]);
                }
            }
    }
}

// ---------------------------------------------------------------- dK, dV (64 keys per wave)

// The same pass for d = 128 without dropout, with 64 keys per wave (256 per
// workgroup): every Q and dO row read and every transposed read feeds two
// products, one per 32-key half, so a wave issues about a third fewer LDS
// reads per product than with 32 keys. K stays in VGPRs as the B operand of
// S; V of the second half moves to LDS and is read row-wise as the B operand
// of dP (the first half's stays in VGPRs); dK^T and
// dV^T of the 64 keys fill the 256 AGPRs. Steps of 32 query rows, in five
// regions pinned by scheduling barriers:
//   S:  the S products of both halves, with the row reads;
//   dP: the dP products, with P of the first 16 rows in their shadow;
//   V0: dV products of rows 0..15, with P of rows 16..31;
//   V1: dV products of rows 16..31, with dS of rows 0..15;
//   K0, K1: dK products, with dS of rows 16..31 and the Q^T reads.
template <int DT, int MASK, bool DROP, int SPLIT>
__global__ __launch_bounds__(256, 1)
void bwd_dkdv_wide_kernel(BwdParams p) {
    constexpr int D = 128;
    constexpr bool CAUSAL = MASK != kMaskNone;
    constexpr bool WINDOW = MASK == kMaskWindow;
    constexpr int NW = 4;
    constexpr int BK = NW * 64;   // keys per workgroup
    constexpr int BQ = 32;        // query rows per step
    constexpr int KS = D / 16;
    constexpr int NDT = D / 32;
    constexpr int QP = sw_pitch(D);  // Q, dO tiles: row reads and transposing reads
    constexpr int VP = D + 8;        // V rows: row reads only
    constexpr int TILE = BQ * QP;
    constexpr int RT = 64;           // row-term slots per buffer (one 64-lane load)
    constexpr int BUF = 2 * TILE * 2 + 2 * RT * 4;
    constexpr int VBYTES = BK * VP * 2;

    __shared__ __attribute__((aligned(16))) unsigned char smem_raw[VBYTES + 2 * BUF];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31;
    const int h = lane >> 5;
    const int N = p.N;

    // Workgroup index: key block (ascending: heaviest first when causal),
    // then the part of the group's query heads (hsplit parts), then the KV
    // head, fastest.
    const int BHk = p.B * p.Hkv;
    constexpr int S = SPLIT;  // = p.hsplit
    const int bid = blockIdx.x;
    const int kb = bid / (BHk * S);
    const int rem = bid - kb * BHk * S;
    const int part_i = rem / BHk;
    const int bhk = rem - part_i * BHk;
    const int b = bhk / p.Hkv;
    const int hkv = bhk - b * p.Hkv;
    const int Gs = p.G / S;  // query heads of this workgroup
    const int k0 = kb * BK;
    const int kw0 = k0 + wave * 64;

    const e16* Kh = static_cast<const e16*>(p.k) + b * p.sk.b + hkv * p.sk.h;
    const e16* Vh = static_cast<const e16*>(p.v) + b * p.sv.b + hkv * p.sv.h;

    e16* Vs = reinterpret_cast<e16*>(smem_raw);
    auto qtile = [&](int bufi) { return reinterpret_cast<e16*>(smem_raw + VBYTES + bufi * BUF); };
    auto dotile = [&](int bufi) { return qtile(bufi) + TILE; };
    auto lsetile = [&](int bufi) { return reinterpret_cast<float*>(smem_raw + VBYTES + bufi * BUF + 4 * TILE); };
    auto deltile = [&](int bufi) { return lsetile(bufi) + RT; };

    // K of the wave's two 32-key halves as B operands (lane = key); the V
    // rows of the second half into the wave's part of the V region (zeros
    // past N).
    e16x8 kf[2][KS];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int key = kw0 + 32 * j + l32;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            kf[j][ks] = key < N ? *reinterpret_cast<const e16x8*>(Kh + key * p.sk.n + ks * 16 + h * 8) : e16x8{};
    }
    // V of the first half also stays in VGPRs (room is left for 32 more),
    // which saves half of the V row reads of every step.
    e16x8 vf0[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
        vf0[ks] = kw0 + l32 < N ? *reinterpret_cast<const e16x8*>(Vh + (kw0 + l32) * p.sv.n + ks * 16 + h * 8) : e16x8{};
#pragma unroll
    for (int i = 32 * (D / 8) / 64; i < 64 * (D / 8) / 64; ++i) {
        const int c = i * 64 + lane;
        const int row = c / (D / 8), col = c - row * (D / 8);
        const int key = kw0 + row;
        const uint4 v = key < N ? *reinterpret_cast<const uint4*>(Vh + key * p.sv.n + col * 8) : zero4();
        *reinterpret_cast<uint4*>(Vs + (wave * 64 + row) * VP + col * 8) = v;
    }

    const int nqb = (N + BQ - 1) / BQ;
    const int qb_start = CAUSAL ? (k0 / BQ) : 0;
    const int W = WINDOW ? p.window : 0;
    const int qb_stop = WINDOW ? min(nqb, (k0 + BK - 1 + W - 1) / BQ + 1) : nqb;
    const int nq_iter = qb_stop - qb_start;
    const int total = Gs * nq_iter;
    // Unmasked query blocks [qu_begin, qu_end), as in the 32-key kernel.
    int qu_begin = qb_start, qu_end = qb_stop;
    if (CAUSAL) qu_begin = min(qb_stop, max(qb_start, (k0 + BK - 1 + BQ - 1) / BQ));
    if (WINDOW) {
        const int t = k0 + W - BQ;
        qu_end = max(qu_begin, min(qb_stop, t >= 0 ? t / BQ + 1 : 0));
    }
    const int nu = qu_end - qu_begin;
    const int nmG = Gs * (nq_iter - nu);
    struct Step {
        int g, qb;
        const e16* qh;
        const e16* dh;
        size_t rt;
    };
    const int hq0 = hkv * p.G + part_i * Gs;
    const Step head0{0, 0, static_cast<const e16*>(p.q) + b * p.sq.b + hq0 * p.sq.h,
                     static_cast<const e16*>(p.dout) + b * p.sdo.b + hq0 * p.sdo.h,
                     ((size_t)b * p.Hq + hq0) * N};
    const int qm_first = qb_start < qu_begin ? qb_start : qu_end;
    auto next_head = [&](Step st, int qb) {
        st.g += 1;
        st.qb = qb;
        st.qh += p.sq.h;
        st.dh += p.sdo.h;
        st.rt += N;
        return st;
    };
    auto next_step = [&](Step st, int it_next) {
        if (it_next >= total) return st;
        const int qb = st.qb + 1;
        if (it_next < nmG) {
            const int qn = qb == qu_begin ? qu_end : qb;
            if (qn == qb_stop) return next_head(st, qm_first);
            st.qb = qn;
            return st;
        }
        if (it_next == nmG) {
            Step hh = head0;
            hh.qb = qu_begin;
            return hh;
        }
        if (qb == qu_end) return next_head(st, qu_begin);
        st.qb = qb;
        return st;
    };
    Step first = head0;
    first.qb = nmG > 0 ? qm_first : qu_begin;

    constexpr int CKQ = QP / 8;
    constexpr int NLQ = BQ * CKQ / 64;
    constexpr int LPWQ = (NLQ + NW - 1) / NW;
    static_assert(BQ * CKQ % 64 == 0, "tile must be whole loads");
    uint32_t offq[LPWQ], offd[LPWQ];
    {
        const uint32_t sq2 = (uint32_t)p.sq.n * 2u, sd2 = (uint32_t)p.sdo.n * 2u;
#pragma unroll
        for (int i = 0; i < LPWQ; ++i) {
            const int chunk = (wave + i * NW) * 64 + lane;
            const int row = chunk / CKQ;
            const int lc = (chunk - row * CKQ) ^ sw_swizzle(row);
            offq[i] = lc < D / 8 ? (uint32_t)row * sq2 + (uint32_t)lc * 16u : 0xFFFFFFF0u;
            offd[i] = lc < D / 8 ? (uint32_t)row * sd2 + (uint32_t)lc * 16u : 0xFFFFFFF0u;
        }
    }
    struct Issue {
        const e16* bq;
        const e16* bd;
        const float* br;
        uint32_t nq, nd, nr;
    };
    auto issue_params = [&](const Step& st) {
        const int r0 = st.qb * BQ;
        const uint32_t sq2 = (uint32_t)p.sq.n * 2u, sd2 = (uint32_t)p.sdo.n * 2u;
        Issue x;
        x.bq = st.qh + r0 * (int)p.sq.n;
        x.bd = st.dh + r0 * (int)p.sdo.n;
        x.nq = (uint32_t)(N - r0 - 1) * sq2 + D * 2;
        x.nd = (uint32_t)(N - r0 - 1) * sd2 + D * 2;
        x.br = (wave == 0 ? p.lse2 : p.delta) + st.rt + r0;
        x.nr = (uint32_t)(N - r0) * 4u;
        return x;
    };
    auto issue_loads = [&](const Issue& x, int bufi) {
        const auto rq = buf_rsrc(x.bq, x.nq);
        const auto rd = buf_rsrc(x.bd, x.nd);
        char* qt_lds = reinterpret_cast<char*>(qtile(bufi));
        char* dt_lds = reinterpret_cast<char*>(dotile(bufi));
#pragma unroll
        for (int i = 0; i < LPWQ; ++i) {
            const int j = wave + i * NW;
            if (NLQ % NW == 0 || j < NLQ) {
                buf_load16_to_lds(rq, qt_lds + j * 1024, offq[i]);
                buf_load16_to_lds(rd, dt_lds + j * 1024, offd[i]);
            }
        }
        if (wave < 2)
            buf_load4_to_lds(buf_rsrc(x.br, x.nr), wave == 0 ? lsetile(bufi) : deltile(bufi), (uint32_t)lane * 4u);
    };

    f32x16 dkacc[2][NDT], dvacc[2][NDT];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) { dkacc[j][dt] = f32x16{}; dvacc[j][dt] = f32x16{}; }

    const float c = p.c;
    const int g16 = lane >> 4;
    const int j16 = lane & 15;
    const int tr_row = (g16 >> 1) * 4 + (j16 >> 2);
    const int tr_col = (g16 & 1) * 16 + (j16 & 3) * 4;
    const int qrd[2] = {sw_off(l32, h * 8, QP), sw_off(l32, 16 + h * 8, QP)};
    const int qtr0 = sw_off(tr_row, tr_col, QP), qtr1 = sw_off(tr_row + 8, tr_col, QP);
    const e16* Vl = Vs + (wave * 64 + l32) * VP + h * 8;  // this lane's V row (first half)

    Issue cx{};
    if (total > 0) {
        cx = issue_params(first);
        issue_loads(cx, 0);
        __builtin_amdgcn_s_waitcnt(0);
    }
    __syncthreads();

    auto run_step = [&](int it, Step& cur, auto masked_tag) {
        constexpr bool MASKED = decltype(masked_tag)::value;
        const int bufi = it & 1;
        const int q0 = cur.qb * BQ;
        const int g = cur.g;  // this step's head (cur moves on to the next step below)
        if (!MASKED && cur.qb + 1 < qu_end) {
            const int sqb = BQ * (int)p.sq.n, sdb = BQ * (int)p.sdo.n;
            cx.bq += sqb;
            cx.bd += sdb;
            cx.br += BQ;
            cx.nq -= (uint32_t)sqb * 2u;
            cx.nd -= (uint32_t)sdb * 2u;
            cx.nr -= BQ * 4u;
            cur.qb += 1;
        } else {
            cur = next_step(cur, it + 1);
            cx = issue_params(cur);
        }
        issue_loads(cx, bufi ^ 1);

        const e16* Qs = qtile(bufi);
        const e16* dOs = dotile(bufi);
        const float* Ls = lsetile(bufi);
        const float* Ds = deltile(bufi);
        // register r of a product tile holds local query row qoff(r) + 4h
        auto qoff = [](int r) { return (r >> 2) * 8 + (r & 3); };
        f32x16 s[2], dp[2];
        {
            f32x16 a;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const f32x4 v = *reinterpret_cast<const f32x4*>(Ds + 8 * k + 4 * h);
#pragma unroll
                for (int e = 0; e < 4; ++e) a[4 * k + e] = v[e];
            }
            s[0] = f32x16{};
            s[1] = f32x16{};
            // the dP sums start from -D_i; dropout scales dP alone, so there
            // they start from zero and D_i is subtracted in dS
            dp[0] = DROP ? f32x16{} : a;
            dp[1] = DROP ? f32x16{} : a;
        }
        // Dropout keep bits of each half's key for the step's 32 queries (bit
        // r for register r), as in the 32-key kernel.
        uint32_t keep[2] = {0u, 0u};
        if constexpr (DROP) {
            const uint32_t bh = (uint32_t)(b * p.Hq + hq0 + g);
#pragma unroll
            for (int j = 0; j < 2; ++j)
                keep[j] = keep_bits_key_lane(p.drop, (uint32_t)(kw0 + 32 * j + l32), (uint32_t)(q0 + 4 * h) >> 2, bh);
        }
        const int kq0 = kw0 + l32 - q0 - 4 * h;  // key - query offset, first half
        e16x2 pp[2][2][4], dd[2][2][4];
        e16x8 pb[2][2], dsb[2][2];
        // P of register pair (2e, 2e+1) of rows-half u, both key halves;
        // the probability overwrites the score.
        auto p_pair = [&](int u, int e) {
            const int r = u * 8 + 2 * e;
            // (two float reads: the compiler cannot track a struct float2 read
            // of LDS and would make it wait for the next step's loads)
            const float l2[2] = {Ls[qoff(r) + 4 * h], Ls[qoff(r) + 4 * h + 1]};
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                float pe[2];
#pragma unroll
                for (int w = 0; w < 2; ++w) {
                    pe[w] = fast_exp2(fmaf(s[j][r + w], c, -(w ? l2[1] : l2[0])));
                    const int kq = kq0 + 32 * j;
                    if (MASKED && CAUSAL && kq > qoff(r + w)) pe[w] = 0.0f;
                    if (MASKED && WINDOW && qoff(r + w) > kq + W - 1) pe[w] = 0.0f;
                    s[j][r + w] = pe[w];
                    // dV takes P * M / (1-p)
                    if constexpr (DROP) pe[w] = ((keep[j] >> (r + w)) & 1u) ? pe[w] * p.drop.scale : 0.0f;
                }
                pp[j][u][e] = cvt2<DT>(pe[0], pe[1]);
                asm volatile("" : "+v"(pp[j][u][e]));
            }
        };
        auto ds_pair = [&](int u, int e) {
            const int r = u * 8 + 2 * e;
            if constexpr (DROP) {
                // dS = P ((dP M / (1-p)) - D_i)
                const float nd[2] = {Ds[qoff(r) + 4 * h], Ds[qoff(r) + 4 * h + 1]};
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int w = 0; w < 2; ++w)
                        dp[j][r + w] = (((keep[j] >> (r + w)) & 1u) ? dp[j][r + w] * p.drop.scale : 0.0f) +
                                       (w ? nd[1] : nd[0]);
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                dd[j][u][e] = cvt2<DT>(s[j][r] * dp[j][r], s[j][r + 1] * dp[j][r + 1]);
                asm volatile("" : "+v"(dd[j][u][e]));
            }
        };
        // region S: row reads of Q two products ahead
        e16x8 rq[3];
        e16x8 rdo[2], rv[2][2];
        auto rd_q = [&](int ks) { rq[ks % 3] = lds_read8(Qs + qrd[ks & 1] + (ks >> 1) * 32); };
        auto rd_dv = [&](int ks) {
            rdo[ks & 1] = lds_read8(dOs + qrd[ks & 1] + (ks >> 1) * 32);
            rv[ks & 1][1] = lds_read8(Vl + 32 * VP + ks * 16);
        };
        rd_q(0);
        rd_q(1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if (ks + 2 < KS) rd_q(ks + 2);
            if (ks == KS - 1) rd_dv(0);
            s[0] = mfma32<DT>(rq[ks % 3], kf[0][ks], s[0]);
            s[1] = mfma32<DT>(rq[ks % 3], kf[1][ks], s[1]);
            __builtin_amdgcn_sched_barrier(0);
        }
        // region dP, with P of rows-half 0 (4 pairs x 2 halves)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if (ks + 1 < KS) rd_dv(ks + 1);
            dp[0] = mfma32<DT>(rdo[ks & 1], vf0[ks], dp[0]);
            dp[1] = mfma32<DT>(rdo[ks & 1], rv[ks & 1][1], dp[1]);
            if (ks >= 2 && ks < 6) p_pair(0, ks - 2);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) pb[j][0] = cat8(pp[j][0][0], pp[j][0][1], pp[j][0][2], pp[j][0][3]);
        valu_mfma_gap();
        // dV^T += dO^T P: transposed dO reads one product ahead
        e16x8 od[2];
        auto tr_d = [&](int u, int dt, int slot) {
            const int ob = u * 16 * QP + dt * 32;
            od[slot] = join8(lds_read_tr4(dOs + qtr0 + ob), lds_read_tr4(dOs + qtr1 + ob));
        };
        tr_d(0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {  // region V0, with P of rows-half 1
            tr_d(dt + 1 < NDT ? 0 : 1, (dt + 1) % NDT, (dt + 1) & 1);
            mfma32_agpr<DT>(dvacc[0][dt], od[dt & 1], pb[0][0]);
            mfma32_agpr<DT>(dvacc[1][dt], od[dt & 1], pb[1][0]);
            p_pair(1, dt);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) pb[j][1] = cat8(pp[j][1][0], pp[j][1][1], pp[j][1][2], pp[j][1][3]);
        valu_mfma_gap();
        e16x8 oq[2];
        auto tr_q = [&](int u, int dt, int slot) {
            const int ob = u * 16 * QP + dt * 32;
            oq[slot] = join8(lds_read_tr4(Qs + qtr0 + ob), lds_read_tr4(Qs + qtr1 + ob));
        };
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {  // region V1, with dS of rows-half 0
            if (dt + 1 < NDT) tr_d(1, dt + 1, (dt + 1) & 1);
            else tr_q(0, 0, 0);
            mfma32_agpr<DT>(dvacc[0][dt], od[dt & 1], pb[0][1]);
            mfma32_agpr<DT>(dvacc[1][dt], od[dt & 1], pb[1][1]);
            ds_pair(0, dt);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) dsb[j][0] = cat8(dd[j][0][0], dd[j][0][1], dd[j][0][2], dd[j][0][3]);
        valu_mfma_gap();
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {  // region K0, with dS of rows-half 1
            tr_q(dt + 1 < NDT ? 0 : 1, (dt + 1) % NDT, (dt + 1) & 1);
            mfma32_agpr<DT>(dkacc[0][dt], oq[dt & 1], dsb[0][0]);
            mfma32_agpr<DT>(dkacc[1][dt], oq[dt & 1], dsb[1][0]);
            ds_pair(1, dt);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) dsb[j][1] = cat8(dd[j][1][0], dd[j][1][1], dd[j][1][2], dd[j][1][3]);
        valu_mfma_gap();
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {  // region K1
            if (dt + 1 < NDT) tr_q(1, dt + 1, (dt + 1) & 1);
            mfma32_agpr<DT>(dkacc[0][dt], oq[dt & 1], dsb[0][1]);
            mfma32_agpr<DT>(dkacc[1][dt], oq[dt & 1], dsb[1][1]);
            __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_s_waitcnt(0);  // the next step's tiles have landed in LDS
        __syncthreads();
    };
    int it = 0;
    Step cur = first;
    for (; it < nmG; ++it) run_step(it, cur, std::true_type{});
    for (; it < total; ++it) run_step(it, cur, std::false_type{});

#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            agpr_acc_ready(dkacc[j][dt]);
            agpr_acc_ready(dvacc[j][dt]);
        }
    const float sc = p.scale;
    if constexpr (S > 1) {
        // fp32 partial sums [2][S][B][Hkv][N][D]: dK (scaled), then dV
        const size_t plane = (size_t)S * BHk * N * D;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int key = kw0 + 32 * j + l32;
            if (key < N) {
                float* pk = p.part + (((size_t)part_i * BHk + bhk) * N + key) * D;
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                    for (int g4 = 0; g4 < 4; ++g4) {
                        const int d = dt * 32 + g4 * 8 + h * 4;
                        *reinterpret_cast<f32x4*>(pk + d) =
                            f32x4{dkacc[j][dt][g4 * 4 + 0] * sc, dkacc[j][dt][g4 * 4 + 1] * sc,
                                  dkacc[j][dt][g4 * 4 + 2] * sc, dkacc[j][dt][g4 * 4 + 3] * sc};
                        *reinterpret_cast<f32x4*>(pk + plane + d) =
                            f32x4{dvacc[j][dt][g4 * 4 + 0], dvacc[j][dt][g4 * 4 + 1], dvacc[j][dt][g4 * 4 + 2],
                                  dvacc[j][dt][g4 * 4 + 3]};
                    }
            }
        }
        return;
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int key = kw0 + 32 * j + l32;
        if (key < N) {
            e16* dkrow = static_cast<e16*>(p.dk) + b * p.sdk.b + hkv * p.sdk.h + key * p.sdk.n;
            e16* dvrow = static_cast<e16*>(p.dv) + b * p.sdv.b + hkv * p.sdv.h + key * p.sdv.n;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const int d = dt * 32 + g4 * 8 + h * 4;
                    store4<DT>(dkrow + d, dkacc[j][dt][g4 * 4 + 0] * sc, dkacc[j][dt][g4 * 4 + 1] * sc,
                               dkacc[j][dt][g4 * 4 + 2] * sc, dkacc[j][dt][g4 * 4 + 3] * sc);
                    store4<DT>(dvrow + d, dvacc[j][dt][g4 * 4 + 0], dvacc[j][dt][g4 * 4 + 1],
                               dvacc[j][dt][g4 * 4 + 2], dvacc[j][dt][g4 * 4 + 3]);
                }
        }
    }
}

// Sum of the two partial dK, dV of the head-split 64-key dK/dV kernel or of
// the query-split 32-key one (in part order, so the result is
// deterministic), converted to the element type. One thread per 4 elements
// of a row.
template <int DT, int D>
__global__ __launch_bounds__(256)
void bwd_dkdv_sum_kernel(BwdParams p, long long quads) {
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    if (i >= quads) return;
    const long long row = i / (D / 4);
    const int d = (int)(i - row * (D / 4)) * 4;
    const long long rows = (long long)p.B * p.Hkv * p.N;  // rows of one part
    const int n = (int)(row % p.N);
    const long long bh = row / p.N;
    const int b = (int)(bh / p.Hkv), hkv = (int)(bh - (long long)b * p.Hkv);
    const float* pk = p.part + row * D + d;
    const f32x4 k0 = *reinterpret_cast<const f32x4*>(pk);
    const f32x4 k1 = *reinterpret_cast<const f32x4*>(pk + rows * D);
    const f32x4 v0 = *reinterpret_cast<const f32x4*>(pk + 2 * rows * D);
    const f32x4 v1 = *reinterpret_cast<const f32x4*>(pk + 3 * rows * D);
    e16* dkrow = static_cast<e16*>(p.dk) + b * p.sdk.b + hkv * p.sdk.h + n * p.sdk.n;
    e16* dvrow = static_cast<e16*>(p.dv) + b * p.sdv.b + hkv * p.sdv.h + n * p.sdv.n;
    store4<DT>(dkrow + d, k0[0] + k1[0], k0[1] + k1[1], k0[2] + k1[2], k0[3] + k1[3]);
    store4<DT>(dvrow + d, v0[0] + v1[0], v0[1] + v1[1], v0[2] + v1[2], v0[3] + v1[3]);
}

// ---------------------------------------------------------------- launch

template <int DT, int D, int MASK>
static hipError_t launch_bwd_dc(const BwdParams& p, int passes, hipStream_t stream) {
    if (passes & kBwdPre) {
        const long long rows = (long long)p.B * p.Hq * p.N;
        const long long blocks = (rows + 15) / 16 < kPreMaxBlocks ? (rows + 15) / 16 : kPreMaxBlocks;
        hipLaunchKernelGGL((bwd_pre_kernel<DT, D>), dim3((unsigned)blocks), dim3(256), 0, stream, p, rows);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (passes & kBwdDkDv) {
        if constexpr (D == 128) {
            if (p.dkdv > 0) {
                const dim3 grid((unsigned)((p.N + 255) / 256 * p.B * p.Hkv * p.hsplit));
                if (p.hsplit == 2) {
                    if (p.drop.thr != 0)
                        hipLaunchKernelGGL((bwd_dkdv_wide_kernel<DT, MASK, true, 2>), grid, dim3(256), 0, stream, p);
                    else
                        hipLaunchKernelGGL((bwd_dkdv_wide_kernel<DT, MASK, false, 2>), grid, dim3(256), 0, stream, p);
                } else {
                    if (p.drop.thr != 0)
                        hipLaunchKernelGGL((bwd_dkdv_wide_kernel<DT, MASK, true, 1>), grid, dim3(256), 0, stream, p);
                    else
                        hipLaunchKernelGGL((bwd_dkdv_wide_kernel<DT, MASK, false, 1>), grid, dim3(256), 0, stream, p);
                }
                hipError_t e = hipGetLastError();
                if (e != hipSuccess) return e;
                if (p.hsplit == 2) {
                    const long long quads = (long long)p.B * p.Hkv * p.N * (D / 4);
                    hipLaunchKernelGGL((bwd_dkdv_sum_kernel<DT, D>), dim3((unsigned)((quads + 255) / 256)), dim3(256),
                                       0, stream, p, quads);
                    e = hipGetLastError();
                    if (e != hipSuccess) return e;
                }
                passes &= ~kBwdDkDv;
            }
        }
    }
    if (passes & kBwdDkDv) {
        const long long nkb = (p.N + 127) / 128;
        const dim3 block(256);
        if (p.qsplit == 2) {
            if constexpr (D <= 128) {
                const dim3 grid((unsigned)(nkb * p.B * p.Hkv * 2));
                if (p.drop.thr != 0)
                    hipLaunchKernelGGL((bwd_dkdv_kernel<DT, D, MASK, true, 2>), grid, block, 0, stream, p);
                else
                    hipLaunchKernelGGL((bwd_dkdv_kernel<DT, D, MASK, false, 2>), grid, block, 0, stream, p);
                hipError_t e = hipGetLastError();
                if (e != hipSuccess) return e;
                const long long quads = (long long)p.B * p.Hkv * p.N * (D / 4);
                hipLaunchKernelGGL((bwd_dkdv_sum_kernel<DT, D>), dim3((unsigned)((quads + 255) / 256)), block, 0,
                                   stream, p, quads);
                e = hipGetLastError();
                if (e != hipSuccess) return e;
            } else {
                return hipErrorInvalidValue;  // the split is planned for d <= 128 only
            }
        } else {
            const dim3 grid((unsigned)(nkb * p.B * p.Hkv));
            if (p.drop.thr != 0)
                hipLaunchKernelGGL((bwd_dkdv_kernel<DT, D, MASK, true, 1>), grid, block, 0, stream, p);
            else
                hipLaunchKernelGGL((bwd_dkdv_kernel<DT, D, MASK, false, 1>), grid, block, 0, stream, p);
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
    }
    if (passes & kBwdDq) {
        const hipError_t e = launch_bwd_dq(p, DT, D, MASK, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <int DT, int D>
static hipError_t launch_bwd_d(const BwdParams& p, int mask, int passes, hipStream_t stream) {
    switch (mask) {
        case kMaskNone: return launch_bwd_dc<DT, D, kMaskNone>(p, passes, stream);
        case kMaskCausal: return launch_bwd_dc<DT, D, kMaskCausal>(p, passes, stream);
        case kMaskWindow: return launch_bwd_dc<DT, D, kMaskWindow>(p, passes, stream);
        default: return hipErrorInvalidValue;
    }
}

template <int DT>
static hipError_t launch_bwd_t(const BwdParams& p, int d, int mask, int passes, hipStream_t stream) {
    switch (d) {
#define ATTN_BWD_CASE(D_) \
        case D_: return launch_bwd_d<DT, D_>(p, mask, passes, stream);
        ATTN_FOR_EACH_HEAD_DIM(ATTN_BWD_CASE)
#undef ATTN_BWD_CASE
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_bwd(const BwdParams& p, int dtype, int d, int mask, int passes,
                      hipStream_t stream) {
    switch (dtype) {
        case kBF16: return launch_bwd_t<kBF16>(p, d, mask, passes, stream);
        case kFP16: return launch_bwd_t<kFP16>(p, d, mask, passes, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace attn
