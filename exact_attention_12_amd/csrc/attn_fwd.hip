// attn_fwd.hip - fused tiled attention forward for gfx950.
//
// What it computes (per batch b, query head h, with KV head h / G):
//   O_i   = sum_j softmax_j(scale * <q_i, k_j>) v_j   over allowed keys j
//   LSE_i = ln sum_j exp(scale * <q_i, k_j>)
// following the blockwise online softmax of the CANN ops-transformer
// FlashAttention page (section on online softmax): for each block of keys the
// running row maximum m is raised, the partial output and running sum l are
// rescaled by exp(m_old - m_new), and the block's exp(s - m_new) is
// accumulated; O is divided by l at the end. The lpnh.cn FlashAttention-2
// article (sections 2.1, 2.4) gives the tiling and the parallelisation over
// (batch, head, query block); the yunthe.com GQA page gives the KV-head
// sharing (query head h reads KV head h / (Hq/Hkv)).
//
// Mapping onto the CDNA4 compute unit (4 or 8 waves per workgroup, 32 query rows
// per wave, BLOCK_KV keys per step):
//  * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (_f16 for fp16 inputs): K (from
//    LDS) is the A operand, the wave's 32 query rows (kept in registers for
//    the whole loop) are the B operand. The result puts one query per lane
//    (lane % 32) and 16 keys per lane in registers, so the row maximum is a
//    register reduction plus a single permlane32 swap, and m, l live in one
//    lane pair.
//  * O^T += V^T P^T: the probabilities, rounded to the input type, are
//    already laid out as the B operand (a lane holds 8 keys of its query);
//    V^T is read as the A operand straight from the row-major V tile with
//    the transposing LDS read. O^T keeps one query per lane, so a rescale by
//    exp(m_old - m_new) needs no data movement.
//  * Rescaling is lazy: the reference maximum only moves when a block's row
//    maximum exceeds it by more than 2^8 (probabilities stay <= 2^8; O and l
//    share the reference, so O / l and the LSE are unchanged). On the
//    synthetic workloads this skips the rescale after the first block.
//  * The row sum l is accumulated in fp32 from the unrounded probabilities
//    (only the matrix-product operand is rounded to 16 bits), so LSE carries
//    no rounding bias even for rows with few keys.
//  * Operands are [B, H, N, d] views with any element strides for b, h and n
//    (d contiguous), so BHSD and BSHD tensors are read in place.
//  * Scores are kept in the log2 domain: exp(scale*s - m) = exp2(c*s - m')
//    with c = scale * log2(e).
//  * K/V tiles are double buffered in LDS: the next tile's global loads are
//    issued before the current tile's math, one barrier per step. For
//    d <= 128 buffer loads with the LDS flag write them straight into the
//    other buffer (no staging registers, no LDS stores); larger d stage
//    them in registers and store them after the math.
//  * Causal: key blocks after the workgroup's last query are never loaded; a
//    wave skips the math of blocks after its own last query; the diagonal
//    blocks are masked per element. Heavy (late) query blocks are launched
//    first.
//  * Short sequences take fwd_split_kernel instead (further down): the keys
//    of one 32-row tile are split over the workgroup's waves, which load
//    everything at once and merge in LDS.
//  * Key groups (KG = 2): when the grid is so small that the longest query
//    block's key loop decides the time, the 4 waves form two groups of 2
//    over the same 64 rows (one wave per SIMD, one workgroup per CU); group
//    0 walks the first half of the block's key tiles and group 1 the rest,
//    each with its own double-buffered tiles, and group 1 hands its (m, l,
//    O) to group 0 through LDS at the end. The two partial softmax states
//    combine exactly: M = max(m0, m1), l = sum_g 2^(m_g - M) l_g,
//    O = sum_g 2^(m_g - M) O_g. (Two groups of 4 waves over 128 rows, two
//    waves per SIMD, gained nothing: the groups then share each SIMD.)
//  * d = 128 without dropout on the grids that other head dims run on 8
//    waves: fwd_m16_kernel runs the step loop on 16x16x32 products, which
//    the chip sustains at a higher rate than 32x32x16 ones, pipelined across
//    key blocks (layout and schedule in its own comment), in workgroups of
//    4 waves (128 rows).
#include <type_traits>

#include "attn_device.h"
#include "attn_kernels.h"

namespace attn {

// Two waves per SIMD, except d > 128 and the 4-wave key-group kernel, whose
// tile buffers leave room for one workgroup (one wave per SIMD) per CU.
template <int DT, int D, int MASK, int NW, bool DROP, int KG>
__global__ __launch_bounds__(NW * 64, (D <= 128 && !(KG == 2 && NW == 4) ? 2 : 1))
void fwd_kernel(FwdParams p) {
    constexpr int T = NW * 64;
    constexpr int WG = NW / KG;          // waves per key group
    constexpr int BQ = WG * 32;          // query rows of the workgroup
    constexpr bool CAUSAL = MASK != kMaskNone;
    constexpr bool WINDOW = MASK == kMaskWindow;
    constexpr int BC = FwdTile<D>::BLOCK_KV;
    constexpr int KS = D / 16;            // contraction steps of S^T = K Q^T
    constexpr int NDT = (D + 31) / 32;    // 32-row tiles of O^T
    constexpr int NKT = BC / 32;          // 32-key tiles of S^T
    constexpr int PVS = BC / 16;          // contraction steps of O^T += V^T P^T
    constexpr int KP = k_pitch(D);
    constexpr int VP = v_pitch(D);
    constexpr int CPR = D / 8;            // 16-byte chunks per row
    constexpr int CHUNKS = BC * CPR;
    constexpr int NCH = (CHUNKS + T - 1) / T;
    constexpr int BUF = BC * (KP + VP);
    static_assert(KG == 1 || (KG == 2 && BC == 64 && !DROP), "key groups: d <= 128, no dropout");

    // Buffer j of key group g sits at sBj + g * BUF. The two buffers are
    // separate LDS objects: when the step loop names them at compile time
    // (the mask-free steps run in pairs), the compiler can see that the
    // transposing reads of the current buffer do not alias the loads in
    // flight into the other one, instead of waiting for those loads (vmcnt
    // 0) in the middle of every step.
    __shared__ __attribute__((aligned(16))) e16 sB0[BUF * KG];
    __shared__ __attribute__((aligned(16))) e16 sB1[BUF * KG];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches and buffer resources
    const int grp = KG == 1 ? 0 : wave / WG;  // key group
    const int gw = wave - grp * WG;           // wave within the group = its 32-row tile
    const int l32 = lane & 31;
    const int h = lane >> 5;
    const int N = p.N;

    // Workgroup -> (query block, batch*head). Under the causal mask the
    // latest (heaviest) query blocks come first.
    const int bid = blockIdx.x;
    const int bh = xcd_head(bid % p.BH, p.BH);
    const int qb = causal_block(bid / p.BH, p.nqb, NW == 4 && KG == 1 && gridDim.x <= 512, CAUSAL);
    const int b = bh / p.Hq;
    const int hq = bh - b * p.Hq;
    const int hkv = hq / p.G;

    const e16* Qh = static_cast<const e16*>(p.q) + b * p.sq.b + hq * p.sq.h;
    const e16* Kh = static_cast<const e16*>(p.k) + b * p.sk.b + hkv * p.sk.h;
    const e16* Vh = static_cast<const e16*>(p.v) + b * p.sv.b + hkv * p.sv.h;
    const long long sqn = p.sq.n, skn = p.sk.n, svn = p.sv.n;

    const int q0 = qb * BQ;
    const int qw0 = q0 + gw * 32;
    const int qrow = qw0 + l32;

    // Columns d .. padded width of the V tiles are read by the last O^T tile
    // and must be zero; the loaders never write them.
    if constexpr (NDT * 32 > D) {
        constexpr int PADC = NDT * 32 - D;
        for (int i = tid; i < 2 * KG * BC * PADC; i += T) {
            const int row = i / PADC;
            const int col = D + i % PADC;
            const int bufi = row / BC;  // 2 * group + buffer
            ((bufi & 1) ? sB1 : sB0)[(bufi >> 1) * BUF + BC * KP + (row % BC) * VP + col] = (e16)0;
        }
    }

    // Q operand (B of S^T = K Q^T): lane holds query qrow, dims 16*ks + 8*h .. +7.
    e16x8 qf[KS];
    if (qrow < N) {
        const e16* qp = Qh + qrow * sqn + h * 8;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qf[ks] = *reinterpret_cast<const e16x8*>(qp + ks * 16);
    } else {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qf[ks] = e16x8{};
    }

    const int nkb = (N + BC - 1) / BC;
    const int kb_end = CAUSAL ? min(nkb, (q0 + BQ - 1) / BC + 1) : nkb;
    // Sliding window: keys before the workgroup's first row's band are skipped.
    const int W = WINDOW ? p.window : 0;
    const int kb_begin = WINDOW ? max(0, q0 - W + 1) / BC : 0;

    uint4 kreg[NCH], vreg[NCH];
    // K/V rows kv0 .. kv0+BC-1 through buffer resources ending at row N-1:
    // rows past the end read as zeros, with no per-row bounds arithmetic.
    auto load_tile = [&](int kv0) {
        const uint32_t sk2 = (uint32_t)skn * 2u, sv2 = (uint32_t)svn * 2u;
        const auto rk = buf_rsrc(Kh + (long long)kv0 * skn, (uint32_t)(N - kv0 - 1) * sk2 + D * 2);
        const auto rv = buf_rsrc(Vh + (long long)kv0 * svn, (uint32_t)(N - kv0 - 1) * sv2 + D * 2);
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            const int c = tid + i * T;
            if (CHUNKS % T == 0 || c < CHUNKS) {
                const int row = c / CPR;
                const int col = c - row * CPR;
                kreg[i] = buf_load16(rk, (uint32_t)row * sk2 + (uint32_t)col * 16u);
                vreg[i] = buf_load16(rv, (uint32_t)row * sv2 + (uint32_t)col * 16u);
            }
        }
    };
    auto store_tile = [&](int bufi) {
        e16* Ks = bufi ? sB1 : sB0;
        e16* Vs = Ks + BC * KP;
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            const int c = tid + i * T;
            if (CHUNKS % T == 0 || c < CHUNKS) {
                const int row = c / CPR;
                const int col = c - row * CPR;
                *reinterpret_cast<uint4*>(Ks + row * KP + col * 8) = kreg[i];
                *reinterpret_cast<uint4*>(Vs + row * VP + col * 8) = vreg[i];
            }
        }
    };

    // d <= 128 (64-key tiles): tiles go straight from memory to LDS. Each
    // 64-lane buffer load with the LDS flag writes 64 consecutive 16-byte
    // chunks; lane i of load j covers chunk 64j + i of the padded tile, i.e.
    // row (64j + i) / (pitch / 8), chunk (64j + i) % (pitch / 8). Padding
    // chunks get an offset past the end of the buffer, so they are written
    // with zeros, and so are rows at or past N. No registers or LDS stores
    // are spent on staging.
    constexpr bool DIRECT = BC == 64;
    constexpr int CKK = KP / 8, CKV = VP / 8;           // chunks per padded row
    constexpr int NLK = BC * CKK / 64, NLV = BC * CKV / 64;  // loads per tile
    // A group's tiles are loaded by its own WG waves.
    constexpr int LPWK = (NLK + WG - 1) / WG, LPWV = (NLV + WG - 1) / WG;
    static_assert(!DIRECT || (BC * CKK % 64 == 0 && BC * CKV % 64 == 0), "tile must be whole loads");
    uint32_t offk[DIRECT ? LPWK : 1], offv[DIRECT ? LPWV : 1];
    if constexpr (DIRECT) {
        const uint32_t sk2 = (uint32_t)skn * 2u, sv2 = (uint32_t)svn * 2u;
#pragma unroll
        for (int i = 0; i < LPWK; ++i) {
            const int chunk = (gw + i * WG) * 64 + lane;
            const int row = chunk / CKK, ch = chunk - row * CKK;
            offk[i] = ch < CPR ? (uint32_t)row * sk2 + (uint32_t)ch * 16u : 0xFFFFFFF0u;
        }
#pragma unroll
        for (int i = 0; i < LPWV; ++i) {
            const int chunk = (gw + i * WG) * 64 + lane;
            const int row = chunk / CKV, ch = chunk - row * CKV;
            offv[i] = ch < CPR ? (uint32_t)row * sv2 + (uint32_t)ch * 16u : 0xFFFFFFF0u;
        }
    }
    e16* const g0 = sB0 + grp * BUF;  // this group's two tile buffers
    e16* const g1 = sB1 + grp * BUF;
    auto issue_into = [&](int kv0, e16* buf) {
        const uint32_t sk2 = (uint32_t)skn * 2u, sv2 = (uint32_t)svn * 2u;
        const auto rk = buf_rsrc(Kh + (long long)kv0 * skn, (uint32_t)(N - kv0 - 1) * sk2 + D * 2);
        const auto rv = buf_rsrc(Vh + (long long)kv0 * svn, (uint32_t)(N - kv0 - 1) * sv2 + D * 2);
        char* kb_lds = reinterpret_cast<char*>(buf);
        char* vb_lds = kb_lds + BC * KP * 2;
#pragma unroll
        for (int i = 0; i < LPWK; ++i) {
            const int j = gw + i * WG;
            if (NLK % WG == 0 || j < NLK) buf_load16_to_lds(rk, kb_lds + j * 1024, offk[i]);
        }
#pragma unroll
        for (int i = 0; i < LPWV; ++i) {
            const int j = gw + i * WG;
            if (NLV % WG == 0 || j < NLV) buf_load16_to_lds(rv, vb_lds + j * 1024, offv[i]);
        }
    };
    // A branch rather than a select of the two buffers' addresses: each load
    // then names its LDS object (a selected generic address would have to be
    // cast back to LDS at run time, which unoptimised builds cannot emit).
    auto issue_tile = [&](int kv0, int bufi) {
        if (bufi)
            issue_into(kv0, g1);
        else
            issue_into(kv0, g0);
    };

    // Key tiles of this group: [gs, ge). With one group that is the whole
    // range; with two, group 0 takes the first ceil(n/2) tiles.
    const int kmid = kb_begin + (kb_end - kb_begin + 1) / 2;
    const int gs = KG == 1 ? kb_begin : (grp == 0 ? kb_begin : kmid);
    const int ge = KG == 1 ? kb_end : (grp == 0 ? kmid : kb_end);
    // Key blocks [ku_begin, ku_end) need neither the per-wave skip nor a
    // mask: every key is at or before the workgroup's first query (kv0 + BC
    // - 1 <= q0), inside its last query's band (kv0 >= q0 + BQ - W) and
    // before N. They run in a copy of the step without those tests. With
    // one key group, block kb's tile sits in buffer (kb - ku_begin) & 1.
    int ku_begin = kb_begin, ku_end = min(kb_end, N / BC);
    if (CAUSAL) ku_end = min(ku_end, (q0 + 1) / BC);
    if (WINDOW) {
        const int t = q0 + BQ - W;
        ku_begin = min(kb_end, max(kb_begin, t > 0 ? (t + BC - 1) / BC : 0));
    }
    ku_end = max(ku_end, ku_begin);
    if constexpr (DIRECT) {
        if (KG == 1)
            issue_tile(kb_begin * BC, (kb_begin - ku_begin) & 1);
        else if (gs < ge)
            issue_tile(gs * BC, 0);
        __builtin_amdgcn_s_waitcnt(0);
    } else {
        load_tile(kb_begin * BC);
        store_tile((kb_begin - ku_begin) & 1);
    }
    __syncthreads();

    f32x16 oacc[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) oacc[dt] = f32x16{};
    float m = -__builtin_huge_valf();  // running max of c*s (log2 domain)
    float l = 0.0f;                    // this lane's share of the running sum
    const float c = p.c;

    // Per-lane constant parts of the LDS addresses.
    const int g16 = lane >> 4;          // 16-lane group
    const int j16 = lane & 15;
    const int tr_row = (g16 >> 1) * 4 + (j16 >> 2);
    const int tr_col = (g16 & 1) * 16 + (j16 & 3) * 4;

    // One step: tile kb in buffer bufi, the next tile (kb + 1, at most
    // kb_last) loaded into the other buffer. `has` is false only for the
    // idle last step of a key group with fewer tiles, which just keeps the
    // barrier count.
    auto run_step = [&](int kb, int bufi, int kb_last, bool has, auto masked_tag) {
        constexpr bool MASKED = decltype(masked_tag)::value;
        // The last step reloads its own tile into the idle buffer (never
        // read again), so the loads and stores need no branch.
        if constexpr (DIRECT) {
            if (has) issue_tile(min(kb + 1, kb_last) * BC, bufi ^ 1);
        } else {
            load_tile(min(kb + 1, kb_last) * BC);
        }

        const int kv0 = kb * BC;
        const e16* Ks = bufi ? g1 : g0;
        const e16* Vs = Ks + BC * KP;
        const bool active = has && (!MASKED || !CAUSAL || (kv0 <= qw0 + 31 && (!WINDOW || kv0 + BC - 1 >= qw0 - W + 1)));
        if (active) {
            f32x16 s[NKT];
            if constexpr (D <= 128) {
                // S^T = K Q^T with the K row reads kept two products ahead,
                // pinned in order by scheduling barriers.
                constexpr int NS = NKT * KS;
                e16x8 kr[3];
                auto rdk = [&](int idx) {
                    const int kt = idx / KS, ks = idx % KS;
                    kr[idx % 3] = lds_read8(Ks + (kt * 32 + l32) * KP + h * 8 + ks * 16);
                };
#pragma unroll
                for (int kt = 0; kt < NKT; ++kt) s[kt] = f32x16{};
                rdk(0);
                rdk(1);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int idx = 0; idx < NS; ++idx) {
                    if (idx + 2 < NS) rdk(idx + 2);
                    s[idx / KS] = mfma32<DT>(kr[idx % 3], qf[idx % KS], s[idx / KS]);
                    __builtin_amdgcn_sched_barrier(0);
                }
            } else {
#pragma unroll
                for (int kt = 0; kt < NKT; ++kt) {
                    s[kt] = f32x16{};
                    const e16* kp = Ks + (kt * 32 + l32) * KP + h * 8;
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks)
                        s[kt] = mfma32<DT>(lds_read8(kp + ks * 16), qf[ks], s[kt]);
                }
            }
            // Keys outside [lo, hi] (relative to kv0 + 4h) are masked: the
            // tail beyond N, keys after the row (causal) and keys before its
            // band (sliding window).
            const bool need_mask = MASKED && ((CAUSAL && kv0 + BC - 1 > qw0) || (kv0 + BC > N) ||
                                              (WINDOW && kv0 < qw0 + 32 - W));
            if (need_mask) {
                const int hi = (CAUSAL ? min(qrow, N - 1) : N - 1) - kv0 - 4 * h;
                const int lo = (WINDOW ? qrow - W + 1 : 0) - kv0 - 4 * h;
#pragma unroll
                for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int koff = kt * 32 + (r >> 2) * 8 + (r & 3);
                        s[kt][r] = (koff > hi || koff < lo) ? -__builtin_huge_valf() : s[kt][r];
                    }
            }
            float mx = s[0][0];
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kt][r]);
            // Lazy rescaling: the reference maximum m only moves, and O, l are
            // rescaled, when a row's block maximum exceeds it by more than 2^8;
            // the first block with an allowed key just adopts its maximum.
            const float mb = max_across_halves(mx) * c;
            if (m == -__builtin_huge_valf()) m = mb;
            if (__any(mb > m + 8.0f)) {
                const float m_new = fmaxf(m, mb);
                // (a lane still without an allowed key keeps m = -inf, alpha 1)
                const float alpha = (m_new == -__builtin_huge_valf()) ? 1.0f : fast_exp2(m - m_new);
                m = m_new;
                l *= alpha;
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) oacc[dt] *= alpha;
            }
            // A row that has not met an allowed key yet (possible only under a
            // sliding window) still has m = -inf: use 0 so masked scores give
            // exp2(-inf) = 0 rather than NaN.
            const float m_new = (m == -__builtin_huge_valf()) ? 0.0f : m;

            e16x8 pb[PVS];
            float lsum = 0.0f;
            // Dropout: keep bits of this lane's query for every key of the
            // step (bit r of keep[kt] belongs to register r of s[kt]). The
            // row sum l takes every probability; only the product with V
            // sees the dropped ones as zero, and O is scaled by 1/(1-p).
            uint32_t keep[NKT];
            if constexpr (DROP) {
#pragma unroll
                for (int kt = 0; kt < NKT; ++kt) {
                    keep[kt] = 0;
#pragma unroll
                    for (int gp = 0; gp < 2; ++gp)
                        keep[kt] |= keep_bits_query_lane(p.drop, kv0 + kt * 32 + 16 * gp + 4 * h, qrow, bh)
                                    << (8 * gp);
                }
            }
            // Probabilities of register pair (2e, 2e+1) of contraction step u
            // (16 keys), packed in the B-operand order of O^T += V^T P^T.
            e16x2 pr[PVS][4];
            auto exp_pair = [&](int u, int e) {
                const int kt = u >> 1;
                const int r = (u & 1) * 8 + 2 * e;
                const float a0 = fast_exp2(fmaf(s[kt][r], c, -m_new));
                const float a1 = fast_exp2(fmaf(s[kt][r + 1], c, -m_new));
                lsum += a0 + a1;
                if constexpr (DROP)
                    pr[u][e] = cvt2<DT>(((keep[kt] >> r) & 1u) ? a0 : 0.0f,
                                        ((keep[kt] >> (r + 1)) & 1u) ? a1 : 0.0f);
                else
                    pr[u][e] = cvt2<DT>(a0, a1);
            };
            auto v_op = [&](int u, int dt) {
                const e16* vp = Vs + (u * 16 + tr_row) * VP + tr_col;
                return join8(lds_read_tr4(vp + dt * 32), lds_read_tr4(vp + 8 * VP + dt * 32));
            };
            if constexpr (D <= 128) {
                // The products of step u run with the exponentials of step
                // u + 1 and its transposed V reads in their shadow.
                constexpr int EPD = (4 + NDT - 1) / NDT;  // exp pairs per product
                e16x8 va[2][NDT];
#pragma unroll
                for (int e = 0; e < 4; ++e) exp_pair(0, e);
                pb[0] = cat8(pr[0][0], pr[0][1], pr[0][2], pr[0][3]);
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) va[0][dt] = v_op(0, dt);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int u = 0; u < PVS; ++u) {
#pragma unroll
                    for (int dt = 0; dt < NDT; ++dt) {
                        oacc[dt] = mfma32<DT>(va[u & 1][dt], pb[u], oacc[dt]);
                        if (u + 1 < PVS) {
                            va[(u + 1) & 1][dt] = v_op(u + 1, dt);
#pragma unroll
                            for (int j = 0; j < EPD; ++j)
                                if (dt * EPD + j < 4) exp_pair(u + 1, dt * EPD + j);
                        }
                        __builtin_amdgcn_sched_barrier(0);
                    }
                    if (u + 1 < PVS)
                        pb[u + 1] = cat8(pr[u + 1][0], pr[u + 1][1], pr[u + 1][2], pr[u + 1][3]);
                }
            } else {
#pragma unroll
                for (int u = 0; u < PVS; ++u) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) exp_pair(u, e);
                    pb[u] = cat8(pr[u][0], pr[u][1], pr[u][2], pr[u][3]);
                }
#pragma unroll
                for (int u = 0; u < PVS; ++u)
#pragma unroll
                    for (int dt = 0; dt < NDT; ++dt) oacc[dt] = mfma32<DT>(v_op(u, dt), pb[u], oacc[dt]);
            }
            l += lsum;
        }
        if constexpr (DIRECT)
            __builtin_amdgcn_s_waitcnt(0);  // the next tile has landed in LDS
        else
            store_tile(bufi ^ 1);
        __syncthreads();
    };
    float lt;
    if constexpr (KG == 1) {
        // Mask-free blocks in pairs (buffers known at compile time); a last
        // unpaired one joins the masked blocks after them, whose masks then
        // change nothing. With dropout the second copy of the step costs
        // registers (spills), so there the buffers stay chosen at run time.
        int kb = kb_begin;
        for (; kb < ku_begin; ++kb) run_step(kb, (kb - ku_begin) & 1, kb_end - 1, true, std::true_type{});
        if constexpr (DROP) {
            for (; kb < ku_end; ++kb) run_step(kb, (kb - ku_begin) & 1, kb_end - 1, true, std::false_type{});
        } else {
            for (; kb + 1 < ku_end; kb += 2) {
                run_step(kb, 0, kb_end - 1, true, std::false_type{});
                run_step(kb + 1, 1, kb_end - 1, true, std::false_type{});
            }
        }
        for (; kb < kb_end; ++kb) run_step(kb, (kb - ku_begin) & 1, kb_end - 1, true, std::true_type{});
        lt = sum_across_halves(l);  // the two half-row sums
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
        // Group 1 hands (m, l, O^T) to the wave of group 0 with the same rows,
        // through the tile buffers (every wave has finished with them: each
        // waited for its own loads before the last barrier).
        const float lg = sum_across_halves(l);
        constexpr int OSZ = WG * NDT * 16 * 64;
        static_assert((OSZ + 2 * WG * 64) * 4 <= KG * BUF * 2, "merge data must fit the first tile buffers");
        float* xs = reinterpret_cast<float*>(sB0);
        if (grp == 1) {
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) xs[((gw * NDT + dt) * 16 + r) * 64 + lane] = oacc[dt][r];
            xs[OSZ + gw * 64 + lane] = m;
            xs[OSZ + (WG + gw) * 64 + lane] = lg;
        }
        __syncthreads();
        if (grp == 1) return;
        const float m1 = xs[OSZ + gw * 64 + lane];
        const float l1 = xs[OSZ + (WG + gw) * 64 + lane];
        const float mm = fmaxf(m, m1);
        // a group that met no allowed key of the row has m = -inf and adds nothing
        const float a0 = m == -__builtin_huge_valf() ? (m1 == -__builtin_huge_valf() ? 1.0f : 0.0f) : fast_exp2(m - mm);
        const float a1 = m1 == -__builtin_huge_valf() ? 0.0f : fast_exp2(m1 - mm);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                oacc[dt][r] = a0 * oacc[dt][r] + a1 * xs[((gw * NDT + dt) * 16 + r) * 64 + lane];
        lt = a0 * lg + a1 * l1;
        m = mm;
    }

    // Epilogue: normalise, store O and LSE.
    const float inv = (DROP ? p.drop.scale : 1.0f) / lt;
    if (qrow < N) {
        e16* orow = static_cast<e16*>(p.o) + b * p.so.b + hq * p.so.h + qrow * p.so.n;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int d = dt * 32 + g4 * 8 + h * 4;
                if (d < D)
                    store4<DT>(orow + d, oacc[dt][g4 * 4 + 0] * inv, oacc[dt][g4 * 4 + 1] * inv,
                                 oacc[dt][g4 * 4 + 2] * inv, oacc[dt][g4 * 4 + 3] * inv);
            }
        if (h == 0) p.lse[(size_t)bh * N + qrow] = (m + log2f(lt)) * kLn2;
    }
}

// ------------------------------------------------------------------
// d = 128 without dropout, large grids: the same step loop on 16x16x32 products.
//
// The chip sustains v_mfma_f32_16x16x32_bf16 at a higher clock than the
// 32x32x16 product on the same random operands (the matrix cores are equally
// busy, the power limit lets the clock stay ~12 % higher), so for the
// product-heavy d = 128 loop the wave's work is cut into 16x16 tiles:
//  * 16x16x32 operands and result (wave64): A[16x32]: lane l holds row l % 16,
//    k = 8 (l / 16) .. +7; B[32x16]: lane l holds column l % 16, the same k;
//    D[16x16]: lane l, register r holds D[4 (l / 16) + r][l % 16].
//  * S^T = K Q^T per 64-key step: 4 key tiles x 2 query tiles of 16, 4
//    contraction steps of 32 dims. A K operand (one 16-byte LDS row read)
//    serves both query tiles. A lane then holds, for queries qw0 + l % 16 and
//    qw0 + 16 + l % 16, keys 16 kt + 4 (l / 16) + r: the row maximum and sum
//    combine the lane's 16 values and then the four 16-lane groups (two
//    lane-swap steps).
//  * O^T += V^T P^T over two 32-key halves: B element i of lane group g is
//    key 4g + i (i < 4) or 16 + 4g + i - 4 (i >= 4) of the half, which is
//    exactly what the lane holds of s[2 jj] and s[2 jj + 1], so the
//    probabilities are packed in place. The V^T operand takes the same key
//    order: two transposing reads of 4 keys (rows 4g .. 4g+3 and 16 + 4g ..)
//    by 16 dims. O^T is 8 x 2 tiles of 16x16, one query per lane column.
//  * Both tiles have a pitch of 144 elements (288 bytes, an odd multiple of
//    32). Measured with SQ_LDS_BANK_CONFLICT on the part, that pitch serves
//    both reads of this layout without conflicts: the 16-byte row reads of
//    16 rows x 4 chunks (the S^T operand) and the transposing reads of 4 rows
//    x 32 bytes per 16-lane group (V^T). The 136-element pitch that the
//    32x32x16 kernels' row reads use takes twice the LDS cycles here.
//  * The step loop is software pipelined across key blocks: step j computes
//    the S^T products of block j + 1 while it turns block j's scores into
//    probabilities and runs block j's O^T products (the region plan is in
//    the kernel), so that every stretch of softmax work has matrix products
//    of the same wave beside it. K therefore runs one tile ahead of V.
//  * 16x16x32 products are what the chip runs fastest on random operands:
//    the rate probe (include/attn_probe.h) sustains 2.15 PFLOP/s with 4
//    independent accumulators per wave against 1.33 for 32x32x16.
// Everything else (online softmax with the lazy reference maximum, tile
// loads straight to LDS, causal/window skipping, launch order) is as in
// fwd_kernel.
constexpr int m16_pitch(int d) { return ((2 * d / 32) % 2 == 1 ? 2 * d : 2 * d + 32) / 2; }
static_assert(m16_pitch(128) == 144 && (m16_pitch(128) * 2 / 32) % 2 == 1, "");
// Head dims whose no-dropout step loop runs on 16x16x32 products on large
// grids. (d = 64 is bound by its softmax work, where the two query tiles per
// lane cost more than the products gain; so are the plans of small grids,
// which stay on fwd_kernel.)
template <int D> constexpr bool kProducts16 = D == 128;

template <int DT>
__device__ __forceinline__ f32x4 mfma16(e16x8 a, e16x8 b, f32x4 c) {
    if constexpr (DT == kBF16)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// Lanes l, l ^ 16, l ^ 32 and l ^ 48 combine a value (v_permlane32_swap,
// then v_permlane16_swap).
__device__ __forceinline__ float max_across_quarters(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    const float y = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    auto t = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
    return fmaxf(__uint_as_float(t[0]), __uint_as_float(t[1]));
}
__device__ __forceinline__ float sum_across_quarters(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    const float y = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    auto t = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
    return __uint_as_float(t[0]) + __uint_as_float(t[1]);
}

template <int DT, int D, int MASK, int NW>
__global__ __launch_bounds__(NW * 64, 2)
void fwd_m16_kernel(FwdParams p) {
    constexpr int BQ = NW * 32;
    constexpr bool CAUSAL = MASK != kMaskNone;
    constexpr bool WINDOW = MASK == kMaskWindow;
    constexpr int BC = 64;
    constexpr int KS = D / 32;   // contraction steps of S^T = K Q^T
    constexpr int NDT = D / 16;  // 16-row tiles of O^T
    constexpr int KP = m16_pitch(D);
    constexpr int VP = m16_pitch(D);
    constexpr int CPR = D / 8;
    static_assert(D % 32 == 0 && D <= 128 && FwdTile<D>::BLOCK_KV == BC, "16x16x32 step loop: 64-key tiles");

    // Two K and two V tile buffers, each its own LDS object (see below).
    __shared__ __attribute__((aligned(16))) e16 sK0[BC * KP];
    __shared__ __attribute__((aligned(16))) e16 sK1[BC * KP];
    __shared__ __attribute__((aligned(16))) e16 sV0[BC * VP];
    __shared__ __attribute__((aligned(16))) e16 sV1[BC * VP];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15;
    const int g = lane >> 4;  // 16-lane group
    const int N = p.N;

    const int bid = blockIdx.x;
    const int bh = xcd_head(bid % p.BH, p.BH);
    const int qb = causal_block(bid / p.BH, p.nqb, NW == 4 && gridDim.x <= 512, CAUSAL);
    const int b = bh / p.Hq;
    const int hq = bh - b * p.Hq;
    const int hkv = hq / p.G;

    const e16* Qh = static_cast<const e16*>(p.q) + b * p.sq.b + hq * p.sq.h;
    const e16* Kh = static_cast<const e16*>(p.k) + b * p.sk.b + hkv * p.sk.h;
    const e16* Vh = static_cast<const e16*>(p.v) + b * p.sv.b + hkv * p.sv.h;
    const long long sqn = p.sq.n, skn = p.sk.n, svn = p.sv.n;

    const int q0 = qb * BQ;
    const int qw0 = q0 + wave * 32;
    const int qrow0 = qw0 + l16, qrow1 = qw0 + 16 + l16;

    // Q operand (B of S^T): query qw0 + 16 qt + l16, dims 32 ks + 8 g .. +7.
    e16x8 qf[2][KS];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
        const int qr = qt ? qrow1 : qrow0;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            qf[qt][ks] = qr < N ? *reinterpret_cast<const e16x8*>(Qh + qr * sqn + ks * 32 + g * 8) : e16x8{};
    }

    const int nkb = (N + BC - 1) / BC;
    const int kb_end = CAUSAL ? min(nkb, (q0 + BQ - 1) / BC + 1) : nkb;
    const int W = WINDOW ? p.window : 0;
    const int kb_begin = WINDOW ? max(0, q0 - W + 1) / BC : 0;

    // Tiles go straight from memory to LDS, as in fwd_kernel, but K runs one
    // tile ahead of V: step j reads K of block j + 1 (the next scores) and V
    // of block j, and loads K of block j + 2 and V of block j + 1. Block t's
    // K and V sit in buffer (t - kb_begin) & 1, which the step loop (unrolled
    // by two) knows at compile time. Each buffer being its own __shared__
    // object, the compiler can see that the transposing V reads of the
    // current buffer do not alias the loads in flight into the other one;
    // within one object it would make them wait for those loads (vmcnt 0)
    // half-way through every step.
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
            const int row = chunk / CKK, ch = chunk - row * CKK;
            offk[i] = ch < CPR ? (uint32_t)row * sk2 + (uint32_t)ch * 16u : 0xFFFFFFF0u;
        }
#pragma unroll
        for (int i = 0; i < LPWV; ++i) {
            const int chunk = (wave + i * NW) * 64 + lane;
            const int row = chunk / CKV, ch = chunk - row * CKV;
            offv[i] = ch < CPR ? (uint32_t)row * sv2 + (uint32_t)ch * 16u : 0xFFFFFFF0u;
        }
    }
    auto issue_k = [&](int kb, e16* buf) {
        const int kv0 = kb * BC;
        const auto rk = buf_rsrc(Kh + (long long)kv0 * skn, (uint32_t)(N - kv0 - 1) * (uint32_t)skn * 2u + D * 2);
        char* dst = reinterpret_cast<char*>(buf);
#pragma unroll
        for (int i = 0; i < LPWK; ++i) {
            const int j = wave + i * NW;
            if (NLK % NW == 0 || j < NLK) buf_load16_to_lds(rk, dst + j * 1024, offk[i]);
        }
    };
    auto issue_v = [&](int kb, e16* buf) {
        const int kv0 = kb * BC;
        const auto rv = buf_rsrc(Vh + (long long)kv0 * svn, (uint32_t)(N - kv0 - 1) * (uint32_t)svn * 2u + D * 2);
        char* dst = reinterpret_cast<char*>(buf);
#pragma unroll
        for (int i = 0; i < LPWV; ++i) {
            const int j = wave + i * NW;
            if (NLV % NW == 0 || j < NLV) buf_load16_to_lds(rv, dst + j * 1024, offv[i]);
        }
    };

    f32x4 oacc[NDT][2];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) oacc[dt][0] = oacc[dt][1] = f32x4{};
    float m[2] = {-__builtin_huge_valf(), -__builtin_huge_valf()};  // per query tile, log2 domain
    float l[2] = {0.0f, 0.0f};
    float mn[2] = {0.0f, 0.0f};  // m with -inf read as 0: the exponent offset
    const float c = p.c;
    // Transposing V read: lane 4t+s of group g addresses key row 4g + t, dims 4s .. 4s+3.
    const int v_row = 4 * g + (l16 >> 2);
    const int v_col = 4 * (l16 & 3);

    // A wave computes the blocks from the workgroup's first to the last one
    // that holds a key at or before its last query. (Under a sliding window
    // the later waves' bands start a few blocks after the first; those blocks
    // are masked to -inf in full and add nothing.)
    const int kb_last_w = CAUSAL ? min(kb_end - 1, (qw0 + 31) / BC) : kb_end - 1;
    auto needs_mask = [&](int kb) {
        const int kv0 = kb * BC;
        return (CAUSAL && kv0 + BC - 1 > qw0) || (kv0 + BC > N) || (WINDOW && kv0 < qw0 + 32 - W);
    };
    // s[kt][qt][r]: key kv0 + 16 kt + 4 g + r, query qw0 + 16 qt + l16.
    using Scores = f32x4[4][2];
    // Masks block kb's scores, then takes each query tile's maximum and
    // decides the lazy rescale (as fwd_kernel): the reference m moves only
    // when some row's block maximum exceeds it by more than 8 (log2 units).
    // The lanes' own maxima are combined over the four 16-lane groups only
    // when one of them could move it.
    auto finish_scores = [&](Scores& s, int kb) {
        if (needs_mask(kb)) {
            const int kv0 = kb * BC;
#pragma unroll
            for (int qt = 0; qt < 2; ++qt) {
                const int qr = qt ? qrow1 : qrow0;
                const int hi = (CAUSAL ? min(qr, N - 1) : N - 1) - kv0 - 4 * g;
                const int lo = (WINDOW ? qr - W + 1 : 0) - kv0 - 4 * g;
#pragma unroll
                for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int koff = kt * 16 + r;
                        s[kt][qt][r] = (koff > hi || koff < lo) ? -__builtin_huge_valf() : s[kt][qt][r];
                    }
            }
        }
        float mx[2];
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
            mx[qt] = s[0][qt][0];
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                for (int r = 0; r < 4; ++r) mx[qt] = fmaxf(mx[qt], s[kt][qt][r]);
        }
        const bool moves = mx[0] * c > m[0] + 8.0f || mx[1] * c > m[1] + 8.0f ||
                           m[0] == -__builtin_huge_valf() || m[1] == -__builtin_huge_valf();
        if (__any(moves)) {
            float mb[2];
#pragma unroll
            for (int qt = 0; qt < 2; ++qt) {
                mb[qt] = max_across_quarters(mx[qt]) * c;
                if (m[qt] == -__builtin_huge_valf()) m[qt] = mb[qt];
            }
            if (__any(mb[0] > m[0] + 8.0f || mb[1] > m[1] + 8.0f)) {
#pragma unroll
                for (int qt = 0; qt < 2; ++qt) {
                    const float m_new = fmaxf(m[qt], mb[qt]);
                    const float alpha = (m_new == -__builtin_huge_valf()) ? 1.0f : fast_exp2(m[qt] - m_new);
                    m[qt] = m_new;
                    l[qt] *= alpha;
#pragma unroll
                    for (int dt = 0; dt < NDT; ++dt) oacc[dt][qt] *= alpha;
                }
            }
#pragma unroll
            for (int qt = 0; qt < 2; ++qt) mn[qt] = (m[qt] == -__builtin_huge_valf()) ? 0.0f : m[qt];
        }
    };

    // One step j, in four regions pinned in order by scheduling barriers:
    //   R1: 12 of the 16 S^T product pairs of block j + 1 (K read two pairs
    //       ahead), with the 16 exponentials of block j's first key half;
    //   R2: the 8 O^T product pairs of the first half (V^T read two ahead),
    //       with 10 exponentials of the second half;
    //   R3: the last 4 S^T pairs of block j + 1, with the last 6;
    //   R4: the 8 O^T pairs of the second half, then block j + 1's mask,
    //       maxima and rescale decision.
    // A pair is the two products (query tiles) sharing one A operand. So
    // every region issues softmax work under its own matrix products instead
    // of between them. CUR: this wave computes block j (its scores are in
    // `sc`); NXT: it computes block j + 1 (into `sn`).
    auto step = [&](int j, Scores& sc, Scores& sn, const e16* Ks, const e16* Vs) {
        constexpr bool CUR = true, NXT = true;
        constexpr int NS = 4 * KS;  // S^T product pairs
        e16x8 kr[3];
        auto rdk = [&](int idx) {
            const int ks = idx / 4, kt = idx % 4;
            kr[idx % 3] = lds_read8(Ks + (kt * 16 + l16) * KP + ks * 32 + g * 8);
        };
        auto sprod = [&](int idx) {
            const int ks = idx / 4, kt = idx % 4;
            if (idx + 2 < NS) rdk(idx + 2);
            sn[kt][0] = mfma16<DT>(kr[idx % 3], qf[0][ks], sn[kt][0]);
            sn[kt][1] = mfma16<DT>(kr[idx % 3], qf[1][ks], sn[kt][1]);
        };
        float lsum0 = 0.0f, lsum1 = 0.0f;
        // Probability u (0..31) of the step: key half jj = u / 16 and e = u %
        // 16, query tile e / 8, B element i = e % 8, i.e. register i % 4 of
        // sc[2 jj + i / 4]. Each is computed in three stages a slot apart
        // (a slot being one product pair): the exponent's FMA (A), the
        // exponential (B), then the row sum and, for odd e, the rounding of
        // the pair to 16 bits (C), so that no stage waits on the one before
        // it and the products issue without stalls.
        float ta[32], xb[32];
        e16x2 pp[2][8];
        auto stage_a = [&](int u) {
            const int jj = u >> 4, e = u & 15, qt = e >> 3, i = e & 7;
            ta[u] = fmaf(sc[2 * jj + (i >> 2)][qt][i & 3], c, -mn[qt]);
        };
        auto stage_b = [&](int u) { xb[u] = fast_exp2(ta[u]); };
        auto stage_c = [&](int u) {
            const int jj = u >> 4, e = u & 15;
            if (e >> 3)
                lsum1 += xb[u];
            else
                lsum0 += xb[u];
            if (e & 1) pp[jj][e >> 1] = cvt2<DT>(xb[u - 1], xb[u]);
        };
        // The slot that holds probabilities [lo, hi) starts those two further
        // on (A), takes the next ones through their exponential (B) and
        // finishes its own (C), in that order (a slot of two holds both
        // stages of some probabilities); the first slot also primes the
        // pipeline.
        auto units = [&](int lo, int hi) {
            if (lo == 0) {
                stage_a(0);
                stage_a(1);
                stage_b(0);
            }
            for (int u = lo + 2; u < hi + 2 && u < 32; ++u) stage_a(u);
            for (int u = lo + 1; u < hi + 1 && u < 32; ++u) stage_b(u);
            for (int u = lo; u < hi; ++u) stage_c(u);
        };
        e16x8 pb[2][2];
        auto pack = [&](int jj, int qt) {
            const e16x2* x = &pp[jj][qt * 4];
            pb[jj][qt] = cat8(x[0], x[1], x[2], x[3]);
        };
        e16x8 va[3];
        auto v_op = [&](int idx) {
            const int jj = idx / NDT, dt = idx % NDT;
            const e16* vp = Vs + (jj * 32 + v_row) * VP + v_col + dt * 16;
            va[idx % 3] = join8(lds_read_tr4(vp), lds_read_tr4(vp + 16 * VP));
        };
        constexpr int NP = 2 * NDT;  // O^T product pairs
        auto oprod = [&](int idx) {
            const int jj = idx / NDT, dt = idx % NDT;
            if (idx + 2 < NP) v_op(idx + 2);
            oacc[dt][0] = mfma16<DT>(va[idx % 3], pb[jj][0], oacc[dt][0]);
            oacc[dt][1] = mfma16<DT>(va[idx % 3], pb[jj][1], oacc[dt][1]);
        };
        constexpr int S1 = 12;       // S^T pairs in R1 (the rest in R3)
        static_assert(NS > S1 && NP >= 4, "region split assumes d = 128");
        constexpr int E2 = 10;       // second-half exponentials in R2 (the rest in R3)
        if constexpr (NXT) {
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) sn[kt][0] = sn[kt][1] = f32x4{};
            rdk(0);
            rdk(1);
        }
        __builtin_amdgcn_sched_barrier(0);
        // R1
        if constexpr (CUR) {
#pragma unroll
            for (int i = 0; i < S1; ++i) {
                if constexpr (NXT) sprod(i);
                units((i * 16) / S1, ((i + 1) * 16) / S1);
                __builtin_amdgcn_sched_barrier(0);
            }
            pack(0, 0);
            pack(0, 1);
            v_op(0);
            v_op(1);
            __builtin_amdgcn_sched_barrier(0);
            // R2
#pragma unroll
            for (int i = 0; i < NDT; ++i) {
                oprod(i);
                units(16 + (i * E2) / NDT, 16 + ((i + 1) * E2) / NDT);
                __builtin_amdgcn_sched_barrier(0);
            }
            // R3
            constexpr int S3 = NS - S1;
#pragma unroll
            for (int i = 0; i < S3; ++i) {
                if constexpr (NXT) sprod(S1 + i);
                units(16 + E2 + (i * (16 - E2)) / S3, 16 + E2 + ((i + 1) * (16 - E2)) / S3);
                __builtin_amdgcn_sched_barrier(0);
            }
            pack(1, 0);
            pack(1, 1);
            __builtin_amdgcn_sched_barrier(0);
            // R4
#pragma unroll
            for (int i = NDT; i < NP; ++i) {
                oprod(i);
                __builtin_amdgcn_sched_barrier(0);
            }
            l[0] += lsum0;
            l[1] += lsum1;
        } else if constexpr (NXT) {
#pragma unroll
            for (int i = 0; i < NS; ++i) {
                sprod(i);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        if constexpr (NXT) finish_scores(sn, j + 1);
    };

    // Prologue: K and V of the first block and K of the second; the first
    // block's scores.
    Scores sA, sB;
    issue_k(kb_begin, sK0);
    issue_v(kb_begin, sV0);
    if (kb_begin + 1 < kb_end) issue_k(kb_begin + 1, sK1);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    {
        // The S^T products of the first block alone (step j = kb_begin - 1
        // without a current block), reading K of kb_begin.
        const e16* Ks = sK0;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) sA[kt][0] = sA[kt][1] = f32x4{};
#pragma unroll
        for (int idx = 0; idx < 4 * KS; ++idx) {
            const int ks = idx / 4, kt = idx % 4;
            const e16x8 kr = lds_read8(Ks + (kt * 16 + l16) * KP + ks * 32 + g * 8);
            sA[kt][0] = mfma16<DT>(kr, qf[0][ks], sA[kt][0]);
            sA[kt][1] = mfma16<DT>(kr, qf[1][ks], sA[kt][1]);
        }
        finish_scores(sA, kb_begin);
    }
    __syncthreads();  // K of kb_begin is read; step kb_begin refills its buffer

    // Step j with (j - kb_begin) & 1 == PAR: K of j + 1 is in buffer 1 - PAR,
    // V of j in buffer PAR; K of j + 2 goes to buffer PAR, V of j + 1 to 1 - PAR.
    auto run = [&](int j, Scores& sc, Scores& sn, auto par_tag) {
        constexpr int PAR = decltype(par_tag)::value;
        e16* const Kn = PAR ? sK0 : sK1;
        e16* const Kl = PAR ? sK1 : sK0;
        e16* const Vc = PAR ? sV1 : sV0;
        e16* const Vl = PAR ? sV0 : sV1;
        if (j + 1 < kb_end) issue_v(j + 1, Vl);
        if (j + 2 < kb_end) issue_k(j + 2, Kl);
        // On its last block (and on the grid's last) a wave's step still
        // runs the next block's products, on whatever the K buffer holds;
        // those scores are masked and never used.
        if (j <= kb_last_w) step(j, sc, sn, Kn, Vc);
        __builtin_amdgcn_s_waitcnt(0);  // K of j + 2 and V of j + 1 have landed
        __syncthreads();
    };
    int kb = kb_begin;
    for (; kb + 1 < kb_end; kb += 2) {
        run(kb, sA, sB, std::integral_constant<int, 0>{});
        run(kb + 1, sB, sA, std::integral_constant<int, 1>{});
    }
    if (kb < kb_end) run(kb, sA, sB, std::integral_constant<int, 0>{});
    // Epilogue: the four 16-lane groups' row sums, then O and LSE.
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
        const int qr = qt ? qrow1 : qrow0;
        const float lt = sum_across_quarters(l[qt]);
        const float inv = 1.0f / lt;
        if (qr < N) {
            e16* orow = static_cast<e16*>(p.o) + b * p.so.b + hq * p.so.h + qr * p.so.n;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
                store4<DT>(orow + dt * 16 + 4 * g, oacc[dt][qt][0] * inv, oacc[dt][qt][1] * inv,
                           oacc[dt][qt][2] * inv, oacc[dt][qt][3] * inv);
            if (g == 0) p.lse[(size_t)bh * N + qr] = (m[qt] + log2f(lt)) * kLn2;
        }
    }
}

// Short sequences (at most kSplitMaxKeys keys, small grids): the keys of one
// 32-row query tile are split over the workgroup's waves, one 64-key tile
// each. Every wave issues all of its loads at once (its K tile straight into
// MFMA operand registers, its V tile into its own LDS region), computes its
// tile's probabilities against its own row maximum m_w with sum l_w and
// unnormalised output O_w, and the waves then combine through LDS with the
// same identity the online softmax applies block by block (CANN
// ops-transformer FlashAttention page, section on online softmax):
//   M = max_w m_w,  L = sum_w 2^(m_w - M) l_w,  O = sum_w 2^(m_w - M) O_w / L,
// all in the log2 domain. A workgroup thus waits on memory once instead of
// once per key step, and the grid has a workgroup per 32 rows: the regime
// where the step loop above is bound by latency rather than throughput.
template <int D> struct SplitTile {
    static constexpr int NDT = (D + 31) / 32;
    static constexpr int VBYTES = 64 * v_pitch(D) * 2;       // one wave's V tile
    static constexpr int OP = 40;                             // floats per partial-O row
    static constexpr int OBYTES = NDT * 32 * OP * 4;          // one wave's O_w^T
    static constexpr int AREA = VBYTES > OBYTES ? VBYTES : OBYTES;
    static constexpr int lds_bytes(int nw) { return nw * AREA + nw * 32 * 8; }
};

template <int DT, int D, int MASK, int NW>
__global__ __launch_bounds__(NW * 64, 1)
void fwd_split_kernel(FwdParams p) {
    constexpr int T = NW * 64;
    constexpr bool CAUSAL = MASK != kMaskNone;
    constexpr bool WINDOW = MASK == kMaskWindow;
    constexpr int BC = 64;
    constexpr int KS = D / 16;
    constexpr int NKT = BC / 32;
    constexpr int PVS = BC / 16;
    constexpr int NDT = SplitTile<D>::NDT;
    constexpr int VP = v_pitch(D);
    constexpr int CPR = D / 8;
    constexpr int CKV = VP / 8;
    constexpr int NLV = BC * CKV / 64;
    constexpr int OP = SplitTile<D>::OP;
    constexpr int AREA = SplitTile<D>::AREA;
    static_assert(BC * CKV % 64 == 0, "V tile must be whole loads");
    static_assert(4 * OP % 64 == 32, "the two lane halves of a partial-O store hit disjoint banks");

    __shared__ __attribute__((aligned(16))) char smem[SplitTile<D>::lds_bytes(NW)];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31;
    const int h = lane >> 5;
    const int N = p.N;

    const int bid = blockIdx.x;
    const int bh = xcd_head(bid % p.BH, p.BH);
    const int q0 = (bid / p.BH) * 32;
    const int b = bh / p.Hq;
    const int hq = bh - b * p.Hq;
    const int hkv = hq / p.G;
    const int qrow = q0 + l32;
    const int W = WINDOW ? p.window : 0;

    const e16* Qh = static_cast<const e16*>(p.q) + b * p.sq.b + hq * p.sq.h;
    const e16* Kh = static_cast<const e16*>(p.k) + b * p.sk.b + hkv * p.sk.h;
    const e16* Vh = static_cast<const e16*>(p.v) + b * p.sv.b + hkv * p.sv.h;
    const long long sqn = p.sq.n, skn = p.sk.n, svn = p.sv.n;

    // This wave's keys kv0 .. kv0 + 63; it has work if any of them is
    // allowed for some row of the tile.
    const int kv0 = wave * BC;
    const bool active = kv0 < N && (!CAUSAL || kv0 <= q0 + 31) && (!WINDOW || kv0 + BC - 1 >= q0 - W + 1);

    e16x8 qf[KS];
    e16x8 kf[NKT][KS];
    char* vlds = smem + wave * AREA;
    if (active) {
        // Q operand (B of S^T = K Q^T): query qrow, dims 16*ks + 8*h .. +7.
        if (qrow < N) {
            const e16* qp = Qh + qrow * sqn + h * 8;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) qf[ks] = *reinterpret_cast<const e16x8*>(qp + ks * 16);
        } else {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) qf[ks] = e16x8{};
        }
        // K operand (A): key kv0 + 32*kt + l32, dims 16*ks + 8*h .. +7; keys
        // at or past N read as zeros (buffer range).
        const uint32_t sk2 = (uint32_t)skn * 2u, sv2 = (uint32_t)svn * 2u;
        const auto rk = buf_rsrc(Kh + (long long)kv0 * skn, (uint32_t)(N - kv0 - 1) * sk2 + D * 2);
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const uint4 x = buf_load16(rk, (uint32_t)(kt * 32 + l32) * sk2 + (uint32_t)(h * 8 + ks * 16) * 2u);
                kf[kt][ks] = __builtin_bit_cast(e16x8, x);
            }
        // V tile into this wave's LDS region (row-major, pitch VP): load i
        // fills chunks 64i .. 64i + 63; padding chunks and rows past N are
        // given offsets outside the buffer and arrive as zeros.
        const auto rv = buf_rsrc(Vh + (long long)kv0 * svn, (uint32_t)(N - kv0 - 1) * sv2 + D * 2);
#pragma unroll
        for (int i = 0; i < NLV; ++i) {
            const int chunk = i * 64 + lane;
            const int row = chunk / CKV, ch = chunk - row * CKV;
            const uint32_t off = ch < CPR ? (uint32_t)row * sv2 + (uint32_t)ch * 16u : 0xFFFFFFF0u;
            buf_load16_to_lds(rv, vlds + i * 1024, off);
        }
    }
    __builtin_amdgcn_s_waitcnt(0);  // this wave's K operands and V tile have landed

    f32x16 oacc[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) oacc[dt] = f32x16{};
    float m = -__builtin_huge_valf();  // row maximum of c*s over this wave's keys
    float l = 0.0f;                    // this lane's half of the row sum
    const float c = p.c;
    if (active) {
        f32x16 s[NKT];
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) {
            s[kt] = f32x16{};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) s[kt] = mfma32<DT>(kf[kt][ks], qf[ks], s[kt]);
        }
        // keys outside [lo, hi] (relative to kv0 + 4h): past N, after the
        // row (causal), before its band (window)
        const bool need_mask = (CAUSAL && kv0 + BC - 1 > q0) || (kv0 + BC > N) || (WINDOW && kv0 < q0 + 32 - W);
        if (need_mask) {
            const int hi = (CAUSAL ? min(qrow, N - 1) : N - 1) - kv0 - 4 * h;
            const int lo = (WINDOW ? qrow - W + 1 : 0) - kv0 - 4 * h;
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int koff = kt * 32 + (r >> 2) * 8 + (r & 3);
                    s[kt][r] = (koff > hi || koff < lo) ? -__builtin_huge_valf() : s[kt][r];
                }
        }
        float mx = s[0][0];
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kt][r]);
        m = max_across_halves(mx) * c;
        const float mref = (m == -__builtin_huge_valf()) ? 0.0f : m;
        const int g16 = lane >> 4, j16 = lane & 15;
        const int tr_row = (g16 >> 1) * 4 + (j16 >> 2);
        const int tr_col = (g16 & 1) * 16 + (j16 & 3) * 4;
        const e16* Vs = reinterpret_cast<const e16*>(vlds);
#pragma unroll
        for (int u = 0; u < PVS; ++u) {
            const int kt = u >> 1;
            e16x2 pr[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = (u & 1) * 8 + 2 * e;
                const float a0 = fast_exp2(fmaf(s[kt][r], c, -mref));
                const float a1 = fast_exp2(fmaf(s[kt][r + 1], c, -mref));
                l += a0 + a1;
                pr[e] = cvt2<DT>(a0, a1);
            }
            const e16x8 pb = cat8(pr[0], pr[1], pr[2], pr[3]);
            const e16* vp = Vs + (u * 16 + tr_row) * VP + tr_col;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
                oacc[dt] = mfma32<DT>(join8(lds_read_tr4(vp + dt * 32), lds_read_tr4(vp + 8 * VP + dt * 32)),
                                      pb, oacc[dt]);
        }
        l = sum_across_halves(l);
    }

    // Partial results to LDS: O_w^T as [dim][query] rows of OP floats (the
    // V tiles are dead once every wave is past this barrier), m_w and l_w per
    // query.
    __syncthreads();
    float* ow = reinterpret_cast<float*>(smem + wave * AREA);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) ow[(dt * 32 + (r >> 2) * 8 + 4 * h + (r & 3)) * OP + l32] = oacc[dt][r];
    float* mw = reinterpret_cast<float*>(smem + NW * AREA);
    float* lw = mw + NW * 32;
    if (h == 0) {
        mw[wave * 32 + l32] = m;
        lw[wave * 32 + l32] = l;
    }
    __syncthreads();

    // Combine: thread (query q, dim group g) produces dims g*DPT .. +DPT-1.
    constexpr int GROUPS = T / 32;
    constexpr int DPT = (D + GROUPS - 1) / GROUPS;
    const int q = tid & 31, g = tid >> 5;
    float M = -__builtin_huge_valf();
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, mw[w * 32 + q]);
    float a[NW];
    float L = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const float mv = mw[w * 32 + q];
        a[w] = mv == -__builtin_huge_valf() ? 0.0f : fast_exp2(mv - M);
        L += a[w] * lw[w * 32 + q];
    }
    const int row = q0 + q;
    if (row < N) {
        const float inv = L > 0.0f ? 1.0f / L : 0.0f;
        e16* orow = static_cast<e16*>(p.o) + b * p.so.b + hq * p.so.h + row * p.so.n;
#pragma unroll
        for (int j = 0; j < DPT; ++j) {
            const int dim = g * DPT + j;
            if (dim < D) {
                float acc = 0.0f;
#pragma unroll
                for (int w = 0; w < NW; ++w)
                    acc = fmaf(a[w], reinterpret_cast<const float*>(smem + w * AREA)[dim * OP + q], acc);
                orow[dim] = cvt2<DT>(acc * inv, 0.0f)[0];
            }
        }
        if (g == 0) p.lse[(size_t)bh * N + row] = L > 0.0f ? (M + log2f(L)) * kLn2 : -__builtin_huge_valf();
    }
}

template <int DT, int D, int MASK>
static hipError_t launch_fwd_split(const FwdParams& p, const FwdPlan& plan, hipStream_t stream) {
    const dim3 grid((unsigned)plan.workgroups), block((unsigned)plan.threads);
    if constexpr (D <= kSplitMaxD) {
        switch (plan.key_splits) {
            case 2: hipLaunchKernelGGL((fwd_split_kernel<DT, D, MASK, 2>), grid, block, 0, stream, p); break;
            case 4: hipLaunchKernelGGL((fwd_split_kernel<DT, D, MASK, 4>), grid, block, 0, stream, p); break;
            case 8: hipLaunchKernelGGL((fwd_split_kernel<DT, D, MASK, 8>), grid, block, 0, stream, p); break;
            default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    return hipErrorInvalidValue;
}

template <int DT, int D, int MASK, bool DROP>
static hipError_t launch_fwd_dmd(const FwdParams& p, const FwdPlan& plan, hipStream_t stream) {
    const dim3 grid((unsigned)plan.workgroups), block((unsigned)plan.threads);
    if constexpr (D <= 128) {
        if (plan.key_groups == 2) {
            if constexpr (DROP) {
                return hipErrorInvalidValue;  // the plan never pairs them
            } else {
                if (plan.waves != 4) return hipErrorInvalidValue;
                hipLaunchKernelGGL((fwd_kernel<DT, D, MASK, 4, false, 2>), grid, block, 0, stream, p);
                return hipGetLastError();
            }
        }
        if (plan.waves == 4 && plan.m16) {
            if constexpr (kProducts16<D> && !DROP) {
                hipLaunchKernelGGL((fwd_m16_kernel<DT, D, MASK, 4>), grid, block, 0, stream, p);
                return hipGetLastError();
            } else {
                return hipErrorInvalidValue;
            }
        }
        if (plan.waves == 8) {
            hipLaunchKernelGGL((fwd_kernel<DT, D, MASK, 8, DROP, 1>), grid, block, 0, stream, p);
            return hipGetLastError();
        }
    }
    if (plan.key_groups != 1) return hipErrorInvalidValue;
    hipLaunchKernelGGL((fwd_kernel<DT, D, MASK, 4, DROP, 1>), grid, block, 0, stream, p);
    return hipGetLastError();
}

template <int DT, int D, int MASK>
static hipError_t launch_fwd_dm(const FwdParams& p, const FwdPlan& plan, hipStream_t stream) {
    if (plan.key_splits > 1) {
        if (p.drop.thr != 0) return hipErrorInvalidValue;  // the plan never pairs them
        return launch_fwd_split<DT, D, MASK>(p, plan, stream);
    }
    return p.drop.thr != 0 ? launch_fwd_dmd<DT, D, MASK, true>(p, plan, stream)
                           : launch_fwd_dmd<DT, D, MASK, false>(p, plan, stream);
}

template <int DT, int D>
static hipError_t launch_fwd_d(const FwdParams& p, int mask, const FwdPlan& plan, hipStream_t stream) {
    switch (mask) {
        case kMaskNone: return launch_fwd_dm<DT, D, kMaskNone>(p, plan, stream);
        case kMaskCausal: return launch_fwd_dm<DT, D, kMaskCausal>(p, plan, stream);
        case kMaskWindow: return launch_fwd_dm<DT, D, kMaskWindow>(p, plan, stream);
        default: return hipErrorInvalidValue;
    }
}

template <int DT>
static hipError_t launch_fwd_t(const FwdParams& p, int d, int mask, const FwdPlan& plan,
                               hipStream_t stream) {
    switch (d) {
#define ATTN_FWD_CASE(D_) \
        case D_: return launch_fwd_d<DT, D_>(p, mask, plan, stream);
        ATTN_FOR_EACH_HEAD_DIM(ATTN_FWD_CASE)
#undef ATTN_FWD_CASE
        default: return hipErrorInvalidValue;
    }
}

// Tile plan. 8 waves (256 rows) per workgroup share one K/V pipeline, which
// halves global-load issue and LDS stores per row; used while that still
// gives every CU a workgroup. Shorter sequences use 4 waves (twice the
// workgroups); d > 128 always uses 4. d = 128 without dropout runs those
// large grids on the 16x16x32 kernel with 4 waves instead: its 254 VGPRs
// leave room for 8 waves per CU, so two 128-row workgroups share a CU and
// each one's prologue and epilogue overlap the other's step loop (1-1.5 %
// faster than one 256-row workgroup per CU on the causal 4096- and
// 16384-key shapes, the same on the grouped 8192-key one).
template <int D>
static void plan_d(int B, int Hq, int N, bool causal, bool dropout, FwdPlan* plan) {
    const long long wg256 = (long long)((N + 255) / 256) * B * Hq;
    const long long wg128 = (long long)((N + 127) / 128) * B * Hq;
    plan->key_splits = 1;
    plan->key_groups = 1;
    plan->m16 = 0;
    // Short sequences whose grid of 128-row workgroups would leave CUs idle:
    // the key-split kernel (one workgroup per 32 rows, waves over the keys).
    if (D <= kSplitMaxD && !dropout && N <= kSplitMaxKeys && wg128 < kSplitMaxGrid) {
        const int nkb = (N + 63) / 64;
        const int nw = nkb <= 2 ? 2 : nkb <= 4 ? 4 : 8;
        plan->rows_per_wave = 32;
        plan->waves = nw;
        plan->key_splits = nw;
        plan->block_q = 32;
        plan->block_kv = 64;
        plan->threads = nw * 64;
        plan->workgroups = (long long)((N + 31) / 32) * B * Hq;
        plan->lds_bytes = SplitTile<D <= kSplitMaxD ? D : 32>::lds_bytes(nw);
        return;
    }
    const int BC = FwdTile<D>::BLOCK_KV;
    // Key groups on grids too small to hide the longest query block's key
    // loop (key_groups_pay).
    if (D <= 128 && !dropout) {
        if (key_groups_pay(B, Hq, N, causal)) {
            plan->rows_per_wave = 32;
            plan->waves = 4;
            plan->key_groups = 2;
            plan->block_q = 64;
            plan->block_kv = BC;
            plan->threads = 256;
            plan->workgroups = (long long)((N + 63) / 64) * B * Hq;
            plan->lds_bytes = 2 * 2 * BC * (k_pitch(D) + v_pitch(D)) * 2;
            return;
        }
    }
    int waves = (D <= 128 && wg256 >= (causal ? 512 : 256)) ? 8 : 4;
    if (kProducts16<D> && !dropout && waves == 8) {
        waves = 4;
        plan->m16 = 1;
    }
    const int BQ = waves * 32;
    plan->rows_per_wave = 32;
    plan->waves = waves;
    plan->block_q = BQ;
    plan->block_kv = BC;
    plan->threads = waves * 64;
    plan->workgroups = (long long)((N + BQ - 1) / BQ) * B * Hq;
    plan->lds_bytes = 2 * BC * (plan->m16 ? 2 * m16_pitch(D) : k_pitch(D) + v_pitch(D)) * 2;
}

bool fwd_plan(int B, int Hq, int N, int d, bool causal, bool dropout, FwdPlan* plan) {
    switch (d) {
#define ATTN_PLAN_CASE(D_) \
        case D_: plan_d<D_>(B, Hq, N, causal, dropout, plan); return true;
        ATTN_FOR_EACH_HEAD_DIM(ATTN_PLAN_CASE)
#undef ATTN_PLAN_CASE
        default: return false;
    }
}

hipError_t launch_fwd(const FwdParams& p, int dtype, int d, int mask, const FwdPlan& plan,
                      hipStream_t stream) {
    switch (dtype) {
        case kBF16: return launch_fwd_t<kBF16>(p, d, mask, plan, stream);
        case kFP16: return launch_fwd_t<kFP16>(p, d, mask, plan, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace attn
