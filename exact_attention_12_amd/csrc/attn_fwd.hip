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
#include <type_traits>

#include "attn_device.h"
#include "attn_kernels.h"

namespace attn {

template <int DT, int D, int MASK, int NW, bool DROP>
__global__ __launch_bounds__(NW * 64, (D <= 128 ? 2 : 1))
void fwd_kernel(FwdParams p) {
    constexpr int T = NW * 64;
    constexpr int BQ = NW * 32;
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

    __shared__ __attribute__((aligned(16))) e16 smem[2 * BUF];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches and buffer resources
    const int l32 = lane & 31;
    const int h = lane >> 5;
    const int N = p.N;

    // Workgroup -> (query block, batch*head). Under the causal mask the
    // latest (heaviest) query blocks come first.
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
    const int qrow = qw0 + l32;

    // Columns d .. padded width of the V tiles are read by the last O^T tile
    // and must be zero; the loaders never write them.
    if constexpr (NDT * 32 > D) {
        constexpr int PADC = NDT * 32 - D;
        for (int i = tid; i < 2 * BC * PADC; i += T) {
            const int row = i / PADC;
            const int col = D + i % PADC;
            const int bufi = row / BC;
            smem[bufi * BUF + BC * KP + (row % BC) * VP + col] = (e16)0;
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
        e16* Ks = smem + bufi * BUF;
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
    constexpr int LPWK = (NLK + NW - 1) / NW, LPWV = (NLV + NW - 1) / NW;
    static_assert(!DIRECT || (BC * CKK % 64 == 0 && BC * CKV % 64 == 0), "tile must be whole loads");
    uint32_t offk[DIRECT ? LPWK : 1], offv[DIRECT ? LPWV : 1];
    if constexpr (DIRECT) {
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
    auto issue_tile = [&](int kv0, int bufi) {
        const uint32_t sk2 = (uint32_t)skn * 2u, sv2 = (uint32_t)svn * 2u;
        const auto rk = buf_rsrc(Kh + (long long)kv0 * skn, (uint32_t)(N - kv0 - 1) * sk2 + D * 2);
        const auto rv = buf_rsrc(Vh + (long long)kv0 * svn, (uint32_t)(N - kv0 - 1) * sv2 + D * 2);
        char* kb_lds = reinterpret_cast<char*>(smem + bufi * BUF);
        char* vb_lds = kb_lds + BC * KP * 2;
#pragma unroll
        for (int i = 0; i < LPWK; ++i) {
            const int j = wave + i * NW;
            if (NLK % NW == 0 || j < NLK) buf_load16_to_lds(rk, kb_lds + j * 1024, offk[i]);
        }
#pragma unroll
        for (int i = 0; i < LPWV; ++i) {
            const int j = wave + i * NW;
            if (NLV % NW == 0 || j < NLV) buf_load16_to_lds(rv, vb_lds + j * 1024, offv[i]);
        }
    };

    if constexpr (DIRECT) {
        issue_tile(kb_begin * BC, kb_begin & 1);
        __builtin_amdgcn_s_waitcnt(0);
    } else {
        load_tile(kb_begin * BC);
        store_tile(kb_begin & 1);
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

    auto run_step = [&](int kb, auto masked_tag) {
        constexpr bool MASKED = decltype(masked_tag)::value;
        const int bufi = kb & 1;
        // The last step reloads its own tile into the idle buffer (never
        // read again), so the loads and stores need no branch.
        if constexpr (DIRECT)
            issue_tile(min(kb + 1, kb_end - 1) * BC, bufi ^ 1);
        else
            load_tile(min(kb + 1, kb_end - 1) * BC);

        const int kv0 = kb * BC;
        const e16* Ks = smem + bufi * BUF;
        const e16* Vs = Ks + BC * KP;
        const bool active = !MASKED || !CAUSAL || (kv0 <= qw0 + 31 && (!WINDOW || kv0 + BC - 1 >= qw0 - W + 1));
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
    // Key blocks [ku_begin, ku_end) need neither the per-wave skip nor a
    // mask: every key is at or before the workgroup's first query (kv0 + BC
    // - 1 <= q0), inside its last query's band (kv0 >= q0 + BQ - W) and
    // before N. They run in a copy of the step without those tests.
    int ku_begin = kb_begin, ku_end = min(kb_end, N / BC);
    if (CAUSAL) ku_end = min(ku_end, (q0 + 1) / BC);
    if (WINDOW) {
        const int t = q0 + BQ - W;
        ku_begin = min(kb_end, max(kb_begin, t > 0 ? (t + BC - 1) / BC : 0));
    }
    ku_end = max(ku_end, ku_begin);
    int kb = kb_begin;
    for (; kb < ku_begin; ++kb) run_step(kb, std::true_type{});
    for (; kb < ku_end; ++kb) run_step(kb, std::false_type{});
    for (; kb < kb_end; ++kb) run_step(kb, std::true_type{});

    // Epilogue: combine the two half-row sums, normalise, store O and LSE.
    const float lt = sum_across_halves(l);
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

template <int DT, int D, int MASK, bool DROP>
static hipError_t launch_fwd_dmd(const FwdParams& p, const FwdPlan& plan, hipStream_t stream) {
    const dim3 grid((unsigned)plan.workgroups), block((unsigned)plan.threads);
    if constexpr (D <= 128) {
        if (plan.waves == 8) {
            hipLaunchKernelGGL((fwd_kernel<DT, D, MASK, 8, DROP>), grid, block, 0, stream, p);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((fwd_kernel<DT, D, MASK, 4, DROP>), grid, block, 0, stream, p);
    return hipGetLastError();
}

template <int DT, int D, int MASK>
static hipError_t launch_fwd_dm(const FwdParams& p, const FwdPlan& plan, hipStream_t stream) {
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
// workgroups); d > 128 always uses 4.
template <int D>
static void plan_d(int B, int Hq, int N, bool causal, FwdPlan* plan) {
    const long long wg256 = (long long)((N + 255) / 256) * B * Hq;
    const int waves = (D <= 128 && wg256 >= (causal ? 512 : 256)) ? 8 : 4;
    const int BQ = waves * 32;
    const int BC = FwdTile<D>::BLOCK_KV;
    plan->rows_per_wave = 32;
    plan->waves = waves;
    plan->block_q = BQ;
    plan->block_kv = BC;
    plan->threads = waves * 64;
    plan->workgroups = (long long)((N + BQ - 1) / BQ) * B * Hq;
    plan->lds_bytes = 2 * BC * (k_pitch(D) + v_pitch(D)) * 2;
}

bool fwd_plan(int B, int Hq, int N, int d, bool causal, FwdPlan* plan) {
    switch (d) {
#define ATTN_PLAN_CASE(D_) \
        case D_: plan_d<D_>(B, Hq, N, causal, plan); return true;
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
