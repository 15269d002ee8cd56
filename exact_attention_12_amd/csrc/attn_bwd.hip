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

#include "attn_device.h"
#include "attn_kernels.h"

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

// Loads `rows` rows of a [N, D] bf16 head starting at row r0 into registers
// (16-byte chunks, zero beyond N) and stores them to an LDS tile.
template <int D, int ROWS, int T>
struct TileIO {
    static constexpr int CPR = D / 8;
    static constexpr int CHUNKS = ROWS * CPR;
    static constexpr int NCH = (CHUNKS + T - 1) / T;
    uint4 r[NCH];

    __device__ __forceinline__ void load(const bf16* head, int r0, int N, int tid) {
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            const int c = tid + i * T;
            if (CHUNKS % T == 0 || c < CHUNKS) {
                const int row = c / CPR;
                const int col = c - row * CPR;
                r[i] = (r0 + row < N)
                           ? *reinterpret_cast<const uint4*>(head + (size_t)(r0 + row) * D + col * 8)
                           : zero4();
            }
        }
    }
    __device__ __forceinline__ void store(bf16* tile, int pitch, int tid) const {
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            const int c = tid + i * T;
            if (CHUNKS % T == 0 || c < CHUNKS) {
                const int row = c / CPR;
                const int col = c - row * CPR;
                *reinterpret_cast<uint4*>(tile + row * pitch + col * 8) = r[i];
            }
        }
    }
};

// Zero the columns D .. round_up(D, 32) of `rows` rows of an LDS tile (read
// by the transposing read of the last 32-wide tile, never written by loads).
template <int D>
__device__ __forceinline__ void zero_pad_cols(bf16* tile, int rows, int pitch, int tid, int T) {
    constexpr int PADC = ((D + 31) / 32) * 32 - D;
    if constexpr (PADC > 0) {
        for (int i = tid; i < rows * PADC; i += T) tile[(i / PADC) * pitch + D + i % PADC] = (bf16)0.0f;
    }
}

// ---------------------------------------------------------------- dK, dV

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1)
void bwd_dkdv_kernel(BwdParams p) {
    constexpr int NW = 4;
    constexpr int T = NW * 64;
    constexpr int BK = NW * 32;        // keys per workgroup
    constexpr int BQ = (D <= 128) ? 64 : 32;  // queries per step
    constexpr int NQT = BQ / 32;
    constexpr int PVS = BQ / 16;
    constexpr int KS = D / 16;
    constexpr int NDT = (D + 31) / 32;
    constexpr int QP = v_pitch(D);     // Q, dO tiles: row reads and transposing reads
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
        zero_pad_cols<D>(qtile(bufi), BQ, QP, tid, T);
        zero_pad_cols<D>(dotile(bufi), BQ, QP, tid, T);
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
    const int nq_iter = nqb - qb_start;
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
        qio.store(qtile(bufi), QP, tid);
        doio.store(dotile(bufi), QP, tid);
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
                const bf16* qp = Qs + (qt * 32 + l32) * QP + h * 8;
                const bf16* gp = dOs + (qt * 32 + l32) * QP + h * 8;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    s[qt] = mfma32(lds_read8(qp + ks * 16), kf[ks], s[qt]);
                    dp[qt] = mfma32(lds_read8(gp + ks * 16), vf[ks], dp[qt]);
                }
            }
            // P = exp2(c*S - LSE2) and dS = P (dP - D), packed to bf16 in the
            // B-operand order of the dV/dK products. Under the causal mask the
            // query of register r (local offset qoff(r) + 4h) is masked for
            // this lane's key when key - q0 - 4h > qoff(r): one compare with a
            // constant per element.
            bf16x8 pb[PVS], dsb[PVS];
            {
                const int kq = key - q0 - 4 * h;
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
                const bf16* gp = dOs + (u * 16 + tr_row) * QP + tr_col;
                const bf16* qp = Qs + (u * 16 + tr_row) * QP + tr_col;
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) {
                    ado[dt] = join8(lds_read_tr4(gp + dt * 32), lds_read_tr4(gp + 8 * QP + dt * 32));
                    aq[dt] = join8(lds_read_tr4(qp + dt * 32), lds_read_tr4(qp + 8 * QP + dt * 32));
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

// ---------------------------------------------------------------- dQ

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, (D <= 128 ? 2 : 1))
void bwd_dq_kernel(BwdParams p) {
    constexpr int NW = 4;
    constexpr int T = NW * 64;
    constexpr int BQ = NW * 32;
    constexpr int BC = (D <= 128) ? 64 : 32;
    constexpr int KS = D / 16;
    constexpr int NDT = (D + 31) / 32;
    constexpr int NKT = BC / 32;
    constexpr int PVS = BC / 16;
    constexpr int KP = v_pitch(D);     // K tile: row reads and transposing reads
    constexpr int VP = k_pitch(D);     // V tile: row reads only
    constexpr int BUF = BC * (KP + VP);

    __shared__ __attribute__((aligned(16))) bf16 smem[2 * BUF];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l32 = lane & 31;
    const int h = lane >> 5;
    const int N = p.N;

    const int BH = p.B * p.Hq;
    const int nqb = (N + BQ - 1) / BQ;
    const int bid = blockIdx.x;
    const int bh = bid % BH;
    const int qb = CAUSAL ? (nqb - 1 - bid / BH) : (bid / BH);
    const int b = bh / p.Hq;
    const int hq = bh - b * p.Hq;
    const int hkv = hq / p.G;
    const size_t q_off = (size_t)bh * N;
    const size_t kv_off = ((size_t)b * p.Hkv + hkv) * N * D;
    const bf16* Kh = static_cast<const bf16*>(p.k) + kv_off;
    const bf16* Vh = static_cast<const bf16*>(p.v) + kv_off;

    const int q0 = qb * BQ;
    const int qw0 = q0 + wave * 32;
    const int qrow = qw0 + l32;

    for (int bufi = 0; bufi < 2; ++bufi) zero_pad_cols<D>(smem + bufi * BUF, BC, KP, tid, T);

    bf16x8 qf[KS], gf[KS];
    float lse2 = __builtin_huge_valf(), del = 0.0f;
    if (qrow < N) {
        const bf16* qp = static_cast<const bf16*>(p.q) + (q_off + qrow) * D + h * 8;
        const bf16* gp = static_cast<const bf16*>(p.dout) + (q_off + qrow) * D + h * 8;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            qf[ks] = *reinterpret_cast<const bf16x8*>(qp + ks * 16);
            gf[ks] = *reinterpret_cast<const bf16x8*>(gp + ks * 16);
        }
        lse2 = p.lse[q_off + qrow] * kLog2e;
        del = p.delta[q_off + qrow];
    } else {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) { qf[ks] = bf16x8{}; gf[ks] = bf16x8{}; }
    }

    const int nkb = (N + BC - 1) / BC;
    const int kb_end = CAUSAL ? min(nkb, (q0 + BQ - 1) / BC + 1) : nkb;

    TileIO<D, BC, T> kio, vio;
    kio.load(Kh, 0, N, tid);
    vio.load(Vh, 0, N, tid);
    kio.store(smem, KP, tid);
    vio.store(smem + BC * KP, VP, tid);
    __syncthreads();

    f32x16 dqacc[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) dqacc[dt] = f32x16{};
    const float c = p.c;
    const int g16 = lane >> 4;
    const int j16 = lane & 15;
    const int tr_row = (g16 >> 1) * 4 + (j16 >> 2);
    const int tr_col = (g16 & 1) * 16 + (j16 & 3) * 4;

    for (int kb = 0; kb < kb_end; ++kb) {
        const int bufi = kb & 1;
        const bool has_next = kb + 1 < kb_end;
        if (has_next) {
            kio.load(Kh, (kb + 1) * BC, N, tid);
            vio.load(Vh, (kb + 1) * BC, N, tid);
        }
        const int kv0 = kb * BC;
        const bf16* Ks = smem + bufi * BUF;
        const bf16* Vs = Ks + BC * KP;
        // Branch-free step: blocks past a wave's last query are masked to zero.
        {
            f32x16 s[NKT], dp[NKT];
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt) {
                s[kt] = f32x16{};
                dp[kt] = f32x16{};
                const bf16* kp = Ks + (kt * 32 + l32) * KP + h * 8;
                const bf16* vp = Vs + (kt * 32 + l32) * VP + h * 8;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    s[kt] = mfma32(lds_read8(kp + ks * 16), qf[ks], s[kt]);
                    dp[kt] = mfma32(lds_read8(vp + ks * 16), gf[ks], dp[kt]);
                }
            }
            // dS^T = P^T (dP^T - D) with P^T = exp2(c*S^T - LSE2), packed to bf16
            // in the B-operand order of dQ^T += K^T dS^T. Key kv0 + koff(r) + 4h
            // is masked when it is >= N or (causal) > qrow: one compare with a
            // constant per element, skipped when the block needs no mask.
            bf16x8 dsb[PVS];
            {
                const bool MASKED = CAUSAL || (kv0 + BC > N);
                const int lim = (CAUSAL ? min(qrow, N - 1) : N - 1) - kv0 - 4 * h;
#pragma unroll
                for (int u = 0; u < PVS; ++u) {
                    const int kt = u >> 1;
                    const int r0 = (u & 1) * 8;
                    bf16x2 dd[4];
#pragma unroll
                    for (int e2 = 0; e2 < 4; ++e2) {
                        float dv[2];
#pragma unroll
                        for (int w = 0; w < 2; ++w) {
                            const int r = r0 + 2 * e2 + w;
                            const int koff = kt * 32 + (r >> 2) * 8 + (r & 3);
                            float pe = fast_exp2(fmaf(s[kt][r], c, -lse2));
                            if (MASKED && koff > lim) pe = 0.0f;
                            dv[w] = pe * (dp[kt][r] - del);
                        }
                        dd[e2] = to_bf16x2(dv[0], dv[1]);
                    }
                    dsb[u] = cat8(dd[0], dd[1], dd[2], dd[3]);
                }
            }
#pragma unroll
            for (int u = 0; u < PVS; ++u) {
                const bf16* kp = Ks + (u * 16 + tr_row) * KP + tr_col;
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) {
                    const bf16x8 a = join8(lds_read_tr4(kp + dt * 32), lds_read_tr4(kp + 8 * KP + dt * 32));
                    dqacc[dt] = mfma32(a, dsb[u], dqacc[dt]);
                }
            }
        }
        if (has_next) {
            kio.store(smem + (bufi ^ 1) * BUF, KP, tid);
            vio.store(smem + (bufi ^ 1) * BUF + BC * KP, VP, tid);
        }
        __syncthreads();
    }

    if (qrow < N) {
        bf16* dqrow = static_cast<bf16*>(p.dq) + (q_off + qrow) * D;
        const float sc = p.scale;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int d = dt * 32 + g4 * 8 + h * 4;
                if (d < D)
                    store_bf16x4(dqrow + d, dqacc[dt][g4 * 4 + 0] * sc, dqacc[dt][g4 * 4 + 1] * sc,
                                 dqacc[dt][g4 * 4 + 2] * sc, dqacc[dt][g4 * 4 + 3] * sc);
            }
    }
}

// ---------------------------------------------------------------- launch

template <int D, bool CAUSAL>
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
        hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL>), dim3((unsigned)(nkb * p.B * p.Hkv)), dim3(256),
                           0, stream, p);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (passes & kBwdDq) {
        const long long nqb = (p.N + 127) / 128;
        hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL>), dim3((unsigned)(nqb * p.B * p.Hq)), dim3(256), 0,
                           stream, p);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <int D>
static hipError_t launch_bwd_d(const BwdParams& p, bool causal, int passes, hipStream_t stream) {
    return causal ? launch_bwd_dc<D, true>(p, passes, stream) : launch_bwd_dc<D, false>(p, passes, stream);
}

hipError_t launch_bwd(const BwdParams& p, int d, bool causal, int passes, hipStream_t stream) {
    switch (d) {
        case 64: return launch_bwd_d<64>(p, causal, passes, stream);
        case 80: return launch_bwd_d<80>(p, causal, passes, stream);
        case 128: return launch_bwd_d<128>(p, causal, passes, stream);
        case 256: return launch_bwd_d<256>(p, causal, passes, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace attn
