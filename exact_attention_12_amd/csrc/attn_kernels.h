// attn_kernels.h - host-side view of the kernels: parameter blocks, tile
// plans and launchers. Shared by the C-ABI layer and the kernel sources.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "attn_device.h"

namespace attn {

// Head dimensions with a kernel instantiation (multiples of 16: one MFMA
// contraction step is 16 wide).
#define ATTN_FOR_EACH_HEAD_DIM(X) X(32) X(64) X(80) X(96) X(128) X(192) X(256)

// Forward tile plan per head dimension: 32 query rows per wave, 4 or 8 waves
// per workgroup (chosen per shape), BLOCK_KV keys per inner step. The
// keys-per-step choice keeps two waves per SIMD (LDS double buffer +
// registers) for d <= 128; d > 128 halves it to keep the accumulator and Q
// operand in registers.
template <int D> struct FwdTile {
    static_assert(D % 16 == 0 && D >= 32 && D <= 256, "unsupported head dimension");
    static constexpr int BLOCK_KV = D <= 128 ? 64 : 32;
};

// Row pitches (in 16-bit elements) of the LDS tiles. gfx950's LDS serves
// 64 banks x 4 bytes, i.e. 256 bytes per cycle; measured on the part:
//  * 16-byte row reads (lane i reads row i, same column; the S = K Q^T and
//    dP operands) reach their conflict floor when the pitch is an odd
//    multiple of 16 bytes modulo 256: pitch d + 8 elements;
//  * the transposing read (each 16-lane group reads 4 rows x 32 bytes, two
//    groups per cycle) is conflict free when the pitch is 64 or 192 bytes
//    modulo 256: v_pitch;
//  * a tile read both ways uses the 64-mod-256 pitch with its 16-byte chunks
//    XOR-swizzled by bits 2..3 of the row: sw_pitch and sw_off. With that
//    pitch rows r, r+4, r+8, r+12 start on the same bank; the swizzle moves
//    them to four different 16-byte slots, so the 16 rows of a row read hit
//    every bank once (4 cycles per 16-byte read instead of 8 with a swizzle
//    by (row & 7), counted with SQ_LDS_BANK_CONFLICT), while each transposing
//    read still sees one swizzle value per 4-row group (2 cycles, no
//    conflicts). The swizzle permutes chunks inside aligned groups of 4, and
//    the pitch holds round_up(chunks, 8) chunks.
constexpr int k_pitch(int d) { return d + 8; }
constexpr int pitch_64mod256(int row_bytes) {
    return (row_bytes + (((64 - row_bytes) % 128) + 128) % 128) / 2;
}
constexpr int v_pitch(int d) { return pitch_64mod256(((d + 31) / 32) * 32 * 2); }
constexpr int sw_pitch(int d) { return pitch_64mod256(((d / 8 + 7) / 8) * 8 * 16); }
static_assert(v_pitch(64) == 96 && v_pitch(80) == 96 && v_pitch(128) == 160 && v_pitch(256) == 288, "");
static_assert(sw_pitch(64) == 96 && sw_pitch(80) == 160 && sw_pitch(128) == 160 && sw_pitch(256) == 288, "");

// Element offset of (row, col) in a swizzled tile (chunk = 8 elements).
__host__ __device__ constexpr int sw_swizzle(int row) { return (row >> 2) & 3; }
__host__ __device__ constexpr int sw_off(int row, int col, int pitch) {
    return row * pitch + (((col >> 3) ^ sw_swizzle(row)) << 3) + (col & 7);
}
// The swizzle repeats every 16 rows and stays inside 32-column groups, so
// for 0 <= c < 32: sw_off(r + 16a, c + 32b) = sw_off(r, c) + 16a*pitch + 32b.
// Kernels compute sw_off(r, c) once per lane and reach the other row and
// column blocks through immediate offsets.
constexpr bool sw_off_is_periodic(int pitch) {
    for (int r = 0; r < 16; ++r)
        for (int c = 0; c < 32; ++c)
            for (int a = 0; a < 4; ++a)
                for (int b = 0; b < 8; ++b)
                    if (sw_off(r + 16 * a, c + 32 * b, pitch) != sw_off(r, c, pitch) + 16 * a * pitch + 32 * b)
                        return false;
    return true;
}
static_assert(sw_off_is_periodic(96) && sw_off_is_periodic(160) && sw_off_is_periodic(288), "");

// Head index of a workgroup whose index has j = bid % BH as its fastest
// part. The 8 XCDs of the chip (each with its own L2) receive workgroups
// round robin, so XCD x gets the j = x mod 8; when BH is a multiple of 8 the
// heads are renumbered so that XCD x runs the contiguous heads
// x * BH/8 .. (x+1) * BH/8 - 1, i.e. whole GQA groups, whose query heads then
// read their shared K and V through one L2.
__host__ __device__ constexpr int xcd_head(int j, int BH) {
    return BH % 8 == 0 ? (j % 8) * (BH / 8) + j / 8 : j;
}

constexpr bool xcd_head_is_permutation(int BH) {
    for (int h = 0; h < BH; ++h) {
        int hits = 0;
        for (int j = 0; j < BH; ++j) hits += xcd_head(j, BH) == h;
        if (hits != 1) return false;
    }
    return true;
}
static_assert(xcd_head_is_permutation(8) && xcd_head_is_permutation(32) &&
              xcd_head_is_permutation(64) && xcd_head_is_permutation(12), "");

// Mask modes, one kernel instantiation each: none, causal (keys j <= i) and
// the causal sliding window (keys i - window < j <= i).
enum MaskKind { kMaskNone = 0, kMaskCausal = 1, kMaskWindow = 2 };

// Element strides of one [B, H, N, d] operand (d itself is contiguous):
// element (b, h, n, e) sits at base + b*b_ + h*h_ + n*n_ + e.
struct Strides {
    long long b, h, n;
};

struct FwdParams {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;    // [B, Hq, N], contiguous
    Strides sq, sk, sv, so;
    int N;
    int Hq;
    int Hkv;
    int G;        // Hq / Hkv
    int BH;       // B * Hq
    int nqb;      // query blocks per head
    int window;   // causal band width in keys (query i sees i-window < j <= i); 0 = none
    float c;      // scale * log2(e)
    DropParams drop;
};

struct BwdParams {
    const void* q;
    const void* k;
    const void* v;
    const void* o;
    const float* lse;
    const void* dout;
    void* dq;
    void* dk;
    void* dv;
    float* delta;  // [B, Hq, N] workspace: -D_i = -<dO_i, O_i>
    float* lse2;   // [B, Hq, N] workspace: LSE_i * log2(e), written with D_i
    float* part;   // [2, 2, B, Hkv, N, d] workspace: partial dK, dV (hsplit or qsplit 2 only)
    int dkdv;      // dK/dV kernel (dkdv_wide_split's numbering; 1 and 2 only at d = 128)
    int hsplit;    // workgroups per 256-key block of the 64-key dK/dV kernel (2 iff dkdv == 2)
    int qsplit;    // workgroups per 128-key block of the 32-key dK/dV kernel, each over a part of its queries
    Strides sq, sk, sv, so, sdo, sdq, sdk, sdv;
    int N;
    int Hq;
    int Hkv;
    int G;
    int B;
    int window;    // causal band width in keys; 0 = none
    float scale;
    float c;       // scale * log2(e)
    DropParams drop;
};

// dK/dV kernel for a shape: 0 = 32 keys per wave; 1 = 64 keys per wave (d =
// 128, at least 512 blocks of 256 keys: two rounds of one workgroup per CU);
// 2 = 64 keys per wave with the query heads of each group split over two
// workgroups, which write fp32 partial sums that a second kernel adds (256 to
// 511 blocks and an even group size: one round would leave the CUs with the
// light causal blocks idle).
inline int dkdv_wide_split(int B, int Hq, int Hkv, int N, int d) {
    if (d != 128 || Hkv <= 0) return 0;
    const long long n4 = (long long)((N + 255) / 256) * B * Hkv;
    if (n4 >= 512) return 1;
    if ((Hq / Hkv) % 2 == 0 && 2 * n4 >= 512) return 2;
    return 0;
}

// Query split of the 32-key dK/dV kernel (d <= 128, where neither 64-key
// form is used): when its grid of 128-key blocks holds at most one workgroup
// per CU (causal; half that unmasked, where every block has the same work),
// the heaviest block's query loop decides the time. Two workgroups per block
// then each take half of its query blocks and write fp32 partial dK, dV,
// which a second kernel adds. 1 or 2.
inline int dkdv_query_split(int B, int Hq, int Hkv, int N, int d, bool causal) {
    if (d > 128 || Hkv <= 0 || N < 512 || dkdv_wide_split(B, Hq, Hkv, N, d) != 0) return 1;
    const long long wgs = (long long)((N + 127) / 128) * B * Hkv;
    return wgs <= (causal ? 256 : 128) ? 2 : 1;
}

struct FwdPlan {
    int rows_per_wave;  // query rows per wave (32)
    int waves;          // waves per workgroup
    int block_q;
    int block_kv;
    int threads;
    long long workgroups;
    int lds_bytes;
    int key_splits;     // > 1: the key-split kernel, its waves each take 64 keys of one 32-row tile
    int key_groups;     // 2: the step-loop kernel with its 4 waves in two groups over one 64-row block's keys
    int m16;            // 1: the 16x16x32 step loop (fwd_m16_kernel) on a 4-wave plan
};

// SIMDs of the part (256 compute units x 4), for the load estimate below.
constexpr int kSimds = 1024;

// Whether a pass that walks each query block's 64-key tiles one after the
// other should split every block's tiles over two groups of waves (the
// forward and the dQ pass): when the longest block has at least about twice
// as many tiles (nkb) as the average SIMD has wave steps (32-row tiles times
// their mean key tiles over the chip's SIMDs), the longest blocks decide the
// time. Measured on the forward: 1.06-1.41x at ratios of 1.9 to 8, 0.7-0.95x
// at ratios of 1 to 1.9.
inline bool key_groups_pay(int B, int Hq, int N, bool causal) {
    const int nkb = (N + 63) / 64;
    const double tiles32 = (double)((N + 31) / 32) * B * Hq;
    const double mean_kb = causal ? (nkb + 1) / 2.0 : (double)nkb;
    return nkb >= 4 && nkb >= 1.9 * tiles32 * mean_kb / kSimds;
}

// Key-split forward for short sequences: head dims up to kSplitMaxD, at most
// kSplitMaxKeys keys (one 64-key tile per wave, 8 waves), used when the
// 128-row grid would have fewer than kSplitMaxGrid workgroups.
constexpr int kSplitMaxD = 96;
constexpr int kSplitMaxKeys = 512;
constexpr long long kSplitMaxGrid = 256;

bool fwd_plan(int B, int Hq, int N, int d, bool causal, bool dropout, FwdPlan* plan);
// Query block of rank t (0 = first dispatched) among nqb blocks of a head.
// Under a causal mask late blocks carry the most work. When a CU holds two
// workgroups at once and the whole grid is resident (`paired`), the second
// half of the ranks runs light blocks first, so that the CU that takes rank t
// in the first pass and rank t + half in the second gets a heavy and a light
// block; otherwise the heaviest blocks go first.
__device__ __forceinline__ int causal_block(int t, int nqb, bool paired, bool causal) {
    if (!causal) return t;
    if (!paired) return nqb - 1 - t;
    const int half = (nqb + 1) / 2;
    return t < half ? nqb - 1 - t : t - half;
}


// Decoding against a key/value cache: Nq new queries per sequence, at
// positions L_b - Nq .. L_b - 1 of a cache holding L_b valid rows (of Nk).
// The R = G * Nq query rows of one KV-head group are processed together in
// 32-row tiles; the cache is cut into S splits of LC keys, each split's
// partial (normalised O and log2-domain LSE) goes to the workspace, and a
// second kernel merges the splits. With S == 1 the first kernel writes the
// result directly.
struct DecParams {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;          // [B, Hq, Nq], contiguous
    const int* kv_lens;  // [B] valid cache rows per sequence, or NULL (= Nk)
    float* part_o;       // [B * Hkv * R, S, d] fp32
    float* part_lse;     // [B * Hkv * R, S] fp32, log2 domain
    Strides sq, sk, sv, so;
    int B, Hq, Hkv, G, Nq, Nk;
    int R;       // G * Nq rows per KV-head group
    int RT;      // 32-row tiles per group
    int S;       // key splits
    int LC;      // keys per split (multiple of 32)
    int window;  // sliding window W, 0 = none
    float c;     // scale * log2(e)
};

struct DecPlan {
    int R, RT, S, LC;
    long long workgroups;
    size_t workspace_bytes;
};

bool decode_plan(int B, int Hkv, int G, int Nq, int Nk, int d, DecPlan* plan);
hipError_t launch_decode(const DecParams& p, int dtype, int d, int mask, hipStream_t stream);

// Launchers return the hipError_t of the launch.
// dtype: 0 = bf16, 1 = fp16 (the kernels' DType).
hipError_t launch_fwd(const FwdParams& p, int dtype, int d, int mask, const FwdPlan& plan,
                      hipStream_t stream);
// Backward passes: bit 0 = row-term preprocess, bit 1 = dK/dV, bit 2 = dQ.
enum BwdPass { kBwdPre = 1, kBwdDkDv = 2, kBwdDq = 4, kBwdAll = 7 };
hipError_t launch_bwd(const BwdParams& p, int dtype, int d, int mask, int passes,
                      hipStream_t stream);
hipError_t launch_bwd_dq(const BwdParams& p, int dtype, int d, int mask, hipStream_t stream);

}  // namespace attn
