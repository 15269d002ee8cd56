// attn_kernels.h - host-side view of the kernels: parameter blocks, tile
// plans and launchers. Shared by the C-ABI layer and the kernel sources.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace attn {

// Forward tile plan per head dimension: 4 waves, 32 query rows per wave,
// BLOCK_KV keys per inner step. The keys-per-step choice keeps two
// workgroups resident per CU (LDS double buffer + registers) for d <= 128;
// d = 256 halves it to keep the accumulator and Q operand in registers.
template <int D> struct FwdTile;
template <> struct FwdTile<64>  { static constexpr int WAVES = 4, BLOCK_KV = 64; };
template <> struct FwdTile<80>  { static constexpr int WAVES = 4, BLOCK_KV = 64; };
template <> struct FwdTile<128> { static constexpr int WAVES = 4, BLOCK_KV = 64; };
template <> struct FwdTile<256> { static constexpr int WAVES = 4, BLOCK_KV = 32; };

// Row pitches (in bf16 elements) of the LDS tiles.
//  K tile, read 16 bytes per lane along d: pad one 16-byte chunk per row so
//  that consecutive rows start in different banks.
//  V tile, read with the transposing read (4 rows x 32 bytes per 16 lanes):
//  the row pitch is an odd multiple of 32 bytes modulo 128 so that the four
//  rows of one read land in different banks; rows are at least the padded
//  output width (a multiple of 32 columns), the columns beyond d being zero.
constexpr int k_pitch(int d) { return d + 8; }
constexpr int v_pitch(int d) { return ((d + 31) / 32) * 32 + 16; }

struct FwdParams {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    int N;
    int Hq;
    int Hkv;
    int G;        // Hq / Hkv
    int BH;       // B * Hq
    int nqb;      // query blocks per head
    float c;      // scale * log2(e)
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
    float* delta;  // [B, Hq, N] workspace: D_i = <dO_i, O_i>
    int N;
    int Hq;
    int Hkv;
    int G;
    int B;
    float scale;
    float c;       // scale * log2(e)
};

struct FwdPlan {
    int block_q;
    int block_kv;
    int threads;
    long long workgroups;
    int lds_bytes;
};

bool fwd_plan(int B, int Hq, int N, int d, FwdPlan* plan);

// Launchers return the hipError_t of the launch.
hipError_t launch_fwd(const FwdParams& p, int d, bool causal, long long workgroups,
                      hipStream_t stream);
// Backward passes: bit 0 = row-term preprocess, bit 1 = dK/dV, bit 2 = dQ.
enum BwdPass { kBwdPre = 1, kBwdDkDv = 2, kBwdDq = 4, kBwdAll = 7 };
hipError_t launch_bwd(const BwdParams& p, int d, bool causal, int passes, hipStream_t stream);

}  // namespace attn
