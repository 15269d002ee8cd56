// attn_bwd_common.h - tile helpers shared by the backward kernels.
#pragma once

#include "attn_device.h"
#include "attn_kernels.h"

namespace attn {

// Loads `rows` rows of one head's [N, D] 16-bit operand (row stride sn
// elements) starting at row r0 into registers (16-byte chunks, zero beyond N)
// and stores them to an LDS tile.
template <int D, int ROWS, int T>
struct TileIO {
    static constexpr int CPR = D / 8;
    static constexpr int CHUNKS = ROWS * CPR;
    static constexpr int NCH = (CHUNKS + T - 1) / T;
    uint4 r[NCH];

    // Rows r0 .. r0+ROWS-1 through a buffer resource that ends with row
    // N - 1, so rows at or past N read as zeros with no per-row arithmetic
    // or branch. Requires (N - 1) * sn * 2 + D * 2 < 2^32 and r0 < N.
    __device__ __forceinline__ void load(const e16* head, long long sn, int r0, int N, int tid) {
        const uint32_t sn2 = (uint32_t)sn * 2u;
        const auto rsrc = buf_rsrc(head + (long long)r0 * sn, (uint32_t)(N - r0 - 1) * sn2 + D * 2);
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            const int c = tid + i * T;
            if (CHUNKS % T == 0 || c < CHUNKS) {
                const int row = c / CPR;
                const int col = c - row * CPR;
                r[i] = buf_load16(rsrc, (uint32_t)row * sn2 + (uint32_t)col * 16u);
            }
        }
    }
    __device__ __forceinline__ void store(e16* tile, int pitch, int tid) const {
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
    // Same, into a chunk-swizzled tile (sw_off).
    __device__ __forceinline__ void store_sw(e16* tile, int pitch, int tid) const {
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            const int c = tid + i * T;
            if (CHUNKS % T == 0 || c < CHUNKS) {
                const int row = c / CPR;
                const int col = c - row * CPR;
                *reinterpret_cast<uint4*>(tile + sw_off(row, col * 8, pitch)) = r[i];
            }
        }
    }
};

// Zero the columns D .. round_up(D, 32) of `rows` rows of a chunk-swizzled
// LDS tile (read by the transposing read of the last 32-wide tile, never
// written by the loads).
template <int D>
__device__ __forceinline__ void zero_pad_cols_sw(e16* tile, int rows, int pitch, int tid, int T) {
    constexpr int PADC = ((D + 31) / 32) * 32 - D;
    if constexpr (PADC > 0) {
        for (int i = tid; i < rows * PADC; i += T) tile[sw_off(i / PADC, D + i % PADC, pitch)] = (e16)0;
    }
}

}  // namespace attn
