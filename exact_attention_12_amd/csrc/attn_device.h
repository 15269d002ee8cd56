// attn_device.h - device building blocks for the gfx950 (CDNA4) attention kernels.
//
// Matrix-core conventions used throughout (v_mfma_f32_32x32x16_bf16 and its
// fp16 twin, wave64):
//   D[32x32] += A[32x16] * B[16x32]
//   A operand: lane l holds A[l % 32][8*(l/32) .. 8*(l/32)+7]   (8 values)
//   B operand: lane l holds B[8*(l/32) .. +7][l % 32]          (8 values)
//   D / C:     lane l, register r holds D[8*(r/4) + 4*(l/32) + r%4][l % 32]
// so a lane owns one column of the result and 16 of its rows, in four runs
// of four consecutive rows.
//
// Transposing LDS read (ds_read_b64_tr_b16): inside each group of 16 lanes,
// lane 4t+s supplies the address of 4 consecutive b16 values; together the
// four lanes of sub-group t address row t of a 4x16 matrix. Lane j receives
// column j of that matrix (its 4 values, one per row t). With a row-major
// [key][dim] tile in LDS, this hands each lane 4 keys of one dim column,
// which is the packing a contraction over keys needs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

// 16-bit operands are stored as raw bits (e16) and interpreted by the
// element type DT (bf16 or fp16) only where it matters: the matrix
// instruction, fp32 -> 16-bit rounding and 16-bit -> fp32 widening.
enum DType { kBF16 = 0, kFP16 = 1 };

typedef unsigned short e16;
typedef e16 e16x2 __attribute__((ext_vector_type(2)));
typedef e16 e16x4 __attribute__((ext_vector_type(4)));
typedef e16 e16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// D[32x32] += A[32x16] * B[16x32] (v_mfma_f32_32x32x16_bf16 / _f16).
template <int DT>
__device__ __forceinline__ f32x16 mfma32(e16x8 a, e16x8 b, f32x16 c) {
    if constexpr (DT == kBF16)
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// Accumulating MFMA with the accumulator pinned in AGPRs (acc += a * b).
// Used for long-lived accumulators that only matrix instructions touch inside
// a loop, so that they do not compete with the loop's working set for VGPRs.
// Written as inline assembly, so the compiler's hazard tracking does not see
// it; the hazards it can meet:
//  * a VALU write of an A/B operand VGPR (or of the AGPRs) followed by the
//    MFMA read needs two wait states. Callers produce the operands in an
//    earlier scheduling region and separate the regions with
//    valu_mfma_gap(); the build checks the generated code for any VALU
//    write closer than two wait states to an MFMA that reads it (a nop in
//    every call would cost an issue slot per product). GAP = true puts the
//    two wait states in front of every product instead, for kernels where
//    the compiler moves operand writes past the region boundary;
//  * back-to-back accumulation into the same registers (srcC == vdst) is
//    interlocked by the hardware;
//  * reading the result with VALU instructions needs the MFMA to have drained:
//    call agpr_acc_ready() on the accumulator before any such read.
template <int DT, bool GAP = false>
__device__ __forceinline__ void mfma32_agpr(f32x16& acc, e16x8 a, e16x8 b) {
    if constexpr (GAP) {
        if constexpr (DT == kBF16)
            asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
        else
            asm("s_nop 1\n\tv_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
    } else {
        if constexpr (DT == kBF16)
            asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
        else
            asm("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
    }
}

// Two wait states between everything scheduled before this point and
// everything after it (the VALU -> MFMA operand gap of mfma32_agpr).
__device__ __forceinline__ void valu_mfma_gap() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 1");
    __builtin_amdgcn_sched_barrier(0);
}

// Wait states after the last mfma32_agpr into `acc` before VALU reads of it
// (more than the 8-pass XDL write -> VALU read requirement).
__device__ __forceinline__ void agpr_acc_ready(f32x16& acc) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(acc));
}

// Two floats -> a packed 16-bit pair, rounded to nearest even.
template <int DT>
__device__ __forceinline__ e16x2 cvt2(float a, float b) {
    f32x2 x = {a, b};
    if constexpr (DT == kBF16)
        return __builtin_bit_cast(e16x2, __builtin_convertvector(x, bf16x2));
    else
        return __builtin_bit_cast(e16x2, __builtin_convertvector(x, f16x2));
}

// One 16-bit value -> fp32 (exact).
template <int DT>
__device__ __forceinline__ float widen(e16 x) {
    if constexpr (DT == kBF16)
        return __uint_as_float((unsigned)x << 16);
    else
        return (float)__builtin_bit_cast(_Float16, x);
}

__device__ __forceinline__ e16x8 cat8(e16x2 a, e16x2 b, e16x2 c, e16x2 d) {
    e16x4 lo = __builtin_shufflevector(a, b, 0, 1, 2, 3);
    e16x4 hi = __builtin_shufflevector(c, d, 0, 1, 2, 3);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Lanes l and l^32 exchange a value (v_permlane32_swap); returns the pair
// (own-half copy, other-half copy) combined by `op`.
__device__ __forceinline__ float max_across_halves(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_across_halves(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// 16-byte LDS read (ds_read_b128).
__device__ __forceinline__ e16x8 lds_read8(const e16* p) {
    return *reinterpret_cast<const e16x8*>(p);
}

// Transposing LDS read of 4 b16 values (see the header comment).
__device__ __forceinline__ e16x4 lds_read_tr4(const e16* p) {
    s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
    return __builtin_bit_cast(e16x4, v);
}

__device__ __forceinline__ e16x8 join8(e16x4 a, e16x4 b) {
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ uint4 zero4() { return make_uint4(0u, 0u, 0u, 0u); }

// Raw buffer access: a resource over `bytes` bytes from `base` (wave-uniform);
// 16-byte loads at byte offsets at or past `bytes` return zeros (the buffer
// unit's range check), so tile loaders need no per-row bounds arithmetic.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
}
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0);
    return make_uint4(v.x, v.y, v.z, v.w);
}
// 4-byte variant: the 64 lanes fill 256 consecutive bytes of LDS.
__device__ __forceinline__ void buf_load4_to_lds(__amdgpu_buffer_rsrc_t r, void* lds_dst,
                                                 uint32_t byte_off) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_dst, 4,
                                             byte_off, 0, 0, 0);
}
// The same load written straight to LDS: the 64 lanes of the wave store
// their 16 bytes to 64 consecutive chunks starting at lds_dst (wave-uniform).
__device__ __forceinline__ void buf_load16_to_lds(__amdgpu_buffer_rsrc_t r, void* lds_dst,
                                                  uint32_t byte_off) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_dst, 16,
                                             byte_off, 0, 0, 0);
}

// Stores four fp32 values as four 16-bit values (8 bytes).
template <int DT>
__device__ __forceinline__ void store4(e16* dst, float a, float b, float c, float d) {
    e16x2 lo = cvt2<DT>(a, b);
    e16x2 hi = cvt2<DT>(c, d);
    *reinterpret_cast<e16x4*>(dst) = __builtin_shufflevector(lo, hi, 0, 1, 2, 3);
}

// ------------------------------------------------------------------ dropout
//
// Counter-based random bits: Philox-4x32-10 (Salmon, Moraes, Dror, Shaw,
// "Parallel random numbers: as easy as 1, 2, 3", SC'11). Each round
// multiplies c0 and c2 by the published constants into 64-bit products and
// mixes their halves with c1, c3 and the key; the key advances by the Weyl
// constants between rounds. The key words are wave-uniform, so their updates
// run on the scalar unit.
__device__ __forceinline__ uint4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                               uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r > 0) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
        const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
        // Three-input XOR in one v_bitop3_b32 (truth table 0x96).
        const uint32_t n0 = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c1, k0, 0x96);
        const uint32_t n2 = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c3, k1, 0x96);
        c1 = (uint32_t)p1;
        c3 = (uint32_t)p0;
        c0 = n0;
        c2 = n2;
    }
    return make_uint4(c0, c1, c2, c3);
}

// Dropout stream: score (bh, i, j) is kept when the 16-bit half j % 2 (0:
// low, 1: high) of word i % 4 of philox4x32_10(j / 2, i / 4, bh, offset;
// seed) is >= thr = floor(p * 2^16). One Philox block thus decides a block of
// 4 queries x 2 keys.
struct DropParams {
    uint32_t thr;     // 0 = no dropout
    float scale;      // 1 / (1 - thr / 2^16)
    uint32_t seed_lo, seed_hi, offset;
};

// Keep bits of queries 4*iq .. +3 (k) at keys 2*jp and 2*jp + 1 (jj):
// bit k + 4*jj.
__device__ __forceinline__ uint32_t keep_block(const DropParams& dp, uint32_t jp, uint32_t iq,
                                               uint32_t bh) {
    const uint4 w = philox4x32_10(jp, iq, bh, dp.offset, dp.seed_lo, dp.seed_hi);
    const uint32_t t = dp.thr;
    return (uint32_t)((w.x & 0xFFFFu) >= t) | ((uint32_t)((w.y & 0xFFFFu) >= t) << 1) |
           ((uint32_t)((w.z & 0xFFFFu) >= t) << 2) | ((uint32_t)((w.w & 0xFFFFu) >= t) << 3) |
           ((uint32_t)((w.x >> 16) >= t) << 4) | ((uint32_t)((w.y >> 16) >= t) << 5) |
           ((uint32_t)((w.z >> 16) >= t) << 6) | ((uint32_t)((w.w >> 16) >= t) << 7);
}

// Keep bits for a lane that owns key j (lane % 32 = j % 32, so lanes 2m and
// 2m+1 own an even key and the next one) and the query quads iq0 + 2*gg
// (gg = 0..3): bits 4gg .. 4gg+3 = the four queries of quad gg. Each lane of
// the pair draws two of the four blocks, which cover both keys, and hands the
// other key's half to its partner.
__device__ __forceinline__ uint32_t keep_bits_key_lane(const DropParams& dp, uint32_t j,
                                                       uint32_t iq0, uint32_t bh) {
    const uint32_t jj = j & 1u;
    const uint32_t b0 = keep_block(dp, j >> 1, iq0 + 4u * jj, bh);      // quad gg = 2jj
    const uint32_t b1 = keep_block(dp, j >> 1, iq0 + 4u * jj + 2u, bh); // quad gg = 2jj + 1
    const uint32_t mine = ((b0 >> (4u * jj)) & 0xFu) | (((b1 >> (4u * jj)) & 0xFu) << 4);
    const uint32_t other = ((b0 >> (4u - 4u * jj)) & 0xFu) | (((b1 >> (4u - 4u * jj)) & 0xFu) << 4);
    // partner's value (DPP quad_perm [1, 0, 3, 2]: lanes 2m <-> 2m+1)
    const uint32_t recv = (uint32_t)__builtin_amdgcn_mov_dpp((int)other, 0xB1, 0xF, 0xF, false);
    return jj ? (recv | (mine << 8)) : (mine | (recv << 8));
}

// Value of x held by lane U of this lane's group of four (DPP quad_perm).
template <int U>
__device__ __forceinline__ uint32_t quad_bcast(uint32_t x) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, U * 0x55, 0xF, 0xF, false);
}

// Keep bits for a lane that owns query i (lane % 32 = i % 32, so the four
// lanes of a DPP quad own the queries 4*(i/4) .. +3) and the keys j0 .. j0+3
// (bits 0..3) and j0+8 .. j0+11 (bits 4..7), j0 a multiple of 4. Lane t of
// the quad draws the block of key pair t (j0/2 + t for t < 2, j0/2 + 4 + t - 2
// after), covering all four queries; the bits are then gathered across the
// quad.
__device__ __forceinline__ uint32_t keep_bits_query_lane(const DropParams& dp, uint32_t j0,
                                                         uint32_t i, uint32_t bh) {
    const uint32_t q = i & 3u;
    const uint32_t jp = (j0 >> 1) + (q < 2u ? q : q + 2u);
    const uint32_t blk = keep_block(dp, jp, i >> 2, bh);
    const uint32_t x0 = quad_bcast<0>(blk), x1 = quad_bcast<1>(blk);
    const uint32_t x2 = quad_bcast<2>(blk), x3 = quad_bcast<3>(blk);
    // key j0 + u (u < 4): block of lane u / 2, bit q + 4 * (u % 2)
    return ((x0 >> q) & 1u) | (((x0 >> (q + 4u)) & 1u) << 1) | (((x1 >> q) & 1u) << 2) |
           (((x1 >> (q + 4u)) & 1u) << 3) | (((x2 >> q) & 1u) << 4) | (((x2 >> (q + 4u)) & 1u) << 5) |
           (((x3 >> q) & 1u) << 6) | (((x3 >> (q + 4u)) & 1u) << 7);
}

}  // namespace attn
