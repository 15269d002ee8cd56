// attn_device.h - device building blocks for the gfx950 (CDNA4) attention kernels.
//
// Matrix-core conventions used throughout (v_mfma_f32_32x32x16_bf16, wave64):
//   D[32x32] += A[32x16] * B[16x32]
//   A operand: lane l holds A[l % 32][8*(l/32) .. 8*(l/32)+7]   (8 bf16)
//   B operand: lane l holds B[8*(l/32) .. +7][l % 32]          (8 bf16)
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

typedef __bf16 bf16;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Accumulating MFMA with the accumulator pinned in AGPRs (acc += a * b).
// Used for long-lived accumulators that only matrix instructions touch inside
// a loop, so that they do not compete with the loop's working set for VGPRs.
// Written as inline assembly, so the compiler's hazard tracking does not see
// it; the hazards it can meet are handled here:
//  * a VALU write of an A/B operand VGPR followed by the MFMA read needs two
//    wait states: the s_nop 1 in front of the instruction;
//  * back-to-back accumulation into the same registers (srcC == vdst) is
//    interlocked by the hardware;
//  * reading the result with VALU instructions needs the MFMA to have drained:
//    call agpr_acc_ready() on the accumulator before any such read.
__device__ __forceinline__ void mfma32_agpr(f32x16& acc, bf16x8 a, bf16x8 b) {
    asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// Wait states after the last mfma32_agpr into `acc` before VALU reads of it
// (more than the 8-pass XDL write -> VALU read requirement).
__device__ __forceinline__ void agpr_acc_ready(f32x16& acc) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(acc));
}

// Two floats -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ bf16x2 to_bf16x2(float a, float b) {
    f32x2 x = {a, b};
    return __builtin_convertvector(x, bf16x2);
}

__device__ __forceinline__ bf16x8 cat8(bf16x2 a, bf16x2 b, bf16x2 c, bf16x2 d) {
    bf16x4 lo = __builtin_shufflevector(a, b, 0, 1, 2, 3);
    bf16x4 hi = __builtin_shufflevector(c, d, 0, 1, 2, 3);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Sum of a packed bf16 pair accumulated into c in fp32 (v_dot2c_f32_bf16).
__device__ __forceinline__ float sum_pair(bf16x2 x, float c) {
    const bf16x2 one = {(bf16)1.0f, (bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(x, one, c, false);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

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
__device__ __forceinline__ bf16x8 lds_read8(const bf16* p) {
    return *reinterpret_cast<const bf16x8*>(p);
}

// Transposing LDS read of 4 b16 values (see the header comment).
__device__ __forceinline__ bf16x4 lds_read_tr4(const bf16* p) {
    s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
    return __builtin_bit_cast(bf16x4, v);
}

__device__ __forceinline__ bf16x8 join8(bf16x4 a, bf16x4 b) {
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ uint4 zero4() { return make_uint4(0u, 0u, 0u, 0u); }

// Stores four fp32 values as four bf16 (8 bytes).
__device__ __forceinline__ void store_bf16x4(bf16* dst, float a, float b, float c, float d) {
    bf16x2 lo = to_bf16x2(a, b);
    bf16x2 hi = to_bf16x2(c, d);
    *reinterpret_cast<bf16x4*>(dst) = __builtin_shufflevector(lo, hi, 0, 1, 2, 3);
}

}  // namespace attn
