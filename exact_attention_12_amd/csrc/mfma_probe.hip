// mfma_probe.hip - measurement helper: the matrix-core rate the chip sustains
// on a given operand pattern, as the ceiling the attention kernels' MFMA
// throughput is compared with.
//
// Every wave of every workgroup keeps NACC independent 32x32 accumulators and
// runs v_mfma_f32_32x32x16_bf16 (or 16x16 ones and v_mfma_f32_16x16x32_bf16)
// on operands it reads once from `src` (so
// random operands keep toggling the multiplier array the way attention's
// inputs do), two waves per SIMD like the attention kernels. No LDS, no
// other VALU work in the loop: the result bounds what any kernel that issues
// only these products could reach on the same data.
#include <hip/hip_runtime.h>

#include "attn_device.h"
#include "attn_probe.h"

namespace {

using namespace attn;

constexpr int kThreads = 512;  // 8 waves: two per SIMD

template <int NACC>
__global__ __launch_bounds__(kThreads, 1) void mfma_rate_kernel(const e16* src, float* dst, int iters) {
    const size_t t = (size_t)blockIdx.x * kThreads + threadIdx.x;
    const e16x8 a = *reinterpret_cast<const e16x8*>(src + t * 16);
    const e16x8 b = *reinterpret_cast<const e16x8*>(src + t * 16 + 8);
    f32x16 acc[NACC];
#pragma unroll
    for (int i = 0; i < NACC; ++i) acc[i] = f32x16{};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < NACC; ++i) acc[i] = mfma32<kBF16>(a, b, acc[i]);
    }
    float sum = 0.0f;
#pragma unroll
    for (int i = 0; i < NACC; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) sum += acc[i][r];
    dst[t] = sum;  // keeps the products live
}

// The same on v_mfma_f32_16x16x32_bf16 (half the flops per product, so twice
// the products for the same work): NACC independent 16x16 accumulators.
template <int NACC>
__global__ __launch_bounds__(kThreads, 1) void mfma16_rate_kernel(const e16* src, float* dst, int iters) {
    const size_t t = (size_t)blockIdx.x * kThreads + threadIdx.x;
    const e16x8 a = *reinterpret_cast<const e16x8*>(src + t * 16);
    const e16x8 b = *reinterpret_cast<const e16x8*>(src + t * 16 + 8);
    f32x4 acc[NACC];
#pragma unroll
    for (int i = 0; i < NACC; ++i) acc[i] = f32x4{};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < NACC; ++i)
            acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                            __builtin_bit_cast(bf16x8, b), acc[i], 0, 0, 0);
    }
    float sum = 0.0f;
#pragma unroll
    for (int i = 0; i < NACC; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) sum += acc[i][r];
    dst[t] = sum;
}

}  // namespace

extern "C" {

size_t attn_probe_mfma_src_elems(int blocks) { return (size_t)blocks * kThreads * 16; }

attn_status attn_probe_mfma_rate(const void* src, float* dst, int blocks, int iters, int chains,
                                 hipStream_t stream) {
    if (!src || !dst) return ATTN_ERR_NULL;
    if (blocks < 1 || iters < 1 || blocks > (1 << 20) || iters > (1 << 24)) return ATTN_ERR_SHAPE;
    const e16* s = static_cast<const e16*>(src);
    const dim3 grid((unsigned)blocks), block(kThreads);
    switch (chains) {
        case 1: hipLaunchKernelGGL(mfma_rate_kernel<1>, grid, block, 0, stream, s, dst, iters * 8); break;
        case 2: hipLaunchKernelGGL(mfma_rate_kernel<2>, grid, block, 0, stream, s, dst, iters * 4); break;
        case 4: hipLaunchKernelGGL(mfma_rate_kernel<4>, grid, block, 0, stream, s, dst, iters * 2); break;
        case 8: hipLaunchKernelGGL(mfma_rate_kernel<8>, grid, block, 0, stream, s, dst, iters); break;
        default: return ATTN_ERR_SHAPE;
    }
    return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

attn_status attn_probe_mfma16_rate(const void* src, float* dst, int blocks, int iters, int chains,
                                   hipStream_t stream) {
    if (!src || !dst) return ATTN_ERR_NULL;
    if (blocks < 1 || iters < 1 || blocks > (1 << 20) || iters > (1 << 24)) return ATTN_ERR_SHAPE;
    const e16* s = static_cast<const e16*>(src);
    const dim3 grid((unsigned)blocks), block(kThreads);
    switch (chains) {
        case 1: hipLaunchKernelGGL(mfma16_rate_kernel<1>, grid, block, 0, stream, s, dst, iters * 16); break;
        case 2: hipLaunchKernelGGL(mfma16_rate_kernel<2>, grid, block, 0, stream, s, dst, iters * 8); break;
        case 4: hipLaunchKernelGGL(mfma16_rate_kernel<4>, grid, block, 0, stream, s, dst, iters * 4); break;
        case 8: hipLaunchKernelGGL(mfma16_rate_kernel<8>, grid, block, 0, stream, s, dst, iters * 2); break;
        default: return ATTN_ERR_SHAPE;
    }
    return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

}  // extern "C"
