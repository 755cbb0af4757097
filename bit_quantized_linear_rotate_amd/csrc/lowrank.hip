// Low-rank down projection L = x . proj_down on the raw activation (gfx950).
//
// The source page comfy_kitchen/tensor/svdquant_w4a4.py (module docstring and
// the _w4a4_forward docstring) describes a rank-R correction computed from the
// unshifted, unquantized activation: L (M, R) = x (M, K) . proj_down (K, R),
// later multiplied by proj_up^T in the GEMM epilogue.  L is kept in fp32.
//
// 16-bit activations use v_mfma_f32_16x16x32_{bf16,f16}: one workgroup owns 16
// rows and all R (<= 64) output columns; its four waves take interleaved
// 32-deep K slices and their partial sums are added in a fixed order through
// LDS, so the result does not depend on scheduling.
#include "common.hpp"
#include "kernels.hpp"

namespace w4a4 {

template <int DT, int RT>
__global__ __launch_bounds__(256) void lowrank_mfma_kernel(
    const uint16_t* __restrict__ x, int64_t M, int64_t K, int64_t sm,
    const uint16_t* __restrict__ down, int rank, float* __restrict__ L)
{
    constexpr int NCT = RT / 16;
    __shared__ float part[4][16][RT + 1];
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int j = lane & 15, q = lane >> 4;
    const int64_t m0 = (int64_t)blockIdx.x * 16;
    const int64_t row = m0 + j;
    v4f acc[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) acc[ct] = (v4f){0.f, 0.f, 0.f, 0.f};
    for (int64_t k0 = (int64_t)wave * 32; k0 < K; k0 += 128) {
        v8s af = (v8s){0, 0, 0, 0, 0, 0, 0, 0};
        if (row < M) af = __builtin_bit_cast(v8s, *(const uint4*)(x + row * sm + k0 + q * 8));
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            v8s bf;
            const int col = ct * 16 + j;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                bf[e] = col < rank ? (short)down[(k0 + q * 8 + e) * rank + col] : (short)0;
            if constexpr (DT == BF16)
                acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(v8bf, af), __builtin_bit_cast(v8bf, bf), acc[ct], 0, 0, 0);
            else
                acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                    __builtin_bit_cast(v8h, af), __builtin_bit_cast(v8h, bf), acc[ct], 0, 0, 0);
        }
    }
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r) part[wave][4 * q + r][ct * 16 + j] = acc[ct][r];
    __syncthreads();
    for (int i = tid; i < 16 * rank; i += 256) {
        const int rr = i / rank, c = i - rr * rank;
        if (m0 + rr < M) {
            float s = add_rn(add_rn(part[0][rr][c], part[1][rr][c]),
                             add_rn(part[2][rr][c], part[3][rr][c]));
            L[(m0 + rr) * rank + c] = s;
        }
    }
}

template <int DT>
__global__ __launch_bounds__(256) void lowrank_generic_kernel(
    const void* __restrict__ x, int64_t M, int64_t K, int64_t sm, int64_t sk,
    const void* __restrict__ down, int rank, float* __restrict__ L)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= M * rank) return;
    const int64_t m = i / rank;
    const int r = (int)(i - m * rank);
    float s = 0.0f;
    for (int64_t k = 0; k < K; ++k)
        s = fmaf(load_as_f32<DT>(x, m * sm + k * sk), load_as_f32<DT>(down, k * rank + r), s);
    L[i] = s;
}

hipError_t launch_lowrank_down(const LowRankArgs& a, hipStream_t st)
{
    const bool mf = (a.dtype == BF16 || a.dtype == F16) && a.sk == 1 && (a.sm % 8) == 0 &&
                    (a.K % 32) == 0 && ((uintptr_t)a.x % 16) == 0 && a.rank <= 64;
    if (mf) {
        const unsigned grid = (unsigned)((a.M + 15) / 16);
        const int rt = a.rank <= 16 ? 16 : a.rank <= 32 ? 32 : 64;
#define W4A4_LR(DTV, RTV)                                                                         \
    hipLaunchKernelGGL((lowrank_mfma_kernel<DTV, RTV>), dim3(grid), dim3(256), 0, st,            \
                       (const uint16_t*)a.x, a.M, a.K, a.sm, (const uint16_t*)a.down, a.rank, a.lora)
        if (a.dtype == BF16) {
            if (rt == 16) W4A4_LR(BF16, 16);
            else if (rt == 32) W4A4_LR(BF16, 32);
            else W4A4_LR(BF16, 64);
        } else {
            if (rt == 16) W4A4_LR(F16, 16);
            else if (rt == 32) W4A4_LR(F16, 32);
            else W4A4_LR(F16, 64);
        }
#undef W4A4_LR
        return hipGetLastError();
    }
    const unsigned grid = (unsigned)((a.M * a.rank + 255) / 256);
    switch (a.dtype) {
    case F32:
        hipLaunchKernelGGL(lowrank_generic_kernel<F32>, dim3(grid), dim3(256), 0, st, a.x, a.M, a.K,
                           a.sm, a.sk, a.down, a.rank, a.lora);
        break;
    case F16:
        hipLaunchKernelGGL(lowrank_generic_kernel<F16>, dim3(grid), dim3(256), 0, st, a.x, a.M, a.K,
                           a.sm, a.sk, a.down, a.rank, a.lora);
        break;
    default:
        hipLaunchKernelGGL(lowrank_generic_kernel<BF16>, dim3(grid), dim3(256), 0, st, a.x, a.M,
                           a.K, a.sm, a.sk, a.down, a.rank, a.lora);
    }
    return hipGetLastError();
}

}  // namespace w4a4
