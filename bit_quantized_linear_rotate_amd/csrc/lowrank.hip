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

// Wide variant for rank == RT (16, 32 or 64) and a 16-byte aligned proj_down:
// one workgroup of sixteen waves per 16 rows (one workgroup per CU at
// prefill sizes, four waves per SIMD). Wave w takes the 32-deep K slices
// w, w + 16, w + 32, ...; a slice of proj_down (32 x RT values, contiguous)
// is read with 16-byte loads and transposed through a wave-private LDS tile
// into the MFMA's B layout (a lane holds eight consecutive k of one column,
// 16-byte chunks swizzled per column),
// four slices' loads in flight at a time. The sixteen partial sums are added
// in wave order through LDS.
template <int DT, int RT>
__global__ __launch_bounds__(1024) void lowrank_wide_kernel(
    const uint16_t* __restrict__ x, int64_t M, int64_t K, int64_t sm,
    const uint16_t* __restrict__ down, float* __restrict__ L)
{
    constexpr int NCT = RT / 16;  // 16-column MFMA tiles
    constexpr int NLD = RT / 16;  // 16-byte proj_down loads per lane per slice
    constexpr int DP = 40;        // LDS pitch (values) of a transposed column
    constexpr int UNR = 4;        // slices in flight
    constexpr int TILE_B = RT * DP * 2;
    constexpr int PART_B = 16 * 16 * (RT + 1) * 4;
    constexpr int SMEM_B = 16 * TILE_B > PART_B ? 16 * TILE_B : PART_B;
    __shared__ __align__(16) unsigned char smem[SMEM_B];
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int j = lane & 15, q = lane >> 4;
    uint16_t* Dw = (uint16_t*)(smem + wave * TILE_B);
    // column c's four 8-value k chunks are stored in the order chunk ^ swz(c):
    // the transposing 2-byte stores and the 16-byte fragment reads are then
    // free of bank conflicts (64 banks of 4 bytes) for R = 16, 32 and 64
    auto swz = [](int c) { return ((c >> 4) * 3) & 3; };
    const int64_t m0 = (int64_t)blockIdx.x * 16;
    const int64_t row = m0 + j;
    const int64_t nsl = K / 32;

    v4f acc[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) acc[ct] = (v4f){0.f, 0.f, 0.f, 0.f};

    for (int64_t t0 = wave; t0 < nsl; t0 += 16 * UNR) {
        uint4 xa[UNR], da[UNR][NLD];
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
            const int64_t t = t0 + 16 * u;
            const bool ok = t < nsl;
            xa[u] = make_uint4(0, 0, 0, 0);
            if (ok && row < M) xa[u] = *(const uint4*)(x + row * sm + t * 32 + q * 8);
#pragma unroll
            for (int i = 0; i < NLD; ++i) {
                da[u][i] = make_uint4(0, 0, 0, 0);
                if (ok) da[u][i] = *(const uint4*)(down + t * 32 * RT + lane * 8 + i * 512);
            }
        }
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
            // value e of this lane's load i is proj_down[k = e0 / RT][c0 + e]
#pragma unroll
            for (int i = 0; i < NLD; ++i) {
                const int e0 = lane * 8 + i * 512;
                const int kl = e0 / RT, c0 = e0 % RT;
                const uint32_t w[4] = {da[u][i].x, da[u][i].y, da[u][i].z, da[u][i].w};
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int c = c0 + e;
                    Dw[c * DP + ((((kl >> 3) ^ swz(c)) << 3) | (kl & 7))] =
                        (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
                }
            }
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                const int c = ct * 16 + j;
                const v8s bf = *(const v8s*)(&Dw[c * DP + ((q ^ swz(c)) << 3)]);
                const v8s af = __builtin_bit_cast(v8s, xa[u]);
                if constexpr (DT == BF16)
                    acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(v8bf, af), __builtin_bit_cast(v8bf, bf), acc[ct], 0, 0, 0);
                else
                    acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                        __builtin_bit_cast(v8h, af), __builtin_bit_cast(v8h, bf), acc[ct], 0, 0, 0);
            }
            __builtin_amdgcn_wave_barrier();
        }
    }
    __syncthreads();
    float* part = (float*)smem;  // [16 waves][16 rows][RT + 1]
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r) part[(wave * 16 + 4 * q + r) * (RT + 1) + ct * 16 + j] = acc[ct][r];
    __syncthreads();
    if (tid < 16 * RT) {
        const int rr = tid / RT, c = tid % RT;
        if (m0 + rr < M) {
            float s = part[rr * (RT + 1) + c];
            for (int w = 1; w < 16; ++w) s = add_rn(s, part[(w * 16 + rr) * (RT + 1) + c]);
            L[(m0 + rr) * RT + c] = s;
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
    if (mf && (a.rank == 16 || a.rank == 32 || a.rank == 64) && ((uintptr_t)a.down % 16) == 0) {
        const unsigned grid = (unsigned)((a.M + 15) / 16);
#define W4A4_LRW(DTV, RTV)                                                                        \
    hipLaunchKernelGGL((lowrank_wide_kernel<DTV, RTV>), dim3(grid), dim3(1024), 0, st,           \
                       (const uint16_t*)a.x, a.M, a.K, a.sm, (const uint16_t*)a.down, a.lora)
        if (a.dtype == BF16) {
            if (a.rank == 16) W4A4_LRW(BF16, 16);
            else if (a.rank == 32) W4A4_LRW(BF16, 32);
            else W4A4_LRW(BF16, 64);
        } else {
            if (a.rank == 16) W4A4_LRW(F16, 16);
            else if (a.rank == 32) W4A4_LRW(F16, 32);
            else W4A4_LRW(F16, 64);
        }
#undef W4A4_LRW
        return hipGetLastError();
    }
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
