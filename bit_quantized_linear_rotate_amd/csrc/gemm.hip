// W4A4 GEMM on INT8 MFMA with W4 nibble unpack into LDS and a fused
// scale / bias / cast epilogue (gfx950).
//
// What is computed (web page "[Feat][Ascend] Consolidate INT8, RotateQuant,
// RoPE and ConvRot W4A4 backends", section "W4A4 correctness and performance
// scope"; per-64-group weight scales and the low-rank term from the source
// page comfy_kitchen/tensor/svdquant_w4a4.py, module docstring):
//   acc[m,n] = sum_k c[m,k] * w[n,k]                 exact integer sum
//   out[m,n] = O( ((f32(acc) * s_a[m]) * s_w[n]) [+ l[m,n]] [+ bias[n]] )
// or, with per-64-group weight scales,
//   out[m,n] = O( ((sum_G f32(acc_G) * s_w[G,n]) * s_a[m]) [+ l] [+ bias] )
// with l[m,n] = sum_r L[m,r] * up[n,r]; every listed multiply and add is a
// separately rounded fp32 operation.
//
// Design for CDNA4:
//   * 128 x 128 output tile per 256-thread workgroup, 4 waves in 2 x 2, each
//     wave a 64 x 64 block of 4 x 4 v_mfma_i32_16x16x64_i8 tiles; K advances
//     64 per step with double-buffered LDS (one barrier per step) and the next
//     step's global loads in flight during the MFMAs.
//   * Packed weights are read as bytes (N, K/2) and unpacked once per tile
//     into LDS as 16*w: the low nibble shifted into the high half of a byte
//     and the high nibble masked in place are both already sign-correct int8
//     values, so unpacking is shift/and/perm with no sign extension.  The
//     integer result is divided by 16 (an exact arithmetic shift) before the
//     epilogue.
//   * LDS rows are padded to 80 bytes so the 16 lanes of a ds_read_b128
//     phase hit distinct banks.
//   * When K is too large for INT32 (16 * 7 * 8 * K > 2^31 - 1) or a chunk
//     size is forced, each workgroup accumulates one K-chunk and adds it into
//     an int64 workspace with 64-bit atomics (exact and order-independent);
//     a second kernel applies the epilogue.
#include "common.hpp"
#include "kernels.hpp"

namespace w4a4 {

constexpr int BM = 128, BN = 128, BK = 64, LDR = 80;

__device__ __forceinline__ void unpack16(uint32_t p, uint32_t& lo4, uint32_t& hi4)
{
    // p holds 8 nibbles for k0..k7 (even k in the low nibble of each byte).
    const uint32_t L = (p << 4) & 0xf0f0f0f0u;  // 16*w(k0), 16*w(k2), 16*w(k4), 16*w(k6)
    const uint32_t H = p & 0xf0f0f0f0u;         // 16*w(k1), 16*w(k3), ...
    lo4 = __builtin_amdgcn_perm(H, L, 0x05010400u);  // k0 k1 k2 k3
    hi4 = __builtin_amdgcn_perm(H, L, 0x07030602u);  // k4 k5 k6 k7
}

__device__ __forceinline__ float epilogue_tail(float t, const GemmArgs& a, int64_t row, int64_t col)
{
    if (a.lora) {
        const float* lr = a.lora + row * a.rank;
        float l = 0.0f;
        for (int r = 0; r < a.rank; ++r)
            l = fmaf(lr[r], load_any_f32(a.up_dtype, a.up, col * a.rank + r), l);
        t = add_rn(t, l);
    }
    if (a.bias) t = add_rn(t, load_any_f32(a.bias_dtype, a.bias, col));
    return t;
}

template <bool GROUP, bool SPLIT, bool ALIGNED>
__global__ __launch_bounds__(256) void w4a4_gemm_kernel(GemmArgs a, int64_t kc)
{
    __shared__ __align__(16) int8_t As[2][BM * LDR];
    __shared__ __align__(16) int8_t Bs[2][BN * LDR];

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int j = lane & 15, q = lane >> 4;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t n0 = (int64_t)blockIdx.x * BN;
    const int64_t m0 = (int64_t)blockIdx.y * BM;
    const int64_t K = a.K, M = a.M, N = a.N;
    const int64_t kbeg = (int64_t)blockIdx.z * kc;
    const int64_t kend = min(K, kbeg + kc);
    const int nsteps = (int)((kend - kbeg + BK - 1) / BK);

    // global -> register staging
    uint4 ra[2];
    uint4 rw;
    auto gload = [&](int64_t k) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int c = tid + 256 * i;
            const int row = c >> 2, c16 = c & 3;
            const int64_t gm = m0 + row, gk = k + c16 * 16;
            if constexpr (ALIGNED) {
                if (gm < M && gk < kend) ra[i] = *(const uint4*)(a.codes + gm * K + gk);
                else ra[i] = make_uint4(0, 0, 0, 0);
            } else {
                uint32_t wv[4] = {0, 0, 0, 0};
                if (gm < M)
                    for (int e = 0; e < 16; ++e)
                        if (gk + e < kend)
                            wv[e >> 2] |= (uint32_t)(uint8_t)a.codes[gm * K + gk + e] << (8 * (e & 3));
                ra[i] = make_uint4(wv[0], wv[1], wv[2], wv[3]);
            }
        }
        const int n = tid >> 1, half = tid & 1;
        const int64_t gn = n0 + n;
        const int64_t kp = (k >> 1) + half * 16;  // packed byte index
        if constexpr (ALIGNED) {
            if (gn < N && 2 * kp < kend) rw = *(const uint4*)(a.wp + gn * (K >> 1) + kp);
            else rw = make_uint4(0, 0, 0, 0);
        } else {
            uint32_t wv[4] = {0, 0, 0, 0};
            if (gn < N)
                for (int e = 0; e < 16; ++e)
                    if (2 * (kp + e) < kend)
                        wv[e >> 2] |= (uint32_t)a.wp[gn * (K >> 1) + kp + e] << (8 * (e & 3));
            rw = make_uint4(wv[0], wv[1], wv[2], wv[3]);
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int c = tid + 256 * i;
            const int row = c >> 2, c16 = c & 3;
            *(uint4*)(&As[buf][row * LDR + c16 * 16]) = ra[i];
        }
        const int n = tid >> 1, half = tid & 1;
        uint4 u0, u1;
        unpack16(rw.x, u0.x, u0.y);
        unpack16(rw.y, u0.z, u0.w);
        unpack16(rw.z, u1.x, u1.y);
        unpack16(rw.w, u1.z, u1.w);
        *(uint4*)(&Bs[buf][n * LDR + half * 32]) = u0;
        *(uint4*)(&Bs[buf][n * LDR + half * 32 + 16]) = u1;
    };

    v4i acc[4][4];
    v4f facc[GROUP ? 4 : 1][GROUP ? 4 : 1];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = (v4i){0, 0, 0, 0};
    if constexpr (GROUP) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) facc[mt][nt] = (v4f){0.f, 0.f, 0.f, 0.f};
    }

    if (nsteps > 0) {
        gload(kbeg);
        sstore(0);
    }
    __syncthreads();
    for (int s = 0; s < nsteps; ++s) {
        const int buf = s & 1;
        if (s + 1 < nsteps) gload(kbeg + (int64_t)(s + 1) * BK);
        v4i af[4], bf[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
            af[mt] = *(const v4i*)(&As[buf][(wm * 64 + mt * 16 + j) * LDR + q * 16]);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
            bf[nt] = *(const v4i*)(&Bs[buf][(wn * 64 + nt * 16 + j) * LDR + q * 16]);
        if constexpr (GROUP) {
            const int64_t gidx = (kbeg + (int64_t)s * BK) / 64;
            float swv[4];
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
                const int64_t col = n0 + wn * 64 + nt * 16 + j;
                swv[nt] = col < N ? load_any_f32(a.sw_dtype, a.sw, gidx * N + col) : 0.0f;
            }
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) {
                    v4i t = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[mt], bf[nt], (v4i){0, 0, 0, 0},
                                                                  0, 0, 0);
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        facc[mt][nt][r] = add_rn(facc[mt][nt][r], mul_rn((float)(t[r] >> 4), swv[nt]));
                }
        } else {
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int nt = 0; nt < 4; ++nt)
                    acc[mt][nt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[mt], bf[nt], acc[mt][nt],
                                                                        0, 0, 0);
        }
        if (s + 1 < nsteps) sstore(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue: lane (j, q) holds rows 4q..4q+3, column j of each tile.
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t row = m0 + wm * 64 + mt * 16 + 4 * q + r;
                const int64_t col = n0 + wn * 64 + nt * 16 + j;
                if (row >= M || col >= N) continue;
                if constexpr (SPLIT) {
                    atomicAdd((unsigned long long*)(a.acc64 + row * N + col),
                              (unsigned long long)(int64_t)(acc[mt][nt][r] >> 4));
                } else {
                    float t;
                    if constexpr (GROUP) {
                        t = mul_rn(facc[mt][nt][r], a.sa[row]);
                    } else {
                        const int32_t iv = acc[mt][nt][r] >> 4;
                        if (a.acc_out) a.acc_out[row * N + col] = iv;
                        t = (float)iv;
                        t = mul_rn(t, a.sa[row]);
                        t = mul_rn(t, load_any_f32(a.sw_dtype, a.sw, col));
                    }
                    t = epilogue_tail(t, a, row, col);
                    store_any(a.out_dtype, a.out, row * N + col, t);
                }
            }
}

__global__ void fill_zero_i64(int64_t* p, int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0;
}

__global__ void split_epilogue_kernel(GemmArgs a)
{
    const int64_t total = a.M * a.N;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t row = i / a.N, col = i - row * a.N;
        const int64_t v = a.acc64[i];
        if (a.acc_out) a.acc_out[i] = (int32_t)v;  // meaningful while |acc| < 2^31
        float t = (float)v;                        // nearest-even for |v| >= 2^24
        t = mul_rn(t, a.sa[row]);
        t = mul_rn(t, load_any_f32(a.sw_dtype, a.sw, col));
        t = epilogue_tail(t, a, row, col);
        store_any(a.out_dtype, a.out, i, t);
    }
}

hipError_t launch_gemm(const GemmArgs& a, hipStream_t st)
{
    const bool aligned = (a.K % 32) == 0 && ((uintptr_t)a.codes % 16) == 0 &&
                         ((uintptr_t)a.wp % 16) == 0;
    const bool group = a.sw_group > 0;
    const unsigned gx = (unsigned)((a.N + BN - 1) / BN);
    const unsigned gy = (unsigned)((a.M + BM - 1) / BM);
    if (a.k_chunk > 0 && !group) {
        const int64_t kc = a.k_chunk;
        const unsigned gz = (unsigned)((a.K + kc - 1) / kc);
        const int64_t n = a.M * a.N;
        hipLaunchKernelGGL(fill_zero_i64, dim3(1024), dim3(256), 0, st, a.acc64, n);
        if (aligned)
            hipLaunchKernelGGL((w4a4_gemm_kernel<false, true, true>), dim3(gx, gy, gz), dim3(256), 0,
                               st, a, kc);
        else
            hipLaunchKernelGGL((w4a4_gemm_kernel<false, true, false>), dim3(gx, gy, gz), dim3(256), 0,
                               st, a, kc);
        hipLaunchKernelGGL(split_epilogue_kernel, dim3(2048), dim3(256), 0, st, a);
        return hipGetLastError();
    }
    const int64_t kc = a.K;
    if (group) {
        if (aligned)
            hipLaunchKernelGGL((w4a4_gemm_kernel<true, false, true>), dim3(gx, gy, 1), dim3(256), 0,
                               st, a, kc);
        else
            hipLaunchKernelGGL((w4a4_gemm_kernel<true, false, false>), dim3(gx, gy, 1), dim3(256), 0,
                               st, a, kc);
    } else {
        if (aligned)
            hipLaunchKernelGGL((w4a4_gemm_kernel<false, false, true>), dim3(gx, gy, 1), dim3(256), 0,
                               st, a, kc);
        else
            hipLaunchKernelGGL((w4a4_gemm_kernel<false, false, false>), dim3(gx, gy, 1), dim3(256), 0,
                               st, a, kc);
    }
    return hipGetLastError();
}

}  // namespace w4a4
