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
#ifndef W4A4_GEMM_KERNEL
#define W4A4_GEMM_KERNEL 1
#endif
// 5: four-wave 256x256 (AGPR accumulators); 8: eight-wave 256x256;
// 4: first four-wave 256x256; 1: 128x128
constexpr bool kUseFourWaveV2 = W4A4_GEMM_KERNEL == 5;
constexpr bool kUseEightWave = W4A4_GEMM_KERNEL == 8;
constexpr bool kUseBig = W4A4_GEMM_KERNEL >= 4;

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
    // Workgroups are dealt round-robin over the 8 XCDs; give each XCD a
    // contiguous range of tiles, M-grouped, so its L2 sees shared code rows and
    // weight columns.
    const int tiles_n = (int)gridDim.x, tiles_m = (int)gridDim.y;
    const int ntiles = tiles_m * tiles_n;
    const int bid = (int)(blockIdx.y * gridDim.x + blockIdx.x);
    const int q8 = ntiles >> 3, r8 = ntiles & 7;
    const int xcd = bid & 7, loc = bid >> 3;
    const int tile = xcd * q8 + min(xcd, r8) + loc;
    constexpr int GROUP_M = 16;
    const int per_group = GROUP_M * tiles_n;
    const int first_m = (tile / per_group) * GROUP_M;
    const int gsize = min(tiles_m - first_m, GROUP_M);
    const int in_g = tile - (tile / per_group) * per_group;
    const int64_t m0 = (int64_t)(first_m + in_g % gsize) * BM;
    const int64_t n0 = (int64_t)(in_g / gsize) * BN;
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


// -------------------------------------------------------------------------
// Large-tile kernel (per-channel scales, M > 128): 256 x 256 output tile per
// workgroup, four waves in 2 x 2, each a 128 x 128 block of 8 x 8
// v_mfma_i32_16x16x64_i8 tiles (256 INT32 accumulators per lane).  Only the
// codes are staged through LDS (double-buffered, 80-byte padded rows); each
// wave reads its packed weight fragments straight from global memory (8 bytes
// = 16 nibbles per lane per tile) and unpacks them in registers, so weights
// never touch LDS.  Tiles are numbered so that each XCD (workgroups are
// dealt round-robin over 8) works on a contiguous, M-grouped range of tiles
// and its L2 sees the same weight slices and code rows.
// -------------------------------------------------------------------------
constexpr int BBM = 256, BBN = 256;

__device__ __forceinline__ v4i unpack_frag(uint2 p)
{
    v4i r;
    uint32_t a, b, c, d;
    unpack16(p.x, a, b);
    unpack16(p.y, c, d);
    r[0] = (int)a; r[1] = (int)b; r[2] = (int)c; r[3] = (int)d;
    return r;
}

template <int ODT, bool SPLIT>
__global__ __launch_bounds__(256) void w4a4_gemm_big_kernel(GemmArgs a, int64_t kc, int tiles_m,
                                                            int tiles_n)
{
    // main loop: A tiles, double-buffered; epilogue: per-wave 16 x 128 int32
    // strips with rows padded to 132 words (reuses the same LDS).
    constexpr int EPR = 132;
    constexpr int LDS_BYTES = (2 * BBM * LDR > 4 * 16 * EPR * 4) ? 2 * BBM * LDR : 4 * 16 * EPR * 4;
    __shared__ __align__(16) int8_t smem[LDS_BYTES];
    int8_t (*As)[BBM * LDR] = (int8_t (*)[BBM * LDR])smem;

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int j = lane & 15, q = lane >> 4;
    const int wm = wave >> 1, wn = wave & 1;

    // XCD-contiguous tile ranges, then M-grouped order inside a range.
    const int ntiles = tiles_m * tiles_n;
    const int bid = blockIdx.x;
    const int q8 = ntiles >> 3, r8 = ntiles & 7;
    const int xcd = bid & 7, loc = bid >> 3;
    const int tile = xcd * q8 + min(xcd, r8) + loc;
    constexpr int GROUP_M = 8;
    const int per_group = GROUP_M * tiles_n;
    const int first_m = (tile / per_group) * GROUP_M;
    const int gsize = min(tiles_m - first_m, GROUP_M);
    const int in_g = tile - (tile / per_group) * per_group;
    const int tm = first_m + in_g % gsize;
    const int tn = in_g / gsize;

    const int64_t m0 = (int64_t)tm * BBM, n0 = (int64_t)tn * BBN;
    const int64_t K = a.K, M = a.M, N = a.N;
    const int64_t kbeg = (int64_t)blockIdx.z * kc;
    const int64_t kend = min(K, kbeg + kc);
    const int nsteps = (int)((kend - kbeg + BK - 1) / BK);

    uint4 ra[4];
    auto aload = [&](int64_t k) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = tid + 256 * i;
            const int row = c >> 2, c16 = c & 3;
            const int64_t gm = m0 + row, gk = k + c16 * 16;
            ra[i] = (gm < M && gk < kend) ? *(const uint4*)(a.codes + gm * K + gk)
                                          : make_uint4(0, 0, 0, 0);
        }
    };
    auto astore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = tid + 256 * i;
            const int row = c >> 2, c16 = c & 3;
            *(uint4*)(&As[buf][row * LDR + c16 * 16]) = ra[i];
        }
    };
    // packed weight fragments: column n0 + wn*128 + nt*16 + j, k + q*16 .. +16
    const uint8_t* wrow[8];
    bool wok[8];
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
        const int64_t col = n0 + wn * 128 + nt * 16 + j;
        wok[nt] = col < N;
        wrow[nt] = a.wp + (wok[nt] ? col : 0) * (K >> 1) + q * 8;
    }
    uint2 bq[8];
    auto bload = [&](int64_t k) {
#pragma unroll
        for (int nt = 0; nt < 8; ++nt)
            bq[nt] = (wok[nt] && k + q * 16 < kend) ? *(const uint2*)(wrow[nt] + (k >> 1))
                                                    : make_uint2(0, 0);
    };

    v4i acc[8][8];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) acc[mt][nt] = (v4i){0, 0, 0, 0};

    if (nsteps > 0) {
        aload(kbeg);
        astore(0);
        bload(kbeg);
    }
    __syncthreads();
    for (int s = 0; s < nsteps; ++s) {
        const int buf = s & 1;
        const bool more = s + 1 < nsteps;
        const int64_t knext = kbeg + (int64_t)(s + 1) * BK;
        if (more) aload(knext);
        v4i bf[8];
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) bf[nt] = unpack_frag(bq[nt]);
        if (more) bload(knext);
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
            const v4i af = *(const v4i*)(&As[buf][(wm * 128 + mt * 16 + j) * LDR + q * 16]);
#pragma unroll
            for (int nt = 0; nt < 8; ++nt)
                acc[mt][nt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af, bf[nt], acc[mt][nt], 0, 0, 0);
        }
        if (more) astore(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue, one 16-row strip at a time per wave: lane (j, q) holds
    // rows 4q..4q+3 / column j of each 16 x 16 tile; after the LDS transpose a
    // lane owns 32 consecutive columns of one row.
    int* strip = (int*)smem + wave * 16 * EPR;
    const int er = lane >> 2;            // row within the strip
    const int ec = (lane & 3) * 32;      // first of 32 columns (of 128)
    const int64_t col0 = n0 + wn * 128 + ec;
    float swv[32], bsv[32];
#pragma unroll
    for (int c = 0; c < 32; ++c) {
        const int64_t col = col0 + c;
        swv[c] = col < N ? load_any_f32(a.sw_dtype, a.sw, col) : 0.0f;
        bsv[c] = (a.bias && col < N) ? load_any_f32(a.bias_dtype, a.bias, col) : 0.0f;
    }
    const bool has_bias = a.bias != nullptr;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
#pragma unroll
        for (int nt = 0; nt < 8; ++nt)
#pragma unroll
            for (int r = 0; r < 4; ++r) strip[(4 * q + r) * EPR + nt * 16 + j] = acc[mt][nt][r] >> 4;
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): strip writes of this wave done
        __builtin_amdgcn_wave_barrier();
        const int64_t row = m0 + wm * 128 + mt * 16 + er;
        int iv[32];
#pragma unroll
        for (int c4 = 0; c4 < 8; ++c4) {
            const int4 v = *(const int4*)(strip + er * EPR + ec + 4 * c4);
            iv[4 * c4] = v.x; iv[4 * c4 + 1] = v.y; iv[4 * c4 + 2] = v.z; iv[4 * c4 + 3] = v.w;
        }
        __builtin_amdgcn_wave_barrier();
        if (row < M) {
            const bool full = col0 + 32 <= N;
            if constexpr (SPLIT) {
#pragma unroll
                for (int c = 0; c < 32; ++c)
                    if (col0 + c < N)
                        atomicAdd((unsigned long long*)(a.acc64 + row * N + col0 + c),
                                  (unsigned long long)(int64_t)iv[c]);
            } else {
                if (a.acc_out) {
#pragma unroll
                    for (int c = 0; c < 32; ++c)
                        if (col0 + c < N) a.acc_out[row * N + col0 + c] = iv[c];
                }
                const float sa = a.sa[row];
                float o[32];
#pragma unroll
                for (int c = 0; c < 32; ++c) {
                    float t = mul_rn(mul_rn((float)iv[c], sa), swv[c]);
                    if (has_bias) t = add_rn(t, bsv[c]);
                    o[c] = t;
                }
                if constexpr (ODT == F32) {
                    float* dst = (float*)a.out + row * N + col0;
                    if (full && (N % 4) == 0) {
#pragma unroll
                        for (int c4 = 0; c4 < 8; ++c4)
                            *(float4*)(dst + 4 * c4) = make_float4(o[4 * c4], o[4 * c4 + 1],
                                                                   o[4 * c4 + 2], o[4 * c4 + 3]);
                    } else {
#pragma unroll
                        for (int c = 0; c < 32; ++c)
                            if (col0 + c < N) dst[c] = o[c];
                    }
                } else {
                    uint16_t* dst = (uint16_t*)a.out + row * N + col0;
                    uint32_t pk[16];
#pragma unroll
                    for (int c2 = 0; c2 < 16; ++c2)
                        pk[c2] = (uint32_t)f32_to_h<ODT>(o[2 * c2]) |
                                 ((uint32_t)f32_to_h<ODT>(o[2 * c2 + 1]) << 16);
                    if (full && (N % 8) == 0) {
#pragma unroll
                        for (int c8 = 0; c8 < 4; ++c8)
                            *(uint4*)(dst + 8 * c8) = make_uint4(pk[4 * c8], pk[4 * c8 + 1],
                                                                 pk[4 * c8 + 2], pk[4 * c8 + 3]);
                    } else {
#pragma unroll
                        for (int c = 0; c < 32; ++c)
                            if (col0 + c < N) dst[c] = (uint16_t)(pk[c >> 1] >> (16 * (c & 1)));
                    }
                }
            }
        }
    }
}


// -------------------------------------------------------------------------
// Eight-wave kernel (per-channel scales, M > 128, K % 64 == 0): 256 x 256
// tile per 512-thread workgroup, waves in 4 (M) x 2 (N), each a 64 x 128 block
// of 4 x 8 v_mfma_i32_16x16x64_i8 tiles (128 INT32 accumulators per lane), two
// waves per SIMD.  All global reads are buffer loads whose out-of-range lanes
// return zero (no branches around loads).  Codes go through LDS; while they
// are staged, each 16-byte chunk is reordered to (even k of the first 8,
// odd k of the first 8, even k of the last 8, odd k of the last 8), which is
// the order in which a packed weight dword unpacks with no byte permutes:
// (p & 0x0f0f0f0f) << 4 gives 16*w of the even k, p & 0xf0f0f0f0 the odd k.
// The MFMA contracts over k, so any order shared by both operands is exact.
// -------------------------------------------------------------------------
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint64_t bytes)
{
    const uint32_t n = bytes > 0xffffffffull ? 0xffffffffu : (uint32_t)bytes;
    return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)n, 0x00020000);
}

__device__ __forceinline__ v4i unpack_frag_eo(v2u p)
{
    v4i r;
    r[0] = (int)((p.x & 0x0f0f0f0fu) << 4);
    r[1] = (int)(p.x & 0xf0f0f0f0u);
    r[2] = (int)((p.y & 0x0f0f0f0fu) << 4);
    r[3] = (int)(p.y & 0xf0f0f0f0u);
    return r;
}

__device__ __forceinline__ uint4 reorder_even_odd(v4u d)
{
    uint4 r;
    r.x = __builtin_amdgcn_perm(d.y, d.x, 0x06040200u);  // k0 k2 k4 k6
    r.y = __builtin_amdgcn_perm(d.y, d.x, 0x07050301u);  // k1 k3 k5 k7
    r.z = __builtin_amdgcn_perm(d.w, d.z, 0x06040200u);  // k8 .. k14
    r.w = __builtin_amdgcn_perm(d.w, d.z, 0x07050301u);  // k9 .. k15
    return r;
}

constexpr int W8_EPR = 132;
constexpr int W8_LDS = 8 * 16 * W8_EPR * 4;  // epilogue strips; >= 2 * 256 * LDR

template <int ODT, bool SPLIT>
__global__ __launch_bounds__(512) void w4a4_gemm_w8_kernel(GemmArgs a, int64_t kc, int tiles_m,
                                                           int tiles_n)
{
    extern __shared__ __align__(16) int8_t smem[];
    int8_t (*As)[BBM * LDR] = (int8_t (*)[BBM * LDR])smem;

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int j = lane & 15, q = lane >> 4;
    const int wm = wave >> 1, wn = wave & 1;

    const int ntiles = tiles_m * tiles_n;
    const int bid = blockIdx.x;
    const int q8 = ntiles >> 3, r8 = ntiles & 7;
    const int xcd = bid & 7, loc = bid >> 3;
    const int tile = xcd * q8 + min(xcd, r8) + loc;
    constexpr int GROUP_M = 8;
    const int per_group = GROUP_M * tiles_n;
    const int first_m = (tile / per_group) * GROUP_M;
    const int gsize = min(tiles_m - first_m, GROUP_M);
    const int in_g = tile - (tile / per_group) * per_group;
    const int tm = first_m + in_g % gsize;
    const int tn = in_g / gsize;

    const int64_t m0 = (int64_t)tm * BBM, n0 = (int64_t)tn * BBN;
    const int64_t K = a.K, M = a.M, N = a.N;
    const int64_t kbeg = (int64_t)blockIdx.z * kc;
    const int64_t kend = min(K, kbeg + kc);
    const int nsteps = (int)((kend - kbeg) / BK);

    const __amdgpu_buffer_rsrc_t ra_rsrc = make_rsrc(a.codes + m0 * K, (uint64_t)(M - m0) * K);
    const __amdgpu_buffer_rsrc_t rw_rsrc =
        make_rsrc(a.wp + n0 * (K >> 1), (uint64_t)(N - n0) * (K >> 1));

    // code staging: two 16-byte chunks per thread (rows r and r + 128).  Only
    // one lane-varying offset per operand lives in a VGPR; the row/column
    // step between chunks and the K position go into the scalar offset.
    const int arow = tid >> 2, ac16 = tid & 3;
    const int aoff = (int)(arow * K + ac16 * 16);
    const int a_step = (int)(128 * K);
    const int lds_off = arow * LDR + ac16 * 16;
    const int woff = (int)((wn * 128 + j) * (K >> 1) + q * 8);
    const int w_step = (int)(16 * (K >> 1));

    auto aload = [&](v4u* r, int64_t k) {
        r[0] = __builtin_amdgcn_raw_buffer_load_b128(ra_rsrc, aoff, (int)k, 0);
        r[1] = __builtin_amdgcn_raw_buffer_load_b128(ra_rsrc, aoff, (int)k + a_step, 0);
    };
    auto astore = [&](const v4u* r, int buf) {
        *(uint4*)(&As[buf][lds_off]) = reorder_even_odd(r[0]);
        *(uint4*)(&As[buf][lds_off + 128 * LDR]) = reorder_even_odd(r[1]);
    };
    auto bload = [&](v2u* dst, int64_t k) {
#pragma unroll
        for (int nt = 0; nt < 8; ++nt)
            dst[nt] = __builtin_amdgcn_raw_buffer_load_b64(rw_rsrc, woff, (int)(k >> 1) + nt * w_step, 0);
    };

    v4i acc[4][8];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) acc[mt][nt] = (v4i){0, 0, 0, 0};

    auto mma = [&](int buf, const v2u* w) {
        v4i af[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
            af[mt] = *(const v4i*)(&As[buf][(wm * 64 + mt * 16 + j) * LDR + q * 16]);
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) {
            const v4i bf = unpack_frag_eo(w[nt]);
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
                acc[mt][nt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[mt], bf, acc[mt][nt], 0, 0, 0);
        }
    };

    // Pipeline: codes for step s+2 are fetched during step s and written to
    // LDS at the end of step s+1; weights for step s+1 are fetched during s.
    // Two named register sets alternate, so no register copies (and no early
    // waits on in-flight loads) are needed.
    v4u ra0[2], ra1[2];
    v2u w0[8], w1[8];
    auto kat = [&](int st) { return kbeg + (int64_t)st * BK; };
    if (nsteps > 0) {
        aload(ra0, kat(0));
        bload(w0, kat(0));
        if (nsteps > 1) aload(ra1, kat(1));
        astore(ra0, 0);
    }
    __syncthreads();
    for (int s = 0; s < nsteps; s += 2) {
        // even step s: A(s) in LDS buf 0, W(s) in w0, A(s+1) in ra1
        if (s + 2 < nsteps) aload(ra0, kat(s + 2));
        if (s + 1 < nsteps) bload(w1, kat(s + 1));
        mma(0, w0);
        if (s + 1 < nsteps) astore(ra1, 1);
        __syncthreads();
        if (s + 1 >= nsteps) break;
        // odd step s+1: A(s+1) in LDS buf 1, W(s+1) in w1, A(s+2) in ra0
        if (s + 3 < nsteps) aload(ra1, kat(s + 3));
        if (s + 2 < nsteps) bload(w0, kat(s + 2));
        mma(1, w1);
        if (s + 2 < nsteps) astore(ra0, 0);
        __syncthreads();
    }

    // ---- epilogue through per-wave 16 x 128 LDS strips (as in the 4-wave
    // kernel); scales and bias are read per strip to keep registers free.
    int* strip = (int*)smem + wave * 16 * W8_EPR;
    const int er = lane >> 2;
    const int ec = (lane & 3) * 32;
    const int64_t col0 = n0 + wn * 128 + ec;
    const bool has_bias = a.bias != nullptr;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
        for (int nt = 0; nt < 8; ++nt)
#pragma unroll
            for (int r = 0; r < 4; ++r) strip[(4 * q + r) * W8_EPR + nt * 16 + j] = acc[mt][nt][r] >> 4;
        __builtin_amdgcn_s_waitcnt(0xc07f);
        __builtin_amdgcn_wave_barrier();
        const int64_t row = m0 + wm * 64 + mt * 16 + er;
        int iv[32];
#pragma unroll
        for (int c4 = 0; c4 < 8; ++c4) {
            const int4 v = *(const int4*)(strip + er * W8_EPR + ec + 4 * c4);
            iv[4 * c4] = v.x; iv[4 * c4 + 1] = v.y; iv[4 * c4 + 2] = v.z; iv[4 * c4 + 3] = v.w;
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);
        __builtin_amdgcn_wave_barrier();
        if (row >= M) continue;
        const bool full = col0 + 32 <= N;
        if constexpr (SPLIT) {
#pragma unroll
            for (int c = 0; c < 32; ++c)
                if (col0 + c < N)
                    atomicAdd((unsigned long long*)(a.acc64 + row * N + col0 + c),
                              (unsigned long long)(int64_t)iv[c]);
        } else {
            if (a.acc_out) {
#pragma unroll
                for (int c = 0; c < 32; ++c)
                    if (col0 + c < N) a.acc_out[row * N + col0 + c] = iv[c];
            }
            const float sa = a.sa[row];
#pragma unroll
            for (int c8 = 0; c8 < 4; ++c8) {
                float o[8];
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    const int64_t col = col0 + c8 * 8 + c;
                    const int64_t cc = col < N ? col : N - 1;
                    float t = mul_rn(mul_rn((float)iv[c8 * 8 + c], sa),
                                     load_any_f32(a.sw_dtype, a.sw, cc));
                    if (has_bias) t = add_rn(t, load_any_f32(a.bias_dtype, a.bias, cc));
                    o[c] = t;
                }
                if constexpr (ODT == F32) {
                    float* dst = (float*)a.out + row * N + col0 + c8 * 8;
                    if (full && (N % 4) == 0) {
                        *(float4*)dst = make_float4(o[0], o[1], o[2], o[3]);
                        *(float4*)(dst + 4) = make_float4(o[4], o[5], o[6], o[7]);
                    } else {
#pragma unroll
                        for (int c = 0; c < 8; ++c)
                            if (col0 + c8 * 8 + c < N) dst[c] = o[c];
                    }
                } else {
                    uint16_t* dst = (uint16_t*)a.out + row * N + col0 + c8 * 8;
                    uint32_t pk[4];
#pragma unroll
                    for (int c2 = 0; c2 < 4; ++c2)
                        pk[c2] = (uint32_t)f32_to_h<ODT>(o[2 * c2]) |
                                 ((uint32_t)f32_to_h<ODT>(o[2 * c2 + 1]) << 16);
                    if (full && (N % 8) == 0) {
                        *(uint4*)dst = make_uint4(pk[0], pk[1], pk[2], pk[3]);
                    } else {
#pragma unroll
                        for (int c = 0; c < 8; ++c)
                            if (col0 + c8 * 8 + c < N) dst[c] = (uint16_t)(pk[c >> 1] >> (16 * (c & 1)));
                    }
                }
            }
        }
    }
}

// -------------------------------------------------------------------------
// Four-wave 256 x 256 kernel, one wave per SIMD: each wave owns a 128 x 128
// block of 8 x 8 v_mfma_i32_16x16x64_i8 tiles whose 256 INT32 accumulators
// live in AGPRs, which halves LDS and weight traffic per MFMA compared with a
// 64 x 128 block.  Loads are buffer loads (zero outside the operands),
// addressed with one lane offset plus a scalar offset; codes are fetched two
// K-steps ahead and weights one step ahead into alternating register sets
// (the loop body covers two steps, so no register copies are needed).
// -------------------------------------------------------------------------
template <int ODT, bool SPLIT>
__global__ __launch_bounds__(256) void w4a4_gemm_w4_kernel(GemmArgs a, int64_t kc, int tiles_m,
                                                           int tiles_n)
{
    extern __shared__ __align__(16) int8_t smem[];
    int8_t (*As)[BBM * LDR] = (int8_t (*)[BBM * LDR])smem;

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int j = lane & 15, q = lane >> 4;
    const int wm = wave >> 1, wn = wave & 1;

    const int ntiles = tiles_m * tiles_n;
    const int bid = blockIdx.x;
    const int q8 = ntiles >> 3, r8 = ntiles & 7;
    const int xcd = bid & 7, loc = bid >> 3;
    const int tile = xcd * q8 + min(xcd, r8) + loc;
    constexpr int GROUP_M = 8;
    const int per_group = GROUP_M * tiles_n;
    const int first_m = (tile / per_group) * GROUP_M;
    const int gsize = min(tiles_m - first_m, GROUP_M);
    const int in_g = tile - (tile / per_group) * per_group;
    const int tm = first_m + in_g % gsize;
    const int tn = in_g / gsize;

    const int64_t m0 = (int64_t)tm * BBM, n0 = (int64_t)tn * BBN;
    const int64_t K = a.K, M = a.M, N = a.N;
    const int64_t kbeg = (int64_t)blockIdx.z * kc;
    const int64_t kend = min(K, kbeg + kc);
    const int nsteps = (int)((kend - kbeg) / BK);

    const __amdgpu_buffer_rsrc_t ra_rsrc = make_rsrc(a.codes + m0 * K, (uint64_t)(M - m0) * K);
    const __amdgpu_buffer_rsrc_t rw_rsrc =
        make_rsrc(a.wp + n0 * (K >> 1), (uint64_t)(N - n0) * (K >> 1));

    // codes: four 16-byte chunks per thread, rows r, r+64, r+128, r+192
    const int arow = tid >> 2, ac16 = tid & 3;
    const int aoff = (int)(arow * K + ac16 * 16);
    const int a_step = (int)(64 * K);
    const int lds_off = arow * LDR + ac16 * 16;
    const int woff = (int)((wn * 128 + j) * (K >> 1) + q * 8);
    const int w_step = (int)(16 * (K >> 1));

    auto aload = [&](v4u* r, int64_t k) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            r[i] = __builtin_amdgcn_raw_buffer_load_b128(ra_rsrc, aoff, (int)k + i * a_step, 0);
    };
    auto astore = [&](const v4u* r, int buf) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            *(uint4*)(&As[buf][lds_off + i * 64 * LDR]) = reorder_even_odd(r[i]);
    };
    auto bload = [&](v2u* dst, int64_t k) {
#pragma unroll
        for (int nt = 0; nt < 8; ++nt)
            dst[nt] = __builtin_amdgcn_raw_buffer_load_b64(rw_rsrc, woff, (int)(k >> 1) + nt * w_step, 0);
    };

    v4i acc[8][8];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) acc[mt][nt] = (v4i){0, 0, 0, 0};

    auto mma = [&](int buf, const v2u* w) {
        v4i bf[8];
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) bf[nt] = unpack_frag_eo(w[nt]);
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
            const v4i af = *(const v4i*)(&As[buf][(wm * 128 + mt * 16 + j) * LDR + q * 16]);
#pragma unroll
            for (int nt = 0; nt < 8; ++nt)
                acc[mt][nt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af, bf[nt], acc[mt][nt], 0, 0, 0);
        }
    };

    v4u ra0[4], ra1[4];
    v2u w0[8], w1[8];
    auto kat = [&](int st) { return kbeg + (int64_t)st * BK; };
    if (nsteps > 0) {
        aload(ra0, kat(0));
        bload(w0, kat(0));
        if (nsteps > 1) aload(ra1, kat(1));
        astore(ra0, 0);
    }
    __syncthreads();
    // pairs of steps; an odd final step is peeled after the loop so the
    // accumulators have a single loop-carried path
    int s = 0;
    for (; s + 1 < nsteps; s += 2) {
        if (s + 2 < nsteps) aload(ra0, kat(s + 2));
        bload(w1, kat(s + 1));
        mma(0, w0);
        astore(ra1, 1);
        __syncthreads();
        if (s + 3 < nsteps) aload(ra1, kat(s + 3));
        if (s + 2 < nsteps) bload(w0, kat(s + 2));
        mma(1, w1);
        if (s + 2 < nsteps) astore(ra0, 0);
        __syncthreads();
    }
    if (s < nsteps) mma(0, w0);

    // ---- epilogue: the tile's weight scales and bias are widened to fp32 in
    // LDS once; then per-wave 16 x 128 int32 strips go through LDS so that a
    // lane owns 32 consecutive columns of one row (16-byte output stores).
    float* scol = (float*)(smem + 4 * 16 * W8_EPR * 4);
    float* bcol = scol + BBN;
    {
        const int64_t col = n0 + tid;
        const int64_t cc = col < N ? col : N - 1;
        scol[tid] = load_any_f32(a.sw_dtype, a.sw, cc);
        bcol[tid] = a.bias ? load_any_f32(a.bias_dtype, a.bias, cc) : 0.0f;
    }
    __syncthreads();
    int* strip = (int*)smem + wave * 16 * W8_EPR;
    const int er = lane >> 2;
    const int ec = (lane & 3) * 32;
    const int64_t col0 = n0 + wn * 128 + ec;
    const float* sc = scol + wn * 128 + ec;
    const float* bc = bcol + wn * 128 + ec;
    const bool has_bias = a.bias != nullptr;
    const bool vec_ok = (col0 + 32 <= N) && (N % 8) == 0;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
#pragma unroll
        for (int nt = 0; nt < 8; ++nt)
#pragma unroll
            for (int r = 0; r < 4; ++r) strip[(4 * q + r) * W8_EPR + nt * 16 + j] = acc[mt][nt][r] >> 4;
        __builtin_amdgcn_s_waitcnt(0xc07f);
        __builtin_amdgcn_wave_barrier();
        const int64_t row = m0 + wm * 128 + mt * 16 + er;
        int iv[32];
#pragma unroll
        for (int c4 = 0; c4 < 8; ++c4) {
            const int4 v = *(const int4*)(strip + er * W8_EPR + ec + 4 * c4);
            iv[4 * c4] = v.x; iv[4 * c4 + 1] = v.y; iv[4 * c4 + 2] = v.z; iv[4 * c4 + 3] = v.w;
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);
        __builtin_amdgcn_wave_barrier();
        if (row < M) {
            if constexpr (SPLIT) {
#pragma unroll
                for (int c = 0; c < 32; ++c)
                    if (col0 + c < N)
                        atomicAdd((unsigned long long*)(a.acc64 + row * N + col0 + c),
                                  (unsigned long long)(int64_t)iv[c]);
            } else {
                const float sa = a.sa[row];
                float o[32];
#pragma unroll
                for (int c = 0; c < 32; ++c) {
                    float t = mul_rn(mul_rn((float)iv[c], sa), sc[c]);
                    o[c] = has_bias ? add_rn(t, bc[c]) : t;
                }
                if constexpr (ODT == F32) {
                    float* dst = (float*)a.out + row * N + col0;
                    if (vec_ok) {
#pragma unroll
                        for (int c4 = 0; c4 < 8; ++c4)
                            *(float4*)(dst + 4 * c4) =
                                make_float4(o[4 * c4], o[4 * c4 + 1], o[4 * c4 + 2], o[4 * c4 + 3]);
                    } else {
                        for (int c = 0; c < 32; ++c)
                            if (col0 + c < N) dst[c] = o[c];
                    }
                } else {
                    uint16_t* dst = (uint16_t*)a.out + row * N + col0;
                    uint32_t pk[16];
#pragma unroll
                    for (int c2 = 0; c2 < 16; ++c2)
                        pk[c2] = (uint32_t)f32_to_h<ODT>(o[2 * c2]) |
                                 ((uint32_t)f32_to_h<ODT>(o[2 * c2 + 1]) << 16);
                    if (vec_ok) {
#pragma unroll
                        for (int c8 = 0; c8 < 4; ++c8)
                            *(uint4*)(dst + 8 * c8) =
                                make_uint4(pk[4 * c8], pk[4 * c8 + 1], pk[4 * c8 + 2], pk[4 * c8 + 3]);
                    } else {
                        for (int c = 0; c < 32; ++c)
                            if (col0 + c < N) dst[c] = (uint16_t)(pk[c >> 1] >> (16 * (c & 1)));
                    }
                }
            }
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
    const bool big = kUseBig && !group && a.lora == nullptr && a.acc_out == nullptr && a.M > 128 &&
                     (a.K % 64) == 0 && aligned;
    if (big && kUseFourWaveV2) {
        const int tm = (int)((a.M + BBM - 1) / BBM), tn = (int)((a.N + BBN - 1) / BBN);
        const unsigned nt = (unsigned)(tm * tn);
        const int64_t kc = a.k_chunk > 0 ? a.k_chunk : a.K;
        const unsigned gz = (unsigned)((a.K + kc - 1) / kc);
        constexpr int epi = 4 * 16 * W8_EPR * 4 + 2 * BBN * 4;
        constexpr int lds = epi > 2 * BBM * LDR ? epi : 2 * BBM * LDR;
        auto go = [&](auto kern) -> hipError_t {
            hipLaunchKernelGGL(kern, dim3(nt, 1, gz), dim3(256), lds, st, a, kc, tm, tn);
            return hipGetLastError();
        };
        if (a.k_chunk > 0) {
            hipLaunchKernelGGL(fill_zero_i64, dim3(1024), dim3(256), 0, st, a.acc64, a.M * a.N);
            hipError_t e = go(w4a4_gemm_w4_kernel<F32, true>);
            if (e != hipSuccess) return e;
            hipLaunchKernelGGL(split_epilogue_kernel, dim3(2048), dim3(256), 0, st, a);
            return hipGetLastError();
        }
        if (a.out_dtype == F32) return go(w4a4_gemm_w4_kernel<F32, false>);
        if (a.out_dtype == F16) return go(w4a4_gemm_w4_kernel<F16, false>);
        return go(w4a4_gemm_w4_kernel<BF16, false>);
    }
    if (big && kUseEightWave) {
        const int tm = (int)((a.M + BBM - 1) / BBM), tn = (int)((a.N + BBN - 1) / BBN);
        const unsigned nt = (unsigned)(tm * tn);
        const int64_t kc = a.k_chunk > 0 ? a.k_chunk : a.K;
        const unsigned gz = (unsigned)((a.K + kc - 1) / kc);
        auto go = [&](auto kern) -> hipError_t {
            hipError_t e = hipFuncSetAttribute((const void*)kern,
                                               hipFuncAttributeMaxDynamicSharedMemorySize, W8_LDS);
            if (e != hipSuccess) return e;
            hipLaunchKernelGGL(kern, dim3(nt, 1, gz), dim3(512), W8_LDS, st, a, kc, tm, tn);
            return hipGetLastError();
        };
        hipError_t e;
        if (a.k_chunk > 0) {
            hipLaunchKernelGGL(fill_zero_i64, dim3(1024), dim3(256), 0, st, a.acc64, a.M * a.N);
            e = go(w4a4_gemm_w8_kernel<F32, true>);
            if (e != hipSuccess) return e;
            hipLaunchKernelGGL(split_epilogue_kernel, dim3(2048), dim3(256), 0, st, a);
            return hipGetLastError();
        }
        if (a.out_dtype == F32) return go(w4a4_gemm_w8_kernel<F32, false>);
        if (a.out_dtype == F16) return go(w4a4_gemm_w8_kernel<F16, false>);
        return go(w4a4_gemm_w8_kernel<BF16, false>);
    }
    if (big) {
        const int tm = (int)((a.M + BBM - 1) / BBM), tn = (int)((a.N + BBN - 1) / BBN);
        const unsigned nt = (unsigned)(tm * tn);
        if (a.k_chunk > 0) {
            const int64_t kc = a.k_chunk;
            const unsigned gz = (unsigned)((a.K + kc - 1) / kc);
            hipLaunchKernelGGL(fill_zero_i64, dim3(1024), dim3(256), 0, st, a.acc64, a.M * a.N);
            hipLaunchKernelGGL((w4a4_gemm_big_kernel<F32, true>), dim3(nt, 1, gz), dim3(256), 0, st,
                               a, kc, tm, tn);
            hipLaunchKernelGGL(split_epilogue_kernel, dim3(2048), dim3(256), 0, st, a);
        } else if (a.out_dtype == F32) {
            hipLaunchKernelGGL((w4a4_gemm_big_kernel<F32, false>), dim3(nt, 1, 1), dim3(256), 0, st,
                               a, a.K, tm, tn);
        } else if (a.out_dtype == F16) {
            hipLaunchKernelGGL((w4a4_gemm_big_kernel<F16, false>), dim3(nt, 1, 1), dim3(256), 0, st,
                               a, a.K, tm, tn);
        } else {
            hipLaunchKernelGGL((w4a4_gemm_big_kernel<BF16, false>), dim3(nt, 1, 1), dim3(256), 0, st,
                               a, a.K, tm, tn);
        }
        return hipGetLastError();
    }
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
