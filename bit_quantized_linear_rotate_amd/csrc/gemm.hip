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
// Design for CDNA4 (three kernels; launch_gemm picks one per call):
//   * w4a4_gemm_ring3_kernel, for prefill-sized layers: persistent, one
//     workgroup per CU walking 256 x 256 output tiles; eight waves, two per
//     SIMD, each a 128 x 64 block of 8 x 4 v_mfma_i32_16x16x64_i8 tiles with
//     its 128 INT32 accumulators in VGPRs.  Codes and packed weights stream
//     global -> LDS through buffer_load ... lds into a three-stage ring, so two
//     K-steps are in flight while one is multiplied; the weights are unpacked
//     in registers right before the MFMAs.
//   * w4a4_gemm_skinny_kernel, for decode-sized M (<= 64): one 1024-thread
//     workgroup per 16 output columns; its sixteen waves split K and their
//     INT32 tiles are summed exactly in LDS.
//   * w4a4_gemm_kernel, for everything else (per-64-group weight scales, the
//     low-rank term with group scales, INT32 export, K-chunked runs, M <= 128):
//     128 x 128 output tile, 4 waves in 2 x 2, each a 64 x 64 block of 4 x 4
//     MFMA tiles; K advances 64 per step with double-buffered LDS and the next
//     step's global loads in flight during the MFMAs.  With group scales each
//     step's INT32 tile is converted and accumulated in fp32 in the order
//     above, with the group's scales staged through LDS alongside the operands.
//   * Packed weights are read as bytes (N, K/2) and unpacked as 16*w: the low
//     nibble shifted into the high half of a byte and the high nibble masked
//     in place are both already sign-correct int8 values, so unpacking is
//     shift/and/perm with no sign extension.  The integer result is divided
//     by 16 (an exact arithmetic shift) before the epilogue.
//   * Workgroups are dealt round-robin over the 8 XCDs; tiles are renumbered
//     so that each XCD works on a contiguous, M-grouped range and its L2 sees
//     shared code rows and weight columns.
//   * When K is too large for INT32 (16 * 7 * 8 * K > 2^31 - 1) or a chunk
//     size is forced, each workgroup accumulates one K-chunk and adds it into
//     an int64 workspace with 64-bit atomics (exact and order-independent);
//     a second kernel applies the epilogue.
#include "common.hpp"
#include "kernels.hpp"

#include <type_traits>

namespace w4a4 {

constexpr int BM = 128, BN = 128, BK = 64, LDR = 80;
constexpr float kMagicF = 12582912.0f;  // C = 1.5 * 2^23: C + i is exact for |i| < 2^22
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

// Buffer resource over `bytes` bytes at `base`: loads past the end read zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint64_t bytes)
{
    const uint32_t n = bytes > 0xffffffffull ? 0xffffffffu : (uint32_t)bytes;
    return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)n, 0x00020000);
}

// GSW: -1 for one weight scale per column, else the dtype of the per-64-group
// weight scales (F32, F16 or BF16)
template <int GSW, bool SPLIT, bool ALIGNED, bool W8 = false, bool AG = false>
__global__ __launch_bounds__(256) void w4a4_gemm_kernel(GemmArgs a, int64_t kc)
{
    // W8: INT8 weights (N, K) taken as they are (no unpack, no factor 16)
    static_assert(!(W8 && GSW >= 0), "INT8 weights come with per-channel scales");
    // AG: activation scales per row and 64-wide K group, sa (M, K / 64): every
    // K step (one group) converts its INT32 tile and accumulates
    // (f32(acc) * sa[row][g]) [* sw[g][col]] in fp32, in increasing g
    static_assert(!(AG && (W8 || SPLIT)), "activation group scales: INT4 weights, whole K");
    constexpr int SHIFT = W8 ? 0 : 4;
    constexpr bool GROUP = GSW >= 0;
    constexpr bool FACC = GROUP || AG;   // per-step fp32 accumulation
    __shared__ __align__(16) int8_t As[2][BM * LDR];
    __shared__ __align__(16) int8_t Bs[2][BN * LDR];
    __shared__ __align__(16) float Ss[GSW >= 0 ? 2 : 1][GSW >= 0 ? 256 : 4];
    // (16-bit group scales on the fast path: -kMagicF * scale / 16 beside each)
    constexpr bool MAGIC = GSW == F16 || GSW == BF16;
    __shared__ __align__(16) float Sc[MAGIC ? 2 : 1][MAGIC ? 256 : 4];
    __shared__ __align__(16) float Sa[AG ? 2 : 1][AG ? BM : 4];

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
    uint4 rw, rw1;
    // ALIGNED without K-chunks (K % 64 == 0): buffer loads over the tile's
    // code rows and weight columns.  The step's k is added to the per-lane
    // offset, never passed as the scalar offset: the range check covers only
    // the per-lane part, so every byte must travel there.  Rows past M and
    // columns past N read zeros; the load past the last step reads the next
    // row of the tile (only into the idle buffer) or, on the tile's last row,
    // falls outside the range and reads zeros.
    constexpr bool BUF = ALIGNED && !SPLIT;
    const __amdgpu_buffer_rsrc_t rca =
        make_rsrc(a.codes + (m0 < M ? m0 : 0) * K, (uint64_t)(m0 < M ? min(M - m0, (int64_t)BM) : 0) * K);
    const int64_t wrow = W8 ? K : (K >> 1);   // weight bytes per column
    const __amdgpu_buffer_rsrc_t rcw = make_rsrc(
        a.wp + (n0 < N ? n0 : 0) * wrow, (uint64_t)(n0 < N ? min(N - n0, (int64_t)BN) : 0) * wrow);
    auto gload = [&](int64_t k) {
        if constexpr (BUF) {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int c = tid + 256 * i;
                ra[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                    rca, (int)((c >> 2) * K + (c & 3) * 16 + k), 0, 0));
            }
            if constexpr (W8) {
                const int wo = (int)((tid >> 1) * K + (tid & 1) * 32 + k);
                rw = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rcw, wo, 0, 0));
                rw1 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rcw, wo + 16, 0, 0));
            } else {
                rw = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                    rcw, (int)((tid >> 1) * (K >> 1) + (tid & 1) * 16 + (k >> 1)), 0, 0));
            }
            return;
        }
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
        if constexpr (W8) {
            const int64_t kw = k + half * 32;   // this thread's 32 weight bytes
            if constexpr (ALIGNED) {
                if (gn < N && kw < kend) {
                    rw = *(const uint4*)(a.wp + gn * K + kw);
                    rw1 = *(const uint4*)(a.wp + gn * K + kw + 16);
                } else {
                    rw = make_uint4(0, 0, 0, 0);
                    rw1 = make_uint4(0, 0, 0, 0);
                }
            } else {
                uint32_t wv[8] = {0, 0, 0, 0, 0, 0, 0, 0};
                if (gn < N)
                    for (int e = 0; e < 32; ++e)
                        if (kw + e < kend)
                            wv[e >> 2] |= (uint32_t)a.wp[gn * K + kw + e] << (8 * (e & 3));
                rw = make_uint4(wv[0], wv[1], wv[2], wv[3]);
                rw1 = make_uint4(wv[4], wv[5], wv[6], wv[7]);
            }
            return;
        }
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
        if constexpr (W8) {
            *(uint4*)(&Bs[buf][n * LDR + half * 32]) = rw;
            *(uint4*)(&Bs[buf][n * LDR + half * 32 + 16]) = rw1;
            return;
        }
        uint4 u0, u1;
        unpack16(rw.x, u0.x, u0.y);
        unpack16(rw.y, u0.z, u0.w);
        unpack16(rw.z, u1.x, u1.y);
        unpack16(rw.w, u1.z, u1.w);
        *(uint4*)(&Bs[buf][n * LDR + half * 32]) = u0;
        *(uint4*)(&Bs[buf][n * LDR + half * 32 + 16]) = u1;
    };

    v4i acc[4][4];
    v4f facc[FACC ? 4 : 1][FACC ? 4 : 1];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = (v4i){0, 0, 0, 0};
    if constexpr (FACC) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) facc[mt][nt] = (v4f){0.f, 0.f, 0.f, 0.f};
    }

    // The K loop. With group scales the MFMA sums carry the weights' factor
    // 16 (high-nibble unpack); FAST multiplies float(16 s) by scale / 16,
    // which is the same real number as s * scale and so rounds to the same
    // float, whenever scale / 16 is exact (every scale but subnormal or NaN
    // ones). It returns false if some scale was not; the workgroup then runs
    // the loop again with the shift back to s.
    // With 16-bit scales FAST also drops the conversion: each group's MFMA
    // starts from the bit pattern of C = 1.5 * 2^23, so the INT32 result is the
    // pattern of the float C + 16 s (|16 s| < 2^22), and one fma
    // (C + 16 s) * (scale / 16) + (-C * scale / 16) rounds the exact real
    // 16 s * scale / 16 = s * scale once: the product the exact path rounds.
    // -C * scale / 16 is exact for a 16-bit scale (at most 11 significant
    // bits, times 3) unless it overflows; a scale whose term is not exact or
    // not finite (Inf, NaN, huge) sends the tile to the exact path too.
    auto kloop = [&](auto fast_c) -> bool {
        constexpr bool FAST = decltype(fast_c)::value;
        bool exact = true;
        // Group scales ride the operand pipeline: thread t loads the scale of
        // column c(t) = (t / 64 % 2) * 64 + (t % 4) * 16 + (t / 4) % 16 with its
        // step's operands and stores it to LDS at slot t (FAST: divided by 16
        // and checked), so that a lane's four columns are one 16-byte read.
        // Threads 128..255 repeat threads 0..127 (no branch: a branch here
        // lets the compiler sink the MFMA conversions past the operand wait).
        // Columns past N read column N - 1 and steps past the end the last
        // group: those values are never used.
        uint32_t rsw = 0;
        const int scl = ((tid >> 6) & 1) * 64 + (tid & 3) * 16 + ((tid >> 2) & 15);
        const uint32_t sc = (uint32_t)min(n0 + scl, N - 1);
        auto sgload = [&](int step) {
            if constexpr (GROUP) {
                const int64_t gidx = min((kbeg + (int64_t)step * BK) / 64, (K + 63) / 64 - 1);
                if constexpr (GSW == F32) rsw = ((const uint32_t*)a.sw + gidx * N)[sc];
                else rsw = ((const uint16_t*)a.sw + gidx * N)[sc];
            }
        };
        auto ssstore = [&](int buf) {
            if constexpr (GROUP) {
                const float v = GSW == F32 ? __uint_as_float(rsw) : h_to_f32<GSW>((uint16_t)rsw);
                float w = v;
                if constexpr (FAST) {
                    w = v * 0.0625f;
                    exact = exact && w * 16.0f == v;
                    if constexpr (MAGIC) {
                        const float c = -kMagicF * w;
                        exact = exact && __builtin_fmaf(-kMagicF, w, -c) == 0.0f && fabsf(c) < 0x1p127f;
                        Sc[buf][tid] = c;
                    }
                }
                Ss[buf][tid] = w;
            }
        };
        // activation scales of the step's group for the tile's 128 rows:
        // thread t loads row t mod 128 (threads 128..255 repeat them, no
        // branch); rows past M read row M - 1 and steps past the end the last
        // group (never used)
        float rsa = 0.0f;
        const int64_t sarow = min(m0 + (tid & 127), M - 1);
        const int64_t G64 = (K + 63) / 64;
        auto saload = [&](int step) {
            if constexpr (AG) {
                const int64_t gidx = min((kbeg + (int64_t)step * BK) / 64, G64 - 1);
                rsa = a.sa[sarow * G64 + gidx];
            }
        };
        auto sastore = [&](int buf) {
            if constexpr (AG) Sa[buf][tid & 127] = rsa;
        };
        if (nsteps > 0) {
            sgload(0);
            saload(0);
            gload(kbeg);
            sstore(0);
            ssstore(0);
            sastore(0);
        }
        __syncthreads();
        for (int s = 0; s < nsteps; ++s) {
            const int buf = s & 1;
            // (past the last step the loads are masked off and the stores
            // fill the idle buffer with zeros: no branch in the loop)
            sgload(s + 1);
            saload(s + 1);
            gload(kbeg + (int64_t)(s + 1) * BK);
            v4i af[4], bf[4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
                af[mt] = *(const v4i*)(&As[buf][(wm * 64 + mt * 16 + j) * LDR + q * 16]);
#pragma unroll
            for (int nt = 0; nt < 4; ++nt)
                bf[nt] = *(const v4i*)(&Bs[buf][(wn * 64 + nt * 16 + j) * LDR + q * 16]);
            if constexpr (AG) {
                v4f swv = (v4f){1.f, 1.f, 1.f, 1.f};
                if constexpr (GROUP) swv = *(const v4f*)(&Ss[buf][(wn * 16 + j) * 4]);
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) {
                    const v4f sav = *(const v4f*)(&Sa[buf][wm * 64 + mt * 16 + 4 * q]);
#pragma unroll
                    for (int nt = 0; nt < 4; ++nt) {
                        v4i t = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[mt], bf[nt], (v4i){0, 0, 0, 0},
                                                                      0, 0, 0);
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            float p = mul_rn((float)(t[r] >> SHIFT), sav[r]);
                            if constexpr (GROUP) p = mul_rn(p, swv[nt]);
                            facc[mt][nt][r] = add_rn(facc[mt][nt][r], p);
                        }
                    }
                }
            } else if constexpr (GROUP && FAST && MAGIC) {
                const v4f swv = *(const v4f*)(&Ss[buf][(wn * 16 + j) * 4]);
                const v4f cv = *(const v4f*)(&Sc[buf][(wn * 16 + j) * 4]);
                const int mg = __float_as_int(-kMagicF) & 0x7fffffff;  // pattern of C
                const v4i c0 = (v4i){mg, mg, mg, mg};
#pragma unroll
                for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                    for (int nt = 0; nt < 4; ++nt) {
                        const v4i t = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[mt], bf[nt], c0, 0, 0, 0);
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            facc[mt][nt][r] = add_rn(facc[mt][nt][r],
                                                     __builtin_fmaf(__int_as_float(t[r]), swv[nt], cv[nt]));
                    }
                // one MFMA, then eight VALU instructions (an earlier result's
                // fma and add), sixteen times
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
                }
            } else if constexpr (GROUP) {
                const v4f swv = *(const v4f*)(&Ss[buf][(wn * 16 + j) * 4]);
#pragma unroll
                for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                    for (int nt = 0; nt < 4; ++nt) {
                        v4i t = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[mt], bf[nt], (v4i){0, 0, 0, 0},
                                                                      0, 0, 0);
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            facc[mt][nt][r] = add_rn(facc[mt][nt][r],
                                                     mul_rn((float)(FAST ? t[r] : t[r] >> 4), swv[nt]));
                    }
                if constexpr (FAST) {
                    // one MFMA, then twelve VALU instructions (converting an
                    // earlier result), sixteen times
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                        __builtin_amdgcn_sched_group_barrier(0x002, 12, 0);
                    }
                }
            } else {
#pragma unroll
                for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                    for (int nt = 0; nt < 4; ++nt)
                        acc[mt][nt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[mt], bf[nt], acc[mt][nt],
                                                                            0, 0, 0);
            }
            // (keep the stores after the MFMAs and conversions: they wait for
            // this step's loads)
            __builtin_amdgcn_sched_barrier(0);
            sstore(buf ^ 1);
            ssstore(buf ^ 1);
            sastore(buf ^ 1);
            __syncthreads();
        }
        return exact;
    };
    if constexpr (GROUP && !AG) {
        if (__syncthreads_or(!kloop(std::true_type{}))) {
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) facc[mt][nt] = (v4f){0.f, 0.f, 0.f, 0.f};
            kloop(std::false_type{});
        }
    } else {
        kloop(std::false_type{});
    }

    // ---- low-rank term (rank <= 32): the tile's rows of L and columns of
    // proj_up go to LDS as fp32 (the staging buffers are free after the loop;
    // ranks padded with zeros to a multiple of 4), and each lane sums
    // l[m,n] = sum_r L[m,r] * up[n,r] for its outputs, one row block at a
    // time, in increasing r with fmaf, four terms per read: the same
    // operations as epilogue_tail
    constexpr int LDL = 36;  // fp32 row stride: 16-byte reads of 16 columns hit distinct banks
    static_assert(BM * LDL * 4 <= 2 * BM * LDR && BN * LDL * 4 <= 2 * BN * LDR, "low-rank staging");
    const bool lds_lora = !SPLIT && a.lora != nullptr && a.rank >= 1 && a.rank <= 32;
    const float* Ls = (const float*)&As[0][0];
    const float* Us = (const float*)&Bs[0][0];
    const int RP = (a.rank + 3) & ~3;
    if (lds_lora) {
        float* Lw = (float*)&As[0][0];
        float* Uw = (float*)&Bs[0][0];
        const int R = a.rank;
        for (int i = tid; i < BM * RP; i += 256) {
            const int rr = i / RP, c = i - rr * RP;
            const int64_t gm = m0 + rr;
            Lw[rr * LDL + c] = (gm < M && c < R) ? a.lora[gm * R + c] : 0.0f;
        }
        for (int i = tid; i < BN * RP; i += 256) {
            const int cc = i / RP, c = i - cc * RP;
            const int64_t gn = n0 + cc;
            Uw[cc * LDL + c] = (gn < N && c < R) ? load_any_f32(a.up_dtype, a.up, gn * R + c) : 0.0f;
        }
        __syncthreads();
    }

    // ---- epilogue: lane (j, q) holds rows 4q..4q+3, column j of each tile.
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
        float lsum[4][4];
        if (lds_lora) {
#pragma unroll
            for (int nt = 0; nt < 4; ++nt)
#pragma unroll
                for (int r = 0; r < 4; ++r) lsum[nt][r] = 0.0f;
            for (int c4 = 0; c4 < RP; c4 += 4) {
                v4f lr[4];
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    lr[r] = *(const v4f*)(Ls + (wm * 64 + mt * 16 + 4 * q + r) * LDL + c4);
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) {
                    const v4f u = *(const v4f*)(Us + (wn * 64 + nt * 16 + j) * LDL + c4);
#pragma unroll
                    for (int r = 0; r < 4; ++r)
#pragma unroll
                        for (int e = 0; e < 4; ++e) lsum[nt][r] = fmaf(lr[r][e], u[e], lsum[nt][r]);
                }
            }
        }
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t row = m0 + wm * 64 + mt * 16 + 4 * q + r;
                const int64_t col = n0 + wn * 64 + nt * 16 + j;
                if (row >= M || col >= N) continue;
                if constexpr (SPLIT) {
                    atomicAdd((unsigned long long*)(a.acc64 + row * N + col),
                              (unsigned long long)(int64_t)(acc[mt][nt][r] >> SHIFT));
                } else {
                    float t;
                    if constexpr (AG) {
                        // activation scales already applied per group; a
                        // per-channel weight scale follows the sum
                        t = facc[mt][nt][r];
                        if constexpr (!GROUP) t = mul_rn(t, load_any_f32(a.sw_dtype, a.sw, col));
                    } else if constexpr (GROUP) {
                        t = mul_rn(facc[mt][nt][r], a.sa[row]);
                    } else {
                        const int32_t iv = acc[mt][nt][r] >> SHIFT;
                        if (a.acc_out) a.acc_out[row * N + col] = iv;
                        t = (float)iv;
                        t = mul_rn(t, a.sa[row]);
                        t = mul_rn(t, load_any_f32(a.sw_dtype, a.sw, col));
                    }
                    if (lds_lora) {
                        t = add_rn(t, lsum[nt][r]);
                        if (a.bias) t = add_rn(t, load_any_f32(a.bias_dtype, a.bias, col));
                    } else {
                        t = epilogue_tail(t, a, row, col);
                    }
                    store_any(a.out_dtype, a.out, row * N + col, t);
                }
            }
    }
}



constexpr int BBM = 256, BBN = 256;

typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v8i __attribute__((ext_vector_type(8)));


// -------------------------------------------------------------------------
// Three-stage persistent kernel (per-channel scales, M > 128, K % 128 == 0):
// one 512-thread workgroup per CU walks its 256 x 256 output tiles; eight
// waves in 2 (M) x 4 (N), two per SIMD, each a 128 x 64 block of 8 x 4
// v_mfma_i32_16x16x64_i8 tiles with its 128 INT32 accumulators in VGPRs; K
// advances 128 per step.
//   * Codes (32 KB per step) and packed weights (16 KB per step) go global ->
//     LDS with buffer_load ... lds (no VGPR staging) into a ring of three
//     48 KB slots.  The ring runs across tiles: the last two steps of a tile
//     fetch the first two stages of the workgroup's next tile, and the
//     epilogue of a tile works in the slot its last step freed, so output
//     stores overlap the next tile's loads.
//   * Codes keep 128-byte rows; eight consecutive fetch lanes read one row's
//     K-slice, so each load instruction covers eight whole 128-byte segments.
//     16-byte chunk c of row r sits at c ^ r3_swz(r).  On gfx950 a
//     ds_read_b128 serves the 64 lanes in four cycles, two per pair of 16-lane
//     groups, split by lane index j (group g lanes with j in {0-3, 12-15}
//     together with group g+1 lanes with j in {4-11}), over 64 four-byte
//     banks; with this swizzle the fragment reads of both k-substeps hit 16
//     distinct 16-byte bank groups in every cycle.
//   * Packed weights keep their 64-byte rows (one per output column), 16-byte
//     chunk c of column n stored at c ^ ((n >> 1) & 3), which spreads a
//     fragment read over all banks.
//   * Every byte offset, row and k included, travels in the per-lane voffset,
//     so the buffer range check covers it: rows past M or N and k past K read
//     as zero, and a missing next tile is a zero-sized buffer.
//   * Waves 0-3 issue all operand loads (twelve 1 KB loads per stage each).
//     Every step they wait only for its own stage (vmcnt leaves the next
//     stage's loads in flight), meet the other waves at a bare s_barrier
//     (__syncthreads would also wait for the loads still in flight) and then
//     put stage s+2 in flight before computing stage s.
//   * Epilogue: each wave rounds its own outputs in registers and stores
//     them through a per-wave LDS strip as 16-byte row-contiguous stores.
//     vmcnt retires in issue order on gfx9, so a loader's output stores,
//     issued after the next tile's first two stages, only delay that tile's
//     first two waits, which count them (a partial tile, whose store count
//     varies, drains them and issues dropped stand-ins instead).
//   * Two waves per SIMD keep the matrix core busy while the other waits on
//     LDS or the barrier; with at most 256 registers per lane the compiler
//     keeps the accumulators in VGPRs, where every MFMA updates its
//     accumulator in place.  A 64-column block per wave keeps the nibble
//     unpacking (VALU) at four weight fragments per step.
//   * Tiles are numbered so that each XCD (workgroups are dealt round-robin
//     over 8, and the grid is a multiple of 8) owns a contiguous, M-grouped
//     range of tiles.
// Lane (j, q) covers k = q*32 .. q*32+31 of a step: k-substep t uses
// k = q*32 + t*16 .. +15 for both operands (low / high half of the lane's 16
// packed weight bytes).
//
// INT8 weights (W8) take the same kernel with K advancing 64 per step: codes
// and weights then both keep 64-byte rows (16 KB each per stage, 32 KB
// slots), 16-byte chunk c of row r at c ^ r3_swz8(r) (with the lane pairing
// above, the 16 lanes of every read cycle hit 16 distinct bank groups), one
// k-substep of 16 bytes per lane, the weights used as they are (no unpack, no
// factor 16), and the epilogue in an LDS area of its own after the three
// slots (an fp32 epilogue does not fit in a 32 KB slot).
// -------------------------------------------------------------------------
constexpr int R3_BK = 128;
constexpr int R3_WAVES = 8;
constexpr int R3_LOADERS = 4;                             // waves 0-3 issue every operand load
// per-variant stage geometry (W8: INT8 weights)
template <bool W8> struct R3Geo {
    static constexpr int BK = W8 ? 64 : R3_BK;                    // K per step
    static constexpr int ASTAGE = BBM * BK;                       // codes: 32 KB / 16 KB
    static constexpr int WSTAGE = W8 ? BBN * BK : BBN * BK / 2;   // weights: 16 KB either way
    static constexpr int SLOT = ASTAGE + WSTAGE;
    static constexpr int ALOADS = ASTAGE / 1024 / R3_LOADERS;     // 1 KB per load: 8 / 4 per loader
    static constexpr int WLOADS = WSTAGE / 1024 / R3_LOADERS;     // 4 per loader
    static constexpr int LPS = ALOADS + WLOADS;                   // loads per stage per loader
    static constexpr int RPL = 1024 / BK;                         // code rows per load
};
constexpr int R3_SLOT = R3Geo<false>::SLOT;
// epilogue strip (16 output rows x 64 columns of one wave) row stride in
// bytes: 64 values + 16 bytes, so that the four 16-lane groups of a 2- or
// 4-byte strip write hit distinct banks and 16-byte reads stay aligned
template <int ODT> constexpr int r3_srb() { return ODT == F32 ? 64 * 4 + 16 : 64 * 2 + 16; }
// one strip per wave, then the column scales, the bias and the row scales
template <int ODT> constexpr int r3_epi_bytes()
{
    return R3_WAVES * 16 * r3_srb<ODT>() + 2 * BBN * 4 + BBM * 4;
}
// output store instructions per wave in a full tile's epilogue (8 row tiles,
// 16 x 64 outputs each, 16 bytes per lane and store)
template <int ODT> constexpr int r3_stores() { return 8 * (16 * 64 * (ODT == F32 ? 4 : 2)) / (64 * 16); }
// s_waitcnt immediate for vmcnt(n), expcnt and lgkmcnt not waited on (gfx9)
constexpr int r3_vmcnt(int n) { return ((n >> 4) << 14) | 0x0f70 | (n & 15); }
static_assert(r3_epi_bytes<F32>() <= R3_SLOT && r3_epi_bytes<BF16>() <= R3_SLOT, "epilogue must fit in one slot");
template <int ODT, bool W8> constexpr int r3_lds_bytes()
{
    return 3 * R3Geo<W8>::SLOT + (W8 ? r3_epi_bytes<ODT>() : 0);
}
static_assert(r3_lds_bytes<F32, true>() <= 160 * 1024 && r3_lds_bytes<F32, false>() <= 160 * 1024, "LDS");

__device__ __forceinline__ v4i r3_half(v4u p, int t)
{
    uint32_t a, b, c, d;
    unpack16(t ? p.z : p.x, a, b);
    unpack16(t ? p.w : p.y, c, d);
    return (v4i){(int)a, (int)b, (int)c, (int)d};
}

// Element i of an n-element fp32/fp16/bf16 vector, with no control flow on
// the dtype, so that several such loads issue before one wait: the dword
// that holds it (r3_scalar_word), then its value (r3_scalar_value).  A
// 16-bit element comes from the aligned dword that holds it; the range check
// covers the vector rounded up to whole dwords (an allocation always spans
// the dword that holds its last 16-bit element).
__device__ __forceinline__ uint32_t r3_scalar_word(const void* base, int dt, int64_t n, int64_t i)
{
    const bool w32 = dt == F32;
    const uint64_t bytes = w32 ? (uint64_t)n * 4 : (((uint64_t)n * 2 + 3) & ~(uint64_t)3);
    const __amdgpu_buffer_rsrc_t r = make_rsrc(base, bytes);
    const int off = w32 ? (int)(i * 4) : (int)((i * 2) & ~(int64_t)3);
    return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
__device__ __forceinline__ float r3_scalar_value(uint32_t w, int dt, int64_t i)
{
    const uint32_t h = (i & 1) ? (w >> 16) : (w & 0xffffu);
    const float hf = dt == BF16 ? __uint_as_float(h << 16) : f16_to_f32((uint16_t)h);
    return dt == F32 ? __uint_as_float(w) : hf;
}

// chunk permutation of code row r in LDS (depends on bits 1 and 2 of r)
__device__ __forceinline__ int r3_swz(int r) { return (((r >> 1) & 1) << 2) | ((r >> 2) & 1); }
// the same for the 64-byte rows of the INT8 variant: 0, 3, 2, 1 by bits 2-3
__device__ __forceinline__ int r3_swz8(int r) { return (4 - ((r >> 2) & 3)) & 3; }

struct R3Tile {
    int64_t m0, n0;
    __amdgpu_buffer_rsrc_t ra, rw;
};

template <bool W8>
__device__ __forceinline__ R3Tile r3_tile(const GemmArgs& a, int t, int ntiles, int tiles_n)
{
    R3Tile r;
    if (t >= ntiles) {  // no such tile: zero-sized buffers, every load reads zero
        r.m0 = 0; r.n0 = 0;
        r.ra = make_rsrc(a.codes, 0);
        r.rw = make_rsrc(a.wp, 0);
        return r;
    }
    const int q8 = ntiles >> 3, r8 = ntiles & 7;
    const int xcd = t & 7, loc = t >> 3;
    const int tile = xcd * q8 + min(xcd, r8) + loc;
    // groups of four tile rows: an XCD's 32 concurrent tiles then span 4 row
    // blocks and 8 column blocks, the pair that keeps the fewest operand bytes
    // (a code row block is twice a packed weight column block) across its L2
    constexpr int GROUP_M = 4;
    const int tiles_m = ntiles / tiles_n;
    const int per_group = GROUP_M * tiles_n;
    const int first_m = (tile / per_group) * GROUP_M;
    const int gsize = min(tiles_m - first_m, GROUP_M);
    const int in_g = tile - (tile / per_group) * per_group;
    r.m0 = (int64_t)(first_m + in_g % gsize) * BBM;
    r.n0 = (int64_t)(in_g / gsize) * BBN;
    r.ra = make_rsrc(a.codes + r.m0 * a.K, (uint64_t)(a.M - r.m0) * a.K);
    const int64_t wrow = W8 ? a.K : (a.K >> 1);   // weight bytes per column
    r.rw = make_rsrc(a.wp + r.n0 * wrow, (uint64_t)(a.N - r.n0) * wrow);
    return r;
}

template <int ODT, bool W8 = false>
__global__ __launch_bounds__(512) void w4a4_gemm_ring3_kernel(GemmArgs a, int tiles_m, int tiles_n)
{
    using G3 = R3Geo<W8>;
    constexpr int BK = G3::BK, SLOT = G3::SLOT, ASTAGE = G3::ASTAGE, LPS = G3::LPS, RPL = G3::RPL;
    constexpr int SHIFT = W8 ? 0 : 4;   // INT4 weights are unpacked as 16 * w
    __shared__ __align__(16) int8_t smem[r3_lds_bytes<ODT, W8>()];

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int j = lane & 15, q = lane >> 4;
    const int wm = wave & 1, wn = wave >> 1;  // 128-row block wm, 64-column block wn

    const int ntiles = tiles_m * tiles_n;
    const int64_t K = a.K, M = a.M, N = a.N;
    const int nsteps = (int)(K / BK);
    int t = blockIdx.x;
    const int G = gridDim.x;

    // Waves 0-3 (one per SIMD) issue every operand load and are the only
    // waves that wait on vmcnt in the K loop; waves 4-7 load the epilogue's
    // scales (their vmcnt never holds an operand load, so that wait does not
    // drain the next tile's stages).
    const bool loader = wave < R3_LOADERS;
    const int lw = wave & (R3_LOADERS - 1);
    // codes: loader lw fills tile rows lw*64 .. lw*64+63, RPL rows per
    // load; lane l writes chunk (l % CPR) of row (l / CPR), i.e. logical
    // chunk (l % CPR) ^ swizzle(row) (the row's low bits are l / CPR).
    constexpr int CPR = BK / 16;   // 16-byte chunks per code row
    const int arow = lane / CPR;
    const int a_vo = (int)(arow * K + (((lane % CPR) ^ (W8 ? r3_swz8(arow) : r3_swz(arow))) * 16));
    const int a_rowl = (int)(RPL * K);
    // weights: loader lw fills tile columns lw*64 .. lw*64+63, sixteen per
    // load; lane l writes chunk (l & 3) of column (l >> 2).
    const int64_t wrow = W8 ? K : (K >> 1);
    const int wsw = W8 ? r3_swz8(lane >> 2) : ((lane >> 3) & 3);
    const int w_vo = (int)((lw * 64 + (lane >> 2)) * wrow + (((lane & 3) ^ wsw) * 16));
    const int w_col16 = (int)(16 * wrow);
    constexpr int WB = W8 ? BK : BK / 2;   // weight bytes per column and step
    auto issue = [&](int slot, const __amdgpu_buffer_rsrc_t& ra, const __amdgpu_buffer_rsrc_t& rw, int st) {
        if (!loader) return;
        int8_t* as = smem + slot * SLOT;
        int8_t* ws = as + ASTAGE;
        const int ka = st * BK, kw = st * WB;
#pragma unroll
        for (int i = 0; i < G3::ALOADS; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                ra, (__attribute__((address_space(3))) void*)(as + (lw * 64 + i * RPL) * BK), 16,
                a_vo + (lw * (64 / RPL) + i) * a_rowl + ka, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < G3::WLOADS; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rw, (__attribute__((address_space(3))) void*)(ws + (lw * 64 + i * 16) * WB), 16,
                w_vo + i * w_col16 + kw, 0, 0, 0);
    };

    v4i acc[8][4];
    // fragment offsets inside a slot
    const int w_ro = W8 ? ASTAGE + (wn * 64 + j) * BK + ((q ^ r3_swz8(j)) * 16)
                        : ASTAGE + (wn * 64 + j) * (BK / 2) + ((q ^ ((j >> 1) & 3)) * 16);
    const int a_ro = (wm * 128 + j) * BK + (W8 ? ((q ^ r3_swz8(j)) * 16) : 0);
    const int a_c0 = ((q * 2) ^ r3_swz(j)) * 16, a_c1 = ((q * 2 + 1) ^ r3_swz(j)) * 16;
    // One step: the weight fragments and the code fragments of substep 0,
    // then those of substep 1 while substep 0 multiplies (W8: one substep).
    auto compute = [&](int slot) {
        const int8_t* as = smem + slot * SLOT + a_ro;
        const int8_t* ws = smem + slot * SLOT + w_ro;
        if constexpr (W8) {
            v4i bf[4], af[8];
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) bf[nt] = *(const v4i*)(ws + nt * 16 * BK);
#pragma unroll
            for (int mt = 0; mt < 8; ++mt) af[mt] = *(const v4i*)(as + mt * 16 * BK);
#pragma unroll
            for (int nt = 0; nt < 4; ++nt)
#pragma unroll
                for (int mt = 0; mt < 8; ++mt)
                    acc[mt][nt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[mt], bf[nt], acc[mt][nt], 0, 0, 0);
            return;
        }
        v4u wp[4];
        v4i af[2][8];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) wp[nt] = *(const v4u*)(ws + nt * 16 * (R3_BK / 2));
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int mt = 0; mt < 8; ++mt)
                af[tt][mt] = *(const v4i*)(as + mt * 16 * BK + (tt ? a_c1 : a_c0));
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
                const v4i bf = r3_half(wp[nt], tt);
#pragma unroll
                for (int mt = 0; mt < 8; ++mt)
                    acc[mt][nt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[tt][mt], bf, acc[mt][nt], 0, 0, 0);
            }
    };

    R3Tile cur_t = r3_tile<W8>(a, t, ntiles, tiles_n);
    R3Tile nxt_t = r3_tile<W8>(a, t + G, ntiles, tiles_n);
    // Loads are issued unconditionally: stages past the end of a tile belong
    // to the next tile (or read zeros when there is none), so the loop carries
    // no control flow around them.
    issue(0, cur_t.ra, cur_t.rw, 0);
    issue(1, cur_t.ra, cur_t.rw, 1);
    int cur = 0, nxt2 = 2;
    // vmcnt retires in issue order (gfx9): after a full tile's epilogue the
    // loader's own r3_stores() output stores sit behind the next tile's first
    // two stages, so steps 0 and 1 may leave them in flight
    static_assert(LPS + r3_stores<ODT>() <= 63, "vmcnt range");
    // exactly r3_stores() stores behind the first two stages, as after every
    // full tile: dropped stores through a zero-sized buffer
    auto pad_stores = [&]() {
        if (!loader) return;
        const __amdgpu_buffer_rsrc_t none = make_rsrc(a.out, 0);
        // distinct offsets and the volatile bit: none of them may be merged
        // or dropped by the compiler (the hardware drops them all)
#pragma unroll
        for (int i = 0; i < r3_stores<ODT>(); ++i)
            __builtin_amdgcn_raw_buffer_store_b32(0u, none, 4 * i, 0, (int)0x80000000);
    };
    pad_stores();
    for (;;) {
#pragma unroll
        for (int mt = 0; mt < 8; ++mt)
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = (v4i){0, 0, 0, 0};
        for (int s = 0; s < nsteps; ++s) {
            if (loader) {
                // Stage s has landed once vmcnt drops to LPS (the next stage's
                // loads may still be in flight); in steps 0 and 1 the previous
                // tile's r3_stores() output stores (or as many dropped stand-ins),
                // issued after this tile's first two stages, may be in flight
                // too.  One asm block with its own scalar branch, so that the
                // loop body keeps a single basic block around the MFMAs.
                asm volatile(
                    "s_cmp_lt_u32 %0, 2\n\t"
                    "s_cbranch_scc0 1f\n\t"
                    "s_waitcnt vmcnt(%1)\n\t"
                    "s_branch 2f\n"
                    "1:\n\t"
                    "s_waitcnt vmcnt(%2)\n"
                    "2:" ::"s"(s), "n"(LPS + r3_stores<ODT>()), "n"(LPS) : "memory", "scc");
            }
            __builtin_amdgcn_s_barrier();
            const bool same = s + 2 < nsteps;
            issue(nxt2, same ? cur_t.ra : nxt_t.ra, same ? cur_t.rw : nxt_t.rw,
                  same ? s + 2 : s + 2 - nsteps);
            __builtin_amdgcn_sched_barrier(0);
            compute(cur);
            cur = cur == 2 ? 0 : cur + 1;
            nxt2 = nxt2 == 2 ? 0 : nxt2 + 1;
        }

        // ---- epilogue in the slot the last step used (every wave has left it
        // after the barrier below); the next tile's first two stages are
        // already in flight into the other two.  Waves 4-7 stage the column
        // scales, bias and row scales in LDS.  Every wave then applies the
        // epilogue to its own accumulators in registers, writes each row
        // tile's rounded 16 x 64 outputs as a strip in LDS, reads it back
        // row-contiguous and stores it with 16-byte stores.  A loader wave's
        // stores stay in flight into the next tile's first two steps (the
        // wait there counts them).
        // (W8: the area after the three slots)
        int8_t* eslot = W8 ? smem + 3 * SLOT : smem + nxt2 * SLOT;  // == slot of the step just computed
        __builtin_amdgcn_s_barrier();
        constexpr int SRB = r3_srb<ODT>();
        constexpr int ESZ = ODT == F32 ? 4 : 2;
        int8_t* strips = eslot;
        float* scol = (float*)(eslot + R3_WAVES * 16 * SRB);
        float* bcol = scol + BBN;
        float* srow = bcol + BBN;
        const int64_t m0 = cur_t.m0, n0 = cur_t.n0;
        const bool has_bias = a.bias != nullptr;
        if (!loader) {
            // one round trip per tile for the column scales, the bias and the
            // row scales (waves 4-7 only: their vmcnt holds no operand
            // load); three branch-free loads, then one wait
            const int c = tid - R3_LOADERS * 64;
            const int64_t col = n0 + c, row = m0 + c;
            const int64_t cc = col < N ? col : N - 1;
            const int bdt = has_bias ? a.bias_dtype : a.sw_dtype;
            const uint32_t ws = r3_scalar_word(a.sw, a.sw_dtype, N, cc);
            const uint32_t wb = r3_scalar_word(has_bias ? a.bias : a.sw, bdt, N, cc);
            const uint32_t wr = r3_scalar_word(a.sa, F32, M, row < M ? row : M - 1);
            scol[c] = r3_scalar_value(ws, a.sw_dtype, cc);
            bcol[c] = has_bias ? r3_scalar_value(wb, bdt, cc) : 0.0f;
            srow[c] = __uint_as_float(wr);
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): LDS writes done
        __builtin_amdgcn_s_barrier();
        float scl[4], bia[4];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            scl[nt] = scol[wn * 64 + nt * 16 + j];
            bia[nt] = bcol[wn * 64 + nt * 16 + j];
        }
        // a full tile with 16-byte aligned rows stores with no per-lane checks
        const bool full = m0 + BBM <= M && n0 + BBN <= N && (N % 8) == 0;
        // each wave writes its own strip: 16-byte chunk `ch` of strip row `rr`;
        // VPC outputs per chunk, CPR chunks per strip row
        constexpr int VPC = 16 / ESZ, CPR = 64 / VPC, CHUNKS = 16 * CPR, PER_LANE = CHUNKS / 64;
        static_assert(PER_LANE == 2 || PER_LANE == 4, "strip read asm below");
        int8_t* mine = strips + wave * 16 * SRB;
        using lds_ptr = const __attribute__((address_space(3))) int8_t*;
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
            // this wave's 16 x 64 outputs of row tile mt, rounded, into its strip
            const float* sr = srow + wm * 128 + mt * 16 + 4 * q;
            const float sa[4] = {sr[0], sr[1], sr[2], sr[3]};
#pragma unroll
            for (int nt = 0; nt < 4; ++nt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float tv = mul_rn(mul_rn((float)(acc[mt][nt][r] >> SHIFT), sa[r]), scl[nt]);
                    const float o = has_bias ? add_rn(tv, bia[nt]) : tv;
                    int8_t* dst = mine + (4 * q + r) * SRB + (nt * 16 + j) * ESZ;
                    if constexpr (ODT == F32)
                        *(float*)dst = o;
                    else
                        *(uint16_t*)dst = f32_to_h<ODT>(o);
                }
            // read the strip back row-contiguous: one asm block with its own
            // wait, since the compiler would otherwise put a vmcnt(0) before
            // the first read (it cannot tell the strip from the LDS-DMA
            // targets), which would stall on this wave's stores and loads
            v4u vv[PER_LANE];
            lds_ptr la[PER_LANE];
#pragma unroll
            for (int i = 0; i < PER_LANE; ++i) {
                const int c = lane + 64 * i;
                la[i] = (lds_ptr)(mine + (c / CPR) * SRB + (c % CPR) * 16);
            }
            __builtin_amdgcn_s_waitcnt(0xc07f);
            __builtin_amdgcn_wave_barrier();
            if constexpr (PER_LANE == 2) {
                asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %3\n\ts_waitcnt lgkmcnt(0)"
                             : "=v"(vv[0]), "=v"(vv[1]) : "v"(la[0]), "v"(la[1]) : "memory");
            } else {
                asm volatile("ds_read_b128 %0, %4\n\tds_read_b128 %1, %5\n\t"
                             "ds_read_b128 %2, %6\n\tds_read_b128 %3, %7\n\ts_waitcnt lgkmcnt(0)"
                             : "=v"(vv[0]), "=v"(vv[1]), "=v"(vv[2]), "=v"(vv[3])
                             : "v"(la[0]), "v"(la[1]), "v"(la[2]), "v"(la[3]) : "memory");
            }
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int i = 0; i < PER_LANE; ++i) {
                const int c = lane + 64 * i;
                const int rr = c / CPR, ch = c % CPR;
                const uint4 v = make_uint4(vv[i][0], vv[i][1], vv[i][2], vv[i][3]);
                const int64_t row = m0 + wm * 128 + mt * 16 + rr;
                const int64_t col0 = n0 + wn * 64 + ch * VPC;
                int8_t* dst = (int8_t*)a.out + (row * N + col0) * ESZ;
                if (full) {
                    *(uint4*)dst = v;
                } else if (row < M) {
                    if (col0 + VPC <= N && (N % 8) == 0) {
                        *(uint4*)dst = v;
                    } else {
                        const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                        for (int e = 0; e < VPC; ++e) {
                            if (col0 + e >= N) break;
                            if constexpr (ODT == F32)
                                ((uint32_t*)dst)[e] = w4[e];
                            else
                                ((uint16_t*)dst)[e] = (uint16_t)(w4[e >> 1] >> (16 * (e & 1)));
                        }
                    }
                }
            }
            // one row tile at a time: only its accumulators and addresses live
            __builtin_amdgcn_sched_barrier(0);
        }
        if (!full && loader) {
            // a partial tile's stores vary in number: drain them (and the
            // next tile's first two stages), then stand in for them
            __builtin_amdgcn_s_waitcnt(r3_vmcnt(0));
            pad_stores();
        }
        t += G;
        if (t >= ntiles) break;
        cur_t = nxt_t;
        nxt_t = r3_tile<W8>(a, t + G, ntiles, tiles_n);
    }
    __builtin_amdgcn_s_waitcnt(0x0070);
}

// -------------------------------------------------------------------------
// w4a4_gemm_pp_kernel: the prefill kernel with the two waves of every SIMD
// taking turns ("ping-pong").  Same 256 x 256 tiles, 128-deep K steps, three
// 48 KB LDS-DMA slots, LDS layout of the codes and XCD-aware tile order as
// the kernel above, but:
//   * The eight waves form two groups of four, one wave of each per SIMD
//     (group A: waves 0-3, group B: waves 4-7).  Each wave alternates a
//     memory phase (the LDS fragment reads of one K step, then its group's
//     part of the stage two steps ahead: group A's waves the codes, group B's
//     the packed weights) and a compute phase (the step's 64
//     MFMAs, the nibble unpack of the weights interleaved with them at 1.25
//     VALU instructions per MFMA, which the SIMD issues beside the matrix
//     core).  Group B runs one phase behind group A, so on every SIMD one wave
//     computes while the other reads: the matrix core is fed by one wave at a
//     time and does not wait for LDS.  Every phase ends at a workgroup
//     barrier.
//   * A stage's slot is read only in the two groups' memory phases of its
//     step; each group puts its part of stage s+2 in flight into the slot of
//     stage s-1 in its memory phase of step s (after both groups' reads of
//     step s-1), and waits for its part of stage s+1 before the barrier that
//     precedes group A's memory phase of step s+1: group A at the end of its
//     compute phase of step s (its codes have four phases to land), group B
//     at the end of its memory phase of step s (its weights, a third of the
//     bytes, have two).  Splitting the loads shortens group A's memory
//     phase, the longer of the two.
//   * The MFMA takes the weights as its first operand: lane (j, q) then holds
//     output row j and output columns 4q .. 4q+3 of every 16 x 16 tile.  The
//     weight columns of a wave's four column tiles are interleaved (tile nt,
//     MFMA row c is column 16 (c >> 2) + 4 nt + (c & 3)), so a lane holds
//     sixteen consecutive columns of one row and the epilogue writes them
//     from registers with 16-byte stores.  Packed weight column n keeps its
//     16-byte chunk c at c ^ pp_wswz(n) in LDS, which spreads these reads
//     over all banks.
//   * A tile's column scales, bias and row scales are staged in LDS by group
//     B in the tile's first two memory phases (two buffers, used by
//     alternate tiles).
//   * Each group's epilogue is a phase of its own; group A's overlaps group
//     B's last compute phase.  Output rows past M and columns past N are
//     dropped by the buffer range check, so every wave issues the same
//     number of stores in every tile (the wait that counts them stays exact).
// Lane (j, q) covers k = q*32 .. q*32+31 of a step, k-substep t the sixteen
// from q*32 + t*16, as in the kernel above.
// -------------------------------------------------------------------------
constexpr int PP_SCL = 3 * BBN * 4;                 // column scales, bias, row scales (f32)
constexpr int PP_LDS = 3 * R3_SLOT + 2 * PP_SCL;    // 150 KB
static_assert(BBM == BBN && PP_LDS <= 160 * 1024, "LDS");
// output store instructions per wave and tile (8 row tiles, 16 values per lane)
template <int ODT> constexpr int pp_stores() { return 8 * (ODT == F32 ? 4 : 2); }
// chunk permutation of packed weight column n in LDS (bits 4-5 of n: 0, 2, 3, 1)
__device__ __forceinline__ int pp_wswz(int n) { return (0x78 >> (2 * ((n >> 4) & 3))) & 3; }

// two f32 values rounded to the 16-bit output format, low half first
template <int ODT> __device__ __forceinline__ uint32_t pp_pack2(float lo, float hi)
{
    typedef float f2 __attribute__((ext_vector_type(2)));
    if constexpr (ODT == BF16) {
        typedef __bf16 h2 __attribute__((ext_vector_type(2)));
        return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2){lo, hi}, h2));
    } else {
        typedef _Float16 h2 __attribute__((ext_vector_type(2)));
        return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2){lo, hi}, h2));
    }
}

template <int ODT>
__global__ __launch_bounds__(512) void w4a4_gemm_pp_kernel(GemmArgs a, int tiles_m, int tiles_n)
{
    // loads per stage and wave: LPS for both parts (the first two stages, by
    // group A), LPA codes (group A), LPB weights (group B)
    constexpr int BK = R3_BK, SLOT = R3_SLOT, ASTAGE = BBM * BK, LPS = 12, LPA = 8, LPB = 4;
    constexpr int ST = pp_stores<ODT>(), ESZ = ODT == F32 ? 4 : 2;
    using lds_vptr = __attribute__((address_space(3))) void*;
    __shared__ __align__(16) int8_t smem[PP_LDS];

    const int tid = threadIdx.x;
    // (the wave index is uniform: LDS destinations of the DMA stay scalar)
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int j = lane & 15, q = lane >> 4;
    const bool grp_a = wave < 4;
    const int wm = wave & 1, wn = wave >> 1;  // 128-row block wm, 64-column block wn

    const int ntiles = tiles_m * tiles_n;
    const int64_t K = a.K, M = a.M, N = a.N;
    const int nsteps = (int)(K / BK);
    int t = blockIdx.x;
    const int G = gridDim.x;
    if (t >= ntiles) return;  // (the whole workgroup)

    // DMA by group A, wave lw: code rows lw*64 + 8 i + (lane >> 3) (chunk
    // (lane & 7) of the row's 128 bytes, stored at position (lane & 7)), packed
    // weight columns lw*64 + 16 i + (lane >> 2) (chunk (lane & 3) ^ swizzle
    // stored at position (lane & 3)).  Row and column offsets travel in the
    // voffset, so the range check drops rows past M and columns past N; the
    // step's K offset is the scalar offset.
    const int lw = wave & 3;
    const int arow = lane >> 3;
    const int a_vo = (int)((lw * 64 + arow) * K + (((lane & 7) ^ r3_swz(arow)) * 16));
    const int a_rowl = (int)(8 * K);
    const int64_t wrow = K >> 1;
    const int w_vo = (int)((lw * 64 + (lane >> 2)) * wrow);
    const int w_col16 = (int)(16 * wrow);
    // part: 1 the codes, 2 the weights, 3 both
    auto issue = [&](int slot, const __amdgpu_buffer_rsrc_t& ra, const __amdgpu_buffer_rsrc_t& rw, int st, int part,
                     bool rev) {
        int8_t* as = smem + slot * SLOT;
        int8_t* ws = as + ASTAGE;
        // tiles of odd rounds walk K backward: their first steps read the
        // code slices the previous round read last, still in L2 (the integer
        // sum does not depend on the order)
        const int kst = rev ? nsteps - 1 - st : st;
        const int ka = kst * BK, kw = kst * (BK / 2);
        if (part & 1)
#pragma unroll
        for (int i = 0; i < 8; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_vptr)(as + (lw * 64 + i * 8) * BK), 16,
                                                     a_vo + i * a_rowl, ka, 0, 0);
        if (part & 2)
#pragma unroll
        for (int i = 0; i < 4; ++i)  // column lw*64 + 16 i + c has swizzle pp_wswz = entry i
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rw, (lds_vptr)(ws + (lw * 64 + i * 16) * (BK / 2)), 16,
                w_vo + i * w_col16 + (((lane & 3) ^ ((0x78 >> (2 * i)) & 3)) * 16), kw, 0, 0);
    };

    // fragment offsets inside a slot: code row wm*128 + 16 mt + j, chunks
    // 2q and 2q+1; weight column wcol + 4 nt, chunk q
    const int a_ro = (wm * 128 + j) * BK;
    const int a_c0 = ((q * 2) ^ r3_swz(j)) * 16, a_c1 = ((q * 2 + 1) ^ r3_swz(j)) * 16;
    const int wcol = wn * 64 + 16 * (j >> 2) + (j & 3);
    const int w_ro = ASTAGE + wcol * (BK / 2) + ((q ^ pp_wswz(wcol)) * 16);
    v4u wp[4];
    v4i af[2][8];
    v4i acc[8][4];
    auto mem = [&](int slot) {
        const int8_t* as = smem + slot * SLOT + a_ro;
        const int8_t* ws = smem + slot * SLOT + w_ro;
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) wp[nt] = *(const v4u*)(ws + nt * 4 * (BK / 2));
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int mt = 0; mt < 8; ++mt)
                af[tt][mt] = *(const v4i*)(as + mt * 16 * BK + (tt ? a_c1 : a_c0));
    };
    // compute phase: eight groups of eight MFMAs (group g: substep g >> 2,
    // column tile g & 3); group 0's weights are unpacked at the end of the
    // memory phase, group g+1's (ten VALU instructions) two at a time between
    // group g's first five MFMAs, each group a scheduling region of its own
    v4i bfc;
    auto unpack0 = [&]() { bfc = r3_half(wp[0], 0); };
    auto comp = [&]() {
#pragma unroll
        for (int g = 0; g < 8; ++g) {
            const int tt = g >> 2, nt = g & 3;
            const v4i bfn = g < 7 ? r3_half(wp[(g + 1) & 3], (g + 1) >> 2) : bfc;
#pragma unroll
            for (int mt = 0; mt < 8; ++mt)
                acc[mt][nt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(bfc, af[tt][mt], acc[mt][nt], 0, 0, 0);
            if (g < 7) {
#pragma unroll
                for (int m = 0; m < 5; ++m) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
                }
                __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
            bfc = bfn;
        }
    };

    // group B stages the tile's column scales, bias and row scales in LDS
    // as they are stored (DMA, no registers): wave b = wave - 4 moves bytes
    // 256 b .. 256 b + 255 of each; the epilogue widens them to f32.  Always
    // three loads a wave (a zero-sized resource where there is nothing to
    // move: zeros into an unused part of the buffer), so that group B's wait
    // counts a fixed number of operations
    const bool has_bias = a.bias != nullptr;
    const int sw_sz = a.sw_dtype == F32 ? 4 : 2, b_sz = has_bias && a.bias_dtype != F32 ? 2 : 4;
    auto scale_issue = [&](int par, int64_t m0, int64_t n0) {
        int8_t* sc = smem + 3 * SLOT + par * PP_SCL;
        const int b = wave - 4;
        const int vo = b * 256 + lane * 4;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            make_rsrc((const int8_t*)a.sw + n0 * sw_sz, b * 256 < BBN * sw_sz ? (uint64_t)(N - n0) * sw_sz : 0),
            (lds_vptr)(sc + b * 256), 4, vo, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            make_rsrc(has_bias ? (const int8_t*)a.bias + n0 * b_sz : (const int8_t*)a.sw,
                      has_bias && b * 256 < BBN * b_sz ? (uint64_t)(N - n0) * b_sz : 0),
            (lds_vptr)(sc + BBN * 4 + b * 256), 4, vo, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(a.sa + m0, (uint64_t)(M - m0) * 4),
                                                 (lds_vptr)(sc + 2 * BBN * 4 + b * 256), 4, vo, 0, 0, 0);
    };

    // epilogue: lane (j, q) of wave (wm, wn) holds, for row tile mt, row
    // wm*128 + 16 mt + j and columns c0 .. c0+15, value i = 4 nt + r in
    // acc[mt][nt][r]
    const int c0 = wn * 64 + 16 * q;
    auto epi = [&](int par, int64_t m0, int64_t n0) {
        // The lane's offsets are formed here, every tile, from values the
        // compiler cannot see through: hoisted out of the tile loop they
        // would take registers the K loop needs.
        int scl = c0 * 4, row0 = (wm * 128 + j) * 4;
        asm volatile("" : "+v"(scl), "+v"(row0));
        const int8_t* sc = smem + 3 * SLOT + par * PP_SCL;
        // the sixteen column scales and biases of this lane, widened to f32
        v4f swv[4], bv[4];
        auto widen = [&](v4f* dst, const int8_t* base, int dt) {
            if (dt == F32) {
#pragma unroll
                for (int i = 0; i < 4; ++i) dst[i] = *(const v4f*)(base + scl + 16 * i);
            } else {
                const v4u h0 = *(const v4u*)(base + scl / 2), h1 = *(const v4u*)(base + scl / 2 + 16);
                const uint32_t w[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const uint16_t hb = (uint16_t)(w[i >> 1] >> (16 * (i & 1)));
                    dst[i >> 2][i & 3] = dt == BF16 ? bf16_to_f32(hb) : f16_to_f32(hb);
                }
            }
        };
        widen(swv, sc, a.sw_dtype);
        if (has_bias) widen(bv, sc + BBN * 4, a.bias_dtype);
        const int64_t rows = M - m0 < BBM ? M - m0 : BBM;
        const uint32_t nrec = (uint32_t)((rows * N - n0) * ESZ);
        const __amdgpu_buffer_rsrc_t ro =
            __builtin_amdgcn_make_buffer_rsrc((void*)((int8_t*)a.out + (m0 * N + n0) * ESZ), (short)0, (int)nrec,
                                              0x00020000);
        // byte offset of (row wm*128 + j, column c0), or past the end for
        // columns past N (dropped); row tile mt adds 16 mt rows
        uint32_t off = n0 + c0 < N ? (uint32_t)(((wm * 128 + j) * N + c0) * ESZ) : nrec;
        asm volatile("" : "+v"(off));
        const uint32_t rstep = (uint32_t)(16 * N * ESZ);
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
            const float sa = *(const float*)(sc + 2 * BBN * 4 + row0 + 64 * mt);
            float o[16];
#pragma unroll
            for (int nt = 0; nt < 4; ++nt)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float tv = mul_rn(mul_rn((float)(acc[mt][nt][e] >> 4), sa), swv[nt][e]);
                    o[4 * nt + e] = has_bias ? add_rn(tv, bv[nt][e]) : tv;
                }
            const uint32_t o_mt = off + mt * rstep;
            if constexpr (ODT == F32) {
#pragma unroll
                for (int h = 0; h < 4; ++h)
                    __builtin_amdgcn_raw_buffer_store_b128(
                        (v4u){__float_as_uint(o[4 * h]), __float_as_uint(o[4 * h + 1]), __float_as_uint(o[4 * h + 2]),
                              __float_as_uint(o[4 * h + 3])},
                        ro, o_mt + 16 * h, 0, 0);
            } else {
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    __builtin_amdgcn_raw_buffer_store_b128(
                        (v4u){pp_pack2<ODT>(o[8 * h], o[8 * h + 1]), pp_pack2<ODT>(o[8 * h + 2], o[8 * h + 3]),
                              pp_pack2<ODT>(o[8 * h + 4], o[8 * h + 5]), pp_pack2<ODT>(o[8 * h + 6], o[8 * h + 7])},
                        ro, o_mt + 16 * h, 0, 0);
            }
        }
    };

    R3Tile cur_t = r3_tile<false>(a, t, ntiles, tiles_n);
    R3Tile nxt_t = r3_tile<false>(a, t + G, ntiles, tiles_n);
    if (grp_a) {
        issue(0, cur_t.ra, cur_t.rw, 0, 3, (t / G) & 1);
        issue(1, cur_t.ra, cur_t.rw, 1, 3, (t / G) & 1);
        // stand-ins for a previous tile's output stores, so that the wait of
        // every tile's first compute phase counts the same operations
        const __amdgpu_buffer_rsrc_t none = make_rsrc(a.out, 0);
#pragma unroll
        for (int i = 0; i < ST; ++i) __builtin_amdgcn_raw_buffer_store_b32(0u, none, 4 * i, 0, (int)0x80000000);
        __builtin_amdgcn_s_waitcnt(r3_vmcnt(LPS + ST));  // stage 0 landed
    }
    __builtin_amdgcn_s_barrier();
    if (!grp_a) __builtin_amdgcn_s_barrier();  // group B: one phase behind
    __builtin_amdgcn_sched_barrier(0);
    int slot = 0, par = 0;
    for (;;) {
#pragma unroll
        for (int mt = 0; mt < 8; ++mt)
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = (v4i){0, 0, 0, 0};
        for (int s = 0; s < nsteps; ++s) {
            // ---- memory phase: the fragment reads first, then the group's
            // DMA, whose issue takes a while, under their latency
            const int nslot = slot == 0 ? 2 : slot - 1;  // (slot + 2) % 3
            mem(slot);
            {
                const bool same = s + 2 < nsteps;
                if (!grp_a && s == 0) scale_issue(par, cur_t.m0, cur_t.n0);
                issue(nslot, same ? cur_t.ra : nxt_t.ra, same ? cur_t.rw : nxt_t.rw, same ? s + 2 : s + 2 - nsteps,
                      grp_a ? 1 : 2, ((same ? t : t + G) / G) & 1);
            }
            if (!grp_a) {
                // group B: its weights of stage s+1 landed (the scales of the
                // tile, issued before its stage-2 weights, by step 1).  After
                // them this wave has issued this step's weights and, in a
                // tile's first step, the previous tile's output stores and the
                // scale loads before them (the first tile: stage 1 came from
                // group A, so the wait has nothing to do)
                asm volatile(
                    "s_cmp_eq_u32 %0, 0\n\t"
                    "s_cbranch_scc0 1f\n\t"
                    "s_waitcnt vmcnt(%1)\n\t"
                    "s_branch 2f\n"
                    "1:\n\t"
                    "s_waitcnt vmcnt(%2)\n"
                    "2:" ::"s"(s), "n"(ST + 3 + LPB), "n"(LPB) : "memory", "scc");
            }
            __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): fragments in
            unpack0();
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);
            // ---- compute phase
            comp();
            if (grp_a) {
                // its codes of stage s+1 landed: after them this wave has
                // issued stage s+2's codes and, in a tile's first step, the
                // previous tile's output stores (or their stand-ins) before
                // them
                asm volatile(
                    "s_cmp_eq_u32 %0, 0\n\t"
                    "s_cbranch_scc0 1f\n\t"
                    "s_waitcnt vmcnt(%1)\n\t"
                    "s_branch 2f\n"
                    "1:\n\t"
                    "s_waitcnt vmcnt(%2)\n"
                    "2:" ::"s"(s), "n"(LPA + ST), "n"(LPA) : "memory", "scc");
            }
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);
            slot = slot == 2 ? 0 : slot + 1;
        }
        // ---- epilogue phase
        epi(par, cur_t.m0, cur_t.n0);
        t += G;
        if (t >= ntiles) break;
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        cur_t = nxt_t;
        nxt_t = r3_tile<false>(a, t + G, ntiles, tiles_n);
        par ^= 1;
    }
    if (grp_a) __builtin_amdgcn_s_barrier();  // pairs with group B's last
}

// -------------------------------------------------------------------------
// FP6 variant of the persistent kernel (gfx950 f8f6f4 MFMA).  Codes in
// [-7, 7] and weights in [-8, 7] are exact in bf6 (e3m2: sign, 3 exponent bits
// with bias 3, 2 mantissa bits), their products are small integers, and the
// fp32 accumulator holds every partial sum exactly while |sum| < 2^24 (56 K <
// 2^24): the accumulator is the exact integer sum, the same value the INT8
// kernels convert, so the epilogue gives the same bits.  v_mfma_f32_16x16x128
// _f8f6f4 takes 128 K per instruction at twice the INT8 rate.
//   * Format of both operands ("bf6 blocks"): each run of 32 consecutive K
//     values is 24 bytes, value e in bits 6e .. 6e+5 of the little-endian
//     192-bit block, followed by 8 unused bytes; a row of K values is K bytes
//     (the layout of one lane's MFMA operand: lane (i, q) holds K values
//     32 q .. 32 q + 31 of row or column i).
//   * 256 x 128 tiles, K 128 per step; codes (32 KB) and weights (16 KB) per
//     stage both keep 128-byte rows in LDS with the INT4 kernel's chunk
//     swizzle and buffer_load ... lds pattern (twelve 1 KB loads per loader
//     wave and stage), three 48 KB slots, the ring running across tiles.
//   * Eight waves in 4 (M) x 2 (N), each a 64 x 64 block of 4 x 4 MFMAs with
//     fp32 accumulators; a fragment is the 16 + 8 bytes of chunks 2q and 2q+1.
//   * Epilogue, loader roles and waits as in the INT4 kernel.
// -------------------------------------------------------------------------
constexpr int B6_BN = 128;
constexpr int B6_BK = 128;                              // K per step (bytes per row per step)
constexpr int B6_ASTAGE = BBM * B6_BK;                  // 32 KB
constexpr int B6_WSTAGE = B6_BN * B6_BK;                // 16 KB
constexpr int B6_SLOT = B6_ASTAGE + B6_WSTAGE;
constexpr int B6_ALOADS = B6_ASTAGE / 1024 / R3_LOADERS;   // 8
constexpr int B6_WLOADS = B6_WSTAGE / 1024 / R3_LOADERS;   // 4
constexpr int B6_LPS = B6_ALOADS + B6_WLOADS;
template <int ODT> constexpr int b6_stores() { return 4 * (16 * 64 * (ODT == F32 ? 4 : 2)) / (64 * 16); }
template <int ODT> constexpr int b6_epi_bytes() { return R3_WAVES * 16 * r3_srb<ODT>() + 2 * B6_BN * 4 + BBM * 4; }
static_assert(b6_epi_bytes<F32>() <= B6_SLOT, "bf6 epilogue must fit in one slot");
// the largest K whose sums stay exact in the fp32 accumulator
constexpr int64_t kGemmMaxKBf6 = ((int64_t)1 << 24) / 56 / B6_BK * B6_BK;

__device__ __forceinline__ R3Tile b6_tile(const GemmArgs& a, int t, int ntiles, int tiles_n)
{
    R3Tile r;
    if (t >= ntiles) {
        r.m0 = 0; r.n0 = 0;
        r.ra = make_rsrc(a.codes, 0);
        r.rw = make_rsrc(a.wp, 0);
        return r;
    }
    const int q8 = ntiles >> 3, r8 = ntiles & 7;
    const int xcd = t & 7, loc = t >> 3;
    const int tile = xcd * q8 + min(xcd, r8) + loc;
    // groups of four tile rows: an XCD's 32 concurrent tiles then span 4 row
    // blocks and 8 column blocks, the pair that keeps the fewest operand bytes
    // (a code row block is twice a packed weight column block) across its L2
    constexpr int GROUP_M = 4;
    const int tiles_m = ntiles / tiles_n;
    const int per_group = GROUP_M * tiles_n;
    const int first_m = (tile / per_group) * GROUP_M;
    const int gsize = min(tiles_m - first_m, GROUP_M);
    const int in_g = tile - (tile / per_group) * per_group;
    r.m0 = (int64_t)(first_m + in_g % gsize) * BBM;
    r.n0 = (int64_t)(in_g / gsize) * B6_BN;
    r.ra = make_rsrc(a.codes + r.m0 * a.K, (uint64_t)(a.M - r.m0) * a.K);
    r.rw = make_rsrc(a.wp + r.n0 * a.K, (uint64_t)(a.N - r.n0) * a.K);
    return r;
}

template <int ODT>
__global__ __launch_bounds__(512) void w4a4_gemm_bf6_kernel(GemmArgs a, int tiles_m, int tiles_n)
{
    __shared__ __align__(16) int8_t smem[3 * B6_SLOT];
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int j = lane & 15, q = lane >> 4;
    const int wm = wave & 3, wn = wave >> 2;   // 64-row block wm, 64-column block wn

    const int ntiles = tiles_m * tiles_n;
    const int64_t K = a.K, M = a.M, N = a.N;
    const int nsteps = (int)(K / B6_BK);
    int t = blockIdx.x;
    const int G = gridDim.x;

    const bool loader = wave < R3_LOADERS;
    const int lw = wave & (R3_LOADERS - 1);
    // both operands: lane l of a 1 KB load writes chunk (l & 7) of row
    // (l >> 3), i.e. logical chunk (l & 7) ^ r3_swz(row)
    const int arow = lane >> 3;
    const int c_vo = (int)(arow * K + (((lane & 7) ^ r3_swz(arow)) * 16));
    const int row8 = (int)(8 * K);
    auto issue = [&](int slot, const __amdgpu_buffer_rsrc_t& ra, const __amdgpu_buffer_rsrc_t& rw, int st) {
        if (!loader) return;
        int8_t* as = smem + slot * B6_SLOT;
        int8_t* ws = as + B6_ASTAGE;
        const int k0 = st * B6_BK;
        // codes: rows lw*64 .. lw*64+63; weights: columns lw*32 .. lw*32+31
#pragma unroll
        for (int i = 0; i < B6_ALOADS; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                ra, (__attribute__((address_space(3))) void*)(as + (lw * 64 + i * 8) * B6_BK), 16,
                c_vo + (lw * 8 + i) * row8 + k0, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < B6_WLOADS; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rw, (__attribute__((address_space(3))) void*)(ws + (lw * 32 + i * 8) * B6_BK), 16,
                c_vo + (lw * 4 + i) * row8 + k0, 0, 0, 0);
    };

    v4f acc[4][4];
    // fragment: chunk 2q (16 bytes) and the first 8 bytes of chunk 2q + 1 of
    // row (code) or column (weight) j of each 16-row tile
    const int c0 = ((q * 2) ^ r3_swz(j)) * 16, c1 = ((q * 2 + 1) ^ r3_swz(j)) * 16;
    const int a_ro = (wm * 64 + j) * B6_BK;
    const int w_ro = B6_ASTAGE + (wn * 64 + j) * B6_BK;
    auto frag = [&](const int8_t* p) {
        const v4i lo = *(const v4i*)(p + c0);
        const v2i hi = *(const v2i*)(p + c1);
        return (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], 0, 0};
    };
    auto compute = [&](int slot) {
        const int8_t* as = smem + slot * B6_SLOT + a_ro;
        const int8_t* ws = smem + slot * B6_SLOT + w_ro;
        v8i bfr[4], afr[4];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) bfr[nt] = frag(ws + nt * 16 * B6_BK);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) afr[mt] = frag(as + mt * 16 * B6_BK);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
                acc[mt][nt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(afr[mt], bfr[nt], acc[mt][nt],
                                                                               3, 3, 0, 0, 0, 0);
    };

    R3Tile cur_t = b6_tile(a, t, ntiles, tiles_n);
    R3Tile nxt_t = b6_tile(a, t + G, ntiles, tiles_n);
    issue(0, cur_t.ra, cur_t.rw, 0);
    issue(1, cur_t.ra, cur_t.rw, 1);
    int cur = 0, nxt2 = 2;
    static_assert(B6_LPS + b6_stores<ODT>() <= 63, "vmcnt range");
    auto pad_stores = [&]() {
        if (!loader) return;
        const __amdgpu_buffer_rsrc_t none = make_rsrc(a.out, 0);
#pragma unroll
        for (int i = 0; i < b6_stores<ODT>(); ++i)
            __builtin_amdgcn_raw_buffer_store_b32(0u, none, 4 * i, 0, (int)0x80000000);
    };
    pad_stores();
    for (;;) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = (v4f){0.f, 0.f, 0.f, 0.f};
        for (int s = 0; s < nsteps; ++s) {
            if (loader) {
                // stage s has landed once vmcnt drops to B6_LPS; in steps 0
                // and 1 the previous tile's stores (or their stand-ins) may be
                // in flight too (vmcnt retires in issue order)
                asm volatile(
                    "s_cmp_lt_u32 %0, 2\n\t"
                    "s_cbranch_scc0 1f\n\t"
                    "s_waitcnt vmcnt(%1)\n\t"
                    "s_branch 2f\n"
                    "1:\n\t"
                    "s_waitcnt vmcnt(%2)\n"
                    "2:" ::"s"(s), "n"(B6_LPS + b6_stores<ODT>()), "n"(B6_LPS) : "memory", "scc");
            }
            __builtin_amdgcn_s_barrier();
            const bool same = s + 2 < nsteps;
            issue(nxt2, same ? cur_t.ra : nxt_t.ra, same ? cur_t.rw : nxt_t.rw, same ? s + 2 : s + 2 - nsteps);
            __builtin_amdgcn_sched_barrier(0);
            compute(cur);
            cur = cur == 2 ? 0 : cur + 1;
            nxt2 = nxt2 == 2 ? 0 : nxt2 + 1;
        }

        // ---- epilogue in the slot the last step used (see the INT4 kernel)
        int8_t* eslot = smem + nxt2 * B6_SLOT;
        __builtin_amdgcn_s_barrier();
        constexpr int SRB = r3_srb<ODT>();
        constexpr int ESZ = ODT == F32 ? 4 : 2;
        int8_t* strips = eslot;
        float* scol = (float*)(eslot + R3_WAVES * 16 * SRB);
        float* bcol = scol + B6_BN;
        float* srow = bcol + B6_BN;
        const int64_t m0 = cur_t.m0, n0 = cur_t.n0;
        const bool has_bias = a.bias != nullptr;
        if (!loader) {
            // waves 4-7: 256 threads; columns from the first 128, rows all 256
            const int c = tid - R3_LOADERS * 64;
            const int64_t col = n0 + (c & (B6_BN - 1)), row = m0 + c;
            const int64_t cc = col < N ? col : N - 1;
            const int bdt = has_bias ? a.bias_dtype : a.sw_dtype;
            const uint32_t ws = r3_scalar_word(a.sw, a.sw_dtype, N, cc);
            const uint32_t wb = r3_scalar_word(has_bias ? a.bias : a.sw, bdt, N, cc);
            const uint32_t wr = r3_scalar_word(a.sa, F32, M, row < M ? row : M - 1);
            if (c < B6_BN) {
                scol[c] = r3_scalar_value(ws, a.sw_dtype, cc);
                bcol[c] = has_bias ? r3_scalar_value(wb, bdt, cc) : 0.0f;
            }
            srow[c] = __uint_as_float(wr);
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);
        __builtin_amdgcn_s_barrier();
        float scl[4], bia[4];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            scl[nt] = scol[wn * 64 + nt * 16 + j];
            bia[nt] = bcol[wn * 64 + nt * 16 + j];
        }
        const bool full = m0 + BBM <= M && n0 + B6_BN <= N && (N % 8) == 0;
        constexpr int VPC = 16 / ESZ, CPR = 64 / VPC, CHUNKS = 16 * CPR, PER_LANE = CHUNKS / 64;
        static_assert(PER_LANE == 2 || PER_LANE == 4, "strip read asm below");
        int8_t* mine = strips + wave * 16 * SRB;
        using lds_ptr = const __attribute__((address_space(3))) int8_t*;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            const float* sr = srow + wm * 64 + mt * 16 + 4 * q;
            const float sa[4] = {sr[0], sr[1], sr[2], sr[3]};
#pragma unroll
            for (int nt = 0; nt < 4; ++nt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    // the accumulator is the exact integer sum (below 2^24)
                    const float tv = mul_rn(mul_rn(acc[mt][nt][r], sa[r]), scl[nt]);
                    const float o = has_bias ? add_rn(tv, bia[nt]) : tv;
                    int8_t* dst = mine + (4 * q + r) * SRB + (nt * 16 + j) * ESZ;
                    if constexpr (ODT == F32)
                        *(float*)dst = o;
                    else
                        *(uint16_t*)dst = f32_to_h<ODT>(o);
                }
            v4u vv[PER_LANE];
            lds_ptr la[PER_LANE];
#pragma unroll
            for (int i = 0; i < PER_LANE; ++i) {
                const int c = lane + 64 * i;
                la[i] = (lds_ptr)(mine + (c / CPR) * SRB + (c % CPR) * 16);
            }
            __builtin_amdgcn_s_waitcnt(0xc07f);
            __builtin_amdgcn_wave_barrier();
            if constexpr (PER_LANE == 2) {
                asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %3\n\ts_waitcnt lgkmcnt(0)"
                             : "=v"(vv[0]), "=v"(vv[1]) : "v"(la[0]), "v"(la[1]) : "memory");
            } else {
                asm volatile("ds_read_b128 %0, %4\n\tds_read_b128 %1, %5\n\t"
                             "ds_read_b128 %2, %6\n\tds_read_b128 %3, %7\n\ts_waitcnt lgkmcnt(0)"
                             : "=v"(vv[0]), "=v"(vv[1]), "=v"(vv[2]), "=v"(vv[3])
                             : "v"(la[0]), "v"(la[1]), "v"(la[2]), "v"(la[3]) : "memory");
            }
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int i = 0; i < PER_LANE; ++i) {
                const int c = lane + 64 * i;
                const int rr = c / CPR, ch = c % CPR;
                const uint4 v = make_uint4(vv[i][0], vv[i][1], vv[i][2], vv[i][3]);
                const int64_t row = m0 + wm * 64 + mt * 16 + rr;
                const int64_t col0 = n0 + wn * 64 + ch * VPC;
                int8_t* dst = (int8_t*)a.out + (row * N + col0) * ESZ;
                if (full) {
                    *(uint4*)dst = v;
                } else if (row < M) {
                    if (col0 + VPC <= N && (N % 8) == 0) {
                        *(uint4*)dst = v;
                    } else {
                        const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                        for (int e = 0; e < VPC; ++e) {
                            if (col0 + e >= N) break;
                            if constexpr (ODT == F32)
                                ((uint32_t*)dst)[e] = w4[e];
                            else
                                ((uint16_t*)dst)[e] = (uint16_t)(w4[e >> 1] >> (16 * (e & 1)));
                        }
                    }
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        if (!full && loader) {
            __builtin_amdgcn_s_waitcnt(r3_vmcnt(0));
            pad_stores();
        }
        t += G;
        if (t >= ntiles) break;
        cur_t = nxt_t;
        nxt_t = b6_tile(a, t + G, ntiles, tiles_n);
    }
    __builtin_amdgcn_s_waitcnt(0x0070);
}

// ---- bf6 block encoders (codes and weights -> the FP6 kernel's operands)
// e3m2 patterns of the integers 0..8 (sign in bit 5)
__device__ __forceinline__ uint32_t bf6_of(int v)
{
    const int m = v < 0 ? -v : v;
    // 0, 1, 2, 3, 4, 5, 6, 7, 8 -> 0x00 0x0C 0x10 0x12 0x14 0x15 0x16 0x17 0x18
    const uint32_t e = m == 0 ? 0u : m == 1 ? 0x0Cu : m == 2 ? 0x10u : m == 3 ? 0x12u : (uint32_t)(0x10 + m);
    return e | (v < 0 ? 0x20u : 0u);
}

// one 32-value block per thread: 6 payload dwords and 2 zero dwords
__device__ __forceinline__ void bf6_store(uint8_t* dst, const int (&v)[32])
{
    uint32_t w[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int e = 0; e < 32; ++e) {
        const uint32_t b = bf6_of(v[e]);
        const int bit = 6 * e;
        w[bit >> 5] |= b << (bit & 31);
        if ((bit & 31) > 26) w[(bit >> 5) + 1] |= b >> (32 - (bit & 31));
    }
    *(uint4*)dst = make_uint4(w[0], w[1], w[2], w[3]);
    *(uint4*)(dst + 16) = make_uint4(w[4], w[5], 0u, 0u);
}

__global__ void codes_to_bf6_kernel(const int8_t* __restrict__ codes, int64_t nblk, uint8_t* __restrict__ out)
{
    for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < nblk;
         b += (int64_t)gridDim.x * blockDim.x) {
        const uint4 p0 = *(const uint4*)(codes + 32 * b), p1 = *(const uint4*)(codes + 32 * b + 16);
        const uint32_t d[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
        int v[32];
#pragma unroll
        for (int e = 0; e < 32; ++e) v[e] = (int)(int8_t)(d[e >> 2] >> (8 * (e & 3)));
        bf6_store(out + 32 * b, v);
    }
}

__global__ void weights_to_bf6_kernel(const uint8_t* __restrict__ wp, int64_t nblk, uint8_t* __restrict__ out)
{
    for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < nblk;
         b += (int64_t)gridDim.x * blockDim.x) {
        const uint4 p = *(const uint4*)(wp + 16 * b);
        const uint32_t d[4] = {p.x, p.y, p.z, p.w};
        int v[32];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const uint32_t byte = (d[i >> 2] >> (8 * (i & 3))) & 0xffu;
            const int lo = (int)(byte & 0xfu), hi = (int)(byte >> 4);
            v[2 * i] = lo >= 8 ? lo - 16 : lo;          // low nibble: k = 2i
            v[2 * i + 1] = hi >= 8 ? hi - 16 : hi;      // high nibble: k = 2i + 1
        }
        bf6_store(out + 32 * b, v);
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
// -------------------------------------------------------------------------
// Skinny-M kernel (M <= 64, per-channel weight scales, no K-chunks): the
// packed-weight stream is the whole cost, so the grid is one 1024-thread
// workgroup per 16 output columns and its 16 waves split the K steps of 64
// (wave w takes steps w, w + 16, ...).  A wave issues the code and weight
// loads of up to SK_MAXS steps at once, straight into registers (buffer loads:
// rows past M and columns past N read zeros), then multiplies them with
// v_mfma_i32_16x16x64_i8 (weights unpacked as 16*w).  The 16 partial tiles
// are summed in LDS as exact integers; one thread per output applies the
// epilogue.
// -------------------------------------------------------------------------
constexpr int SK_WAVES = 16;
constexpr int SK_MAXS = 4;    // K steps per wave in flight at once
constexpr int SK_LD = 20;     // LDS row stride of a partial tile, in words

template <int MT>
__global__ __launch_bounds__(1024) void w4a4_gemm_skinny_kernel(GemmArgs a)
{
    __shared__ int32_t part[SK_WAVES][MT * 16 * SK_LD];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int j = lane & 15, kq = lane >> 4;
    const int64_t M = a.M, K = a.K, N = a.N;
    const int64_t n0 = (int64_t)blockIdx.x * 16;
    const int nsteps = (int)(K / 64);
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(a.codes, (uint64_t)M * K);
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(a.wp + n0 * (K >> 1), (uint64_t)(N - n0) * (K >> 1));
    // lane (j, kq): code row mt*16 + j, bytes kq*16 .. +15 of a step; weight
    // column n0 + j, packed bytes kq*8 .. +7 of a step
    const int a_off = (int)(j * K + kq * 16);
    const int w_off = (int)(j * (K >> 1) + kq * 8);

    v4i acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = (v4i){0, 0, 0, 0};
    for (int s0 = wave; s0 < nsteps; s0 += SK_WAVES * SK_MAXS) {
        v4u af[SK_MAXS][MT];
        v2u wf[SK_MAXS];
#pragma unroll
        for (int i = 0; i < SK_MAXS; ++i) {
            const int st = s0 + i * SK_WAVES;
            const int k0 = st * 64;
            if (st < nsteps) {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    af[i][mt] = __builtin_amdgcn_raw_buffer_load_b128(rc, a_off + (int)(mt * 16 * K) + k0, 0, 0);
                wf[i] = __builtin_amdgcn_raw_buffer_load_b64(rw, w_off + (k0 >> 1), 0, 0);
            } else {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) af[i][mt] = (v4u){0u, 0u, 0u, 0u};
                wf[i] = (v2u){0u, 0u};
            }
        }
#pragma unroll
        for (int i = 0; i < SK_MAXS; ++i) {
            uint32_t b0, b1, b2, b3;
            unpack16(wf[i].x, b0, b1);
            unpack16(wf[i].y, b2, b3);
            const v4i bf = (v4i){(int)b0, (int)b1, (int)b2, (int)b3};
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                acc[mt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(v4i, af[i][mt]), bf, acc[mt], 0, 0, 0);
        }
    }
    // lane (j, kq) holds rows 4 kq + r, column j of each 16 x 16 tile
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) part[wave][(mt * 16 + 4 * kq + r) * SK_LD + j] = acc[mt][r];
    __syncthreads();
    if (tid < MT * 16 * 16) {
        const int m = tid >> 4, n = tid & 15;
        int32_t sum = 0;
#pragma unroll
        for (int w = 0; w < SK_WAVES; ++w) sum += part[w][m * SK_LD + n];
        const int64_t row = m, col = n0 + n;
        if (row < M && col < N) {
            const int32_t iv = sum >> 4;
            if (a.acc_out) a.acc_out[row * N + col] = iv;
            float t = mul_rn((float)iv, a.sa[row]);
            t = mul_rn(t, load_any_f32(a.sw_dtype, a.sw, col));
            t = epilogue_tail(t, a, row, col);
            store_any(a.out_dtype, a.out, row * N + col, t);
        }
    }
}

int gemm_path(const GemmArgs& a)
{
    const bool aligned = (a.K % 32) == 0 && ((uintptr_t)a.codes % 16) == 0 &&
                         ((uintptr_t)a.wp % 16) == 0;
    const bool group = a.sw_group > 0;
    // activation scales per 64-wide group: the 128 x 128 kernel (no K chunks:
    // every group's INT32 sums are converted at once)
    if (a.sa_group) return kGemmTile;
    // INT8 weights: the three-stage kernel (64-deep K steps) for
    // prefill-sized layers, else the 128 x 128 kernel
    if (a.w8) {
        if (a.k_chunk == 0 && a.acc_out == nullptr && a.M > 128 && (a.K % R3Geo<true>::BK) == 0 &&
            a.K >= 2 * R3Geo<true>::BK && aligned && ((uintptr_t)a.out % 16) == 0)
            return kGemmRing3;
        return a.k_chunk > 0 ? kGemmTileSplitK : kGemmTile;
    }
    // decode-sized M: the skinny kernel (every epilogue variant but group
    // scales and K-chunks)
    if (!group && a.k_chunk == 0 && a.M >= 1 && a.M <= 64 && (a.K % 64) == 0 &&
        ((uintptr_t)a.codes % 16) == 0 && ((uintptr_t)a.wp % 8) == 0)
        return kGemmSkinny;
    // Prefill-sized layers take a 256 x 256 three-stage kernel: the
    // ping-pong one when whole 16-column output pieces exist (N % 16 == 0)
    // and a tile's output offsets fit its 32-bit range check, else the ring
    // kernel; everything else (small M, group scales, low-rank term, INT32
    // export, K chunks, K not a multiple of 128, unaligned operands) the
    // 128 x 128 kernel.
    if (!group && a.lora == nullptr && a.acc_out == nullptr && a.k_chunk == 0 && a.M > 128 &&
        (a.K % R3_BK) == 0 && a.K >= 2 * R3_BK && aligned && ((uintptr_t)a.out % 16) == 0) {
        const uint64_t esz = a.out_dtype == F32 ? 4 : 2;
        if (a.N % 16 == 0 && (uint64_t)a.N * esz * 512 < (1ull << 32)) return kGemmPP;
        return kGemmRing3;
    }
    if (a.k_chunk > 0 && !group) return kGemmTileSplitK;
    return kGemmTile;
}

hipError_t launch_gemm(const GemmArgs& a, hipStream_t st)
{
    const bool aligned = (a.K % 32) == 0 && ((uintptr_t)a.codes % 16) == 0 &&
                         ((uintptr_t)a.wp % 16) == 0;
    const bool group = a.sw_group > 0;
    const int path = gemm_path(a);
    if (path == kGemmSkinny) {
        const unsigned gx = (unsigned)((a.N + 15) / 16);
        if (a.M <= 16)
            hipLaunchKernelGGL(w4a4_gemm_skinny_kernel<1>, dim3(gx), dim3(1024), 0, st, a);
        else if (a.M <= 32)
            hipLaunchKernelGGL(w4a4_gemm_skinny_kernel<2>, dim3(gx), dim3(1024), 0, st, a);
        else
            hipLaunchKernelGGL(w4a4_gemm_skinny_kernel<4>, dim3(gx), dim3(1024), 0, st, a);
        return hipGetLastError();
    }
    if (path == kGemmRing3 || path == kGemmPP) {
        const int tm = (int)((a.M + BBM - 1) / BBM), tn = (int)((a.N + BBN - 1) / BBN);
        const int nt = tm * tn;
        // persistent grid: one workgroup per CU (a multiple of 8 so that a
        // workgroup's tiles all fall in its XCD), or one per tile if fewer
        static int n_cu = 0;
        if (n_cu == 0) {
            int dev = 0, v = 0;
            if (hipGetDevice(&dev) == hipSuccess &&
                hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v >= 8)
                n_cu = v & ~7;
            else
                n_cu = 256;
        }
        const unsigned grid = (unsigned)(nt < n_cu ? nt : n_cu);
        if (path == kGemmPP) {
            if (a.out_dtype == F32)
                hipLaunchKernelGGL(w4a4_gemm_pp_kernel<F32>, dim3(grid), dim3(512), 0, st, a, tm, tn);
            else if (a.out_dtype == F16)
                hipLaunchKernelGGL(w4a4_gemm_pp_kernel<F16>, dim3(grid), dim3(512), 0, st, a, tm, tn);
            else
                hipLaunchKernelGGL(w4a4_gemm_pp_kernel<BF16>, dim3(grid), dim3(512), 0, st, a, tm, tn);
            return hipGetLastError();
        }
        if (a.w8) {
            if (a.out_dtype == F32)
                hipLaunchKernelGGL((w4a4_gemm_ring3_kernel<F32, true>), dim3(grid), dim3(512), 0, st, a, tm, tn);
            else if (a.out_dtype == F16)
                hipLaunchKernelGGL((w4a4_gemm_ring3_kernel<F16, true>), dim3(grid), dim3(512), 0, st, a, tm, tn);
            else
                hipLaunchKernelGGL((w4a4_gemm_ring3_kernel<BF16, true>), dim3(grid), dim3(512), 0, st, a, tm, tn);
            return hipGetLastError();
        }
        if (a.out_dtype == F32)
            hipLaunchKernelGGL(w4a4_gemm_ring3_kernel<F32>, dim3(grid), dim3(512), 0, st, a, tm, tn);
        else if (a.out_dtype == F16)
            hipLaunchKernelGGL(w4a4_gemm_ring3_kernel<F16>, dim3(grid), dim3(512), 0, st, a, tm, tn);
        else
            hipLaunchKernelGGL(w4a4_gemm_ring3_kernel<BF16>, dim3(grid), dim3(512), 0, st, a, tm, tn);
        return hipGetLastError();
    }
    const unsigned gx = (unsigned)((a.N + BN - 1) / BN);
    const unsigned gy = (unsigned)((a.M + BM - 1) / BM);
    if (path == kGemmTileSplitK) {
        const int64_t kc = a.k_chunk;
        const unsigned gz = (unsigned)((a.K + kc - 1) / kc);
        const int64_t n = a.M * a.N;
        hipLaunchKernelGGL(fill_zero_i64, dim3(1024), dim3(256), 0, st, a.acc64, n);
        if (a.w8) {
            if (aligned)
                hipLaunchKernelGGL((w4a4_gemm_kernel<-1, true, true, true>), dim3(gx, gy, gz), dim3(256), 0,
                                   st, a, kc);
            else
                hipLaunchKernelGGL((w4a4_gemm_kernel<-1, true, false, true>), dim3(gx, gy, gz), dim3(256), 0,
                                   st, a, kc);
        } else if (aligned) {
            hipLaunchKernelGGL((w4a4_gemm_kernel<-1, true, true>), dim3(gx, gy, gz), dim3(256), 0,
                               st, a, kc);
        } else {
            hipLaunchKernelGGL((w4a4_gemm_kernel<-1, true, false>), dim3(gx, gy, gz), dim3(256), 0,
                               st, a, kc);
        }
        hipLaunchKernelGGL(split_epilogue_kernel, dim3(2048), dim3(256), 0, st, a);
        return hipGetLastError();
    }
    const int64_t kc = a.K;
    // (the aligned kernels without K-chunks stage through buffer loads that
    // need whole 64-deep K steps and 32-bit offsets within a 128-row tile)
    const bool aligned_buf = aligned && (a.K % 64) == 0 && a.K < (1 << 24);
    if (a.sa_group) {
#define W4A4_AG_LAUNCH(DT)                                                                                  \
    do {                                                                                                    \
        if (aligned_buf)                                                                                    \
            hipLaunchKernelGGL((w4a4_gemm_kernel<DT, false, true, false, true>), dim3(gx, gy, 1), dim3(256), \
                               0, st, a, kc);                                                               \
        else                                                                                                \
            hipLaunchKernelGGL((w4a4_gemm_kernel<DT, false, false, false, true>), dim3(gx, gy, 1),          \
                               dim3(256), 0, st, a, kc);                                                    \
    } while (0)
        if (!group) W4A4_AG_LAUNCH(-1);
        else if (a.sw_dtype == F32) W4A4_AG_LAUNCH(F32);
        else if (a.sw_dtype == F16) W4A4_AG_LAUNCH(F16);
        else W4A4_AG_LAUNCH(BF16);
#undef W4A4_AG_LAUNCH
        return hipGetLastError();
    }
    if (group) {
#define W4A4_GROUP_LAUNCH(DT)                                                                    \
    do {                                                                                         \
        if (aligned_buf)                                                                         \
            hipLaunchKernelGGL((w4a4_gemm_kernel<DT, false, true>), dim3(gx, gy, 1), dim3(256), 0, \
                               st, a, kc);                                                       \
        else                                                                                     \
            hipLaunchKernelGGL((w4a4_gemm_kernel<DT, false, false>), dim3(gx, gy, 1), dim3(256), \
                               0, st, a, kc);                                                    \
    } while (0)
        if (a.sw_dtype == F32) W4A4_GROUP_LAUNCH(F32);
        else if (a.sw_dtype == F16) W4A4_GROUP_LAUNCH(F16);
        else W4A4_GROUP_LAUNCH(BF16);
#undef W4A4_GROUP_LAUNCH
    } else if (a.w8) {
        if (aligned_buf)
            hipLaunchKernelGGL((w4a4_gemm_kernel<-1, false, true, true>), dim3(gx, gy, 1), dim3(256), 0,
                               st, a, kc);
        else
            hipLaunchKernelGGL((w4a4_gemm_kernel<-1, false, false, true>), dim3(gx, gy, 1), dim3(256), 0,
                               st, a, kc);
    } else {
        if (aligned_buf)
            hipLaunchKernelGGL((w4a4_gemm_kernel<-1, false, true>), dim3(gx, gy, 1), dim3(256), 0,
                               st, a, kc);
        else
            hipLaunchKernelGGL((w4a4_gemm_kernel<-1, false, false>), dim3(gx, gy, 1), dim3(256), 0,
                               st, a, kc);
    }
    return hipGetLastError();
}

// ---- FP6 path (host) ---------------------------------------------------

bool gemm_bf6_ok(const GemmArgs& a)
{
    return a.M > 0 && a.N > 0 && (a.K % B6_BK) == 0 && a.K >= 2 * B6_BK && a.K <= kGemmMaxKBf6 &&
           a.sw_group == 0 && a.lora == nullptr && a.acc_out == nullptr && a.k_chunk == 0 &&
           ((uintptr_t)a.codes % 16) == 0 && ((uintptr_t)a.wp % 16) == 0 && ((uintptr_t)a.out % 16) == 0;
}

int64_t gemm_bf6_max_k() { return kGemmMaxKBf6; }

hipError_t launch_gemm_bf6(const GemmArgs& a, hipStream_t st)
{
    if (!gemm_bf6_ok(a)) return hipErrorNotSupported;
    const int tm = (int)((a.M + BBM - 1) / BBM), tn = (int)((a.N + B6_BN - 1) / B6_BN);
    const int nt = tm * tn;
    static int n_cu = 0;
    if (n_cu == 0) {
        int dev = 0, v = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v >= 8)
            n_cu = v & ~7;
        else
            n_cu = 256;
    }
    const unsigned grid = (unsigned)(nt < n_cu ? nt : n_cu);
    if (a.out_dtype == F32)
        hipLaunchKernelGGL(w4a4_gemm_bf6_kernel<F32>, dim3(grid), dim3(512), 0, st, a, tm, tn);
    else if (a.out_dtype == F16)
        hipLaunchKernelGGL(w4a4_gemm_bf6_kernel<F16>, dim3(grid), dim3(512), 0, st, a, tm, tn);
    else
        hipLaunchKernelGGL(w4a4_gemm_bf6_kernel<BF16>, dim3(grid), dim3(512), 0, st, a, tm, tn);
    return hipGetLastError();
}

hipError_t launch_to_bf6(const void* src, bool weights, int64_t nblk, uint8_t* out, hipStream_t st)
{
    const int64_t want = (nblk + 255) / 256;
    const unsigned grid = (unsigned)(want < 4096 ? (want > 0 ? want : 1) : 4096);
    if (weights)
        hipLaunchKernelGGL(weights_to_bf6_kernel, dim3(grid), dim3(256), 0, st, (const uint8_t*)src, nblk, out);
    else
        hipLaunchKernelGGL(codes_to_bf6_kernel, dim3(grid), dim3(256), 0, st, (const int8_t*)src, nblk, out);
    return hipGetLastError();
}

}  // namespace w4a4
