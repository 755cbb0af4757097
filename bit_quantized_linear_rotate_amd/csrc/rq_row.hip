// Row-streaming rotate + quantize for many contiguous 16-bit rows, g = 64
// (gfx950).  Same arithmetic as every rotate-quant kernel of this library
// (web page "[Feat][Ascend] Consolidate INT8, RotateQuant, RoPE and ConvRot
// W4A4 backends", section "W4A4 correctness and performance scope";
// "[Feat][Ascend] Add fused RotateQuant backend", section "What this PR
// does"; codes in int8 storage: "[Perf][Ascend] Avoid activation pack/unpack
// in ConvRot W4A4", section "Summary"):
//   y = T(x_group . T(R)),  s = max(absmax(y) / 7, 2^-126),
//   c = clamp(round_half_even(fp32(y) / s), -7, 7).
//
// Design (a wave owns one whole row at a time, at most 64 groups of 64):
//   * R's MFMA fragments (A operand, rounded to T; 8 KB) sit in LDS, built
//     once per workgroup; a row is up to four tiles of 16 group-rows, each
//     rotated by eight v_mfma_f32_16x16x32 (B = the tile's x, two 16-byte
//     loads a lane), column tile by column tile so that each R fragment is
//     read from LDS once per row and used for every tile (in registers the
//     fragments took 32 VGPRs and a wave per SIMD).
//   * The rotated values are rounded to T in pairs (v_cvt_pk) and kept packed:
//     eight VGPRs a tile.  The row absmax is a packed 16-bit integer max over
//     the sign-cleared patterns (monotone in |y|; a NaN pattern exceeds every
//     other) and one wave reduction: no second rotation, no LDS.
//   * As soon as a row's tiles are rotated, the next row's loads go into the
//     freed x registers, so each wave keeps one row in flight while it
//     quantizes the previous one.  96 VGPRs (bf16): four workgroups of four
//     waves per CU, so 8192 rows give every wave exactly two.
//   * Row indices are 32-bit: every row test is a scalar compare, and the
//     per-row buffer resources (rows past M get a zero-sized one) stay in
//     SGPRs with no exec-masked code around the stores; the scale is stored
//     by a buffer store whose lanes other than 0 fall past its 4-byte range.
//   * Row scale: s = max(a / qmax, 2^-126), 1/s and the outcomes of exact
//     ties depend only on the significand of the 16-bit absmax a, up to a
//     power of two while every value stays normal; a compile-time table per
//     significand (scale_table.hpp), read with scalar loads and shifted by a's
//     exponent, replaces the per-row IEEE divisions.  Rows outside the
//     table's range (zero, a < 2^-119, Inf, NaN) take the divisions.
//   * Codes: with rinv = 1/s, the integers RNE(y * rinv * (1 + 2^-21)) and
//     RNE(y * rinv * (1 - 2^-21)), each one fma against 1.5 * 2^23 (the add
//     rounds the exact product to an integer and leaves it in the low byte),
//     bracket the correctly rounded quotient fl(y / s): when they agree that
//     integer IS the code (rounding is monotone).  They disagree only when
//     y / s lies within 2^-20 of a half-integer, which for 16-bit y and a
//     scale taken from the row's own 16-bit absmax a happens only at exact
//     ties 7 y = (k + 1/2) a, k = 0..6.  All elements of a row that tie at
//     the same k have the same |y|, so a 7-bit mask per row (bit k: the tie
//     at k rounds away from zero) decides every tie; each element takes its
//     code from the two integers and that mask with one bitfield extract and
//     one bitwise select, with no branch and no per-element division.  When
//     7 does not divide the integer significand of a, a tie needs 7 | 2k + 1,
//     i.e. k = 3 only: then the one multiplier that rounds that tie the
//     quantizer's way gives every code with a single fma (most rows).  Rows
//     whose scale is Inf or NaN take the division for every element.
//   * Each lane holds four codes of each of four column tiles; two
//     v_permlane32_swap and two v_permlane16_swap transpose them so that every
//     lane stores 16 consecutive codes (one 1 KB store per tile and wave).
#include "common.hpp"
#include "kernels.hpp"
#include "row_quant.hpp"

namespace w4a4 {

namespace {

typedef unsigned short v2u16 __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef unsigned v4u32 __attribute__((ext_vector_type(4)));
typedef unsigned v2u32 __attribute__((ext_vector_type(2)));

constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23

template <int DT>
__device__ __forceinline__ uint32_t cvt_pair(float a, float b)
{
    if constexpr (DT == BF16) return __builtin_bit_cast(uint32_t, (v2bf){(__bf16)a, (__bf16)b});
    else return __builtin_bit_cast(uint32_t, (v2h){(_Float16)a, (_Float16)b});
}

// value r (0: low half, 1: high half) of a packed pair, as fp32
template <int DT>
__device__ __forceinline__ float unpack_half(uint32_t p, int r)
{
    if constexpr (DT == BF16) return __uint_as_float(r ? (p & 0xffff0000u) : (p << 16));
    else return f16_to_f32((uint16_t)(r ? (p >> 16) : (p & 0xffffu)));
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v)
{
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xb1, 0xf, 0xf, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4e, 0xf, 0xf, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x124, 0xf, 0xf, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xf, 0xf, false));
    const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
    const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
    const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
    const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
    return max(max(r0, r1), max(r2, r3));
}

// buffer resource over `bytes` bytes at `base`: accesses whose per-lane
// offset falls outside read zeros / are dropped
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const void* base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)bytes, 0x00020000);
}

// Tie table of a row with absmax a and finite scale s.  An element whose
// two bracketing roundings differ is an exact tie y = h * a / 7, h = k + 1/2
// (k = 0..6), whose code is either k or k + 1 in magnitude; bit k of the
// result says "k + 1".  Lane k < 7 divides exactly as the quantizer does for
// that y: y_h = fl(fl(h * a) / 7) is exact whenever h * a / 7 is a 16-bit
// value at all (otherwise no element can tie at h), computed at a 2^-64
// scale for large a so that h * a cannot overflow; q_h = fl(y_h / s).  When
// the scale was clamped to 2^-126, y / s = y * 2^126 exactly and a tie
// rounds to even.  The returned mask is indexed by the low five bits of the
// toward-zero code's two's-complement byte: bit k for code k >= 0 and bit
// 32 - k for code -k.
__device__ __forceinline__ uint32_t tie_mask(float a, float s, bool clamped, int lane)
{
    uint32_t b;
    if (clamped) {
        b = 0x2au;  // k odd: h = k + 1/2 rounds to even k + 1
    } else {
        const float h = (float)(lane & 7) + 0.5f;
        const bool big = a > 0x1p64f;
        const float ah = big ? a * 0x1p-64f : a;
        float yh = (h * ah) / 7.0f;
        if (big) yh *= 0x1p64f;
        const float qh = yh / s;
        const bool up = lane < 7 && rintf(qh) > h;
        b = (uint32_t)__builtin_amdgcn_ballot_w64(up) & 0x7fu;
    }
    return b | (__builtin_bitreverse32(b) << 1);
}

// correctly rounded code for a finite or non-finite quotient (NaN -> 0)
template <int QMAX>
__device__ __forceinline__ int code_of_quotient(float qv)
{
    if (qv != qv) return 0;
    return (int)__builtin_amdgcn_fmed3f(rintf(qv), -(float)QMAX, (float)QMAX);
}

}  // namespace

template <int DT, bool SMOOTH, bool YOUT, int TW, int PF, int QMAX>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void rq_row_kernel(
    const uint16_t* __restrict__ x, int M, int64_t K, int64_t sm,
    const float* __restrict__ rot, const uint16_t* __restrict__ smooth,
    int8_t* __restrict__ codes, float* __restrict__ scales, uint16_t* __restrict__ yout,
    int had, const int8_t* __restrict__ sign_in, const int8_t* __restrict__ sign_out)
{
    constexpr int GP = 64, CT = 4, NKS = 2, LPL = 16;
    constexpr int kNT = 2;  // cache policy of the output stores: non-temporal
    const int lane = threadIdx.x & 63;
    const int j = lane & 15, q = lane >> 4;
    const int gpr = (int)(K / GP);
    // row indices are 32-bit (the launcher requires M < 2^30) so that every
    // row test is a scalar compare: the buffer resources built from them stay
    // in SGPRs
    const int nw = (int)gridDim.x * (int)(blockDim.x >> 6);
    // the wave's row is uniform: row pointers live in SGPRs and every load
    // and store is a scalar base plus a 32-bit lane offset
    const int wid = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    int row = (int)blockIdx.x * (int)(blockDim.x >> 6) + wid;

    // this lane's byte offsets in tile u (x, codes); lanes past the row's
    // last group-row get an offset past the row, so their loads read zeros
    // (no effect on the absmax) and their stores are dropped
    int xoff[TW], coff[TW];
#pragma unroll
    for (int u = 0; u < TW; ++u) {
        const int b = u * 16 + j;
        const bool live = b < gpr;
        xoff[u] = live ? (b * GP + q * LPL) * 2 : (int)(2 * K);
        coff[u] = live ? b * GP + q * 16 : (int)K;
    }

    // PF rows in flight per wave, each in its own set of x registers.  Rows
    // past M get a zero-sized resource: their loads read zeros and touch no
    // memory, so the loads need no branch (and the compiler's wait counts
    // stay exact)
    v8s xf[PF][TW][NKS];
    auto load_row = [&](v8s (&buf)[TW][NKS], int r) {
        const bool live = r < M;
        const __amdgpu_buffer_rsrc_t rx = row_rsrc(x + (int64_t)(live ? r : 0) * sm, live ? (uint32_t)(2 * K) : 0u);
#pragma unroll
        for (int u = 0; u < TW; ++u)
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
                buf[u][ks] = __builtin_bit_cast(v8s, __builtin_amdgcn_raw_buffer_load_b128(rx, xoff[u] + 16 * ks, 0, 0));
    };
#pragma unroll
    for (int p = 0; p < PF; ++p) load_row(xf[p], row + p * nw);

    // R's MFMA fragments (A operand), rounded to T: fragment f = ct*2 + ks of
    // lane (j, q) holds T(R[q*16 + ks*8 + e][ct*16 + j]), e = 0..7.  Built
    // once per workgroup from the fp32 matrix after the first rows' loads are
    // on their way
    __shared__ v8s rlds[CT * NKS][64];
    for (int e = threadIdx.x; e < CT * NKS * 64; e += blockDim.x) {
        const int f = e >> 6, jj = e & 15, qq = (e >> 4) & 3;
        v8s v;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int kk = qq * LPL + (f & 1) * 8 + i, cc = (f >> 1) * 16 + jj;
            float rv;
            if (had) {
                // R = diag(sign_in) H_64 diag(sign_out) / 8, H_64 the Sylvester
                // matrix: entry (k, c) is (-1)^popcount(k & c) / 8, exact in T
                const int neg = (__builtin_popcount(kk & cc) ^ (sign_in && sign_in[kk] < 0) ^
                                 (sign_out && sign_out[cc] < 0)) & 1;
                rv = neg ? -0.125f : 0.125f;
            } else {
                rv = rot[kk * GP + cc];
            }
            v[i] = (short)f32_to_h<DT>(rv);
        }
        rlds[f][e & 63] = v;
    }
    __syncthreads();

    // one row: rotate, absmax, refill this buffer with the row PF*nw ahead,
    // scale, codes
    auto process = [&](v8s (&buf)[TW][NKS], int r) {
        if constexpr (SMOOTH) {
            // x' = T(fp32(x) / fp32(smooth)), one IEEE division per value
            // (lanes past the row keep their zeros)
#pragma unroll
            for (int u = 0; u < TW; ++u) {
                if (xoff[u] < (int)(2 * K)) {
#pragma unroll
                    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const int k = xoff[u] / 2 + ks * 8 + e;
                            buf[u][ks][e] = (short)f32_to_h<DT>(h_to_f32<DT>((uint16_t)buf[u][ks][e]) /
                                                               h_to_f32<DT>(smooth[k]));
                        }
                }
            }
        }
        // rotate every tile, one column tile of R at a time; keep the rounded
        // values packed; packed absmax per tile
        // the fragments are re-read from LDS for every row: an opaque lane
        // index keeps the compiler from hoisting them into 32 live VGPRs
        int rlane = lane;
        asm volatile("" : "+v"(rlane));
        uint32_t yp[TW][CT][2];
        v2u16 um[TW];
#pragma unroll
        for (int u = 0; u < TW; ++u) um[u] = (v2u16){0, 0};
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            const v8s a0 = rlds[ct * NKS + 0][rlane], a1 = rlds[ct * NKS + 1][rlane];
#pragma unroll
            for (int u = 0; u < TW; ++u) {
                v4f acc = {0.f, 0.f, 0.f, 0.f};
                if constexpr (DT == BF16) {
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a0),
                                                                 __builtin_bit_cast(v8bf, buf[u][0]), acc, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a1),
                                                                 __builtin_bit_cast(v8bf, buf[u][1]), acc, 0, 0, 0);
                } else {
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, a0),
                                                                __builtin_bit_cast(v8h, buf[u][0]), acc, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, a1),
                                                                __builtin_bit_cast(v8h, buf[u][1]), acc, 0, 0, 0);
                }
                yp[u][ct][0] = cvt_pair<DT>(acc[0], acc[1]);
                yp[u][ct][1] = cvt_pair<DT>(acc[2], acc[3]);
                um[u] = __builtin_elementwise_max(um[u], __builtin_bit_cast(v2u16, yp[u][ct][0] & 0x7fff7fffu));
                um[u] = __builtin_elementwise_max(um[u], __builtin_bit_cast(v2u16, yp[u][ct][1] & 0x7fff7fffu));
            }
            // convert each column tile as soon as it is rotated: only its
            // MFMA results are live at a time
            __builtin_amdgcn_sched_barrier(0);
        }
        v2u16 amax = um[0];
#pragma unroll
        for (int u = 1; u < TW; ++u) amax = __builtin_elementwise_max(amax, um[u]);
        // the row PF*nw ahead goes into the x registers the rotation freed
        load_row(buf, r + PF * nw);

        // row scale s = max(a / qmax, 2^-126), 1/s, the bracketing multipliers
        // and the tie outcomes: from the significand table shifted by a's
        // exponent (a scalar load, no division), or with IEEE divisions for
        // the rows the table does not cover (zero, tiny, Inf, NaN)
        const uint32_t a16 = wave_max_u32(max((uint32_t)amax[0], (uint32_t)amax[1]));
        uint32_t tidx;
        int tE;
        float s, rinv, rh, rl, r1;
        uint32_t tmask;
        bool one;
        if (row_scale_key<DT == BF16>(a16, tidx, tE)) {
            const RowScaleEntry& te = row_scale_entry<DT, QMAX>(tidx);
            s = row_scale_shift(te.s, tE);
            rinv = row_scale_shift(te.rinv, -tE);
            rh = row_scale_shift(te.rh, -tE);
            rl = row_scale_shift(te.rl, -tE);
            r1 = row_scale_shift(te.r1, -tE);
            tmask = te.tie;
            one = te.one != 0u;
        } else {
            const float a = DT == BF16 ? __uint_as_float(a16 << 16) : f16_to_f32((uint16_t)a16);
            s = a / (float)QMAX;
            if (s < 0x1p-126f) s = 0x1p-126f;  // NaN compares false and stays NaN
            const bool clamped = s == 0x1p-126f;
            rinv = 1.0f / s;
            rh = rinv * (1.0f + 0x1p-21f);
            rl = rinv * (1.0f - 0x1p-21f);
            tmask = QMAX == 7 && fabsf(s) < 3.0e38f ? tie_mask(a, s, clamped, lane) : 0u;
            r1 = (tmask & 8u) ? rh : rl;
            // a's integer significand: when 7 does not divide it, the only
            // tie a 16-bit element can make is y = a / 2 (k = 3)
            const uint32_t sig = DT == BF16 ? ((a16 >> 7) & 0xffu ? (a16 & 0x7fu) | 0x80u : a16 & 0x7fu)
                                            : ((a16 >> 10) & 0x1fu ? (a16 & 0x3ffu) | 0x400u : a16 & 0x3ffu);
            one = !clamped && sig % 7u != 0u;
        }
        const bool live = r < M;
        const int64_t rr = live ? r : 0;
        // lane 0 stores the scale; the other lanes' offsets fall past the
        // 4-byte resource and are dropped (no branch)
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(s), row_rsrc(scales + rr, live ? 4u : 0u),
                                              lane == 0 ? 0 : 4, 0, 0);
        const bool finite = fabsf(s) < 3.0e38f;
        const __amdgpu_buffer_rsrc_t rc = row_rsrc(codes + rr * K, live ? (uint32_t)K : 0u);

        // transpose the codes of tile u (4 x 4 dwords across the lane groups:
        // lane group q then holds bytes q*16 .. q*16+15 of its group-row) and
        // store them; the rotated values too when they are exported
        auto store_tile = [&](int u, const uint32_t (&P)[CT]) {
            auto s02 = __builtin_amdgcn_permlane32_swap(P[0], P[2], false, false);
            auto s13 = __builtin_amdgcn_permlane32_swap(P[1], P[3], false, false);
            auto s01 = __builtin_amdgcn_permlane16_swap(s02[0], s13[0], false, false);
            auto s23 = __builtin_amdgcn_permlane16_swap(s02[1], s13[1], false, false);
            __builtin_amdgcn_raw_buffer_store_b128((v4u32){s01[0], s01[1], s23[0], s23[1]}, rc, coff[u], 0, kNT);
            if constexpr (YOUT) {
                // rotated values of columns ct*16 + 4q .. +3: byte offset
                // 2*(b*64) + 32*ct + 8q
                const __amdgpu_buffer_rsrc_t ry = row_rsrc(yout + rr * K, live ? (uint32_t)(2 * K) : 0u);
                const int yo = coff[u] < (int)K ? 2 * (coff[u] - q * 16) + 8 * q : (int)(2 * K);
#pragma unroll
                for (int ct = 0; ct < CT; ++ct)
                    __builtin_amdgcn_raw_buffer_store_b64((v2u32){yp[u][ct][0], yp[u][ct][1]}, ry,
                                                          yo + 32 * ct, 0, kNT);
            }
        };

        if constexpr (QMAX == 127) {
            // INT8 mode: one rounding per element (|y / s| <= 127 (1 + 2^-23),
            // so y * (1/s) is within 2^-15 of fl(y / s)); a quotient within
            // 2^-13 of a half-integer sends its group of four to the IEEE
            // division, as does a scale that is not finite
#pragma unroll
            for (int u = 0; u < TW; ++u) {
                uint32_t P[CT];
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) {
                    uint32_t c[4];
                    bool near = !finite;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float y = unpack_half<DT>(yp[u][ct][i >> 1], i & 1);
                        const float t = __builtin_fmaf(y, rinv, kMagic);
                        const float res = __builtin_fmaf(y, rinv, -(t - kMagic));
                        near |= fabsf(res) > 0.5f - 0x1p-13f;
                        c[i] = __float_as_uint(t);
                    }
                    if (__any(near)) {
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            c[i] = (uint32_t)code_of_quotient<127>(unpack_half<DT>(yp[u][ct][i >> 1], i & 1) / s);
                    }
                    P[ct] = pack_code_bytes(c[0], c[1], c[2], c[3]);
                }
                store_tile(u, P);
            }
        } else if (__builtin_expect(finite && one, 1)) {
            // one rounding per element: of the two bracketing multipliers,
            // the one that takes the k = 3 tie the quantizer's way gives every
            // code (the two agree on every element that is not a tie)
#pragma unroll
            for (int u = 0; u < TW; ++u) {
                uint32_t P[CT];
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) {
                    uint32_t c[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        c[i] = __float_as_uint(__builtin_fmaf(unpack_half<DT>(yp[u][ct][i >> 1], i & 1), r1, kMagic));
                    P[ct] = pack_code_bytes(c[0], c[1], c[2], c[3]);
                }
                store_tile(u, P);
            }
        } else if (finite) {
#pragma unroll
            for (int u = 0; u < TW; ++u) {
                uint32_t P[CT];
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) {
                    uint32_t c[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float y = unpack_half<DT>(yp[u][ct][i >> 1], i & 1);
                        c[i] = tie_select(__builtin_fmaf(y, rh, kMagic), __builtin_fmaf(y, rl, kMagic), tmask);
                    }
                    P[ct] = pack_code_bytes(c[0], c[1], c[2], c[3]);
                }
                store_tile(u, P);
            }
        } else {
            // an Inf or NaN scale: every quotient by IEEE division
#pragma unroll
            for (int u = 0; u < TW; ++u) {
                uint32_t P[CT];
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) {
                    uint32_t w = 0;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float y = unpack_half<DT>(yp[u][ct][i >> 1], i & 1);
                        w |= (uint32_t)(code_of_quotient<QMAX>(y / s) & 0xff) << (8 * i);
                    }
                    P[ct] = w;
                }
                store_tile(u, P);
            }
        }
    };

    // every wave takes at least one pass (a row past M is all zeros in and
    // nothing out), so no branch guards the loop and the first rows' loads
    // stay where they are issued, ahead of R's
    do {
#pragma unroll
        for (int p = 0; p < PF; ++p) {
            process(xf[p], row);
            row += nw;
            if (p + 1 < PF && row >= M) break;
        }
    } while (row < M);
}

// Contiguous 16-bit rows, g = 64, 32 < K/64 <= 64 group-rows (four tiles) or
// 16 < K/64 <= 32 (two tiles), 16-byte aligned rows, codes and smoothing
// factors, 8-byte aligned rotated export, enough rows to fill the GPU.  A
// dense R, or the structured one (signed Sylvester-Hadamard), whose
// fragments the kernel builds itself.
bool row_kernel_ok(const RQArgs& a)
{
    const bool sixteen = a.dtype == F16 || a.dtype == BF16;
    if (!sixteen || !(a.rot || a.hadamard) || a.g != 64 || a.sk != 1 || a.M < 2048 || a.M >= (int64_t(1) << 30))
        return false;
    if ((a.K % 64) != 0) return false;
    const int64_t gpr = a.K / 64;
    if (gpr <= 16 || gpr > 64) return false;
    if ((a.sm % 8) != 0 || ((uintptr_t)a.x % 16) != 0 || ((uintptr_t)a.codes % 16) != 0) return false;
    if ((a.K % 16) != 0) return false;
    if (a.smooth && ((uintptr_t)a.smooth % 16) != 0) return false;
    if (a.yout && ((uintptr_t)a.yout % 8) != 0) return false;
    return true;
}

// rows in flight per wave (two measured no faster than one: the extra
// registers cost a wave per SIMD)
constexpr int kRowPF = 1;

template <int DT, bool SMOOTH, bool YOUT, int TW, int QMAX>
static hipError_t launch_row_t(const RQArgs& a, hipStream_t st)
{
    auto kern = rq_row_kernel<DT, SMOOTH, YOUT, TW, kRowPF, QMAX>;
    static int per_cu = 0, n_cu = 0;
    if (per_cu == 0) {
        int dev = 0;
        hipDeviceProp_t p;
        if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&p, dev) != hipSuccess ||
            hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, 256, 0) != hipSuccess || per_cu < 1) {
            per_cu = 2;
            n_cu = 256;
        } else {
            n_cu = p.multiProcessorCount;
        }
    }
    // at most four workgroups (16 waves) per CU: with 8192 rows every wave
    // then takes exactly two (a fifth workgroup, which the registers would
    // allow, leaves waves with one or two rows and measured slower)
    int64_t grid = (int64_t)(per_cu < 4 ? per_cu : 4) * n_cu;
    const int64_t need = (a.M + 3) / 4;   // four waves (rows) per workgroup
    if (grid > need) grid = need;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(256), 0, st, (const uint16_t*)a.x, (int)a.M, a.K,
                       a.sm, a.rot, (const uint16_t*)a.smooth, a.codes, a.scales, (uint16_t*)a.yout,
                       a.hadamard ? 1 : 0, a.sign_in, a.sign_out);
    return hipGetLastError();
}

template <int DT, bool SMOOTH, bool YOUT, int QMAX>
static hipError_t launch_row_tw(const RQArgs& a, hipStream_t st)
{
    const int64_t gpr = a.K / 64;
    return gpr > 32 ? launch_row_t<DT, SMOOTH, YOUT, 4, QMAX>(a, st) : launch_row_t<DT, SMOOTH, YOUT, 2, QMAX>(a, st);
}

template <int DT, int QMAX>
static hipError_t launch_row_dt(const RQArgs& a, hipStream_t st)
{
    if (a.smooth)
        return a.yout ? launch_row_tw<DT, true, true, QMAX>(a, st) : launch_row_tw<DT, true, false, QMAX>(a, st);
    return a.yout ? launch_row_tw<DT, false, true, QMAX>(a, st) : launch_row_tw<DT, false, false, QMAX>(a, st);
}

hipError_t launch_rotate_quant_row(const RQArgs& a, hipStream_t st)
{
    if (a.qmax == 127) return a.dtype == BF16 ? launch_row_dt<BF16, 127>(a, st) : launch_row_dt<F16, 127>(a, st);
    return a.dtype == BF16 ? launch_row_dt<BF16, 7>(a, st) : launch_row_dt<F16, 7>(a, st);
}

}  // namespace w4a4
