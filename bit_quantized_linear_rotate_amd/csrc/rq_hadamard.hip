// Rotate + quantize with a structured rotation, for contiguous 16-bit rows:
//   R = diag(sign_in) . H_g . diag(sign_out) . c,   c = T(1 / sqrt(g)),
// H_g the Sylvester Hadamard matrix (H_1 = [1], H_2n = [[H_n, H_n], [H_n, -H_n]]),
// entries of R rounded to T exactly as the dense kernels round a given R.
// The layer is the same as everywhere in this library (web page "[Feat][Ascend]
// Consolidate INT8, RotateQuant, RoPE and ConvRot W4A4 backends", section "W4A4
// correctness and performance scope"; "[Feat][Ascend] Add fused RotateQuant
// backend", sections "What this PR does" (the INT8 mode) and "How was this patch
// tested?" (group sizes, asymmetric rotations)):
//   y = T(x_group . R),  s = max(absmax(y) / qmax, 2^-126),
//   c = clamp(round_half_even(fp32(y) / s), -qmax, qmax).
// Only the evaluation of x_group . R differs: it is a fast Walsh-Hadamard
// transform instead of a dense g x g product, i.e. another order of the fp32
// sum of the same exact products x_i * R_ij.
//
// Design (g = 2^L, 16 <= g <= 256; a 16-lane row of a wave holds 512
// consecutive elements of one row of x, lane (j, q) the 16 bytes at elements
// 32 j + 8 q .. + 7):
//   * H_g = H_{g/32} (x) H_32 for g >= 32 (element n = 32 a + b): stage 1 applies
//     c . H_32 to every 32-element chunk as two v_mfma_f32_16x16x32 against
//     constant A fragments (c . H_32 rows 0-15 and 16-31, built in registers
//     once), with the chunk as the B operand; lane (j, q) then holds U[d][a] for
//     d = 16 h + 4 q + r and chunk a = j mod (g/32).  The products are exact
//     (T times +-T(c)), so stage 1 is an fp32 sum of 32 exact products.
//   * Stage 2 applies H_{g/32} across the g/32 chunks of a group, which sit in
//     neighbouring lanes: log2(g/32) butterfly levels (partners at lane
//     distance 1, 2, 4 inside a 16-lane row, moved with DPP), each an fp32
//     a + b / b - a.  Lane (j, q) ends with y[32 j + 16 h + 4 q + r]: four
//     consecutive outputs, so every store is a contiguous 4 bytes of codes
//     (8 of rotated values) and a wave's stores cover 512 elements.
//   * g = 16: a 32-element piece holds two groups; output half h takes c . H_16
//     against group h's inputs only (the other group's are zeroed in the B
//     operand, so an infinite input never meets a zero weight); no stage 2.
//   * Error: stage 1 adds at most 31 roundings of partial sums, stage 2 at
//     most three more, so |y_fp32 - exact| <= 34 * 2^-24 * sum_i |x_i R_ij|,
//     inside the fp32 summation bound g * 2^-24 * sum_i |x_i R_ij| that every
//     dense kernel of this library is held to (g >= 64); for g = 16 and 32
//     the sum has at most g terms, as in the dense kernels.  Partial sums never
//     exceed sum_i |x_i R_ij| (the scale c is applied to the products).
//   * sign_in flips x before stage 1 (sign bit XOR, lane-constant masks);
//     sign_out flips y after stage 2.  Both are exact.
//   * A workgroup of W = ceil(K / 1024) waves (at most 16) works on one row at
//     a time, chunk p to wave p mod W (two chunks a wave: under 80 VGPRs, room
//     for several workgroups a CU); the row absmax is a wave max of the
//     sign-cleared 16-bit patterns (monotone in |y|, NaN above all), then the
//     W waves' through LDS (two buffers by row parity: one barrier per row).
//   * The next row's loads are issued before the current row is transformed,
//     into a second register set (the loop is unrolled so that the two sets
//     swap by name: a register copy would wait for the loads in flight).  All
//     loads and stores are buffer accesses whose range checks drop what lies
//     past the row, so every lane issues the same memory instructions and the
//     waits count them exactly.
//   * Codes: y * (1/s) rounded with one add of 1.5 * 2^23; a quotient within
//     the rounding band of a half-integer (2^-17 for qmax 7, 2^-13 for 127:
//     |y (1/s) - fl(y / s)| <= 2 qmax 2^-24) sends its four values to the IEEE
//     division, as does a scale that is not finite.
#include <cmath>
#include <cstring>

#include "common.hpp"
#include "kernels.hpp"
#include "row_quant.hpp"

namespace w4a4 {
namespace {

constexpr int HD_MAXW = 16;               // waves sharing one row (a 1024-thread workgroup)
constexpr int HD_MAXK = 16384;            // widest row
constexpr float kHdMagic = 12582912.0f;   // 1.5 * 2^23

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}

// partner value at lane distance D (1, 2 or 4) inside a 16-lane row
template <int D>
__device__ __forceinline__ float partner(float v)
{
    if constexpr (D == 1) return dpp_mov<0xb1>(v);           // quad_perm [1, 0, 3, 2]
    else if constexpr (D == 2) return dpp_mov<0x4e>(v);      // quad_perm [2, 3, 0, 1]
    else return dpp_mov<0x1b>(dpp_mov<0x141>(v));            // lane ^ 7, then ^ 3
}

typedef unsigned v2u_hd __attribute__((ext_vector_type(2)));

// buffer resource over [base, base + bytes): accesses past it read zeros and
// drop stores
__device__ __forceinline__ __amdgpu_buffer_rsrc_t hd_rsrc(const void* base, uint64_t bytes)
{
    const uint32_t n = bytes > 0xffffffffull ? 0xffffffffu : (uint32_t)bytes;
    return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)n, 0x00020000);
}

__device__ __forceinline__ uint32_t pack_magic4(float t0, float t1, float t2, float t3)
{
    const uint32_t lo = __builtin_amdgcn_perm(__float_as_uint(t1), __float_as_uint(t0), 0x0c0c0400u);
    const uint32_t hi = __builtin_amdgcn_perm(__float_as_uint(t3), __float_as_uint(t2), 0x0c0c0400u);
    return lo | (hi << 16);
}

template <int QMAX>
__device__ __forceinline__ uint32_t codes_exact4(const float (&y)[4], float s)
{
    uint32_t out = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float q = y[i] / s;
        const float cl = __builtin_amdgcn_fmed3f(rintf(q), -(float)QMAX, (float)QMAX);
        const int c = (q == q) ? (int)cl : 0;
        out |= ((uint32_t)c & 0xffu) << (8 * i);
    }
    return out;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v)
{
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xb1, 0xf, 0xf, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4e, 0xf, 0xf, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x124, 0xf, 0xf, false));  // row_ror:4
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xf, 0xf, false));  // row_ror:8
    const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
    const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
    const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
    const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
    return max(max(r0, r1), max(r2, r3));
}

// P: 512-element chunks per wave and row; PF: rows whose loads are in flight
// ahead of the one being transformed
template <int DT, int G, bool SMOOTH, int QMAX, int P, int PF>
__global__ __launch_bounds__(1024) void rq_hadamard_kernel(
    const uint16_t* __restrict__ x, int64_t M, int64_t K, int64_t sm, uint32_t cbits,
    const int8_t* __restrict__ sign_in, const int8_t* __restrict__ sign_out,
    const uint16_t* __restrict__ smooth, int8_t* __restrict__ codes, float* __restrict__ scales,
    uint16_t* __restrict__ yout)
{
    constexpr int LA = G >= 256 ? 3 : G >= 128 ? 2 : G >= 64 ? 1 : 0;   // stage-2 levels
    static_assert(PF == 1 || PF == 2, "one or two rows in flight");
    __shared__ uint32_t wmax[2][HD_MAXW];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int nw = (int)(blockDim.x >> 6);
    const int j = lane & 15, q = lane >> 4;

    // stage-1 A fragments: row i = j of c . H32 (h = 0) and 16 + j (h = 1),
    // k = 8 q + e; for g = 16 c . H16 in both diagonal blocks (the other
    // blocks meet zeroed inputs, see below)
    v8s af[2];
    const uint16_t cpos = (uint16_t)cbits, cneg = (uint16_t)(cbits | 0x8000u);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int d = 16 * h + j, b = 8 * q + e;
            uint16_t v;
            const int dd = G == 16 ? (d & 15) : d, bb = G == 16 ? (b & 15) : b;
            v = (__builtin_popcount(dd & bb) & 1) ? cneg : cpos;
            af[h][e] = (short)v;
        }
    // sign masks (sign-bit XOR on T patterns): the lane's inputs are
    // n = 32 (j mod g/32) + 8 q + e of a group (for g = 16: (8 q + e) mod 16),
    // its outputs m = 32 (j mod g/32) + 16 h + 4 q + r, two per packed word
    constexpr int AM = (G >= 32 ? G / 32 : 1) - 1;
    v8s smask;
    uint32_t omask[4];
    {
        // the lane's 8 input signs are contiguous, so are its 4 output signs
        // per h: three range-checked loads (a NULL array is a zero-sized
        // buffer: all +1), one wait
        const int n0 = G >= 32 ? 32 * (j & AM) + 8 * q : (8 * q) & 15;
        const __amdgpu_buffer_rsrc_t ri = hd_rsrc(sign_in, sign_in ? G : 0);
        const __amdgpu_buffer_rsrc_t ro = hd_rsrc(sign_out, sign_out ? G : 0);
        const v2u_hd sin8 = __builtin_bit_cast(v2u_hd, __builtin_amdgcn_raw_buffer_load_b64(ri, n0, 0, 0));
        uint32_t so4[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int m0 = G >= 32 ? 32 * (j & AM) + 16 * h + 4 * q : (16 * h + 4 * q) & 15;
            so4[h] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(ro, m0, 0, 0);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e)
            smask[e] = (short)(((sin8[e >> 2] >> (8 * (e & 3) + 7)) & 1u) << 15);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const uint32_t b = so4[w >> 1] >> (16 * (w & 1));   // signs of outputs r = 2 (w & 1), + 1
            omask[w] = (((b >> 7) & 1u) << 15) | (((b >> 15) & 1u) << 31);
        }
    }
    // butterfly signs: +1 where the lane is the lower partner
    const float bs1 = (j & 1) ? -1.0f : 1.0f, bs2 = (j & 2) ? -1.0f : 1.0f, bs4 = (j & 4) ? -1.0f : 1.0f;

    const int lo = 32 * j + 8 * q;                 // the lane's first input in a chunk
    const int oo = 32 * j + 4 * q;                 // its first output (h = 0; + 16 for h = 1)
    auto chunk_of = [&](int i) { return wave + nw * i; };
    // chunk p holds elements 512 p .. 512 p + 511.  Every access is a buffer
    // access whose range check drops what lies past the row (loads read
    // zeros), so each lane issues the same loads and stores and the waits
    // count them exactly: no lane-dependent branches around memory.
    auto load_row = [&](int64_t row, v8s (&xf)[P]) {
        const __amdgpu_buffer_rsrc_t rx =
            hd_rsrc(x + (row < M ? row : 0) * sm, row < M ? (uint64_t)K * 2 : 0);
#pragma unroll
        for (int i = 0; i < P; ++i) {
            const int off = (chunk_of(i) << 9) + lo;
            xf[i] = __builtin_bit_cast(v8s, __builtin_amdgcn_raw_buffer_load_b128(rx, off * 2, 0, 0));
        }
    };
    const __amdgpu_buffer_rsrc_t rsm = hd_rsrc(smooth, SMOOTH ? (uint64_t)K * 2 : 0);
    const __amdgpu_buffer_rsrc_t rsc = hd_rsrc(scales, (uint64_t)M * 4);

    int par = 0;
    // transform, quantize and store one row (a no-op past M; every wave of
    // the workgroup takes the same rows, so the barrier is uniform)
    auto process = [&](int64_t row, const v8s (&xin)[P]) {
        if (row >= M) return;
        uint32_t yp[P][4];                         // packed T values: [h * 2 + r / 2]
        typedef unsigned short v2u16 __attribute__((ext_vector_type(2)));
        v2u16 m2 = {0, 0};                         // max sign-cleared 16-bit patterns, packed
#pragma unroll
        for (int i = 0; i < P; ++i) {
            const int p = chunk_of(i);
            v8s xv = xin[i];
            if constexpr (SMOOTH) {
                // (lanes past K read zero factors: their inputs stay zero
                // instead of becoming 0 / 0)
                const bool in = (p << 9) + lo < K;
                const v8s sv = __builtin_bit_cast(
                    v8s, __builtin_amdgcn_raw_buffer_load_b128(rsm, ((p << 9) + lo) * 2, 0, 0));
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint16_t qb = f32_to_h<DT>(h_to_f32<DT>((uint16_t)xv[e]) / h_to_f32<DT>((uint16_t)sv[e]));
                    xv[e] = (short)(in ? qb : (uint16_t)0);
                }
            }
            xv ^= smask;
            v4f u[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                // g = 16: group h of the piece only (lanes q = 2h, 2h + 1); the
                // other group's inputs are zeroed in B rather than met by zeros
                // in A, so that an infinite input never multiplies a zero
                v8s bv = xv;
                if constexpr (G == 16) {
                    if ((q >> 1) != h) bv = (v8s){0, 0, 0, 0, 0, 0, 0, 0};
                }
                if constexpr (DT == BF16)
                    u[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, af[h]),
                                                                   __builtin_bit_cast(v8bf, bv),
                                                                   (v4f){0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                else
                    u[h] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, af[h]),
                                                                  __builtin_bit_cast(v8h, bv),
                                                                  (v4f){0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
            }
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                uint16_t hv[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float v = u[h][r];
                    if constexpr (LA >= 1) v = __builtin_fmaf(bs1, v, partner<1>(v));
                    if constexpr (LA >= 2) v = __builtin_fmaf(bs2, v, partner<2>(v));
                    if constexpr (LA >= 3) v = __builtin_fmaf(bs4, v, partner<4>(v));
                    hv[r] = f32_to_h<DT>(v);
                }
                yp[i][2 * h] = ((uint32_t)hv[0] | ((uint32_t)hv[1] << 16)) ^ omask[2 * h];
                yp[i][2 * h + 1] = ((uint32_t)hv[2] | ((uint32_t)hv[3] << 16)) ^ omask[2 * h + 1];
                m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(v2u16, yp[i][2 * h] & 0x7fff7fffu));
                m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(v2u16, yp[i][2 * h + 1] & 0x7fff7fffu));
            }
        }
        // lanes past K hold zeros (zero inputs, zero outputs): they do not
        // raise the max
        const uint32_t wm = wave_max_u32(max((uint32_t)m2[0], (uint32_t)m2[1]));
        if (lane == 0) wmax[par][wave] = wm;
        __syncthreads();
        uint32_t mm = wmax[par][0];
        for (int w = 1; w < nw; ++w) mm = max(mm, wmax[par][w]);
        par ^= 1;
        // INT4 codes: the row's quantizer from the significand table (or
        // divisions outside its range), codes from one fma per value (or the
        // two bracketing fmas and the tie mask when 7 divides the absmax's
        // significand); the INT8 mode: product, residual test, exact division
        // near half-integers
        RowQuant rq;
        float sv;
        if constexpr (QMAX == 7) {
            rq = row_quant_thread<DT>(mm);
            sv = rq.s;
        } else {
            const float amax = h_to_f32<DT>((uint16_t)mm);
            sv = amax / (float)QMAX;
            if (sv < 0x1p-126f) sv = 0x1p-126f;        // NaN stays NaN
        }
        // lane 0 of wave 0 writes the scale (the other lanes' offsets are
        // out of range and dropped)
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sv), rsc,
                                              (wave == 0 && lane == 0) ? (int)(row * 4) : (int)(M * 4), 0, 0);
        const float ri = 1.0f / sv;
        constexpr float kBand = QMAX == 7 ? 0x1p-17f : 0x1p-13f;
        constexpr float kQ = (float)QMAX;
        const bool fin = fabsf(sv) < 3.0e38f;
        const __amdgpu_buffer_rsrc_t rc = hd_rsrc(codes + row * K, (uint64_t)K);
        const __amdgpu_buffer_rsrc_t ry = hd_rsrc(yout ? yout + row * K : nullptr, yout ? (uint64_t)K * 2 : 0);
#pragma unroll
        for (int i = 0; i < P; ++i) {
            const int ob = (chunk_of(i) << 9) + oo;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                float yy[4];
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    yy[r] = h_to_f32<DT>((uint16_t)(yp[i][2 * h + (r >> 1)] >> (16 * (r & 1))));
                uint32_t pk;
                if (!fin) {
                    pk = codes_exact4<QMAX>(yy, sv);
                } else if constexpr (QMAX == 7) {
                    pk = rq.exact ? codes_exact4<7>(yy, sv) : rq.one ? quant4_one(yy, rq) : quant4_bracket(yy, rq);
                } else {
                    float t[4];
                    bool nr = false;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float qv = yy[r] * ri;
                        t[r] = __builtin_amdgcn_fmed3f(qv, -kQ, kQ) + kHdMagic;
                        nr |= fabsf(qv - (t[r] - kHdMagic)) > 0.5f - kBand;
                    }
                    pk = pack_magic4(t[0], t[1], t[2], t[3]);
                    if (__any(nr)) pk = codes_exact4<QMAX>(yy, sv);
                }
                __builtin_amdgcn_raw_buffer_store_b32(pk, rc, ob + 16 * h, 0, 0);
                if (yout)
                    __builtin_amdgcn_raw_buffer_store_b64(
                        __builtin_bit_cast(v2u_hd, make_uint2(yp[i][2 * h], yp[i][2 * h + 1])), ry,
                        (ob + 16 * h) * 2, 0, 0);
            }
        }
    };

    // Rows blockIdx.x, + grid, ...: PF + 1 register sets rotate by name (no
    // copies, which would wait for the loads in flight), the loads of row
    // r + PF * grid issued before row r is transformed.
    const int64_t rs = gridDim.x;
    const int64_t r0 = blockIdx.x;
    v8s xa[P], xb[P];
    if constexpr (PF == 1) {
        load_row(r0, xa);
        for (int64_t row = r0; row < M; row += 2 * rs) {
            load_row(row + rs, xb);
            process(row, xa);
            load_row(row + 2 * rs, xa);
            process(row + rs, xb);
        }
    } else {
        v8s xc[P];
        load_row(r0, xa);
        load_row(r0 + rs, xb);
        for (int64_t row = r0; row < M; row += 3 * rs) {
            load_row(row + 2 * rs, xc);
            process(row, xa);
            load_row(row + 3 * rs, xa);
            process(row + rs, xb);
            load_row(row + 4 * rs, xb);
            process(row + 2 * rs, xc);
        }
    }
}

// T(fl32(1 / sqrt(g))) as a 16-bit pattern, on the host: the entry of R
// rounded to T as the dense kernels round an fp32 R (for every supported g
// the same as rounding 1 / sqrt(g) itself).
uint32_t scale_bits(int dt, int g)
{
    const float f = (float)(1.0 / std::sqrt((double)g));
    if (dt == F16) {
        const _Float16 h = (_Float16)f;
        uint16_t b;
        std::memcpy(&b, &h, 2);
        return b;
    }
    uint32_t u;
    std::memcpy(&u, &f, 4);
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;   // nearest even (f is finite)
}

template <int DT, int G, int QMAX>
hipError_t launch_g(const RQArgs& a, hipStream_t st)
{
    static int n_cu = 0;
    if (n_cu == 0) {
        int dev = 0, v = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
            n_cu = v;
        else
            n_cu = 256;
    }
    // two chunks a wave and one row in flight: the fastest of the measured
    // shapes (P in {1, 2, 4}, PF in {1, 2}, 32 or 64 waves a CU)
    constexpr int P = 2, PF = 1;
    const int nchunk = (int)((a.K + 511) / 512);
    const int nw = (nchunk + P - 1) / P;
    // a persistent grid: each workgroup walks rows blockIdx.x, + grid, ...
    const int64_t per_cu = 32 / nw > 0 ? 32 / nw : 1;   // up to 32 waves a CU
    const int64_t want = (int64_t)n_cu * per_cu;
    const unsigned grid = (unsigned)(a.M < want ? a.M : want);
    const uint32_t cb = scale_bits(DT, G);
    auto* xp = (const uint16_t*)a.x;
    auto* sp = (const uint16_t*)a.smooth;
    auto* yp = (uint16_t*)a.yout;
    if (a.smooth)
        hipLaunchKernelGGL((rq_hadamard_kernel<DT, G, true, QMAX, P, PF>), dim3(grid), dim3(64 * nw), 0, st, xp, a.M,
                           a.K, a.sm, cb, a.sign_in, a.sign_out, sp, a.codes, a.scales, yp);
    else
        hipLaunchKernelGGL((rq_hadamard_kernel<DT, G, false, QMAX, P, PF>), dim3(grid), dim3(64 * nw), 0, st, xp, a.M,
                           a.K, a.sm, cb, a.sign_in, a.sign_out, sp, a.codes, a.scales, yp);
    return hipGetLastError();
}

template <int DT, int QMAX>
hipError_t launch_q(const RQArgs& a, hipStream_t st)
{
    switch (a.g) {
    case 16: return launch_g<DT, 16, QMAX>(a, st);
    case 32: return launch_g<DT, 32, QMAX>(a, st);
    case 64: return launch_g<DT, 64, QMAX>(a, st);
    case 128: return launch_g<DT, 128, QMAX>(a, st);
    default: return launch_g<DT, 256, QMAX>(a, st);
    }
}

}  // namespace

// Contiguous 16-bit rows (16-byte aligned, row stride a multiple of 8; fewer
// than 2^29 rows, so that scale offsets fit the buffer offsets), g a
// power of two in [16, 256], K at most 16384, 4-byte
// aligned codes, 8-byte aligned rotated export and sign arrays, 16-byte
// aligned smoothing.
bool hadamard_kernel_ok(const RQArgs& a)
{
    const bool sixteen = a.dtype == F16 || a.dtype == BF16;
    if (!sixteen || a.M <= 0 || a.M >= (1 << 29) || a.sk != 1 || (a.qmax != 7 && a.qmax != 127)) return false;
    if (!(a.g == 16 || a.g == 32 || a.g == 64 || a.g == 128 || a.g == 256)) return false;
    if (a.K <= 0 || (a.K % a.g) != 0 || a.K > HD_MAXK) return false;
    if ((a.sm % 8) != 0 || ((uintptr_t)a.x % 16) != 0) return false;
    if (((uintptr_t)a.codes % 4) != 0 || (a.yout && ((uintptr_t)a.yout % 8) != 0)) return false;
    if (a.smooth && ((uintptr_t)a.smooth % 16) != 0) return false;
    if (((uintptr_t)a.sign_in % 8) != 0 || ((uintptr_t)a.sign_out % 8) != 0) return false;
    return true;
}

hipError_t launch_rotate_quant_hadamard(const RQArgs& a, hipStream_t st)
{
    if (!hadamard_kernel_ok(a)) return hipErrorNotSupported;
    if (a.dtype == BF16)
        return a.qmax == 127 ? launch_q<BF16, 127>(a, st) : launch_q<BF16, 7>(a, st);
    return a.qmax == 127 ? launch_q<F16, 127>(a, st) : launch_q<F16, 7>(a, st);
}

}  // namespace w4a4
