// Fused block rotation + per-row signed-INT4 quantization (gfx950).
//
// What is computed (web page "[Feat][Ascend] Consolidate INT8, RotateQuant,
// RoPE and ConvRot W4A4 backends", section "W4A4 correctness and performance
// scope"; "[Perf][Ascend] Avoid activation pack/unpack in ConvRot W4A4",
// section "Summary"; "[Feat][Ascend] Add fused RotateQuant backend", section
// "What this PR does"):
//   x' = T(fp32(x) / fp32(smooth))            (optional input smoothing)
//   y  = T( x'_group . T(R) )                 (per group of g entries, fp32 sums)
//   s  = max(absmax_row(y) / 7, 2^-126)       (IEEE fp32; NaN row -> NaN)
//   c  = clamp(round_half_even(y / s), -7, 7) (codes kept unpacked in int8)
//
// Design for CDNA4:
//   * 16-bit activations rotate on MFMA (v_mfma_f32_16x16x32_{bf16,f16}):
//     a row is viewed as K/g "group-rows" of g entries; 16 group-rows times the
//     g x g rotation is a small GEMM whose B operand (the rotation) stays in
//     VGPRs for the whole kernel.  For g = 256 the four waves of a workgroup
//     split the 16 output-column tiles so that each holds a quarter of R.
//   * x streams from HBM straight into A-fragment registers (each lane reads a
//     contiguous g/4-element slice of one group-row; a wave covers 16 whole
//     group-rows), so the kernel reads x exactly once.
//   * Rotated values are rounded to T and parked in LDS until the row absmax
//     (an integer max over |y| bit patterns, so a NaN dominates) is known; the
//     quantize pass then streams codes out with 16-byte stores.
//   * y / s is evaluated as y * (1/s) and re-done with an IEEE division only
//     when the product lies within 2^-17 of a rounding boundary, which keeps
//     the code identical to the correctly-rounded quotient's.
#include "common.hpp"
#include "kernels.hpp"
#include "row_quant.hpp"

namespace w4a4 {

// Nearest-even code of the correctly rounded quotient y / s, clamped to
// [-7, 7]; NaN -> 0.  rinv = 1/s (correctly rounded).  Because |y/s| <= 7
// (1 + 2^-23), y * rinv is within 2^-19 of fl(y/s); outside a 2^-17 band
// around a half-integer both round to the same integer.
__device__ __forceinline__ int quant_code(float y, float s, float rinv)
{
    float q = y * rinv;
    float aq = fabsf(q);
    float fr = aq - floorf(aq);
    if (fabsf(fr - 0.5f) < 0x1p-17f) q = y / s;
    if (q != q) return 0;
    float r = rintf(q);
    r = fminf(fmaxf(r, -7.0f), 7.0f);
    return (int)r;
}

// The same for the INT8 mode (|y/s| <= 127 (1 + 2^-23)): y * rinv is within
// 2^-15 of fl(y/s), so outside a 2^-13 band around a half-integer both round
// to the same integer.
__device__ __forceinline__ int quant_code127(float y, float s, float rinv)
{
    float q = y * rinv;
    float aq = fabsf(q);
    float fr = aq - floorf(aq);
    if (fabsf(fr - 0.5f) < 0x1p-13f) q = y / s;
    if (q != q) return 0;
    float r = rintf(q);
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    return (int)r;
}

template <int QMAX>
__device__ __forceinline__ int quant_code_q(float y, float s, float rinv)
{
    if constexpr (QMAX == 7) return quant_code(y, s, rinv);
    else return quant_code127(y, s, rinv);
}

// Four codes packed into one dword (code r in byte r).  quant4_fast uses
// y * (1/s) and raises `near` when any quotient lies within 2^-17 of a
// half-integer, where only the correctly rounded quotient may be trusted;
// quant4_exact divides.  For |y/s| <= 7 (1 + 2^-23) the fast product is within
// 2^-19 of fl(y/s), so outside that band both give the same integer.
__device__ __forceinline__ uint32_t pack_codes(const float (&r)[4])
{
    uint32_t out = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) out |= ((uint32_t)((int)r[i] & 0xff)) << (8 * i);
    return out;
}

__device__ __forceinline__ uint32_t quant4_fast(const float (&y)[4], float rinv, bool& near)
{
    float c[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float q = y[i] * rinv;
        const float r = rintf(q);
        near |= fabsf(fabsf(q - r) - 0.5f) < 0x1p-17f;
        const float cl = __builtin_amdgcn_fmed3f(r, -7.0f, 7.0f);
        c[i] = (q == q) ? cl : 0.0f;
    }
    return pack_codes(c);
}

template <int QMAX = 7>
__device__ __forceinline__ uint32_t quant4_exact(const float (&y)[4], float s)
{
    float c[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float q = y[i] / s;
        const float cl = __builtin_amdgcn_fmed3f(rintf(q), -(float)QMAX, (float)QMAX);
        c[i] = (q == q) ? cl : 0.0f;
    }
    return pack_codes(c);
}

// Fast path for rows whose scale is finite (then every entry is finite).  The
// clamped quotient plus 1.5 * 2^23 is rounded to the nearest even integer by
// the addition itself, and that integer's low byte is the two's-complement
// code; subtracting the constant again gives the rounded value exactly, so
// the residual q - r shows whether q sat within 2^-17 of a half-integer.
constexpr float kRoundMagic = 12582912.0f;  // 1.5 * 2^23

__device__ __forceinline__ uint32_t pack4_magic(float t0, float t1, float t2, float t3)
{
    const uint32_t lo = __builtin_amdgcn_perm(__float_as_uint(t1), __float_as_uint(t0), 0x0c0c0400u);
    const uint32_t hi = __builtin_amdgcn_perm(__float_as_uint(t3), __float_as_uint(t2), 0x0c0c0400u);
    return lo | (hi << 16);
}

// fp32 pattern of T(|v|) for the sign-cleared fp32 pattern of v
template <int DT>
__device__ __forceinline__ uint32_t round_bits(uint32_t vbits)
{
    return __float_as_uint(h_to_f32<DT>(f32_to_h<DT>(__uint_as_float(vbits))));
}

__device__ __forceinline__ float row_scale(uint32_t absmax_bits)
{
    float a = __uint_as_float(absmax_bits);
    float s = a / 7.0f;
    if (s < 0x1p-126f) s = 0x1p-126f;  // NaN compares false and stays NaN
    return s;
}

template <int QMAX>
__device__ __forceinline__ float row_scale_q(uint32_t absmax_bits)
{
    float a = __uint_as_float(absmax_bits);
    float s = a / (float)QMAX;
    if (s < 0x1p-126f) s = 0x1p-126f;  // NaN compares false and stays NaN
    return s;
}

// Wave-wide unsigned max with DPP moves inside each row of 16 lanes (quad
// swaps, then row rotations by 4 and 8) and four lane reads across rows; no
// LDS round trips.
__device__ __forceinline__ uint32_t wave_max_dpp(uint32_t v)
{
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xb1, 0xf, 0xf, false));  // quad [1,0,3,2]
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4e, 0xf, 0xf, false));  // quad [2,3,0,1]
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x124, 0xf, 0xf, false)); // row_ror:4
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xf, 0xf, false)); // row_ror:8
    const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
    const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
    const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
    const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
    return max(max(r0, r1), max(r2, r3));
}

__device__ __forceinline__ uint32_t wave_max16(uint32_t v)
{
    // max over the 16 lanes that share lane/16 (xor partners stay inside)
    v = max(v, (uint32_t)__shfl_xor((int)v, 1));
    v = max(v, (uint32_t)__shfl_xor((int)v, 2));
    v = max(v, (uint32_t)__shfl_xor((int)v, 4));
    v = max(v, (uint32_t)__shfl_xor((int)v, 8));
    return v;
}

// -------------------------------------------------------------------------
// MFMA path for 16-bit activations.
//   GP  = MFMA group width: g for g >= 32, 32 for g = 16 (two groups side by
//         side, the rotation placed twice on the diagonal of a 32 x 32 B).
//   ROT = false skips the rotation (y = x').
// LDS: rowmax[rows] | y buffer, group-row gr at gr * (GP + 8) (16-byte pad
// per group-row keeps the column-tile stores of the four lane groups in
// distinct banks).
// -------------------------------------------------------------------------
template <int DT, int GP, bool CONTIG, bool ROT, bool SMOOTH>
__global__ __launch_bounds__(256) void rq_mfma_kernel(
    const uint16_t* __restrict__ x, int64_t M, int64_t K, int64_t sm, int64_t sk,
    const float* __restrict__ rot, int g, const uint16_t* __restrict__ smooth,
    int8_t* __restrict__ codes, float* __restrict__ scales, uint16_t* __restrict__ yout,
    int rows_per_wg)
{
    constexpr int NCT = GP / 16;              // 16-wide output column tiles
    constexpr int NKS = GP / 32;              // 32-deep MFMA k-steps
    constexpr int NWC = NCT >= 4 ? NCT / 4 : 1;
    constexpr int CT = NCT / NWC;             // column tiles per wave
    constexpr int NTS = 4 / NWC;              // independent tile streams
    constexpr int LPL = GP / 4;               // elements per lane per group-row
    constexpr int PADG = GP + 8;

    extern __shared__ __align__(16) uint8_t smem[];
    uint32_t* rowmax = (uint32_t*)smem;
    float* rowsc = (float*)(smem + 4 * 64);
    float* rowinv = (float*)(smem + 8 * 64);
    uint16_t* ybuf = (uint16_t*)(smem + 12 * 64);

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int j = lane & 15, q = lane >> 4;
    const int cw = wave % NWC, ts = wave / NWC;

    const int64_t m0 = (int64_t)blockIdx.x * rows_per_wg;
    const int nrows = (int)min((int64_t)rows_per_wg, M - m0);
    const int gpr = (int)(K / GP);            // group-rows per row
    const int ngr = nrows * gpr;
    const int ntiles = (ngr + 15) >> 4;

    if (tid < rows_per_wg) rowmax[tid] = 0u;

    // Rotation fragments (B operand), rounded to T, kept for the whole kernel.
    v8s bfr[ROT ? CT : 1][ROT ? NKS : 1];
    if constexpr (ROT) {
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            const int c = (cw * CT + ct) * 16 + j;
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int kk = q * LPL + ks * 8 + e;
                    float rv;
                    if (GP == 32 && g == 16)
                        rv = ((kk >> 4) == (c >> 4)) ? rot[(kk & 15) * 16 + (c & 15)] : 0.0f;
                    else
                        rv = rot[kk * GP + c];
                    bfr[ct][ks][e] = (short)f32_to_h<DT>(rv);
                }
            }
        }
    }
    __syncthreads();

    for (int t = ts; t < ntiles; t += NTS) {
        // ---- A fragments: lane (j, q) holds group-row t*16+j, elements
        //      [q*LPL, q*LPL+LPL) split into NKS chunks of 8.
        const int gra = t * 16 + j;
        const bool va = gra < ngr;
        const int ml = va ? gra / gpr : 0;
        const int b = va ? gra - ml * gpr : 0;
        const int64_t kbase = (int64_t)b * GP + q * LPL;
        v8s afr[NKS];
        if (va) {
            if constexpr (CONTIG) {
                const v4i* src = (const v4i*)(x + (m0 + ml) * sm + kbase);
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    v4i u = __builtin_nontemporal_load(src + ks);
                    afr[ks] = __builtin_bit_cast(v8s, u);
                }
            } else {
                const uint16_t* src = x + (m0 + ml) * sm + kbase * sk;
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
                    for (int e = 0; e < 8; ++e) afr[ks][e] = (short)src[(int64_t)(ks * 8 + e) * sk];
            }
            if constexpr (SMOOTH) {
                const uint4* sp = (const uint4*)(smooth + kbase);
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    v8s sv = __builtin_bit_cast(v8s, sp[ks]);
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        float xv = h_to_f32<DT>((uint16_t)afr[ks][e]);
                        float fv = h_to_f32<DT>((uint16_t)sv[e]);
                        afr[ks][e] = (short)f32_to_h<DT>(xv / fv);
                    }
                }
            }
        } else {
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) afr[ks] = (v8s){0, 0, 0, 0, 0, 0, 0, 0};
        }

        if constexpr (ROT) {
            uint32_t rmax[4] = {0u, 0u, 0u, 0u};
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    if constexpr (DT == BF16)
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(v8bf, afr[ks]), __builtin_bit_cast(v8bf, bfr[ct][ks]),
                            acc, 0, 0, 0);
                    else
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                            __builtin_bit_cast(v8h, afr[ks]), __builtin_bit_cast(v8h, bfr[ct][ks]),
                            acc, 0, 0, 0);
                }
                const int c = (cw * CT + ct) * 16 + j;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int gr = t * 16 + 4 * q + r;
                    uint16_t yb = f32_to_h<DT>(acc[r]);
                    if (gr < ngr) ybuf[gr * PADG + c] = yb;
                    uint32_t ab = __float_as_uint(h_to_f32<DT>(yb)) & 0x7fffffffu;
                    rmax[r] = max(rmax[r], gr < ngr ? ab : 0u);
                }
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                uint32_t v = wave_max16(rmax[r]);
                const int gr = t * 16 + 4 * q + r;
                if (j == 0 && gr < ngr) atomicMax(&rowmax[gr / gpr], v);
            }
        } else {
            uint32_t rm = 0u;
            if (va) {
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    *(v8s*)(ybuf + gra * PADG + q * LPL + ks * 8) = afr[ks];
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        rm = max(rm, __float_as_uint(h_to_f32<DT>((uint16_t)afr[ks][e])) & 0x7fffffffu);
                }
                // lanes q = 0..3 with the same j share one group-row
            }
            rm = max(rm, (uint32_t)__shfl_xor((int)rm, 16));
            rm = max(rm, (uint32_t)__shfl_xor((int)rm, 32));
            if (q == 0 && va) atomicMax(&rowmax[ml], rm);
        }
    }
    __syncthreads();

    if (tid < nrows) {
        float s = row_scale(rowmax[tid]);
        rowsc[tid] = s;
        rowinv[tid] = 1.0f / s;
        scales[m0 + tid] = s;
    }
    __syncthreads();

    // ---- quantize: 16 consecutive entries of one group-row per step.
    const int cpr = (int)(K >> 4);            // 16-entry chunks per row
    const int nch = nrows * cpr;
    for (int ch = tid; ch < nch; ch += 256) {
        const int r = ch / cpr;
        const int k0 = (ch - r * cpr) << 4;
        const int gr = r * gpr + (k0 / GP);
        const uint16_t* yp = ybuf + gr * PADG + (k0 % GP);
        v8s y0 = *(const v8s*)yp;
        v8s y1 = *(const v8s*)(yp + 8);
        const float s = rowsc[r], ri = rowinv[r];
        uint32_t w[4];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            uint32_t packed = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int idx = d * 4 + e;
                uint16_t hb = (uint16_t)(idx < 8 ? y0[idx] : y1[idx - 8]);
                int c = quant_code(h_to_f32<DT>(hb), s, ri);
                packed |= ((uint32_t)(c & 0xff)) << (8 * e);
            }
            w[d] = packed;
        }
        st_stream16(codes + (m0 + r) * K + k0, w[0], w[1], w[2], w[3]);
        if (yout) {
            uint16_t* yo = yout + (m0 + r) * K + k0;
            const uint4 a0 = __builtin_bit_cast(uint4, y0), a1 = __builtin_bit_cast(uint4, y1);
            st_stream16(yo, a0.x, a0.y, a0.z, a0.w);
            st_stream16(yo + 8, a1.x, a1.y, a1.z, a1.w);
        }
    }
}

// -------------------------------------------------------------------------
// Column-major path for 16-bit activations stored with unit row stride
// (x[m, k] at x[k * sk + m], e.g. the transpose of a contiguous (K, M)
// buffer).  One 512-thread workgroup per 32-row block walks the K/g rotation
// groups twice: the first pass rotates and keeps the per-row absmax, the
// second rotates again and quantizes with the now known row scale (the rows
// are too long to park their rotated values on chip).
//   * A group's tile (g k-rows of 32 consecutive x values = 64 bytes) goes
//     global -> LDS with buffer_load ... lds into a ring of tiles, so each
//     load instruction reads 16 whole 64-byte segments; neighbouring row
//     blocks run on the same XCD, where they share 128-byte lines in L2.
//   * The two 32-byte halves of a k-row are swapped in odd quarters of the
//     group (k-rows g/4 .. g/2-1 and 3g/4 ..), so the four lane groups of a
//     transposing read, which read the same rows of k-rows g/4 apart, do not
//     all land on the same banks.
//   * MFMA A operands come straight out of the [k][m] tile with
//     ds_read_b64_tr_b16: within each 16-lane group, lane i receives element
//     (i & 3) of the 4-element reads of lanes 4e + (i >> 2), e = 0..3, so
//     when lane L reads k-row 8q' + (L >> 2) at rows 4 (L & 3) .. +3, lane i
//     gets x[i][8q' + e]; two such reads give the 8 k of a fragment.
//   * The k-slots of each MFMA step match the contiguous-row MFMA kernel
//     (lane group q, step ks: k = q * g/4 + 8 ks + e), so both give the same
//     rotated bits.
//   * The rotation B operand (a slice per wave) stays in VGPRs.
//   * Waves 0-3 issue every tile load and waves 4-7 every store, so each
//     wave's vmcnt counts one kind of operation (loads and stores may retire
//     out of order with respect to each other) and a loader's wait for its
//     own tile leaves the next tile in flight.  Codes (and the optional
//     rotated export) are staged per group in LDS and leave as 16-byte
//     buffer stores whose range check drops rows past M.
// -------------------------------------------------------------------------
// LDS writes visible, then a workgroup barrier that does not wait for the
// loads and stores still in flight (__syncthreads would).
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
}

typedef unsigned v2u32 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rq_rsrc(const void* base, uint64_t bytes)
{
    const uint32_t n = bytes > 0x7fffffffull ? 0x7fffffffu : (uint32_t)bytes;
    return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)n, 0x00020000);
}

constexpr int CM_ROWS = 32;            // rows per workgroup
constexpr int CM_OOB = 0x7ffffff0;     // byte offset past every range used below

typedef short v4s __attribute__((ext_vector_type(4)));

// NKS pairs of transposing reads from LDS byte address a: pair ks reads at
// a + 512 ks and a + 512 ks + 256 (k-rows 8 ks and 8 ks + 4 of a 64-byte-row
// tile).  Written as inline asm because the compiler makes the builtin form
// wait for every outstanding global load first.  The block first waits for
// earlier stores to have read their data registers (expcnt: the compiler
// does not order those against asm outputs) and waits for its own reads
// before it ends, so no register is handed out while a read is in flight;
// the outputs are early-clobber so that none shares the address register,
// which later reads of the block still use.
template <int NKS> struct TrReads;
template <> struct TrReads<8> {
    static __device__ __forceinline__ void run(unsigned a, v4s (&lo)[8], v4s (&hi)[8])
    {
        asm volatile(
            "s_waitcnt expcnt(0)\n\tds_read_b64_tr_b16 %0, %16\n\tds_read_b64_tr_b16 %1, %16 offset:256\n\t"
            "ds_read_b64_tr_b16 %2, %16 offset:512\n\tds_read_b64_tr_b16 %3, %16 offset:768\n\t"
            "ds_read_b64_tr_b16 %4, %16 offset:1024\n\tds_read_b64_tr_b16 %5, %16 offset:1280\n\t"
            "ds_read_b64_tr_b16 %6, %16 offset:1536\n\tds_read_b64_tr_b16 %7, %16 offset:1792\n\t"
            "ds_read_b64_tr_b16 %8, %16 offset:2048\n\tds_read_b64_tr_b16 %9, %16 offset:2304\n\t"
            "ds_read_b64_tr_b16 %10, %16 offset:2560\n\tds_read_b64_tr_b16 %11, %16 offset:2816\n\t"
            "ds_read_b64_tr_b16 %12, %16 offset:3072\n\tds_read_b64_tr_b16 %13, %16 offset:3328\n\t"
            "ds_read_b64_tr_b16 %14, %16 offset:3584\n\tds_read_b64_tr_b16 %15, %16 offset:3840\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(lo[0]), "=&v"(hi[0]), "=&v"(lo[1]), "=&v"(hi[1]), "=&v"(lo[2]), "=&v"(hi[2]),
              "=&v"(lo[3]), "=&v"(hi[3]), "=&v"(lo[4]), "=&v"(hi[4]), "=&v"(lo[5]), "=&v"(hi[5]),
              "=&v"(lo[6]), "=&v"(hi[6]), "=&v"(lo[7]), "=&v"(hi[7])
            : "v"(a)
            : "memory");
    }
};
template <> struct TrReads<4> {
    static __device__ __forceinline__ void run(unsigned a, v4s (&lo)[4], v4s (&hi)[4])
    {
        asm volatile(
            "s_waitcnt expcnt(0)\n\tds_read_b64_tr_b16 %0, %8\n\tds_read_b64_tr_b16 %1, %8 offset:256\n\t"
            "ds_read_b64_tr_b16 %2, %8 offset:512\n\tds_read_b64_tr_b16 %3, %8 offset:768\n\t"
            "ds_read_b64_tr_b16 %4, %8 offset:1024\n\tds_read_b64_tr_b16 %5, %8 offset:1280\n\t"
            "ds_read_b64_tr_b16 %6, %8 offset:1536\n\tds_read_b64_tr_b16 %7, %8 offset:1792\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(lo[0]), "=&v"(hi[0]), "=&v"(lo[1]), "=&v"(hi[1]), "=&v"(lo[2]), "=&v"(hi[2]),
              "=&v"(lo[3]), "=&v"(hi[3])
            : "v"(a)
            : "memory");
    }
};
template <> struct TrReads<2> {
    static __device__ __forceinline__ void run(unsigned a, v4s (&lo)[2], v4s (&hi)[2])
    {
        asm volatile(
            "s_waitcnt expcnt(0)\n\tds_read_b64_tr_b16 %0, %4\n\tds_read_b64_tr_b16 %1, %4 offset:256\n\t"
            "ds_read_b64_tr_b16 %2, %4 offset:512\n\tds_read_b64_tr_b16 %3, %4 offset:768\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(lo[0]), "=&v"(hi[0]), "=&v"(lo[1]), "=&v"(hi[1])
            : "v"(a)
            : "memory");
    }
};

// One 16-byte LDS read, in asm for the same reason as TrReads.
__device__ __forceinline__ v4i lds_read16(const void* p)
{
    v4i v;
    asm volatile("s_waitcnt expcnt(0)\n\tds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)"
                 : "=&v"(v)
                 : "v"((unsigned)(size_t)(__attribute__((address_space(3))) const void*)p)
                 : "memory");
    return v;
}

// LDS stores in asm: as a compiler-visible store after the LDS-DMA loads
// the compiler would first wait for all of them.  Completion is covered by
// the lgkmcnt(0) before the next barrier.
__device__ __forceinline__ void lds_write4(void* p, uint32_t v)
{
    asm volatile("ds_write_b32 %0, %1"
                 :
                 : "v"((unsigned)(size_t)(__attribute__((address_space(3))) void*)p), "v"(v)
                 : "memory");
}

__device__ __forceinline__ void lds_write8(void* p, uint32_t lo, uint32_t hi)
{
    asm volatile("ds_write_b64 %0, %1"
                 :
                 : "v"((unsigned)(size_t)(__attribute__((address_space(3))) void*)p),
                   "v"(__builtin_bit_cast(uint64_t, make_uint2(lo, hi)))
                 : "memory");
}

// TrReads for two row tiles (addresses a0, a1) in one block, so the read
// latency is exposed once per step.
template <int NKS> struct TrReads2;
template <> struct TrReads2<8> {
    static __device__ __forceinline__ void run(unsigned a0, unsigned a1, v4s (&lo0)[8], v4s (&hi0)[8],
                                               v4s (&lo1)[8], v4s (&hi1)[8])
    {
        asm volatile(
            "s_waitcnt expcnt(0)\n\t"
            "ds_read_b64_tr_b16 %0, %32\n\t"
            "ds_read_b64_tr_b16 %1, %32 offset:256\n\t"
            "ds_read_b64_tr_b16 %2, %32 offset:512\n\t"
            "ds_read_b64_tr_b16 %3, %32 offset:768\n\t"
            "ds_read_b64_tr_b16 %4, %32 offset:1024\n\t"
            "ds_read_b64_tr_b16 %5, %32 offset:1280\n\t"
            "ds_read_b64_tr_b16 %6, %32 offset:1536\n\t"
            "ds_read_b64_tr_b16 %7, %32 offset:1792\n\t"
            "ds_read_b64_tr_b16 %8, %32 offset:2048\n\t"
            "ds_read_b64_tr_b16 %9, %32 offset:2304\n\t"
            "ds_read_b64_tr_b16 %10, %32 offset:2560\n\t"
            "ds_read_b64_tr_b16 %11, %32 offset:2816\n\t"
            "ds_read_b64_tr_b16 %12, %32 offset:3072\n\t"
            "ds_read_b64_tr_b16 %13, %32 offset:3328\n\t"
            "ds_read_b64_tr_b16 %14, %32 offset:3584\n\t"
            "ds_read_b64_tr_b16 %15, %32 offset:3840\n\t"
            "ds_read_b64_tr_b16 %16, %33\n\t"
            "ds_read_b64_tr_b16 %17, %33 offset:256\n\t"
            "ds_read_b64_tr_b16 %18, %33 offset:512\n\t"
            "ds_read_b64_tr_b16 %19, %33 offset:768\n\t"
            "ds_read_b64_tr_b16 %20, %33 offset:1024\n\t"
            "ds_read_b64_tr_b16 %21, %33 offset:1280\n\t"
            "ds_read_b64_tr_b16 %22, %33 offset:1536\n\t"
            "ds_read_b64_tr_b16 %23, %33 offset:1792\n\t"
            "ds_read_b64_tr_b16 %24, %33 offset:2048\n\t"
            "ds_read_b64_tr_b16 %25, %33 offset:2304\n\t"
            "ds_read_b64_tr_b16 %26, %33 offset:2560\n\t"
            "ds_read_b64_tr_b16 %27, %33 offset:2816\n\t"
            "ds_read_b64_tr_b16 %28, %33 offset:3072\n\t"
            "ds_read_b64_tr_b16 %29, %33 offset:3328\n\t"
            "ds_read_b64_tr_b16 %30, %33 offset:3584\n\t"
            "ds_read_b64_tr_b16 %31, %33 offset:3840\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(lo0[0]), "=&v"(hi0[0]), "=&v"(lo0[1]), "=&v"(hi0[1]), "=&v"(lo0[2]), "=&v"(hi0[2]), "=&v"(lo0[3]), "=&v"(hi0[3]), "=&v"(lo0[4]), "=&v"(hi0[4]), "=&v"(lo0[5]), "=&v"(hi0[5]), "=&v"(lo0[6]), "=&v"(hi0[6]), "=&v"(lo0[7]), "=&v"(hi0[7]), "=&v"(lo1[0]), "=&v"(hi1[0]), "=&v"(lo1[1]), "=&v"(hi1[1]), "=&v"(lo1[2]), "=&v"(hi1[2]), "=&v"(lo1[3]), "=&v"(hi1[3]), "=&v"(lo1[4]), "=&v"(hi1[4]), "=&v"(lo1[5]), "=&v"(hi1[5]), "=&v"(lo1[6]), "=&v"(hi1[6]), "=&v"(lo1[7]), "=&v"(hi1[7])
            : "v"(a0), "v"(a1)
            : "memory");
    }
};
template <> struct TrReads2<4> {
    static __device__ __forceinline__ void run(unsigned a0, unsigned a1, v4s (&lo0)[4], v4s (&hi0)[4],
                                               v4s (&lo1)[4], v4s (&hi1)[4])
    {
        asm volatile(
            "s_waitcnt expcnt(0)\n\t"
            "ds_read_b64_tr_b16 %0, %16\n\t"
            "ds_read_b64_tr_b16 %1, %16 offset:256\n\t"
            "ds_read_b64_tr_b16 %2, %16 offset:512\n\t"
            "ds_read_b64_tr_b16 %3, %16 offset:768\n\t"
            "ds_read_b64_tr_b16 %4, %16 offset:1024\n\t"
            "ds_read_b64_tr_b16 %5, %16 offset:1280\n\t"
            "ds_read_b64_tr_b16 %6, %16 offset:1536\n\t"
            "ds_read_b64_tr_b16 %7, %16 offset:1792\n\t"
            "ds_read_b64_tr_b16 %8, %17\n\t"
            "ds_read_b64_tr_b16 %9, %17 offset:256\n\t"
            "ds_read_b64_tr_b16 %10, %17 offset:512\n\t"
            "ds_read_b64_tr_b16 %11, %17 offset:768\n\t"
            "ds_read_b64_tr_b16 %12, %17 offset:1024\n\t"
            "ds_read_b64_tr_b16 %13, %17 offset:1280\n\t"
            "ds_read_b64_tr_b16 %14, %17 offset:1536\n\t"
            "ds_read_b64_tr_b16 %15, %17 offset:1792\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(lo0[0]), "=&v"(hi0[0]), "=&v"(lo0[1]), "=&v"(hi0[1]), "=&v"(lo0[2]), "=&v"(hi0[2]), "=&v"(lo0[3]), "=&v"(hi0[3]), "=&v"(lo1[0]), "=&v"(hi1[0]), "=&v"(lo1[1]), "=&v"(hi1[1]), "=&v"(lo1[2]), "=&v"(hi1[2]), "=&v"(lo1[3]), "=&v"(hi1[3])
            : "v"(a0), "v"(a1)
            : "memory");
    }
};

// s_waitcnt immediate for vmcnt(n), n < 64 (expcnt and lgkmcnt not waited)
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0f70; }

template <int DT, int GP, bool SMOOTH, bool YOUT, int NSTG>
__global__ __launch_bounds__(512) void rq_colmajor_kernel(
    const uint16_t* __restrict__ x, int64_t M, int64_t K, int64_t sk,
    const float* __restrict__ rot, const uint16_t* __restrict__ smooth,
    int8_t* __restrict__ codes, float* __restrict__ scales, uint16_t* __restrict__ yout)
{
    constexpr int TROW = CM_ROWS * 2;                 // bytes per k-row of a tile
    constexpr int TILE = GP * TROW;                   // bytes per group tile
    constexpr int NLD = TILE / 1024 / 4;              // 1 KB loads per loader wave per tile
    constexpr int NJT = GP / 16;                      // 16-wide output column tiles
    constexpr int JPW = NJT >= 8 ? NJT / 8 : 1;       // column tiles per wave
    constexpr int MPW = NJT >= 8 ? 2 : 1;             // 16-row tiles per wave
    constexpr int NKS = GP / 32;                      // 32-deep MFMA steps
    constexpr int LPL = GP / 4;                       // k per lane group per group-row
    constexpr int CCH = CM_ROWS * GP / 16;            // 16-byte code chunks per group
    constexpr int YCH = YOUT ? CM_ROWS * GP * 2 / 16 : 0;
    constexpr int NCS = (CCH + 255) / 256;            // code stores per storer thread
    constexpr int NYS = (YCH + 255) / 256;            // rotated-value stores per storer thread
    static_assert(NJT >= 8 || NJT == 4, "group width 64, 128 or 256");
    static_assert(NLD >= 1 && NLD <= 4, "one to four loads per loader wave");

    __shared__ __align__(16) uint8_t stg[NSTG][TILE];
    static_assert(NSTG >= 3 && NLD * (NSTG - 2) < 64, "ring depth");
    __shared__ __align__(16) int8_t ctile[2][CM_ROWS * GP];
    __shared__ __align__(16) uint16_t ytile[2][YOUT ? CM_ROWS * GP : 8];
    __shared__ uint32_t rowmax[CM_ROWS];
    __shared__ RowQuant rowq[CM_ROWS];

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int n = lane & 15, q = lane >> 4;
    const int jt0 = NJT >= 8 ? wave * JPW : (wave & 3);
    const int mt0 = NJT >= 8 ? 0 : (wave >> 2);
    const bool loader = wave < 4;
    const int st_tid = tid - 256;                     // storer thread index (waves 4-7)
    // workgroups are dealt round-robin over the 8 XCDs; give each XCD a
    // contiguous range of row blocks so that the two halves of every
    // 128-byte line (two neighbouring blocks) meet in the same L2
    const int nb = gridDim.x, bid = blockIdx.x;
    const int q8 = nb >> 3, r8 = nb & 7, xcd = bid & 7;
    const int rb = xcd * q8 + min(xcd, r8) + (bid >> 3);
    const int64_t m0 = (int64_t)rb * CM_ROWS;
    const int G = (int)(K / GP);

    if (tid < CM_ROWS) rowmax[tid] = 0u;

    // rotation slice, rounded to T: lane (n, q), step ks holds
    // R[q * LPL + 8 ks + e][column jt * 16 + n]
    v8s bfr[JPW][NKS];
#pragma unroll
    for (int jj = 0; jj < JPW; ++jj)
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int kk = q * LPL + ks * 8 + e;
                bfr[jj][ks][e] = (short)f32_to_h<DT>(rot[kk * GP + (jt0 + jj) * 16 + n]);
            }

    // tile loads: loader wave w issues loads w*NLD .. w*NLD+NLD-1; load i fills
    // k-rows 16 i .. 16 i + 15; lane l takes k-row 16 i + (l >> 2), rows
    // 8 (l & 3) .. +7 of the block
    const uint64_t xelems = (uint64_t)(K - 1) * sk + M;
    auto issue = [&](int stage, int b) {
        const uint64_t base = (uint64_t)b * GP * sk + m0;
        const __amdgpu_buffer_rsrc_t r = rq_rsrc(x + base, (xelems - base) * 2);
#pragma unroll
        for (int u = 0; u < NLD; ++u) {
            const int i = wave * NLD + u;
            // 16-byte chunk (lane & 3) of k-row 16 i + (lane >> 2) holds
            // logical chunk (lane & 3) ^ cm_swz(k-row)
            const int c = (lane & 3) ^ (2 * (((16 * i) / LPL) & 1));
            const int vo = (int)(((lane >> 2) * sk + 8 * c) * 2);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                r, (__attribute__((address_space(3))) void*)(&stg[stage][i * 1024]), 16,
                vo + (int)(16 * i * sk * 2), 0, 0, 0);
        }
    };

    const __amdgpu_buffer_rsrc_t rc = rq_rsrc(codes, (uint64_t)M * K);
    const __amdgpu_buffer_rsrc_t ry = rq_rsrc(yout, YOUT ? (uint64_t)M * K * 2 : 0);
    uint32_t rmax[MPW];
#pragma unroll
    for (int mi = 0; mi < MPW; ++mi) rmax[mi] = 0u;

    // storer waves: codes (and rotated values) of step st from the LDS
    // staging tiles to global memory, 16 bytes per store
    auto store_group = [&](int st) {
        const int bs = 2 * G - 1 - st;
        const int8_t* ct = ctile[st & 1];
#pragma unroll
        for (int u = 0; u < NCS; ++u) {
            const int c = st_tid + 256 * u;
            const int row = c / (GP / 16), ch = c % (GP / 16);
            const v4i v = lds_read16(ct + (c < CCH ? row * GP + ch * 16 : 0));
            const int off = c < CCH ? (int)((m0 + row) * K + (int64_t)bs * GP + ch * 16) : CM_OOB;
            __builtin_amdgcn_raw_buffer_store_b128(v, rc, off, 0, 2);  // non-temporal
        }
        if constexpr (YOUT) {
            const uint16_t* yt = ytile[st & 1];
#pragma unroll
            for (int u = 0; u < NYS; ++u) {
                const int c = st_tid + 256 * u;
                const int row = c / (GP / 8), ch = c % (GP / 8);
                const v4i v = lds_read16(yt + (c < YCH ? row * GP + ch * 8 : 0));
                const int off = c < YCH ? (int)(((m0 + row) * K + (int64_t)bs * GP + ch * 8) * 2) : CM_OOB;
                __builtin_amdgcn_raw_buffer_store_b128(v, ry, off, 0, 2);
            }
        }
    };

    RowQuant rq[MPW];  // quantizer of this lane's row in each row tile (pass 2)
    // group of step s: pass 1 walks the groups forward, pass 2 backward, so
    // that the second pass starts on the tiles the first one read last
    // (still in cache)
    auto step_group = [G](int st) { return st < G ? st : 2 * G - 1 - st; };
    const int nsteps = 2 * G;
    if (loader)
        for (int i = 0; i < NSTG - 1 && i < nsteps; ++i) issue(i, step_group(i));
    int cur = 0;  // ring slot of step s
    for (int s = 0; s < nsteps; ++s) {
        const int b = step_group(s);
        const bool pass2 = s >= G;
        // a loader waits for its part of this step's tile; the next NSTG - 2
        // tiles' loads stay in flight (near the end, none)
        if (loader) {
            if (s + NSTG - 2 < nsteps) __builtin_amdgcn_s_waitcnt(vmcnt_imm(NLD * (NSTG - 2)));
            else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        }
        lds_barrier();  // also publishes the previous step's code tile
        const int nxt = cur == 0 ? NSTG - 1 : cur - 1;  // slot of step s - 1, free now
        if (loader && s + NSTG - 1 < nsteps) issue(nxt, step_group(s + NSTG - 1));
        if (!loader && s > G) store_group(s - 1);
        uint8_t* tile = stg[cur];
        cur = cur == NSTG - 1 ? 0 : cur + 1;
        if constexpr (SMOOTH) {
            // x' = T(x / smooth[k]) in place: thread t handles k-rows t / 4,
            // t / 4 + 128, ..., 16 bytes each
            for (int kr = tid >> 2; kr < GP; kr += 128) {
                const float sv = h_to_f32<DT>(smooth[(int64_t)b * GP + kr]);
                v8s* p = (v8s*)(tile + kr * TROW + (tid & 3) * 16);
                v8s v = *p;
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    v[e] = (short)f32_to_h<DT>(h_to_f32<DT>((uint16_t)v[e]) / sv);
                *p = v;
            }
            lds_barrier();
        }
        v4f acc[MPW][JPW];
#pragma unroll
        for (int mi = 0; mi < MPW; ++mi)
#pragma unroll
            for (int jj = 0; jj < JPW; ++jj) acc[mi][jj] = (v4f){0.f, 0.f, 0.f, 0.f};
        // all x fragments of the step first (LDS returns them in order, so the
        // MFMAs only wait for the ones they use)
        v4s afl[MPW][NKS], afh[MPW][NKS];
        {
            // lane L of group q reads k-rows q * LPL + 8 ks + (L >> 2) (+4),
            // rows 16 mt + 4 (L & 3) .. +3
            static_assert(8 * TROW == 512 && 4 * TROW == 256, "read offsets in TrReads");
            unsigned ad[MPW];
#pragma unroll
            for (int mi = 0; mi < MPW; ++mi) {
                const int kr = q * LPL + (n >> 2);
                const int lc = 2 * (mt0 + mi) + ((n & 3) >> 1);  // logical 16-byte chunk
                const uint8_t* p = tile + kr * TROW + (lc ^ (2 * (q & 1))) * 16 + (n & 1) * 8;
                ad[mi] = (unsigned)(size_t)(__attribute__((address_space(3))) const uint8_t*)p;
            }
            if constexpr (MPW == 2)
                TrReads2<NKS>::run(ad[0], ad[MPW - 1], afl[0], afh[0], afl[MPW - 1], afh[MPW - 1]);
            else
                TrReads<NKS>::run(ad[0], afl[0], afh[0]);
        }
        // y^T = R^T . x^T: lane (n, q) of tile (mt, jt) receives
        // y[16 mt + n][16 jt + 4 q + r], r = 0..3 (four consecutive columns of
        // one row); same products and k order as x . R
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
            for (int mi = 0; mi < MPW; ++mi) {
                const v4s lo = afl[mi][ks], hi = afh[mi][ks];
                const v8s af = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
                for (int jj = 0; jj < JPW; ++jj) {
                    if constexpr (DT == BF16)
                        acc[mi][jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(v8bf, bfr[jj][ks]), __builtin_bit_cast(v8bf, af), acc[mi][jj], 0, 0, 0);
                    else
                        acc[mi][jj] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                            __builtin_bit_cast(v8h, bfr[jj][ks]), __builtin_bit_cast(v8h, af), acc[mi][jj], 0, 0, 0);
                }
            }
        }
        if (!pass2) {
            // the row absmax of the unrounded values as an integer max of the
            // sign-cleared fp32 patterns (a NaN pattern exceeds every other);
            // rounding to T is monotone, so rounding the maximum once per row
            // gives the maximum of the rounded values
#pragma unroll
            for (int mi = 0; mi < MPW; ++mi)
#pragma unroll
                for (int jj = 0; jj < JPW; ++jj) {
                    const v4f a = acc[mi][jj];
                    rmax[mi] = max(rmax[mi], max(__float_as_uint(a[0]) & 0x7fffffffu, __float_as_uint(a[1]) & 0x7fffffffu));
                    rmax[mi] = max(rmax[mi], max(__float_as_uint(a[2]) & 0x7fffffffu, __float_as_uint(a[3]) & 0x7fffffffu));
                }
            if (s == G - 1) {
                // row absmax across the four lane groups, then across waves
#pragma unroll
                for (int mi = 0; mi < MPW; ++mi) {
                    uint32_t v = rmax[mi];
                    v = max(v, (uint32_t)__shfl_xor((int)v, 16));
                    v = max(v, (uint32_t)__shfl_xor((int)v, 32));
                    if (q == 0) atomicMax(&rowmax[(mt0 + mi) * 16 + n], v);
                }
                lds_barrier();
                if (tid < CM_ROWS) {
                    // T(max |y|) of the row, then its quantizer parameters
                    const RowQuant p = row_quant_thread<DT>(f32_to_h<DT>(__uint_as_float(rowmax[tid])));
                    rowq[tid] = p;
                    if (m0 + tid < M) scales[m0 + tid] = p.s;
                }
                lds_barrier();
#pragma unroll
                for (int mi = 0; mi < MPW; ++mi) rq[mi] = rowq[(mt0 + mi) * 16 + n];
            }
            continue;
        }
        // pass 2: quantize four codes of one row at a time into this step's
        // code tile (the storers write out the previous step's tile
        // meanwhile): the two bracketing roundings and the row's tie mask.
        // A non-finite scale, or a row outside the scale table's range, sends
        // the wave to the exact division.
        int8_t* ct = ctile[s & 1];
        float yv[MPW][JPW][4];
        bool near = false;
#pragma unroll
        for (int mi = 0; mi < MPW; ++mi) {
            const int row = (mt0 + mi) * 16 + n;
            near |= !(fabsf(rq[mi].s) < 3.0e38f) || rq[mi].exact;
#pragma unroll
            for (int jj = 0; jj < JPW; ++jj) {
                uint16_t yb[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    yb[r] = f32_to_h<DT>(acc[mi][jj][r]);
                    yv[mi][jj][r] = h_to_f32<DT>(yb[r]);
                }
                const int col = (jt0 + jj) * 16 + 4 * q;
                lds_write4(ct + row * GP + col, quant4_bracket(yv[mi][jj], rq[mi]));
                if constexpr (YOUT)
                    lds_write8(ytile[s & 1] + row * GP + col, (uint32_t)yb[0] | ((uint32_t)yb[1] << 16),
                               (uint32_t)yb[2] | ((uint32_t)yb[3] << 16));
            }
        }
        if (__any(near)) {
#pragma unroll
            for (int mi = 0; mi < MPW; ++mi)
#pragma unroll
                for (int jj = 0; jj < JPW; ++jj)
                    lds_write4(ct + ((mt0 + mi) * 16 + n) * GP + (jt0 + jj) * 16 + 4 * q,
                               quant4_exact(yv[mi][jj], rq[mi].s));
        }
    }
    // the last step's codes
    lds_barrier();
    if (!loader) store_group(nsteps - 1);
}

// -------------------------------------------------------------------------
// Register-resident path for 16-bit activations, group width 32 or 64,
// contiguous rows.  Persistent workgroups (R loaded once per workgroup) walk
// blocks of rows; a block's group-rows are dealt to the four waves as 16-row
// MFMA tiles.  The MFMA is issued as R^T . x^T so that each lane receives four
// consecutive outputs of one group-row: codes then leave as 4-byte stores
// straight from registers, and rotated values never touch LDS.  Only the
// per-row absmax crosses waves (an LDS integer max).
//   TW = tiles per wave per block (1, 2 or 4).
// -------------------------------------------------------------------------
template <int DT, int GP, bool ROT, bool SMOOTH, int TW>
__global__ __launch_bounds__(256) void rq_reg_kernel(
    const uint16_t* __restrict__ x, int64_t M, int64_t K, int64_t sm,
    const float* __restrict__ rot, int g, const uint16_t* __restrict__ smooth,
    int8_t* __restrict__ codes, float* __restrict__ scales, uint16_t* __restrict__ yout,
    int rows_per_blk)
{
    constexpr int NKS = GP / 32;     // 32-deep k-steps
    constexpr int CT = GP / 16;      // 16-wide output column tiles
    constexpr int LPL = GP / 4;      // elements per lane per group-row
    constexpr int NV = ROT ? NKS : CT / 2;  // 16-byte vectors per lane per tile
    __shared__ uint32_t rowmax[3][16];

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int j = lane & 15, q = lane >> 4;
    const int gpr = (int)(K / GP);
    const int64_t nblk = (M + rows_per_blk - 1) / rows_per_blk;

    // R^T fragments (A operand): lane (j, q) holds R[kk][ct*16 + j] for its k-slots
    v8s rfr[ROT ? CT : 1][ROT ? NKS : 1];
    if constexpr (ROT) {
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            const int c = ct * 16 + j;
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int kk = q * LPL + ks * 8 + e;
                    float rv;
                    if (GP == 32 && g == 16)
                        rv = ((kk >> 4) == (c >> 4)) ? rot[(kk & 15) * 16 + (c & 15)] : 0.0f;
                    else
                        rv = rot[kk * GP + c];
                    rfr[ct][ks][e] = (short)f32_to_h<DT>(rv);
                }
        }
    }
    if (tid < 48) rowmax[tid >> 4][tid & 15] = 0u;
    __syncthreads();

    // ---- loads for one block.  With a rotation, lane (j, q) of tile t reads
    // group-row t*16 + j, slice q (the MFMA B layout).  Without one, it reads
    // the entries ct*16 + 4q .. +3 of that group-row that it will quantize.
    auto load_blk = [&](int64_t blk, v8s (*xf)[NV]) {
        const int64_t m0 = blk * rows_per_blk;
        const int nrows = (int)min((int64_t)rows_per_blk, M - m0);
        const int ngr = nrows * gpr;
#pragma unroll
        for (int u = 0; u < TW; ++u) {
            const int gr = (wave * TW + u) * 16 + j;
            if (blk < nblk && gr < ngr) {
                const int rl = gr / gpr, b = gr - rl * gpr;
                const uint16_t* rowp = x + (m0 + rl) * sm + (int64_t)b * GP;
                if constexpr (ROT) {
                    const v4i* src = (const v4i*)(rowp + q * LPL);
#pragma unroll
                    for (int ks = 0; ks < NKS; ++ks)
                        xf[u][ks] = __builtin_bit_cast(v8s, __builtin_nontemporal_load(src + ks));
                } else {
#pragma unroll
                    for (int c2 = 0; c2 < CT / 2; ++c2) {
                        const uint2 lo = *(const uint2*)(rowp + (2 * c2) * 16 + 4 * q);
                        const uint2 hi = *(const uint2*)(rowp + (2 * c2 + 1) * 16 + 4 * q);
                        xf[u][c2] = __builtin_bit_cast(v8s, make_uint4(lo.x, lo.y, hi.x, hi.y));
                    }
                }
            } else {
#pragma unroll
                for (int v = 0; v < NV; ++v) xf[u][v] = (v8s){0, 0, 0, 0, 0, 0, 0, 0};
            }
        }
    };

    auto process_blk = [&](int64_t blk, v8s (*xf)[NV], int buf) {
        const int64_t m0 = blk * rows_per_blk;
        const int nrows = (int)min((int64_t)rows_per_blk, M - m0);
        const int ngr = nrows * gpr;
        int grw[TW];
        uint32_t yv[TW][CT][2];   // 4 values of T per (tile, ct), packed in pairs
        uint32_t tmax[TW];
#pragma unroll
        for (int u = 0; u < TW; ++u) {
            const int gr = (wave * TW + u) * 16 + j;
            grw[u] = gr;
            if constexpr (SMOOTH) {
                if (gr < ngr) {
                    const int rl = gr / gpr, b = gr - rl * gpr;
                    const uint16_t* sp = smooth + (int64_t)b * GP;
#pragma unroll
                    for (int v = 0; v < NV; ++v)
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const int el = ROT ? q * LPL + v * 8 + e
                                               : (2 * v + (e >> 2)) * 16 + 4 * q + (e & 3);
                            xf[u][v][e] = (short)f32_to_h<DT>(h_to_f32<DT>((uint16_t)xf[u][v][e]) /
                                                              h_to_f32<DT>(sp[el]));
                        }
                    (void)rl;
                }
            }
            tmax[u] = 0u;
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                uint16_t h[4];
                if constexpr (ROT) {
                    v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < NKS; ++ks) {
                        if constexpr (DT == BF16)
                            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                __builtin_bit_cast(v8bf, rfr[ct][ks]), __builtin_bit_cast(v8bf, xf[u][ks]),
                                acc, 0, 0, 0);
                        else
                            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                                __builtin_bit_cast(v8h, rfr[ct][ks]), __builtin_bit_cast(v8h, xf[u][ks]),
                                acc, 0, 0, 0);
                    }
#pragma unroll
                    for (int r = 0; r < 4; ++r) h[r] = f32_to_h<DT>(acc[r]);
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r) h[r] = (uint16_t)xf[u][ct >> 1][(ct & 1) * 4 + r];
                }
                yv[u][ct][0] = (uint32_t)h[0] | ((uint32_t)h[1] << 16);
                yv[u][ct][1] = (uint32_t)h[2] | ((uint32_t)h[3] << 16);
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    tmax[u] = max(tmax[u], __float_as_uint(h_to_f32<DT>(h[r])) & 0x7fffffffu);
            }
            if (gr >= ngr) tmax[u] = 0u;
        }

        // per-row absmax over the rows this wave's tiles touch
#pragma unroll
        for (int u = 0; u < TW; ++u) {
            const int t = wave * TW + u;
            const int g_lo = t * 16, g_hi = min(t * 16 + 15, ngr - 1);
            if (g_lo > g_hi) continue;
            const int r_lo = g_lo / gpr, r_hi = g_hi / gpr;
            const int my_r = grw[u] / gpr;
            for (int r = r_lo; r <= r_hi; ++r) {
                uint32_t v = (my_r == r) ? tmax[u] : 0u;
                for (int o = 32; o >= 1; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o));
                if (lane == 0) atomicMax(&rowmax[buf][r], v);
            }
        }
        // block i accumulates into buffer i % 3 and, before its barrier, clears
        // buffer (i + 1) % 3: every wave finished reading that buffer (block
        // i - 2) before the previous barrier, and nobody writes it before this one.
        if (tid < 16) rowmax[buf == 2 ? 0 : buf + 1][tid] = 0u;
        __syncthreads();

        // quantize from registers: 4 consecutive codes per (tile, ct); the
        // division is redone only for tiles where some lane sits near a tie
#pragma unroll
        for (int u = 0; u < TW; ++u) {
            const int gr = grw[u];
            const bool live = gr < ngr;
            const int rl = live ? gr / gpr : 0;
            const int b = live ? gr - rl * gpr : 0;
            const float s = row_scale(rowmax[buf][rl]);
            const float ri = 1.0f / s;
            uint32_t pk[CT];
            bool near = false;
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                float yy[4];
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    yy[r] = h_to_f32<DT>((uint16_t)(yv[u][ct][r >> 1] >> (16 * (r & 1))));
                pk[ct] = quant4_fast(yy, ri, near);
            }
            if (__any(near && live)) {
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) {
                    float yy[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        yy[r] = h_to_f32<DT>((uint16_t)(yv[u][ct][r >> 1] >> (16 * (r & 1))));
                    pk[ct] = quant4_exact(yy, s);
                }
            }
            // Lane (j, q) holds codes ct*16 + 4q .. +3 of group-row j for each
            // ct; the four lanes of a group-row exchange dwords (4 rounds of
            // ds_bpermute) so that each ends up with 16 consecutive codes and
            // a wave stores whole 64-byte group-rows.
            if constexpr (CT == 4) {
                uint32_t o4[4];
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const int send = (q - t) & 3;
                    uint32_t v = pk[0];
                    v = send == 1 ? pk[1] : v;
                    v = send == 2 ? pk[2] : v;
                    v = send == 3 ? pk[3] : v;
                    const uint32_t got = (uint32_t)__shfl((int)v, j + 16 * ((q + t) & 3));
                    o4[(q + t) & 3] = got;   // dword from the lane with that q
                }
                // o4[d] now holds codes q*16 + 4d .. +3 (d = source lane's q)
                uint32_t w0 = o4[0], w1 = o4[1], w2 = o4[2], w3 = o4[3];
                if (live) {
                    int8_t* crow = codes + (m0 + rl) * K + (int64_t)b * GP;
                    st_stream16(crow + q * 16, w0, w1, w2, w3);
                }
            } else {
                if (live) {
                    int8_t* crow = codes + (m0 + rl) * K + (int64_t)b * GP;
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct) *(uint32_t*)(crow + ct * 16 + 4 * q) = pk[ct];
                }
            }
            if (live && yout) {
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) {
                    st_stream8(yout + (m0 + rl) * K + (int64_t)b * GP + ct * 16 + 4 * q, yv[u][ct][0], yv[u][ct][1]);
                }
            }
        }
        if (tid < nrows) scales[m0 + tid] = row_scale(rowmax[buf][tid]);
    };

    // two register sets alternate (the loop covers two blocks), so the next
    // block's loads are in flight while the current one is processed
    v8s xa[TW][NV], xb[TW][NV];
    const int64_t stride = gridDim.x;
    int64_t blk = blockIdx.x;
    int buf = 0;
    load_blk(blk, xa);
    while (blk < nblk) {
        load_blk(blk + stride, xb);
        process_blk(blk, xa, buf);
        buf = buf == 2 ? 0 : buf + 1;
        blk += stride;
        if (blk >= nblk) break;
        load_blk(blk + stride, xa);
        process_blk(blk, xb, buf);
        buf = buf == 2 ? 0 : buf + 1;
        blk += stride;
    }
}

// -------------------------------------------------------------------------
// Wave-per-row-block path (16-bit activations, g <= 64, K/g <= 64): every
// wave owns RPB whole rows (RPB * K/g <= 16 * TW group-rows, one tile of 16
// group-rows per unit of TW), so the row absmax is a wave shuffle and waves
// never wait for each other: no LDS, no barrier.  Loads for the wave's next
// row-block are in flight while the current one is rotated and quantized.
// -------------------------------------------------------------------------
template <int DT, int GP, bool ROT, bool SMOOTH, int TW>
__global__ __launch_bounds__(256, TW >= 4 ? 2 : 3) void rq_wave_kernel(
    const uint16_t* __restrict__ x, int64_t M, int64_t K, int64_t sm,
    const float* __restrict__ rot, int g, const uint16_t* __restrict__ smooth,
    int8_t* __restrict__ codes, float* __restrict__ scales, uint16_t* __restrict__ yout, int rpb)
{
    constexpr int NKS = GP / 32;
    constexpr int CT = GP / 16;
    constexpr int LPL = GP / 4;
    constexpr int NV = ROT ? NKS : CT / 2;

    const int lane = threadIdx.x & 63;
    const int j = lane & 15, q = lane >> 4;
    const int gpr = (int)(K / GP);
    const int64_t nblk = (M + rpb - 1) / rpb;
    const int64_t wid = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x >> 6);

    v8s rfr[ROT ? CT : 1][ROT ? NKS : 1];
    if constexpr (ROT) {
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            const int c = ct * 16 + j;
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int kk = q * LPL + ks * 8 + e;
                    float rv;
                    if (GP == 32 && g == 16)
                        rv = ((kk >> 4) == (c >> 4)) ? rot[(kk & 15) * 16 + (c & 15)] : 0.0f;
                    else
                        rv = rot[kk * GP + c];
                    rfr[ct][ks][e] = (short)f32_to_h<DT>(rv);
                }
        }
    }

    // A lane's place inside a row-block never changes: precompute, per tile,
    // its row within the block and 32-bit offsets into x and the codes.
    int t_row[TW], t_xoff[TW], t_coff[TW], t_b[TW];
#pragma unroll
    for (int u = 0; u < TW; ++u) {
        const int gr = u * 16 + j;
        const int rl = gr / gpr, b = gr - rl * gpr;
        t_row[u] = rl;
        t_b[u] = b;
        t_xoff[u] = (int)(rl * sm + b * GP);
        t_coff[u] = (int)(rl * K + b * GP);
    }

    auto load_blk = [&](int64_t blk, v8s (*xf)[NV]) {
        const int64_t m0 = blk * rpb;
        const int nrows = blk < nblk ? (int)min((int64_t)rpb, M - m0) : 0;
        const uint16_t* xb = x + m0 * sm;
#pragma unroll
        for (int u = 0; u < TW; ++u) {
            if (t_row[u] < nrows) {
                const uint16_t* rowp = xb + t_xoff[u];
                if constexpr (ROT) {
                    const v4i* src = (const v4i*)(rowp + q * LPL);
#pragma unroll
                    for (int ks = 0; ks < NKS; ++ks)
                        xf[u][ks] = __builtin_bit_cast(v8s, __builtin_nontemporal_load(src + ks));
                } else {
#pragma unroll
                    for (int c2 = 0; c2 < CT / 2; ++c2) {
                        const uint2 lo = *(const uint2*)(rowp + (2 * c2) * 16 + 4 * q);
                        const uint2 hi = *(const uint2*)(rowp + (2 * c2 + 1) * 16 + 4 * q);
                        xf[u][c2] = __builtin_bit_cast(v8s, make_uint4(lo.x, lo.y, hi.x, hi.y));
                    }
                }
            } else {
#pragma unroll
                for (int v = 0; v < NV; ++v) xf[u][v] = (v8s){0, 0, 0, 0, 0, 0, 0, 0};
            }
        }
    };

    // fp32 MFMA results of one (tile, ct): 4 consecutive entries of group-row j
    auto rotate4f = [&](const v8s* xt, int ct, float (&f)[4]) {
        if constexpr (ROT) {
            v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                if constexpr (DT == BF16)
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(v8bf, rfr[ct][ks]), __builtin_bit_cast(v8bf, xt[ks]), acc, 0, 0, 0);
                else
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                        __builtin_bit_cast(v8h, rfr[ct][ks]), __builtin_bit_cast(v8h, xt[ks]), acc, 0, 0, 0);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) f[r] = acc[r];
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) f[r] = h_to_f32<DT>((uint16_t)xt[ct >> 1][(ct & 1) * 4 + r]);
        }
    };

    // Two passes over the registers: absmax, then quantize.  The rotation is
    // recomputed in the second pass (a few MFMAs per tile) instead of keeping
    // the rotated values live, which keeps enough waves resident.
    auto process_blk = [&](int64_t blk, v8s (*xf)[NV]) {
        const int64_t m0 = blk * rpb;
        const int nrows = (int)min((int64_t)rpb, M - m0);
        uint32_t tmax[TW];
#pragma unroll
        for (int u = 0; u < TW; ++u) {
            const bool live = t_row[u] < nrows;
            if constexpr (SMOOTH) {
                if (live) {
                    const uint16_t* sp = smooth + t_b[u] * GP;
#pragma unroll
                    for (int v = 0; v < NV; ++v)
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const int el = ROT ? q * LPL + v * 8 + e
                                               : (2 * v + (e >> 2)) * 16 + 4 * q + (e & 3);
                            xf[u][v][e] = (short)f32_to_h<DT>(h_to_f32<DT>((uint16_t)xf[u][v][e]) /
                                                              h_to_f32<DT>(sp[el]));
                        }
                }
            }
            // max |.| of the fp32 results, rounded to T once: rounding is
            // monotone, so this is the max of the rounded values (a NaN, whose
            // bits exceed every finite pattern, still dominates)
            uint32_t m = 0u;
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                float f[4];
                rotate4f(xf[u], ct, f);
                m = max(m, max(max(__float_as_uint(f[0]) & 0x7fffffffu, __float_as_uint(f[1]) & 0x7fffffffu),
                               max(__float_as_uint(f[2]) & 0x7fffffffu, __float_as_uint(f[3]) & 0x7fffffffu)));
            }
            m = __float_as_uint(h_to_f32<DT>(f32_to_h<DT>(__uint_as_float(m)))) & 0x7fffffffu;
            tmax[u] = live ? m : 0u;
            __builtin_amdgcn_sched_barrier(0);
        }
        // row scales: one wave-wide max per row of the block
        float srow[TW], rinv[TW];
#pragma unroll
        for (int u = 0; u < TW; ++u) { srow[u] = 1.0f; rinv[u] = 1.0f; }
        for (int r = 0; r < nrows; ++r) {
            uint32_t v = 0u;
#pragma unroll
            for (int u = 0; u < TW; ++u)
                if (t_row[u] == r) v = max(v, tmax[u]);
            v = wave_max_dpp(v);
            const float sv = row_scale(v);
            if (lane == 0) scales[m0 + r] = sv;
            const float ri = 1.0f / sv;
#pragma unroll
            for (int u = 0; u < TW; ++u)
                if (t_row[u] == r) { srow[u] = sv; rinv[u] = ri; }
        }
        int8_t* cb = codes + m0 * K;
        uint16_t* yb = yout ? yout + m0 * K : nullptr;
        // quantize; exact division only for tiles with a near-tie somewhere
#pragma unroll
        for (int u = 0; u < TW; ++u) {
            const bool live = t_row[u] < nrows;
            uint32_t pk[CT];
            uint32_t yv[CT][2];
            const float sv = srow[u], ri = rinv[u];
            if (__any(live && !(fabsf(sv) < 3.0e38f))) {
                // some row of this tile has a NaN or Inf scale: exact path
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) {
                    float f[4];
                    rotate4f(xf[u], ct, f);
                    uint16_t h[4];
                    float yy[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        h[r] = f32_to_h<DT>(f[r]);
                        yy[r] = h_to_f32<DT>(h[r]);
                    }
                    yv[ct][0] = (uint32_t)h[0] | ((uint32_t)h[1] << 16);
                    yv[ct][1] = (uint32_t)h[2] | ((uint32_t)h[3] << 16);
                    pk[ct] = quant4_exact(yy, sv);
                }
            } else {
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) {
                    float f[4];
                    rotate4f(xf[u], ct, f);
                    uint16_t h[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) h[r] = f32_to_h<DT>(f[r]);
                    yv[ct][0] = (uint32_t)h[0] | ((uint32_t)h[1] << 16);
                    yv[ct][1] = (uint32_t)h[2] | ((uint32_t)h[3] << 16);
                    float t[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float yy = h_to_f32<DT>(h[r]);
                        const float qv = yy * ri;
                        t[r] = __builtin_amdgcn_fmed3f(qv, -7.0f, 7.0f) + kRoundMagic;
                        const bool nr = fabsf(qv - (t[r] - kRoundMagic)) > 0.5f - 0x1p-17f;
                        // a value-slot where some lane sits near a tie is
                        // redone with the correctly rounded quotient
                        if (__any(nr)) t[r] = __builtin_amdgcn_fmed3f(yy / sv, -7.0f, 7.0f) + kRoundMagic;
                    }
                    pk[ct] = pack4_magic(t[0], t[1], t[2], t[3]);
                }
            }
            if constexpr (CT == 4) {
                uint32_t o4[4];
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const int send = (q - t) & 3;
                    uint32_t v = pk[0];
                    v = send == 1 ? pk[1] : v;
                    v = send == 2 ? pk[2] : v;
                    v = send == 3 ? pk[3] : v;
                    o4[(q + t) & 3] = (uint32_t)__shfl((int)v, j + 16 * ((q + t) & 3));
                }
                if (live) st_stream16(cb + t_coff[u] + q * 16, o4[0], o4[1], o4[2], o4[3]);
            } else {
                if (live) {
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct) *(uint32_t*)(cb + t_coff[u] + ct * 16 + 4 * q) = pk[ct];
                }
            }
            if (live && yb) {
#pragma unroll
                for (int ct = 0; ct < CT; ++ct)
                    st_stream8(yb + t_coff[u] + ct * 16 + 4 * q, yv[ct][0], yv[ct][1]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // The next row-block's loads are issued before the current one is
    // processed (the register copy afterwards finds them arrived).
    constexpr bool PF = true;
    v8s xa[TW][NV], xb[PF ? TW : 1][NV];
    load_blk(wid, xa);
    for (int64_t blk = wid; blk < nblk; blk += nwaves) {
        if constexpr (PF) load_blk(blk + nwaves, xb);
        process_blk(blk, xa);
        if constexpr (PF) {
#pragma unroll
            for (int u = 0; u < TW; ++u)
#pragma unroll
                for (int v = 0; v < NV; ++v) xa[u][v] = xb[u][v];
        } else {
            load_blk(blk + nwaves, xa);
        }
    }
}

// -------------------------------------------------------------------------
// g = 256 on contiguous rows (16-bit, K/256 <= 64 group-rows per row): the
// rotation's 128 MFMA A fragments (R^T, rounded to T; 128 KB) live in LDS for
// the life of a persistent workgroup.  Its eight waves take 2 * RPW rows at a
// time: wave (wr, wt) owns the wt-th 16-group-row tile of rows wr*RPW ..
// wr*RPW + RPW - 1, and every R fragment it reads from LDS feeds one MFMA per
// row (the LDS stream of R per row falls by RPW).  x is loaded (and smoothed)
// exactly once, the rotated values stay in registers (two per VGPR), and only
// the row absmax crosses waves, through LDS with one barrier per 2 * RPW
// rows.  The k-slots of each MFMA step are those of the column-major kernel
// (lane group q, step ks: k = 64 q + 8 ks + e), so the two give the same
// rotated bits.  The row absmax is a packed 16-bit max of the sign-cleared
// patterns (a NaN pattern exceeds every other).  INT4 codes come from the two
// bracketing multipliers and the row's tie mask (row_quant.hpp); the INT8
// mode keeps the product with a residual test and an exact division near
// half-integers.
// -------------------------------------------------------------------------
template <int DT, bool SMOOTH, int QMAX = 7, int RPW = 1>
__global__ __launch_bounds__(512) void rq_g256_kernel(
    const uint16_t* __restrict__ x, int64_t M, int64_t K, int64_t sm,
    const float* __restrict__ rot, const uint16_t* __restrict__ smooth,
    int8_t* __restrict__ codes, float* __restrict__ scales, uint16_t* __restrict__ yout)
{
    constexpr int GP = 256, CT = 16, NKS = 8, LPL = 64;
    constexpr int RB = 2 * RPW;                      // rows per workgroup step
    __shared__ __align__(16) v8s rs[CT * NKS][64];   // fragment (ct, ks), lane-major
    __shared__ uint32_t wmax[2][8][RPW];

    // (the wave index is uniform: row bases and buffer resources stay scalar)
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int wr = wave >> 2, wt = wave & 3;     // row pair, tile in the row
    const int q = lane >> 4;
    const int G = (int)(K / GP);
    const int ntile = (G + 15) >> 4;

    // R^T fragments: element (kk, c) of R goes to fragment (c / 16, (kk % 64) / 8),
    // lane (kk / 64) * 16 + c % 16, slot kk % 8 (coalesced reads of R)
#pragma unroll 4
    for (int idx = tid; idx < GP * GP; idx += 512) {
        const int kk = idx >> 8, c = idx & 255;
        uint16_t* dst = (uint16_t*)&rs[(c >> 4) * NKS + ((kk & 63) >> 3)][(kk >> 6) * 16 + (c & 15)];
        dst[kk & 7] = f32_to_h<DT>(rot[idx]);
    }
    __syncthreads();

    const int gr = wt * 16 + (lane & 15);        // this lane's group-row in the row
    const bool tlive = wt < ntile && gr < G;
    const int xo = gr * GP + q * LPL;            // element offset of the lane's slice

    // lanes past the row's last group-row take offsets past the row: their
    // loads read zeros and their stores are dropped by the range check
    const int xoff = tlive ? xo * 2 : (int)(2 * K);
    const int coff = tlive ? gr * GP + 4 * q : (int)K;
    auto load_row = [&](int64_t row, v8s (&xf)[NKS]) {
        const bool rl = row < M;
        // plain loads: each lane reads one whole 128-byte line in eight
        // 16-byte pieces, and only a cached line serves the later seven
        // (non-temporal loads sent every piece to L2)
        const __amdgpu_buffer_rsrc_t rx = rq_rsrc(x + (rl ? row : 0) * sm, rl ? (uint64_t)K * 2 : 0);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
            xf[ks] = __builtin_bit_cast(v8s, __builtin_amdgcn_raw_buffer_load_b128(rx, xoff + 16 * ks, 0, 0));
    };

    // the rows' x in registers; the next rows' loads go into them as soon as
    // the rotation has read them, so they are in flight during the absmax
    // exchange and the quantization
    v8s xa[RPW][NKS];
    int par = 0;
    const int64_t rstep = RB * (int64_t)gridDim.x;
#pragma unroll
    for (int i = 0; i < RPW; ++i) load_row(RB * (int64_t)blockIdx.x + wr * RPW + i, xa[i]);
    for (int64_t row0 = RB * (int64_t)blockIdx.x; row0 < M; row0 += rstep, par ^= 1) {
        const int64_t rowb = row0 + wr * RPW;
        if constexpr (SMOOTH) {
            if (tlive) {
                const v4i* sp = (const v4i*)(smooth + xo);
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    const v8s sv = __builtin_bit_cast(v8s, sp[ks]);
#pragma unroll
                    for (int i = 0; i < RPW; ++i)
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            xa[i][ks][e] = (short)f32_to_h<DT>(h_to_f32<DT>((uint16_t)xa[i][ks][e]) /
                                                               h_to_f32<DT>((uint16_t)sv[e]));
                }
            }
        }
        // rotate: lane (j, q) gets output columns 16 ct + 4 q .. + 3 of
        // group-row j of each of its rows, rounded to T and packed two per
        // register
        typedef unsigned short v2u16 __attribute__((ext_vector_type(2)));
        uint32_t yp[RPW][CT][2];
        v2u16 m2[RPW];
#pragma unroll
        for (int i = 0; i < RPW; ++i) m2[i] = (v2u16){0, 0};
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            v4f acc[RPW];
#pragma unroll
            for (int i = 0; i < RPW; ++i) acc[i] = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const v8s af = rs[ct * NKS + ks][lane];
#pragma unroll
                for (int i = 0; i < RPW; ++i) {
                    if constexpr (DT == BF16)
                        acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, af),
                                                                         __builtin_bit_cast(v8bf, xa[i][ks]), acc[i], 0, 0, 0);
                    else
                        acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, af),
                                                                        __builtin_bit_cast(v8h, xa[i][ks]), acc[i], 0, 0, 0);
                }
            }
#pragma unroll
            for (int i = 0; i < RPW; ++i) {
                yp[i][ct][0] = (uint32_t)f32_to_h<DT>(acc[i][0]) | ((uint32_t)f32_to_h<DT>(acc[i][1]) << 16);
                yp[i][ct][1] = (uint32_t)f32_to_h<DT>(acc[i][2]) | ((uint32_t)f32_to_h<DT>(acc[i][3]) << 16);
                m2[i] = __builtin_elementwise_max(m2[i], __builtin_bit_cast(v2u16, yp[i][ct][0] & 0x7fff7fffu));
                m2[i] = __builtin_elementwise_max(m2[i], __builtin_bit_cast(v2u16, yp[i][ct][1] & 0x7fff7fffu));
            }
            // one column tile at a time: only its fragments and results live
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int i = 0; i < RPW; ++i) load_row(rowb + i + rstep, xa[i]);
        // row absmax: a wave max, then the four waves' through LDS (two
        // buffers by step parity, so one barrier per step suffices)
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
            const uint32_t mi = wave_max_dpp(tlive ? max((uint32_t)m2[i][0], (uint32_t)m2[i][1]) : 0u);
            if (lane == 0) wmax[par][wave][i] = mi;
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
            const int64_t row = rowb + i;
            const uint32_t* wm = &wmax[par][4 * wr][i];
            const uint32_t a16 = max(max(wm[0], wm[RPW]), max(wm[2 * RPW], wm[3 * RPW]));
            const bool rl = row < M;
            const __amdgpu_buffer_rsrc_t rc = rq_rsrc(codes + (rl ? row : 0) * K, rl ? (uint64_t)K : 0);
            const __amdgpu_buffer_rsrc_t ry =
                rq_rsrc(yout + (rl && yout ? row : 0) * K, rl && yout ? (uint64_t)K * 2 : 0);
            if constexpr (QMAX == 7) {
                const RowQuant p = row_quant_thread<DT>(a16);
                if (wt == 0 && lane == 0 && rl) scales[row] = p.s;
                const bool fin = fabsf(p.s) < 3.0e38f;
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) {
                    float yy[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) yy[r] = h_to_f32<DT>((uint16_t)(yp[i][ct][r >> 1] >> (16 * (r & 1))));
                    const uint32_t pk = (!fin || p.exact) ? quant4_exact<7>(yy, p.s)
                                        : p.one ? quant4_one(yy, p) : quant4_bracket(yy, p);
                    __builtin_amdgcn_raw_buffer_store_b32(pk, rc, coff + ct * 16, 0, 0);
                    if (yout)
                        __builtin_amdgcn_raw_buffer_store_b64((v2u32){yp[i][ct][0], yp[i][ct][1]}, ry,
                                                              2 * (coff + ct * 16), 0, 0);
                }
            } else {
                const float sv = row_scale_q<QMAX>(__float_as_uint(h_to_f32<DT>((uint16_t)a16)));
                const float ri = 1.0f / sv;
                if (wt == 0 && lane == 0 && rl) scales[row] = sv;
                // exact division only where a quotient is near a tie or the
                // scale is not finite (|y * ri - fl(y / s)| <= 2 QMAX 2^-24,
                // so the band is 2^-13 in the INT8 mode)
                constexpr float kBand = 0x1p-13f;
                constexpr float kQ = (float)QMAX;
                const bool fin = fabsf(sv) < 3.0e38f;
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) {
                    float yy[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) yy[r] = h_to_f32<DT>((uint16_t)(yp[i][ct][r >> 1] >> (16 * (r & 1))));
                    uint32_t pk;
                    if (!fin) {
                        pk = quant4_exact<QMAX>(yy, sv);
                    } else {
                        float t[4];
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const float qv = yy[r] * ri;
                            t[r] = __builtin_amdgcn_fmed3f(qv, -kQ, kQ) + kRoundMagic;
                            const bool nr = fabsf(qv - (t[r] - kRoundMagic)) > 0.5f - kBand;
                            if (__any(nr)) t[r] = __builtin_amdgcn_fmed3f(yy[r] / sv, -kQ, kQ) + kRoundMagic;
                        }
                        pk = pack4_magic(t[0], t[1], t[2], t[3]);
                    }
                    __builtin_amdgcn_raw_buffer_store_b32(pk, rc, coff + ct * 16, 0, 0);
                    if (yout)
                        __builtin_amdgcn_raw_buffer_store_b64((v2u32){yp[i][ct][0], yp[i][ct][1]}, ry,
                                                              2 * (coff + ct * 16), 0, 0);
                }
            }
        }
    }
}

template <int DT, int QMAX = 7>
static hipError_t launch_g256_dt(const RQArgs& a, hipStream_t st)
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
    // one row per wave: with two (every R fragment read feeding two MFMAs)
    // the registers spilled and the kernel measured no faster
    constexpr int RPW = 1;
    const int64_t blocks = (a.M + 2 * RPW - 1) / (2 * RPW);
    const int64_t grid = blocks < n_cu ? blocks : n_cu;   // one workgroup per CU (128 KB of LDS)
    if (a.smooth)
        hipLaunchKernelGGL((rq_g256_kernel<DT, true, QMAX, RPW>), dim3((unsigned)grid), dim3(512), 0, st,
                           (const uint16_t*)a.x, a.M, a.K, a.sm, a.rot, (const uint16_t*)a.smooth, a.codes, a.scales,
                           (uint16_t*)a.yout);
    else
        hipLaunchKernelGGL((rq_g256_kernel<DT, false, QMAX, RPW>), dim3((unsigned)grid), dim3(512), 0, st,
                           (const uint16_t*)a.x, a.M, a.K, a.sm, a.rot, (const uint16_t*)a.smooth, a.codes, a.scales,
                           (uint16_t*)a.yout);
    return hipGetLastError();
}

// g = 256 with rotation, 16-bit, contiguous 16-byte aligned rows, at most 64
// group-rows per row, 4-byte aligned codes, 8-byte aligned rotated export,
// 16-byte aligned smoothing factors.
static bool g256_ok(const RQArgs& a)
{
    const bool sixteen = a.dtype == F16 || a.dtype == BF16;
    if (!sixteen || !a.rot || a.g != 256 || a.M <= 0 || a.sk != 1) return false;
    if ((a.K % 256) != 0 || a.K / 256 > 64 || (a.sm % 8) != 0 || ((uintptr_t)a.x % 16) != 0) return false;
    if (((uintptr_t)a.codes % 4) != 0 || (a.yout && ((uintptr_t)a.yout % 8) != 0)) return false;
    if (a.smooth && ((uintptr_t)a.smooth % 16) != 0) return false;
    return true;
}

// -------------------------------------------------------------------------
// Generic path (fp32 activations, or shapes the MFMA path does not take):
// one workgroup per row, the (smoothed) row staged in LDS as fp32, the
// rotation evaluated on VALU twice (absmax pass, then quantize pass) as an
// fp64 sum in index order, rounded once to T.
// -------------------------------------------------------------------------
template <int DT>
__device__ __forceinline__ float round_T(float v)
{
    if constexpr (DT == F32) return v;
    else return h_to_f32<DT>(f32_to_h<DT>(v));
}

template <int DT>
__device__ __forceinline__ float ld_T(const void* p, int64_t i) { return load_as_f32<DT>(p, i); }

// fp64 -> T in one rounding.  For T = fp32 that is the plain conversion.  For
// the 16-bit formats the fp64 value is first rounded to fp32 with round-to-odd
// (truncate, then set the last bit if anything was discarded); fp32 keeps more
// than two extra bits beyond fp16/bf16, so the following nearest-even rounding
// to T equals a direct nearest-even rounding of the fp64 value.
__device__ __forceinline__ float f64_to_f32_odd(double v)
{
    float f = (float)v;
    const double df = (double)f;
    if (df == v || f != f) return f;
    if (fabs(df) > fabs(v)) f = __uint_as_float(__float_as_uint(f) - 1u);  // toward zero
    if (isinf(f)) return f;
    return __uint_as_float(__float_as_uint(f) | 1u);
}

template <int DT>
__device__ __forceinline__ float round_f64_to_T(double v)
{
    if constexpr (DT == F32) return (float)v;
    else return round_T<DT>(f64_to_f32_odd(v));
}
template <int DT, bool ROT, bool SMOOTH, int QMAX = 7>
__global__ __launch_bounds__(256) void rq_generic_kernel(
    const void* __restrict__ x, int64_t M, int64_t K, int64_t sm, int64_t sk,
    const float* __restrict__ rot, int g, const void* __restrict__ smooth,
    int8_t* __restrict__ codes, float* __restrict__ scales, void* __restrict__ yout)
{
    extern __shared__ __align__(16) uint8_t smem[];
    float* xs = (float*)smem;
    __shared__ uint32_t red[4];
    const int64_t m = blockIdx.x;
    const int tid = threadIdx.x;
    for (int64_t k = tid; k < K; k += 256) {
        float v = ld_T<DT>(x, m * sm + k * sk);
        if constexpr (SMOOTH) v = round_T<DT>(v / ld_T<DT>(smooth, k));
        xs[k] = v;
    }
    __syncthreads();
    auto ycalc = [&](int64_t k) -> float {
        if constexpr (!ROT) return xs[k];
        const int64_t b = k / g;
        const int jj = (int)(k - b * g);
        const float* xb = xs + b * g;
        // fp32 x fp32 products are exact in fp64, so this is the index-order
        // fp64 sum of exact products, rounded once to T.
        double acc = 0.0;
        for (int i = 0; i < g; ++i)
            acc = fma((double)xb[i], (double)round_T<DT>(rot[i * g + jj]), acc);
        return round_f64_to_T<DT>(acc);
    };
    uint32_t mx = 0u;
    for (int64_t k = tid; k < K; k += 256)
        mx = max(mx, __float_as_uint(ycalc(k)) & 0x7fffffffu);
    for (int o = 32; o >= 1; o >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, o));
    if ((tid & 63) == 0) red[tid >> 6] = mx;
    __syncthreads();
    mx = max(max(red[0], red[1]), max(red[2], red[3]));
    const float s = row_scale_q<QMAX>(mx);
    const float ri = 1.0f / s;
    if (tid == 0) scales[m] = s;
    for (int64_t k = tid; k < K; k += 256) {
        float y = ycalc(k);
        codes[m * K + k] = (int8_t)quant_code_q<QMAX>(y, s, ri);
        if (yout) {
            if constexpr (DT == F32) ((float*)yout)[m * K + k] = y;
            else ((uint16_t*)yout)[m * K + k] = f32_to_h<DT>(y);
        }
    }
}

// -------------------------------------------------------------------------
// Launchers.
// -------------------------------------------------------------------------
static size_t mfma_lds_bytes(int GP, int64_t K, int rows)
{
    return 12 * 64 + (size_t)rows * (size_t)(K / GP) * (GP + 8) * 2;
}

template <int DT, int GP, bool CONTIG, bool ROT, bool SMOOTH>
static hipError_t launch_mfma_t(const RQArgs& a, hipStream_t st)
{
    const size_t per_row = mfma_lds_bytes(GP, a.K, 1) - 12 * 64;
    int rows = (int)((48 * 1024 - 12 * 64) / per_row);
    if (rows < 1) rows = 1;
    if (rows > 64) rows = 64;
    if (rows > a.M) rows = (int)a.M;
    const size_t lds = mfma_lds_bytes(GP, a.K, rows);
    const int64_t grid = (a.M + rows - 1) / rows;
    auto kern = rq_mfma_kernel<DT, GP, CONTIG, ROT, SMOOTH>;
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute((const void*)kern,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(256), lds, st, (const uint16_t*)a.x,
                       a.M, a.K, a.sm, a.sk, a.rot, a.g, (const uint16_t*)a.smooth, a.codes,
                       a.scales, (uint16_t*)a.yout, rows);
    return hipGetLastError();
}

template <int DT, int GP, bool CONTIG>
static hipError_t launch_mfma_rs(const RQArgs& a, hipStream_t st)
{
    const bool rot = a.rot != nullptr, sm = a.smooth != nullptr;
    if (rot && sm) return launch_mfma_t<DT, GP, CONTIG, true, true>(a, st);
    if (rot) return launch_mfma_t<DT, GP, CONTIG, true, false>(a, st);
    if (sm) return launch_mfma_t<DT, GP, CONTIG, false, true>(a, st);
    return launch_mfma_t<DT, GP, CONTIG, false, false>(a, st);
}

template <int DT, int GP>
static hipError_t launch_mfma_c(const RQArgs& a, hipStream_t st, bool contig)
{
    return contig ? launch_mfma_rs<DT, GP, true>(a, st) : launch_mfma_rs<DT, GP, false>(a, st);
}

template <int DT>
static hipError_t launch_mfma_dt(const RQArgs& a, int GP, bool contig, hipStream_t st)
{
    switch (GP) {
    case 32: return launch_mfma_c<DT, 32>(a, st, contig);
    case 64: return launch_mfma_c<DT, 64>(a, st, contig);
    case 128: return launch_mfma_c<DT, 128>(a, st, contig);
    default: return launch_mfma_c<DT, 256>(a, st, contig);
    }
}

template <int DT, int QMAX = 7>
static hipError_t launch_generic_dt(const RQArgs& a, hipStream_t st)
{
    const size_t lds = (size_t)a.K * 4;
    const bool rot = a.rot != nullptr, sm = a.smooth != nullptr;
    auto go = [&](auto kern) -> hipError_t {
        if (lds > 64 * 1024) {
            hipError_t e = hipFuncSetAttribute((const void*)kern,
                                               hipFuncAttributeMaxDynamicSharedMemorySize,
                                               (int)lds);
            if (e != hipSuccess) return e;
        }
        hipLaunchKernelGGL(kern, dim3((unsigned)a.M), dim3(256), lds, st, a.x, a.M, a.K, a.sm,
                           a.sk, a.rot, a.g, a.smooth, a.codes, a.scales, a.yout);
        return hipGetLastError();
    };
    if (rot && sm) return go(rq_generic_kernel<DT, true, true, QMAX>);
    if (rot) return go(rq_generic_kernel<DT, true, false, QMAX>);
    if (sm) return go(rq_generic_kernel<DT, false, true, QMAX>);
    return go(rq_generic_kernel<DT, false, false, QMAX>);
}


template <int DT, int GP, bool ROT, bool SMOOTH>
static hipError_t launch_reg_t(const RQArgs& a, hipStream_t st)
{
    const int gpr = (int)(a.K / GP);
    // rows per block: enough group-rows for one 16-row tile per wave
    int rows = 64 / (gpr > 0 ? gpr : 1);
    if (rows < 1) rows = 1;
    if (rows > 16) rows = 16;
    const int tiles = (rows * gpr + 15) / 16;
    int tw = (tiles + 3) / 4;
    if (tw > 4) return hipErrorNotSupported;
    const int64_t nblk = (a.M + rows - 1) / rows;
    auto go = [&](auto kern) {
        // persistent grid: exactly the workgroups that can be resident
        static int per_cu = 0, n_cu = 0;
        if (per_cu == 0) {
            int dev = 0;
            hipDeviceProp_t p;
            if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&p, dev) != hipSuccess ||
                hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, 256, 0) != hipSuccess ||
                per_cu < 1) {
                per_cu = 2;
                n_cu = 256;
            } else {
                n_cu = p.multiProcessorCount;
            }
        }
        int64_t grid = (int64_t)per_cu * n_cu;
        if (grid > nblk) grid = nblk;
        hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(256), 0, st, (const uint16_t*)a.x, a.M,
                           a.K, a.sm, a.rot, a.g, (const uint16_t*)a.smooth, a.codes, a.scales,
                           (uint16_t*)a.yout, rows);
        return hipGetLastError();
    };
    if (tw == 1) return go(rq_reg_kernel<DT, GP, ROT, SMOOTH, 1>);
    if (tw == 2) return go(rq_reg_kernel<DT, GP, ROT, SMOOTH, 2>);
    return go(rq_reg_kernel<DT, GP, ROT, SMOOTH, 4>);
}

template <int DT>
static hipError_t launch_reg_dt(const RQArgs& a, int GP, hipStream_t st)
{
    const bool rot = a.rot != nullptr, sm = a.smooth != nullptr;
    if (GP == 32) {
        if (rot && sm) return launch_reg_t<DT, 32, true, true>(a, st);
        if (rot) return launch_reg_t<DT, 32, true, false>(a, st);
        if (sm) return launch_reg_t<DT, 32, false, true>(a, st);
        return launch_reg_t<DT, 32, false, false>(a, st);
    }
    if (rot && sm) return launch_reg_t<DT, 64, true, true>(a, st);
    if (rot) return launch_reg_t<DT, 64, true, false>(a, st);
    if (sm) return launch_reg_t<DT, 64, false, true>(a, st);
    return launch_reg_t<DT, 64, false, false>(a, st);
}


template <int DT, int GP, bool ROT, bool SMOOTH>
static hipError_t launch_wave_t(const RQArgs& a, hipStream_t st)
{
    const int gpr = (int)(a.K / GP);
    int tw = (gpr + 15) / 16;
    tw = tw <= 1 ? 1 : tw <= 2 ? 2 : 4;
    if (gpr > 64) return hipErrorNotSupported;
    int rpb = (16 * tw) / gpr;
    if (rpb < 1) rpb = 1;
    const int64_t nblk = (a.M + rpb - 1) / rpb;
    auto go = [&](auto kern) {
        static int per_cu = 0, n_cu = 0;
        if (per_cu == 0) {
            int dev = 0;
            hipDeviceProp_t p;
            if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&p, dev) != hipSuccess ||
                hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, 256, 0) != hipSuccess ||
                per_cu < 1) {
                per_cu = 2;
                n_cu = 256;
            } else {
                n_cu = p.multiProcessorCount;
            }
        }
        int64_t grid = (int64_t)per_cu * n_cu;
        const int64_t need = (nblk + 3) / 4;          // four waves per workgroup
        if (grid > need) grid = need;
        hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(256), 0, st, (const uint16_t*)a.x, a.M,
                           a.K, a.sm, a.rot, a.g, (const uint16_t*)a.smooth, a.codes, a.scales,
                           (uint16_t*)a.yout, rpb);
        return hipGetLastError();
    };
    if (tw == 1) return go(rq_wave_kernel<DT, GP, ROT, SMOOTH, 1>);
    if (tw == 2) return go(rq_wave_kernel<DT, GP, ROT, SMOOTH, 2>);
    return go(rq_wave_kernel<DT, GP, ROT, SMOOTH, 4>);
}

template <int DT>
static hipError_t launch_wave_dt(const RQArgs& a, int GP, hipStream_t st)
{
    const bool rot = a.rot != nullptr, sm = a.smooth != nullptr;
    if (GP == 32) {
        if (rot && sm) return launch_wave_t<DT, 32, true, true>(a, st);
        if (rot) return launch_wave_t<DT, 32, true, false>(a, st);
        if (sm) return launch_wave_t<DT, 32, false, true>(a, st);
        return launch_wave_t<DT, 32, false, false>(a, st);
    }
    if (rot && sm) return launch_wave_t<DT, 64, true, true>(a, st);
    if (rot) return launch_wave_t<DT, 64, true, false>(a, st);
    if (sm) return launch_wave_t<DT, 64, false, true>(a, st);
    return launch_wave_t<DT, 64, false, false>(a, st);
}

// ring depth: as many tiles in flight as fit next to the staging tiles
template <int GP, bool YOUT> constexpr int cm_stages() { return GP == 256 ? (YOUT ? 5 : 6) : 8; }

template <int DT, int GP, bool SMOOTH, bool YOUT>
static hipError_t launch_colmajor_t(const RQArgs& a, hipStream_t st)
{
    const unsigned grid = (unsigned)((a.M + CM_ROWS - 1) / CM_ROWS);
    hipLaunchKernelGGL((rq_colmajor_kernel<DT, GP, SMOOTH, YOUT, cm_stages<GP, YOUT>()>), dim3(grid), dim3(512), 0, st,
                       (const uint16_t*)a.x, a.M, a.K, a.sk, a.rot, (const uint16_t*)a.smooth, a.codes,
                       a.scales, (uint16_t*)a.yout);
    return hipGetLastError();
}

template <int DT, int GP>
static hipError_t launch_colmajor_g(const RQArgs& a, hipStream_t st)
{
    if (a.smooth)
        return a.yout ? launch_colmajor_t<DT, GP, true, true>(a, st) : launch_colmajor_t<DT, GP, true, false>(a, st);
    return a.yout ? launch_colmajor_t<DT, GP, false, true>(a, st) : launch_colmajor_t<DT, GP, false, false>(a, st);
}

template <int DT>
static hipError_t launch_colmajor_dt(const RQArgs& a, hipStream_t st)
{
    if (a.g == 64) return launch_colmajor_g<DT, 64>(a, st);
    if (a.g == 128) return launch_colmajor_g<DT, 128>(a, st);
    return launch_colmajor_g<DT, 256>(a, st);
}

// Unit row stride (a transposed view): the column-major kernel applies when
// its loads and stores line up on 16 bytes and every buffer offset fits in
// 31 bits.
static bool colmajor_ok(const RQArgs& a)
{
    const bool sixteen = a.dtype == F16 || a.dtype == BF16;
    if (!sixteen || !a.rot || a.sm != 1 || a.sk < a.M || a.M <= 0) return false;
    if (!(a.g == 64 || a.g == 128 || a.g == 256) || (a.K % a.g) != 0) return false;
    if ((a.M % 8) != 0 || (a.sk % 8) != 0) return false;
    if (((uintptr_t)a.x % 16) != 0 || ((uintptr_t)a.codes % 16) != 0) return false;
    if (a.yout && ((uintptr_t)a.yout % 16) != 0) return false;
    const int64_t lim = 0x7ffffff0ll;
    if (a.M * a.K > lim || (a.yout && 2 * a.M * a.K > lim)) return false;
    if (2 * (int64_t)a.g * a.sk > lim) return false;
    return true;
}

// Which kernel serves a call (decided on the host from shapes, strides and
// alignments alone): 0 generic, 1 MFMA with an LDS row buffer, 2 MFMA
// registers, 3 wave per row block, 4 column-major, 5 g = 256 row-major,
// 6 row-streaming g = 64 (rq_row.hip); -1
// when none does (a row too long for the generic kernel's LDS buffer).
int rotate_quant_path(const RQArgs& a)
{
    // structured (Hadamard) rotation: at g = 64 on many contiguous rows the
    // row-streaming kernel (it builds R's fragments from the signs; faster
    // than the transform at this width), else the fast Walsh-Hadamard kernel
    if (a.hadamard) return row_kernel_ok(a) ? 6 : hadamard_kernel_ok(a) ? 7 : -1;
    // INT8 mode: the row-streaming and g = 256 kernels, else the generic one
    if (a.qmax == 127) {
        if (g256_ok(a)) return 5;
        if (row_kernel_ok(a)) return 6;
        if ((size_t)a.K * 4 > 160 * 1024) return -1;  // row does not fit in LDS
        return 0;
    }
    if (a.qmax != 7) return -1;
    // MFMA path: 16-bit activations, group width 16..256, K a multiple of
    // the MFMA group width, 16-byte aligned operands for the vector loads.
    int GP = 0;
    if (a.rot) GP = a.g < 32 ? 32 : a.g;
    else GP = 32;
    const bool sixteen = a.dtype == F16 || a.dtype == BF16;
    bool ok = sixteen && GP <= 256 && (a.K % GP) == 0 && ((uintptr_t)a.codes % 16) == 0 &&
              (a.yout == nullptr || ((uintptr_t)a.yout % 16) == 0) &&
              (a.smooth == nullptr || ((uintptr_t)a.smooth % 16) == 0);
    if (a.rot && !(a.g == 16 || a.g == 32 || a.g == 64 || a.g == 128 || a.g == 256)) ok = false;
    // g = 16 would run as 32-wide MFMA groups with R twice on the diagonal of
    // a zero-padded 32 x 32 operand; an infinite input then meets a padding
    // zero (Inf * 0 = NaN) and poisons the neighbouring group.  Those calls
    // take the generic kernel, which sums each group on its own.
    if (a.rot && a.g == 16) ok = false;
    if (colmajor_ok(a)) return 4;
    if (g256_ok(a)) return 5;
    if (row_kernel_ok(a)) return 6;
    if (ok && mfma_lds_bytes(GP, a.K, 1) > 160 * 1024) ok = false;
    const bool contig = a.sk == 1 && (a.sm % 8) == 0 && ((uintptr_t)a.x % 16) == 0;
    // The wave-per-row-block kernel needs many row blocks to keep the GPU
    // busy (each wave works through its rows alone); with fewer, the
    // register kernel, which spreads a block's tiles over four waves, is
    // faster (measured crossover near 1,500 blocks at K/g = 60).
    bool many_blocks = false;
    if (GP <= 64 && a.K / GP <= 64) {
        const int gpr = (int)(a.K / GP);
        int tw = (gpr + 15) / 16;
        tw = tw <= 1 ? 1 : tw <= 2 ? 2 : 4;
        int rpb = (16 * tw) / (gpr > 0 ? gpr : 1);
        if (rpb < 1) rpb = 1;
        many_blocks = (a.M + rpb - 1) / rpb >= 1536;
    }
    if (ok && contig && GP <= 64 && a.K / GP <= 64 && many_blocks &&
        (a.yout == nullptr || ((uintptr_t)a.yout % 8) == 0) && ((uintptr_t)a.codes % 16) == 0)
        return 3;
    if (ok && contig && GP <= 64 && a.K / GP <= 256 &&
        (a.yout == nullptr || ((uintptr_t)a.yout % 8) == 0) && ((uintptr_t)a.codes % 4) == 0)
        return 2;
    if (ok) return 1;
    if ((size_t)a.K * 4 > 160 * 1024) return -1;  // row does not fit in LDS
    return 0;
}

hipError_t launch_rotate_quant(const RQArgs& a, hipStream_t st, int* path)
{
    const int p = rotate_quant_path(a);
    if (path) *path = p;
    const bool bf = a.dtype == BF16;
    const int GP = a.rot ? (a.g < 32 ? 32 : a.g) : 32;
    const bool contig = a.sk == 1 && (a.sm % 8) == 0 && ((uintptr_t)a.x % 16) == 0;
    if (p == 7) return launch_rotate_quant_hadamard(a, st);
    if (a.qmax == 127) {
        switch (p) {
        case 5: return bf ? launch_g256_dt<BF16, 127>(a, st) : launch_g256_dt<F16, 127>(a, st);
        case 6: return launch_rotate_quant_row(a, st);
        case 0:
            switch (a.dtype) {
            case F32: return launch_generic_dt<F32, 127>(a, st);
            case F16: return launch_generic_dt<F16, 127>(a, st);
            default: return launch_generic_dt<BF16, 127>(a, st);
            }
        default: return hipErrorNotSupported;
        }
    }
    switch (p) {
    case 4: return bf ? launch_colmajor_dt<BF16>(a, st) : launch_colmajor_dt<F16>(a, st);
    case 5: return bf ? launch_g256_dt<BF16>(a, st) : launch_g256_dt<F16>(a, st);
    case 6: return launch_rotate_quant_row(a, st);
    case 3: return bf ? launch_wave_dt<BF16>(a, GP, st) : launch_wave_dt<F16>(a, GP, st);
    case 2: return bf ? launch_reg_dt<BF16>(a, GP, st) : launch_reg_dt<F16>(a, GP, st);
    case 1: return bf ? launch_mfma_dt<BF16>(a, GP, contig, st) : launch_mfma_dt<F16>(a, GP, contig, st);
    case 0:
        switch (a.dtype) {
        case F32: return launch_generic_dt<F32>(a, st);
        case F16: return launch_generic_dt<F16>(a, st);
        default: return launch_generic_dt<BF16>(a, st);
        }
    default: return hipErrorNotSupported;
    }
}

}  // namespace w4a4
