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

__device__ __forceinline__ float row_scale(uint32_t absmax_bits)
{
    float a = __uint_as_float(absmax_bits);
    float s = a / 7.0f;
    if (s < 0x1p-126f) s = 0x1p-126f;  // NaN compares false and stays NaN
    return s;
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
        uint4 out = {w[0], w[1], w[2], w[3]};
        *(uint4*)(codes + (m0 + r) * K + k0) = out;
        if (yout) {
            uint4* yo = (uint4*)(yout + (m0 + r) * K + k0);
            yo[0] = __builtin_bit_cast(uint4, y0);
            yo[1] = __builtin_bit_cast(uint4, y1);
        }
    }
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
template <int DT, bool ROT, bool SMOOTH>
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
    const float s = row_scale(mx);
    const float ri = 1.0f / s;
    if (tid == 0) scales[m] = s;
    for (int64_t k = tid; k < K; k += 256) {
        float y = ycalc(k);
        codes[m * K + k] = (int8_t)quant_code(y, s, ri);
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

template <int DT>
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
    if (rot && sm) return go(rq_generic_kernel<DT, true, true>);
    if (rot) return go(rq_generic_kernel<DT, true, false>);
    if (sm) return go(rq_generic_kernel<DT, false, true>);
    return go(rq_generic_kernel<DT, false, false>);
}

// Chooses the kernel; returns the path taken in *path (0 generic, 1 MFMA).
hipError_t launch_rotate_quant(const RQArgs& a, hipStream_t st, int* path)
{
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
    if (ok && mfma_lds_bytes(GP, a.K, 1) > 160 * 1024) ok = false;
    const bool contig = a.sk == 1 && (a.sm % 8) == 0 && ((uintptr_t)a.x % 16) == 0;
    if (ok) {
        if (path) *path = 1;
        return a.dtype == BF16 ? launch_mfma_dt<BF16>(a, GP, contig, st)
                               : launch_mfma_dt<F16>(a, GP, contig, st);
    }
    if (path) *path = 0;
    if ((size_t)a.K * 4 > 160 * 1024) return hipErrorNotSupported;  // row does not fit in LDS
    switch (a.dtype) {
    case F32: return launch_generic_dt<F32>(a, st);
    case F16: return launch_generic_dt<F16>(a, st);
    default: return launch_generic_dt<BF16>(a, st);
    }
}

}  // namespace w4a4
