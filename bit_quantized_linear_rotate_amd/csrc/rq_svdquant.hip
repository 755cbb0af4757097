// Activation quantizer of the SVDQuant layer (source page
// comfy_kitchen/tensor/svdquant_w4a4.py: the _w4a4_forward docstring, the
// shift 0.171875 of act_unsigned layers onto the unsigned [0, 15] grid; the
// module docstring, INT4 group size 64), for contiguous 16-bit rows:
//   x_main = T(fp32(x) + 0.171875)            (act_unsigned only)
//   x_s    = T(fp32(x_main) / fp32(smooth))   (when smoothing factors are given)
//   per row (group 0) or per 64-wide group of a row (group 64):
//   s = max(absmax / qmax, 2^-126), qmax = 7 (signed) or 15 (unsigned grid),
//   c = clamp(round_half_even(fp32(x_s) / s), -7, 7)  or  (..., 0, 15).
// No rotation: the SVDQuant layer has none.
//
// Design: a workgroup of W = ceil(K / 1024) waves takes one row at a time,
// 512-element chunk p to wave p mod W; lane l holds the 8 consecutive
// elements 8 l .. 8 l + 7 of its chunk (16-byte loads, 8-byte code stores), so
// a 64-wide group is 8 neighbouring lanes and its absmax a three-step DPP max.
// A whole-row scale crosses waves through LDS (one barrier a row).  As in the
// other streaming kernels, the next row's loads are in flight in a second
// register set while a row is quantized, and every access is a range-checked
// buffer access (no lane-dependent branches around memory).
#include "common.hpp"
#include "kernels.hpp"

namespace w4a4 {
namespace {

constexpr int SQ_MAXW = 16;
constexpr int SQ_P = 2;                   // chunks a wave and row
constexpr float kSqMagic = 12582912.0f;   // 1.5 * 2^23
typedef unsigned v2u_sq __attribute__((ext_vector_type(2)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t sq_rsrc(const void* base, uint64_t bytes)
{
    const uint32_t n = bytes > 0xffffffffull ? 0xffffffffu : (uint32_t)bytes;
    return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)n, 0x00020000);
}

template <int CTRL>
__device__ __forceinline__ uint32_t sq_dpp(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xf, 0xf, false);
}

// max over the 8 lanes 8t .. 8t + 7 (quad swaps, then the mirror inside the
// half row: lane i meets lane i ^ 7)
__device__ __forceinline__ uint32_t max8(uint32_t v)
{
    v = max(v, sq_dpp<0xb1>(v));
    v = max(v, sq_dpp<0x4e>(v));
    return max(v, sq_dpp<0x141>(v));
}

__device__ __forceinline__ uint32_t max_wave(uint32_t v)
{
    v = max8(v);
    v = max(v, sq_dpp<0x128>(v));   // row_ror:8
    const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
    const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
    const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
    const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
    return max(max(r0, r1), max(r2, r3));
}

template <int LO, int HI>
__device__ __forceinline__ uint32_t codes4_exact(const float (&y)[4], float s)
{
    uint32_t out = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float q = y[i] / s;
        const float cl = __builtin_amdgcn_fmed3f(rintf(q), (float)LO, (float)HI);
        const int c = (q == q) ? (int)cl : 0;
        out |= ((uint32_t)c & 0xffu) << (8 * i);
    }
    return out;
}

__device__ __forceinline__ uint32_t pack_magic(float t0, float t1, float t2, float t3)
{
    const uint32_t lo = __builtin_amdgcn_perm(__float_as_uint(t1), __float_as_uint(t0), 0x0c0c0400u);
    const uint32_t hi = __builtin_amdgcn_perm(__float_as_uint(t3), __float_as_uint(t2), 0x0c0c0400u);
    return lo | (hi << 16);
}

// four codes of one block: y * (1/s) rounded by an add of 1.5 * 2^23, the
// IEEE division where a quotient lies near a half-integer or is clamped
// (|y (1/s) - fl(y / s)| <= 2 * 15 * 2^-24 < 2^-19 inside the grid)
template <int LO, int HI>
__device__ __forceinline__ uint32_t codes4(const float (&y)[4], float s, float ri, bool fin)
{
    if (!fin) return codes4_exact<LO, HI>(y, s);
    float t[4];
    bool nr = false;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const float qv = y[r] * ri;
        t[r] = __builtin_amdgcn_fmed3f(qv, (float)LO, (float)HI) + kSqMagic;
        nr |= fabsf(qv - (t[r] - kSqMagic)) > 0.5f - 0x1p-17f;
    }
    const uint32_t pk = pack_magic(t[0], t[1], t[2], t[3]);
    return __any(nr) ? codes4_exact<LO, HI>(y, s) : pk;
}

template <int DT, int GRP, bool UNS, bool SHIFT, bool SMOOTH>
__global__ __launch_bounds__(1024) void rq_svd_kernel(
    const uint16_t* __restrict__ x, int64_t M, int64_t K, int64_t sm, const uint16_t* __restrict__ smooth,
    int8_t* __restrict__ codes, float* __restrict__ scales)
{
    constexpr int P = SQ_P;
    constexpr int QM = UNS ? 15 : 7, LO = UNS ? 0 : -7;
    __shared__ uint32_t wmax[2][SQ_MAXW];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int nw = (int)(blockDim.x >> 6);
    const int lo = 8 * lane;                        // the lane's first element in a chunk
    const int G = GRP ? (int)(K / GRP) : 1;         // scales per row
    auto chunk_of = [&](int i) { return wave + nw * i; };

    auto load_row = [&](int64_t row, v8s (&xf)[P]) {
        const __amdgpu_buffer_rsrc_t rx = sq_rsrc(x + (row < M ? row : 0) * sm, row < M ? (uint64_t)K * 2 : 0);
#pragma unroll
        for (int i = 0; i < P; ++i)
            xf[i] = __builtin_bit_cast(v8s, __builtin_amdgcn_raw_buffer_load_b128(
                                                rx, ((chunk_of(i) << 9) + lo) * 2, 0, 0));
    };
    const __amdgpu_buffer_rsrc_t rsm = sq_rsrc(smooth, SMOOTH ? (uint64_t)K * 2 : 0);
    const __amdgpu_buffer_rsrc_t rsc = sq_rsrc(scales, (uint64_t)M * G * 4);
    int par = 0;

    auto process = [&](int64_t row, const v8s (&xin)[P]) {
        if (row >= M) return;
        float y[P][8];
        uint32_t m16[P];
#pragma unroll
        for (int i = 0; i < P; ++i) {
            const int off = (chunk_of(i) << 9) + lo;
            const bool in = off < K;
            v8s sv = {0, 0, 0, 0, 0, 0, 0, 0};
            if constexpr (SMOOTH) sv = __builtin_bit_cast(v8s, __builtin_amdgcn_raw_buffer_load_b128(rsm, off * 2, 0, 0));
            m16[i] = 0u;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                uint16_t b = (uint16_t)xin[i][e];
                if constexpr (SHIFT) b = f32_to_h<DT>(h_to_f32<DT>(b) + 0.171875f);
                if constexpr (SMOOTH) b = f32_to_h<DT>(h_to_f32<DT>(b) / h_to_f32<DT>((uint16_t)sv[e]));
                // lanes past K hold zeros (the shift and 0 / 0 must not reach them)
                b = in ? b : (uint16_t)0;
                y[i][e] = h_to_f32<DT>(b);
                m16[i] = max(m16[i], (uint32_t)(b & 0x7fffu));
            }
        }
        const __amdgpu_buffer_rsrc_t rc = sq_rsrc(codes + row * K, (uint64_t)K);
        if constexpr (GRP == 64) {
            // one scale per 8-lane group; lane 8t of the group writes it
#pragma unroll
            for (int i = 0; i < P; ++i) {
                const uint32_t gm = max8(m16[i]);
                float s = h_to_f32<DT>((uint16_t)gm) / (float)QM;
                if (s < 0x1p-126f) s = 0x1p-126f;
                const int off = (chunk_of(i) << 9) + lo;
                const int gi = off >> 6;
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(s), rsc,
                                                      ((lane & 7) == 0 && off < K) ? (int)((row * G + gi) * 4)
                                                                                   : (int)(M * G * 4), 0, 0);
                const float ri = 1.0f / s;
                const bool fin = fabsf(s) < 3.0e38f;
                const float y0[4] = {y[i][0], y[i][1], y[i][2], y[i][3]};
                const float y1[4] = {y[i][4], y[i][5], y[i][6], y[i][7]};
                const v2u_sq pk = {codes4<LO, QM>(y0, s, ri, fin), codes4<LO, QM>(y1, s, ri, fin)};
                __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(v2u_sq, pk), rc, off, 0, 0);
            }
        } else {
            uint32_t mm = m16[0];
#pragma unroll
            for (int i = 1; i < P; ++i) mm = max(mm, m16[i]);
            const uint32_t wm = max_wave(mm);
            if (lane == 0) wmax[par][wave] = wm;
            __syncthreads();
            mm = wmax[par][0];
            for (int w = 1; w < nw; ++w) mm = max(mm, wmax[par][w]);
            par ^= 1;
            float s = h_to_f32<DT>((uint16_t)mm) / (float)QM;
            if (s < 0x1p-126f) s = 0x1p-126f;
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(s), rsc,
                                                  (wave == 0 && lane == 0) ? (int)(row * 4) : (int)(M * 4), 0, 0);
            const float ri = 1.0f / s;
            const bool fin = fabsf(s) < 3.0e38f;
#pragma unroll
            for (int i = 0; i < P; ++i) {
                const int off = (chunk_of(i) << 9) + lo;
                const float y0[4] = {y[i][0], y[i][1], y[i][2], y[i][3]};
                const float y1[4] = {y[i][4], y[i][5], y[i][6], y[i][7]};
                const v2u_sq pk = {codes4<LO, QM>(y0, s, ri, fin), codes4<LO, QM>(y1, s, ri, fin)};
                __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(v2u_sq, pk), rc, off, 0, 0);
            }
        }
    };

    const int64_t rs = gridDim.x;
    const int64_t r0 = blockIdx.x;
    v8s xa[P], xb[P];
    load_row(r0, xa);
    for (int64_t row = r0; row < M; row += 2 * rs) {
        load_row(row + rs, xb);
        process(row, xa);
        load_row(row + 2 * rs, xa);
        process(row + rs, xb);
    }
}

template <int DT, int GRP, bool UNS>
hipError_t launch_sq3(const RQArgs& a, bool shift, hipStream_t st)
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
    const int nchunk = (int)((a.K + 511) / 512);
    const int nw = (nchunk + SQ_P - 1) / SQ_P;
    const int64_t per_cu = 32 / nw > 0 ? 32 / nw : 1;
    const int64_t want = (int64_t)n_cu * per_cu;
    const unsigned grid = (unsigned)(a.M < want ? a.M : want);
    auto* xp = (const uint16_t*)a.x;
    auto* sp = (const uint16_t*)a.smooth;
#define W4A4_SQ(SH, SM)                                                                                     \
    hipLaunchKernelGGL((rq_svd_kernel<DT, GRP, UNS, SH, SM>), dim3(grid), dim3(64 * nw), 0, st, xp, a.M, a.K, \
                       a.sm, sp, a.codes, a.scales)
    if (shift) {
        if (a.smooth) W4A4_SQ(true, true);
        else W4A4_SQ(true, false);
    } else {
        if (a.smooth) W4A4_SQ(false, true);
        else W4A4_SQ(false, false);
    }
#undef W4A4_SQ
    return hipGetLastError();
}

template <int DT>
hipError_t launch_sq_dt(const RQArgs& a, int group, bool uns, hipStream_t st)
{
    // the unsigned grid always comes with the shift (act_unsigned layers)
    if (group == 64)
        return uns ? launch_sq3<DT, 64, true>(a, true, st) : launch_sq3<DT, 64, false>(a, false, st);
    return uns ? launch_sq3<DT, 0, true>(a, true, st) : launch_sq3<DT, 0, false>(a, false, st);
}

}  // namespace

// Contiguous 16-bit rows (16-byte aligned, row stride a multiple of 8), K a
// multiple of 64 for per-group scales (else of 8), K <= 16384, fewer than
// 2^29 rows (scale offsets fit the buffer offsets), 8-byte aligned codes,
// 16-byte aligned smoothing factors.
bool svd_quant_ok(const RQArgs& a, int group)
{
    const bool sixteen = a.dtype == F16 || a.dtype == BF16;
    if (!sixteen || a.M <= 0 || a.M >= (1 << 29) || a.sk != 1 || a.rot) return false;
    if (group != 0 && group != 64) return false;
    if (a.K <= 0 || a.K > 16384 || (a.K % (group ? 64 : 8)) != 0) return false;
    if ((int64_t)a.M * (a.K / 64) >= (int64_t)1 << 29) return false;
    if ((a.sm % 8) != 0 || ((uintptr_t)a.x % 16) != 0 || ((uintptr_t)a.codes % 8) != 0) return false;
    if (a.smooth && ((uintptr_t)a.smooth % 16) != 0) return false;
    return true;
}

hipError_t launch_svd_quant(const RQArgs& a, int group, bool act_unsigned, hipStream_t st)
{
    if (!svd_quant_ok(a, group)) return hipErrorNotSupported;
    return a.dtype == BF16 ? launch_sq_dt<BF16>(a, group, act_unsigned, st)
                           : launch_sq_dt<F16>(a, group, act_unsigned, st);
}

}  // namespace w4a4
