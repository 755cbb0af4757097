// Row quantizer parameters and the bracketed code rounding shared by the
// rotate-quant kernels (device code).
//
// The quantizer ("[Feat][Ascend] Consolidate INT8, RotateQuant, RoPE and
// ConvRot W4A4 backends", section "W4A4 correctness and performance scope")
// takes s = max(a / 7, 2^-126) for a row with absmax a and codes
// c = clamp(RNE(y / s), -7, 7).  For a finite s, with rinv = 1/s, the
// integers RNE(y * rinv * (1 + 2^-21)) and RNE(y * rinv * (1 - 2^-21)) (one
// fma each against 1.5 * 2^23, which leaves the integer in the low byte)
// bracket the correctly rounded quotient; for 16-bit y and a taken from the
// row's own 16-bit values they differ only at exact ties 7 y = (k + 1/2) a,
// whose outcome (rounds to k or to k + 1) is the same for every element of the
// row with that k: a 7-bit mask per row decides them all.
#pragma once
#include "common.hpp"
#include "scale_table.hpp"

namespace w4a4 {

constexpr float kBracketMagic = 12582912.0f;  // 1.5 * 2^23

// per-significand row scales (exact: see scale_table.hpp), one copy per
// translation unit; read with scalar loads where the row is uniform across
// a wave
static __constant__ const RowScaleTable<7> kRowScaleBf16Q7 = make_row_scale_table<7, 7>();
static __constant__ const RowScaleTable<7> kRowScaleBf16Q127 = make_row_scale_table<7, 127>();
static __constant__ const RowScaleTable<10> kRowScaleF16Q7 = make_row_scale_table<10, 7>();
static __constant__ const RowScaleTable<10> kRowScaleF16Q127 = make_row_scale_table<10, 127>();

template <int DT, int QMAX>
__device__ __forceinline__ const RowScaleEntry& row_scale_entry(uint32_t idx)
{
    if constexpr (DT == BF16) return QMAX == 7 ? kRowScaleBf16Q7.e[idx] : kRowScaleBf16Q127.e[idx];
    else return QMAX == 7 ? kRowScaleF16Q7.e[idx] : kRowScaleF16Q127.e[idx];
}

struct RowQuant {
    float s;       // the row's scale
    float rh, rl;  // rinv * (1 + 2^-21), rinv * (1 - 2^-21)
    float r1;      // the bracketing multiplier that rounds the k = 3 tie the quantizer's way
    uint32_t tie;  // tie mask, bit k and its mirror bit 32 - k (see tie_select)
    bool one;      // 7 does not divide a's significand: r1 alone gives every code
    bool exact;    // outside the table's range: every code by IEEE division
};

// Parameters of one row from its 16-bit absmax pattern a16, computed by one
// thread: the significand table shifted by a's exponent.  For the patterns
// the table does not cover (zero, a < 2^-119, Inf, NaN) the scale is one IEEE
// division; a row whose scale is the smallest one (2^-126: zero and tiny rows)
// keeps the bracketed codes, exact at that scale, and every other such row
// (Inf, NaN, absmax in [7 * 2^-126, 2^-119)) sets `exact`, which sends its
// codes to the IEEE division of every element, the quantizer's own formula.
template <int DT>
__device__ __forceinline__ RowQuant row_quant_thread(uint32_t a16)
{
    RowQuant p;
    uint32_t idx;
    int E;
    if (row_scale_key<DT == BF16>(a16, idx, E)) {
        const RowScaleEntry& e = row_scale_entry<DT, 7>(idx);
        p.s = row_scale_shift(e.s, E);
        p.rh = row_scale_shift(e.rh, -E);
        p.rl = row_scale_shift(e.rl, -E);
        p.r1 = row_scale_shift(e.r1, -E);
        p.tie = e.tie;
        p.one = e.one != 0u;
        p.exact = false;
        return p;
    }
    const float a = h_to_f32<DT>((uint16_t)a16);
    float s = a / 7.0f;
    if (s < 0x1p-126f) s = 0x1p-126f;  // NaN compares false and stays NaN
    p.s = s;
    p.one = false;
    if (s == 0x1p-126f) {
        // the smallest scale (zero and tiny rows): y / s = y * 2^126 exactly,
        // so the bracketing multipliers are exact scalings and a tie rounds
        // to even (k odd rounds up)
        p.rh = 0x1p126f * (1.0f + 0x1p-21f);
        p.rl = 0x1p126f * (1.0f - 0x1p-21f);
        p.r1 = p.rh;
        p.tie = 0x2au | (__builtin_bitreverse32(0x2au) << 1);
        p.exact = false;
    } else {
        p.rh = p.rl = p.r1 = 0.0f;
        p.tie = 0u;
        p.exact = true;
    }
    return p;
}

// code byte of y from its two bracketing roundings (magic sums) and the tie
// mask: t_dn when they agree (then t_up == t_dn), else the tie's outcome.
// The mask bit, sign-extended to all ones or zero, selects t_up or t_dn.
__device__ __forceinline__ uint32_t tie_select(float t_up, float t_dn, uint32_t mask)
{
    const uint32_t u = __float_as_uint(t_up), d = __float_as_uint(t_dn);
    const uint32_t sel = (uint32_t)__builtin_amdgcn_sbfe((int)mask, (int)(d & 31u), 1);
    return (sel & u) | (~sel & d);
}

// four code bytes (in the low byte of each value) in one dword
__device__ __forceinline__ uint32_t pack_code_bytes(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3)
{
    const uint32_t lo = __builtin_amdgcn_perm(c1, c0, 0x0c0c0400u);
    const uint32_t hi = __builtin_amdgcn_perm(c3, c2, 0x0c0c0400u);
    return lo | (hi << 16);
}

// codes of four finite-scale values of a row whose tie can only be k = 3
// (p.one): one fma each
__device__ __forceinline__ uint32_t quant4_one(const float (&y)[4], const RowQuant& p)
{
    uint32_t c[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) c[i] = __float_as_uint(__builtin_fmaf(y[i], p.r1, kBracketMagic));
    return pack_code_bytes(c[0], c[1], c[2], c[3]);
}

// codes of four finite-scale values of one row
__device__ __forceinline__ uint32_t quant4_bracket(const float (&y)[4], const RowQuant& p)
{
    uint32_t c[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        c[i] = tie_select(__builtin_fmaf(y[i], p.rh, kBracketMagic), __builtin_fmaf(y[i], p.rl, kBracketMagic), p.tie);
    return pack_code_bytes(c[0], c[1], c[2], c[3]);
}

}  // namespace w4a4
