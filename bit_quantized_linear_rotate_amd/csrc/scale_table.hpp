// Per-significand row-scale table for 16-bit row absmax values (host and
// device; no HIP dependency, so host code can check it).
//
// The quantizer's scale is s = max(a / qmax, 2^-126) with a the row's absmax
// ("[Feat][Ascend] Consolidate INT8, RotateQuant, RoPE and ConvRot W4A4
// backends", section "W4A4 correctness and performance scope": per-row
// absmax scale; qmax = 7 for INT4 codes, 127 for the INT8 mode of "[Feat]
// [Ascend] Add fused RotateQuant backend").  A row kernel also needs, per
// row, 1/s, the two multipliers 1/s * (1 +- 2^-21) that bracket every
// quotient y / s, and the outcome of each exact tie 7 y = (k + 1/2) a.
//
// When a is a 16-bit value, a = a_n * 2^E with a_n in [1, 2) holding at most
// 8 (bf16) or 11 (fp16) significant bits.  Every one of those quantities is
// a correctly rounded quotient or product of a_n-derived values; while the
// results stay normal, scaling the operands by 2^E scales the rounded result
// by the same power of two (or its inverse).  So each is the entry for a_n,
// shifted by E in the exponent field: one table row per fraction pattern
// (128 for bf16, 1024 for fp16), computed at compile time with IEEE
// round-to-nearest-even arithmetic.  Rows where the shifted values would
// leave the normal range (a < 2^-119, zero, Inf, NaN) are not covered: the
// caller computes those with divisions.
#pragma once
#include <stdint.h>

#if defined(__HIPCC__)
#define W4A4_HD __host__ __device__
#else
#define W4A4_HD
#endif

namespace w4a4 {

struct RowScaleEntry {
    float s;      // fl(a_n / qmax)
    float rinv;   // fl(1 / s)
    float rh;     // fl(rinv * (1 + 2^-21))
    float rl;     // fl(rinv * (1 - 2^-21))
    float r1;     // qmax 7: the one multiplier that rounds every code when 7 does not divide
                  // the significand (it takes the only possible tie, k = 3, the quantizer's way)
    uint32_t tie; // qmax 7: tie outcomes, bit k set when the tie at k + 1/2 rounds to k + 1,
                  // mirrored to bit 32 - k for the tie at -(k + 1/2) (indexed by the low five
                  // bits of the toward-zero code's two's-complement byte)
    uint32_t one; // qmax 7: nonzero when 7 does not divide the significand (r1 gives every code)
    uint32_t pad; // 32-byte entries: one scalar load each
};

template <int FB>
struct RowScaleTable {
    RowScaleEntry e[1 << FB];
};

namespace scale_table_detail {

constexpr float rne(float x)
{
    // round to the nearest integer, ties to even (|x| < 2^22)
    return x >= 0.0f ? (x + 12582912.0f) - 12582912.0f : -((-x + 12582912.0f) - 12582912.0f);
}

constexpr uint32_t bitrev32(uint32_t v)
{
    uint32_t r = 0;
    for (int i = 0; i < 32; ++i) r |= ((v >> i) & 1u) << (31 - i);
    return r;
}

}  // namespace scale_table_detail

// FB fraction bits (7: bf16, 10: fp16); QMAX 7 or 127
template <int FB, int QMAX>
constexpr RowScaleTable<FB> make_row_scale_table()
{
    using namespace scale_table_detail;
    RowScaleTable<FB> t{};
    for (int f = 0; f < (1 << FB); ++f) {
        const float an = 1.0f + (float)f / (float)(1 << FB);
        RowScaleEntry& e = t.e[f];
        e.s = an / (float)QMAX;
        e.rinv = 1.0f / e.s;
        e.rh = e.rinv * (1.0f + 1.0f / 2097152.0f);
        e.rl = e.rinv * (1.0f - 1.0f / 2097152.0f);
        uint32_t b = 0;
        for (int k = 0; k < 7; ++k) {
            const float h = (float)k + 0.5f;
            const float yh = (h * an) / 7.0f;
            const float qh = yh / e.s;
            if (rne(qh) > h) b |= 1u << k;
        }
        e.r1 = (b & 8u) ? e.rh : e.rl;
        const uint32_t sig = (uint32_t)((1 << FB) + f);
        e.tie = b | (bitrev32(b) << 1);
        e.one = sig % 7u != 0u ? 1u : 0u;
    }
    return t;
}

// Table key of a 16-bit absmax pattern a16 (bf16 when BF, else fp16): the
// fraction index of a = a_n * 2^E and E.  Returns false when the table does
// not cover a (zero, Inf, NaN, a < 2^-119: some shifted value would not be
// normal); fp16 subnormals are normalised first.
template <bool BF>
W4A4_HD inline bool row_scale_key(uint32_t a16, uint32_t& idx, int& E)
{
    if (BF) {
        const uint32_t eb = (a16 >> 7) & 0xffu;
        if (eb < 8u || eb == 0xffu) return false;
        idx = a16 & 0x7fu;
        E = (int)eb - 127;
        return true;
    }
    const uint32_t eb = (a16 >> 10) & 0x1fu, fr = a16 & 0x3ffu;
    if (eb == 0x1fu || (eb == 0u && fr == 0u)) return false;
    if (eb != 0u) {
        idx = fr;
        E = (int)eb - 15;
        return true;
    }
    const int p = 31 - __builtin_clz(fr);  // position of the subnormal fraction's top bit
    idx = (fr << (10 - p)) & 0x3ffu;
    E = p - 24;
    return true;
}

// v * 2^E for a normal v whose result is normal: an add to the exponent field
W4A4_HD inline float row_scale_shift(float v, int E)
{
    return __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, v) + ((uint32_t)E << 23));
}

}  // namespace w4a4
