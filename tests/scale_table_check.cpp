// Host check of the row-scale table (csrc/scale_table.hpp): for every 16-bit
// absmax pattern of both formats and both code ranges, the table's values
// shifted by the pattern's exponent must equal, bit for bit, what the row
// kernel computes with IEEE divisions when the table does not cover a row:
//   s = max(a / qmax, 2^-126), rinv = 1 / s, rh/rl = rinv * (1 +- 2^-21),
//   bit k of the tie mask: rint(fl(fl(fl((k + 1/2) * a) / 7) / s)) > k + 1/2
//   (at a 2^-64 scale for a > 2^64), and whether 7 divides a's significand.
// Built with g++ -ffp-contract=off (SSE arithmetic: every operation is one
// IEEE round-to-nearest-even rounding).  Prints the number of covered
// patterns per case; exits nonzero at the first mismatch.
#include <cmath>
#include <cstdio>
#include <cstring>

#include "scale_table.hpp"

using namespace w4a4;

static float bits_to_f(uint32_t u) { float f; std::memcpy(&f, &u, 4); return f; }
static uint32_t f_to_bits(float f) { uint32_t u; std::memcpy(&u, &f, 4); return u; }

static float f16_value(uint32_t h)
{
    const uint32_t e = (h >> 10) & 0x1f, m = h & 0x3ff;
    float v;
    if (e == 0) v = std::ldexp((float)m, -24);
    else if (e == 31) v = m ? NAN : INFINITY;
    else v = std::ldexp((float)(m | 0x400), (int)e - 25);
    return (h & 0x8000) ? -v : v;
}

struct Ref { float s, rinv, rh, rl; uint32_t tie, one; };

static Ref reference(float a, uint32_t sig, int qmax)
{
    Ref r;
    r.s = a / (float)qmax;
    if (r.s < 0x1p-126f) r.s = 0x1p-126f;
    r.rinv = 1.0f / r.s;
    r.rh = r.rinv * (1.0f + 0x1p-21f);
    r.rl = r.rinv * (1.0f - 0x1p-21f);
    uint32_t b = 0;
    for (int k = 0; k < 7; ++k) {
        const float h = (float)k + 0.5f;
        const bool big = a > 0x1p64f;
        const float ah = big ? a * 0x1p-64f : a;
        float yh = (h * ah) / 7.0f;
        if (big) yh *= 0x1p64f;
        const float qh = yh / r.s;
        if (std::rint(qh) > h) b |= 1u << k;
    }
    uint32_t rev = 0;
    for (int i = 0; i < 32; ++i) rev |= ((b >> i) & 1u) << (31 - i);
    r.tie = b | (rev << 1);
    r.one = sig % 7u != 0u;
    return r;
}

template <bool BF, int FB, int QMAX>
static int check(const RowScaleTable<FB>& tab, const char* name)
{
    int covered = 0;
    for (uint32_t a16 = 0; a16 < 0x8000u; ++a16) {
        uint32_t idx;
        int E;
        if (!row_scale_key<BF>(a16, idx, E)) continue;
        const float a = BF ? bits_to_f(a16 << 16) : f16_value(a16);
        const uint32_t sig = BF ? (((a16 >> 7) & 0xff) ? ((a16 & 0x7f) | 0x80) : (a16 & 0x7f))
                                : (((a16 >> 10) & 0x1f) ? ((a16 & 0x3ff) | 0x400) : (a16 & 0x3ff));
        const Ref r = reference(a, sig, QMAX);
        const RowScaleEntry& e = tab.e[idx];
        const float s = row_scale_shift(e.s, E), rinv = row_scale_shift(e.rinv, -E);
        const float rh = row_scale_shift(e.rh, -E), rl = row_scale_shift(e.rl, -E);
        bool ok = f_to_bits(s) == f_to_bits(r.s) && f_to_bits(rinv) == f_to_bits(r.rinv) &&
                  f_to_bits(rh) == f_to_bits(r.rh) && f_to_bits(rl) == f_to_bits(r.rl);
        if (QMAX == 7) {
            const float r1 = row_scale_shift(e.r1, -E);
            const float r1_ref = (r.tie & 8u) ? r.rh : r.rl;
            ok = ok && e.tie == r.tie && (e.one != 0) == (r.one != 0) && f_to_bits(r1) == f_to_bits(r1_ref);
        }
        if (!ok) {
            std::printf("%s: mismatch at pattern 0x%04x (a = %a): s %a/%a rinv %a/%a tie %08x/%08x\n", name, a16,
                        (double)a, (double)s, (double)r.s, (double)rinv, (double)r.rinv, e.tie, r.tie);
            return -1;
        }
        ++covered;
    }
    std::printf("%s: %d patterns covered, all equal\n", name, covered);
    return covered;
}

int main()
{
    static const RowScaleTable<7> bf7 = make_row_scale_table<7, 7>();
    static const RowScaleTable<7> bf127 = make_row_scale_table<7, 127>();
    static const RowScaleTable<10> h7 = make_row_scale_table<10, 7>();
    static const RowScaleTable<10> h127 = make_row_scale_table<10, 127>();
    if (check<true, 7, 7>(bf7, "bf16 qmax 7") < 0) return 1;
    if (check<true, 7, 127>(bf127, "bf16 qmax 127") < 0) return 1;
    if (check<false, 10, 7>(h7, "fp16 qmax 7") < 0) return 1;
    if (check<false, 10, 127>(h127, "fp16 qmax 127") < 0) return 1;
    return 0;
}
