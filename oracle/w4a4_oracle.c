/*
 * CPU oracle for the ConvRot-style W4A4 linear layer.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously-correct
 * reference that the GPU path is checked against.  Only the tests, the smoke
 * check and the benchmark's CPU-baseline leg may load it; the product path
 * (the HIP library and its Python binding) never does, and shares no code,
 * header, table or helper with it.
 *
 * Sources (web pages, cited by title and section):
 *   [P1] "[Feat][Ascend] Consolidate INT8, RotateQuant, RoPE and ConvRot W4A4
 *        backends" (comfy-kitchen PR #198), section "W4A4 correctness and
 *        performance scope".
 *   [P2] "[Perf][Ascend] Avoid activation pack/unpack in ConvRot W4A4"
 *        (PR #201), sections "Summary" and "Correctness and tests".
 *   [P3] "[Feat][Ascend] Add fused RotateQuant backend" (PR #155), sections
 *        "What this PR does / why we need it", "How was this patch tested?"
 *        and the review comment on zero scales.
 *   [P4] source page comfy_kitchen/tensor/svdquant_w4a4.py: module docstring
 *        (tensor shapes) and the _w4a4_forward docstring (low-rank branch).
 *
 * Floating point: every step that the method leaves to "a matmul" is done in
 * fp64 and rounded once; steps that the readings fix in fp32 (scale,
 * quotient, epilogue) are done in IEEE binary32.  Build with
 * -ffp-contract=off -fno-fast-math so that no multiply-add is fused.
 *
 * Readings of points the pages leave open (R1..R19) are stated at each step.
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_F32 = 0, ORC_F16 = 1, ORC_BF16 = 2 };

/* ------------------------------------------------------------------------ */
/* Number formats.                                                           */
/* ------------------------------------------------------------------------ */

/* Round v to the nearest value of a binary format with p significand bits,
 * smallest normal 2^emin and largest finite (2 - 2^(1-p)) * 2^emax, ties to
 * even, overflow to infinity.  The scaling by powers of two is exact in
 * double, so the only rounding is the nearbyint() (round-half-even in the
 * default rounding mode). */
static double round_format(double v, int p, int emin, int emax)
{
    if (isnan(v) || isinf(v) || v == 0.0) return v;
    int e;
    (void)frexp(v, &e); /* |v| in [2^(e-1), 2^e) */
    int top = e - 1;
    if (top < emin) top = emin; /* subnormal range: fixed quantum */
    int q_exp = top - (p - 1);
    double r = ldexp(nearbyint(ldexp(v, -q_exp)), q_exp);
    double maxf = ldexp(2.0 - ldexp(1.0, 1 - p), emax);
    if (fabs(r) > maxf) return copysign(INFINITY, v);
    return r;
}

static double round_to(int dt, double v)
{
    switch (dt) {
    case ORC_F32: return round_format(v, 24, -126, 127);
    case ORC_F16: return round_format(v, 11, -14, 15);
    default: return round_format(v, 8, -126, 127);
    }
}

static double decode_f16(uint16_t b)
{
    int s = b >> 15, ex = (b >> 10) & 31, m = b & 1023;
    double v;
    if (ex == 0) v = ldexp((double)m, -24);
    else if (ex == 31) v = m ? NAN : INFINITY;
    else v = ldexp((double)(1024 + m), ex - 25);
    return s ? -v : v;
}

/* v must already be representable in binary16 (or be Inf/NaN). */
static uint16_t encode_f16(double v)
{
    uint16_t s = signbit(v) ? 0x8000 : 0;
    if (isnan(v)) return 0x7E00;
    if (isinf(v)) return s | 0x7C00;
    double a = fabs(v);
    if (a == 0.0) return s;
    int e;
    double f = frexp(a, &e); /* a = f * 2^e, f in [0.5,1) */
    int ex = e - 1 + 15;
    if (ex >= 1) return s | (uint16_t)(ex << 10) | (uint16_t)(f * 2048.0 - 1024.0);
    return s | (uint16_t)ldexp(a, 24); /* subnormal: multiple of 2^-24 */
}

static double load_T(int dt, const void *p, int64_t i)
{
    if (dt == ORC_F32) return (double)((const float *)p)[i];
    uint16_t b = ((const uint16_t *)p)[i];
    if (dt == ORC_F16) return decode_f16(b);
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* v must already be representable in T (or be Inf/NaN). */
static void store_T(int dt, void *p, int64_t i, double v)
{
    if (dt == ORC_F32) { ((float *)p)[i] = (float)v; return; }
    if (dt == ORC_F16) { ((uint16_t *)p)[i] = encode_f16(v); return; }
    if (isnan(v)) { ((uint16_t *)p)[i] = 0x7FC0; return; }
    float f = (float)v;
    uint32_t u;
    memcpy(&u, &f, 4);
    ((uint16_t *)p)[i] = (uint16_t)(u >> 16);
}

/* Exposed for the pins: round an array of doubles to T and return the values
 * (as doubles) and the stored bit patterns. */
int orc_round_to(int dt, const double *v, int64_t n, double *out_val, void *out_bits)
{
    for (int64_t i = 0; i < n; ++i) {
        double r = round_to(dt, v[i]);
        if (out_val) out_val[i] = r;
        if (out_bits) store_T(dt, out_bits, i, r);
    }
    return 0;
}

int orc_decode(int dt, const void *bits, int64_t n, double *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = load_T(dt, bits, i);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* a1  Input-side smoothing ([P4] module docstring: smooth_factor (K,)).     */
/* Reading R3: divide the activation by the factor, one IEEE fp32 division,  */
/* then round to the activation dtype T.                                     */
/* ------------------------------------------------------------------------ */
int orc_smooth(int dt, const void *x, int64_t M, int64_t K, const void *smooth, void *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t k = 0; k < K; ++k) {
            float xv = (float)load_T(dt, x, m * K + k);
            float sv = (float)load_T(dt, smooth, k);
            float q = xv / sv;
            store_T(dt, out, m * K + k, round_to(dt, (double)q));
        }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* a2  Block-diagonal rotation ([P1] W4A4 scope: rotation keeps the          */
/* activation dtype; [P3] tested with group sizes 16/64/256 and asymmetric   */
/* rotations).                                                               */
/* Readings R1/R2: each group of g consecutive entries of a row is a row     */
/* vector multiplied on the right by R:  y_j = sum_i x_i * R[i][j].  R is    */
/* first rounded to T; the exact products are summed in fp64 and the sum is  */
/* rounded once to T.                                                        */
/* ------------------------------------------------------------------------ */
int orc_rotate(int dt, const void *x, int64_t M, int64_t K, const double *R, int g, void *y)
{
    if (g <= 0 || K % g) return -1;
    if (g > 256) return -1;
    double *rt = (double *)malloc(sizeof(double) * g * g);
    if (!rt) return -2;
    for (int i = 0; i < g * g; ++i) rt[i] = round_to(dt, R[i]);
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        double xs[256];
        for (int64_t b = 0; b < K / g; ++b) {
            for (int i = 0; i < g; ++i) xs[i] = load_T(dt, x, m * K + b * g + i);
            for (int j = 0; j < g; ++j) {
                double acc = 0.0;
                for (int i = 0; i < g; ++i) acc += xs[i] * rt[i * g + j];
                store_T(dt, y, m * K + b * g + j, round_to(dt, acc));
            }
        }
    }
    free(rt);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* a3/a4  Per-row symmetric quantizer with codes kept in INT8 storage        */
/* ([P1] W4A4 scope: the reference signed-INT4 quantizer; [P2] Summary: the  */
/* same codes stay in INT8 storage; [P3] zero scales are replaced by the     */
/* finite minimum before division, public scales stay positive).             */
/* Readings R4/R5: a = max |y| over the row in fp32 (a NaN anywhere makes    */
/* the scale NaN); s = a / qmax in IEEE fp32; s below the smallest normal    */
/* fp32 becomes 2^-126.  q = y / s (IEEE fp32 division, not a reciprocal     */
/* multiply); code = clamp(round-half-even(q), -qmax, qmax); a NaN quotient  */
/* gives code 0.  qmax = 7 for the INT4 codes of the W4A4 layer; qmax = 127  */
/* for the INT8 mode of the fused RotateQuant of [P3] "What this PR does"    */
/* (reading R16: the same rule on the symmetric INT8 grid, -128 unused).     */
/* ------------------------------------------------------------------------ */
int orc_quantize_q(int dt, const void *y, int64_t M, int64_t K, int qmax, int8_t *codes, float *scales)
{
    if (qmax != 7 && qmax != 127) return 1;
    const float fq = (float)qmax;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        float a = 0.0f;
        int nan_row = 0;
        for (int64_t k = 0; k < K; ++k) {
            float v = (float)load_T(dt, y, m * K + k);
            if (isnan(v)) nan_row = 1;
            else if (fabsf(v) > a) a = fabsf(v);
        }
        float s;
        if (nan_row) s = NAN;
        else {
            s = a / fq;
            if (s < FLT_MIN) s = FLT_MIN; /* 2^-126 */
        }
        scales[m] = s;
        for (int64_t k = 0; k < K; ++k) {
            float v = (float)load_T(dt, y, m * K + k);
            float q = v / s;
            int8_t c = 0;
            if (!isnan(q)) {
                float r = nearbyintf(q);
                if (r > fq) r = fq;
                if (r < -fq) r = -fq;
                c = (int8_t)r;
            }
            codes[m * K + k] = c;
        }
    }
    return 0;
}

int orc_quantize(int dt, const void *y, int64_t M, int64_t K, int8_t *codes, float *scales)
{
    return orc_quantize_q(dt, y, M, K, 7, codes, scales);
}

/* ------------------------------------------------------------------------ */
/* SVDQuant activation quantizer ([P4] _w4a4_forward docstring: post-GELU    */
/* layers flagged act_unsigned add the shift 0.171875 to the main-path       */
/* activation so that it falls into the unsigned [0, 15] grid; the low-rank  */
/* branch keeps the raw activation; module docstring: INT4 group size 64).   */
/* Reading R18: the shifted activation is T(fp32(x) + 0.171875), one fp32    */
/* add rounded to T, as an elementwise add of a scalar to a T tensor.        */
/* ------------------------------------------------------------------------ */
int orc_shift(int dt, const void *x, int64_t M, int64_t K, double c, void *out)
{
    const float fc = (float)c;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t k = 0; k < K; ++k) {
            float v = (float)load_T(dt, x, m * K + k) + fc;
            store_T(dt, out, m * K + k, round_to(dt, (double)v));
        }
    return 0;
}

/* Readings R18/R19: the quantizer of a3/a4 applied to each block of `group`  */
/* consecutive entries of a row (group = 0: the whole row), scales (M, K /   */
/* group) row-major (or (M,)).  Signed: s = max(absmax / 7, 2^-126), codes   */
/* clamp(rne(y / s), -7, 7).  Unsigned grid: s = max(absmax / 15, 2^-126),   */
/* codes clamp(rne(y / s), 0, 15) (a value below zero gives 0).  NaN in a    */
/* block makes its scale NaN and a NaN quotient gives code 0, as in a4.      */
/* ------------------------------------------------------------------------ */
int orc_quantize_ex(int dt, const void *y, int64_t M, int64_t K, int is_unsigned, int group,
                    int8_t *codes, float *scales)
{
    if (group < 0 || (group > 0 && K % group)) return 1;
    const int64_t glen = group > 0 ? group : K;
    const int64_t G = group > 0 ? K / group : 1;
    const float fq = is_unsigned ? 15.0f : 7.0f;
    const float lo = is_unsigned ? 0.0f : -7.0f;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t gi = 0; gi < G; ++gi) {
            const int64_t k0 = gi * glen;
            float a = 0.0f;
            int nan_blk = 0;
            for (int64_t k = k0; k < k0 + glen; ++k) {
                float v = (float)load_T(dt, y, m * K + k);
                if (isnan(v)) nan_blk = 1;
                else if (fabsf(v) > a) a = fabsf(v);
            }
            float s;
            if (nan_blk) s = NAN;
            else {
                s = a / fq;
                if (s < FLT_MIN) s = FLT_MIN;
            }
            scales[m * G + gi] = s;
            for (int64_t k = k0; k < k0 + glen; ++k) {
                float q = (float)load_T(dt, y, m * K + k) / s;
                int8_t c = 0;
                if (!isnan(q)) {
                    float r = nearbyintf(q);
                    if (r > fq) r = fq;
                    if (r < lo) r = lo;
                    c = (int8_t)r;
                }
                codes[m * K + k] = c;
            }
        }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* a6  Weight nibble unpack ([P1] W4A4 scope: the W4 codes are unpacked to   */
/* INT8; [P4] module docstring: qweight is (N, K/2) packed).                 */
/* Reading R6: byte j of a row holds k = 2j in its low nibble and k = 2j+1   */
/* in its high nibble, each a 4-bit two's-complement value (0x8 = -8).       */
/* ------------------------------------------------------------------------ */
static int sext4(unsigned v) { return (v & 8u) ? (int)v - 16 : (int)v; }

int orc_unpack(const uint8_t *wp, int64_t N, int64_t K, int8_t *w)
{
    if (K % 2) return -1;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t j = 0; j < K / 2; ++j) {
            uint8_t b = wp[n * (K / 2) + j];
            w[n * K + 2 * j] = (int8_t)sext4(b & 15u);
            w[n * K + 2 * j + 1] = (int8_t)sext4(b >> 4);
        }
    return 0;
}

/* Inverse of orc_unpack (a test utility: builds packed weights from codes in
 * [-8, 7]).  Returns -1 on a code outside that range. */
int orc_pack(const int8_t *w, int64_t N, int64_t K, uint8_t *wp)
{
    if (K % 2) return -1;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t j = 0; j < K / 2; ++j) {
            int lo = w[n * K + 2 * j], hi = w[n * K + 2 * j + 1];
            if (lo < -8 || lo > 7 || hi < -8 || hi > 7) return -1;
            wp[n * (K / 2) + j] = (uint8_t)((lo & 15) | ((hi & 15) << 4));
        }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* a7  Exact integer GEMM ([P1] W4A4 scope: INT8 codes multiplied with unit  */
/* scale and no per-token scale, accumulated in INT32).  Reading R7/R8: the  */
/* oracle sums in int64, which is the exact value whatever chunking the GPU  */
/* uses to keep its INT32 accumulators from overflowing.                     */
/* acc[m][n] = sum_k c[m][k] * w[n][k].                                      */
/* If group > 0, acc is (M, K/group, N): one partial sum per K-group.        */
/* ------------------------------------------------------------------------ */
int orc_gemm(const int8_t *c, int64_t M, int64_t K, const int8_t *w, int64_t N,
             int group, int64_t *acc)
{
    int64_t G = group > 0 ? K / group : 1;
    int64_t glen = group > 0 ? group : K;
    if (group > 0 && K % group) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t gi = 0; gi < G; ++gi)
            for (int64_t n = 0; n < N; ++n) {
                int64_t s = 0;
                for (int64_t k = gi * glen; k < (gi + 1) * glen; ++k)
                    s += (int64_t)c[m * K + k] * (int64_t)w[n * K + k];
                acc[(m * G + gi) * N + n] = s;
            }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* a5  Low-rank down projection ([P4] _w4a4_forward docstring: the low-rank  */
/* branch sees the raw, unsmoothed, unrotated activation).  Reading R11:     */
/* L[m][r] = fp32( sum_k x[m][k] * down[k][r] ), summed in fp64.             */
/* ------------------------------------------------------------------------ */
int orc_lowrank_down(int dt, const void *x, int64_t M, int64_t K, const void *down, int R,
                     float *L)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int r = 0; r < R; ++r) {
            double s = 0.0;
            for (int64_t k = 0; k < K; ++k) s += load_T(dt, x, m * K + k) * load_T(dt, down, k * R + r);
            L[m * R + r] = (float)round_to(ORC_F32, s);
        }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* a9  Epilogue ([P1] W4A4 scope: cast, then activation scale, weight scale  */
/* and bias in eager's order; no FP16 intermediate for FP32/BF16 outputs).   */
/* Reading R9 (order E-B): t = fp32(acc); t = t * s_a; t = t * s_w;          */
/* [t = t + l]; [t = t + bias]; out = round-half-even to the output dtype.   */
/* Each is a separately rounded fp32 operation (no fused multiply-add).      */
/* Reading R10 (per-64-group weight scales, [P4] module docstring):          */
/* t = sum over groups in increasing K order of fp32(acc_G) * s_w[G][n],     */
/* each product and each sum rounded in fp32; then t = t * s_a; the         */
/* low-rank term l and the bias follow as above.                             */
/* Reading R11: l[m][n] = fp32( sum_r L[m][r] * up[n][r] ) summed in fp64.   */
/*                                                                           */
/* acc: (M, N) int64 when group == 0, (M, K/group, N) when group > 0.        */
/* sw:  (N,) in sw_dt when group == 0, (K/group, N) when group > 0.          */
/* bias (N,) in bias_dt or NULL; L (M,R) fp32 and up (N,R) in up_dt or NULL. */
/* ------------------------------------------------------------------------ */
int orc_epilogue(const int64_t *acc, int64_t M, int64_t N, int64_t G, int group,
                 const float *sa, const void *sw, int sw_dt, const void *bias, int bias_dt,
                 const float *L, const void *up, int up_dt, int R, void *out, int out_dt)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            float t;
            if (group > 0) {
                t = 0.0f;
                for (int64_t gi = 0; gi < G; ++gi) {
                    float a = (float)round_to(ORC_F32, (double)acc[(m * G + gi) * N + n]);
                    float p = a * (float)load_T(sw_dt, sw, gi * N + n);
                    t = t + p;
                }
                t = t * sa[m];
            } else {
                t = (float)round_to(ORC_F32, (double)acc[m * N + n]);
                t = t * sa[m];
                t = t * (float)load_T(sw_dt, sw, n);
            }
            if (L && up) {
                double s = 0.0;
                for (int r = 0; r < R; ++r) s += (double)L[m * R + r] * load_T(up_dt, up, (int64_t)n * R + r);
                float l = (float)round_to(ORC_F32, s);
                t = t + l;
            }
            if (bias) t = t + (float)load_T(bias_dt, bias, n);
            store_T(out_dt, out, m * N + n, round_to(out_dt, (double)t));
        }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Epilogue with per-group activation scales (reading R19, [P4]: the SVDQuant */
/* kernel takes activation scales `ascales` with the INT4 group size 64).    */
/* acc (M, G, N) per-group sums; sa (M, G).  With per-group weight scales:   */
/* t = sum over G in increasing K order of (fp32(acc_G) * sa[m][G]) *        */
/* sw[G][n]; with per-channel weight scales: t = (sum over G of fp32(acc_G)  */
/* * sa[m][G]) * sw[n].  Each product and sum is a separately rounded fp32   */
/* operation; the low-rank term and the bias follow as in the epilogue above. */
/* ------------------------------------------------------------------------ */
int orc_epilogue_ag(const int64_t *acc, int64_t M, int64_t N, int64_t G, const float *sa,
                    const void *sw, int sw_dt, int sw_group, const void *bias, int bias_dt,
                    const float *L, const void *up, int up_dt, int R, void *out, int out_dt)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            float t = 0.0f;
            for (int64_t gi = 0; gi < G; ++gi) {
                float a = (float)round_to(ORC_F32, (double)acc[(m * G + gi) * N + n]);
                float p = a * sa[m * G + gi];
                if (sw_group > 0) p = p * (float)load_T(sw_dt, sw, gi * N + n);
                t = t + p;
            }
            if (sw_group == 0) t = t * (float)load_T(sw_dt, sw, n);
            if (L && up) {
                double s = 0.0;
                for (int r = 0; r < R; ++r) s += (double)L[m * R + r] * load_T(up_dt, up, (int64_t)n * R + r);
                float l = (float)round_to(ORC_F32, s);
                t = t + l;
            }
            if (bias) t = t + (float)load_T(bias_dt, bias, n);
            store_T(out_dt, out, m * N + n, round_to(out_dt, (double)t));
        }
    return 0;
}

int orc_num_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}
