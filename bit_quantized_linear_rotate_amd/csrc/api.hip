// Host side of the C ABI declared in include/w4a4.h: argument validation,
// status codes, the INT32 overflow guard, workspace layout and kernel
// selection.  No device allocation, no synchronisation.
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "../../include/w4a4.h"
#include "kernels.hpp"

using namespace w4a4;

namespace {

thread_local char g_err[512];

int fail(int code, const char* fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return code;
}

int hip_fail(hipError_t e, const char* where)
{
    return fail(W4A4_HIP_ERROR, "%s: %s", where, hipGetErrorString(e));
}

bool dtype_ok(int dt) { return dt == W4A4_F32 || dt == W4A4_F16 || dt == W4A4_BF16; }
size_t dsize(int dt) { return dt == W4A4_F32 ? 4 : 2; }
size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// Cached per device: is it gfx950?
int device_check()
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    static int cache[64];  // 0 unknown, 1 yes, 2 no
    if (dev >= 0 && dev < 64 && cache[dev]) {
        return cache[dev] == 1 ? W4A4_OK
                               : fail(W4A4_UNSUPPORTED, "device %d is not gfx950", dev);
    }
    hipDeviceProp_t p;
    e = hipGetDeviceProperties(&p, dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
    const bool ok = strncmp(p.gcnArchName, "gfx950", 6) == 0;
    if (dev >= 0 && dev < 64) cache[dev] = ok ? 1 : 2;
    return ok ? W4A4_OK : fail(W4A4_UNSUPPORTED, "device %d is %s, not gfx950", dev, p.gcnArchName);
}

bool pow2_g(int g) { return g == 16 || g == 32 || g == 64 || g == 128 || g == 256; }

int check_activation(const void* x, int dt, int64_t M, int64_t K, int64_t sm, int64_t sk)
{
    if (M < 0 || K < 0) return fail(W4A4_INVALID, "negative size M=%lld K=%lld", (long long)M, (long long)K);
    if (sm < 0 || sk < 0) return fail(W4A4_INVALID, "negative stride");
    if (!dtype_ok(dt)) return fail(W4A4_UNSUPPORTED, "unknown activation dtype %d", dt);
    if (K % 2) return fail(W4A4_INVALID, "K=%lld is odd: INT4 rows need an even width", (long long)K);
    if (M > 0 && K > 0 && !x) return fail(W4A4_INVALID, "x is NULL");
    return W4A4_OK;
}

int rq_validate(const void* x, int dt, int64_t M, int64_t K, int64_t sm, int64_t sk, const float* rot,
                int g, int8_t* codes, float* scales)
{
    int rc = check_activation(x, dt, M, K, sm, sk);
    if (rc) return rc;
    if (rot) {
        if (g <= 0) return fail(W4A4_INVALID, "group size g=%d", g);
        if (K % g) return fail(W4A4_INVALID, "K=%lld is not a multiple of g=%d", (long long)K, g);
        if (!pow2_g(g)) return fail(W4A4_UNSUPPORTED, "g=%d is not a power of two in [16, 256]", g);
    }
    if (M > 0 && (!codes || !scales)) return fail(W4A4_INVALID, "codes/scales is NULL");
    if (M > 0 && K == 0) return fail(W4A4_INVALID, "K=0 with M>0");
    return W4A4_OK;
}

int64_t guard_chunk(int64_t K) { return K > kGemmMaxK ? kGemmMaxK : 0; }

int gemm_validate(const int8_t* codes, const float* scales, int64_t M, int64_t K, const uint8_t* wp,
                  int64_t N, const void* sw, int sw_dt, int sw_group, const void* bias, int bias_dt,
                  const float* lora, const void* up, int up_dt, int rank, void* out, int out_dt,
                  int64_t k_chunk)
{
    if (M < 0 || K < 0 || N < 0) return fail(W4A4_INVALID, "negative size");
    if (K % 2) return fail(W4A4_INVALID, "K=%lld is odd", (long long)K);
    if (!dtype_ok(sw_dt) || !dtype_ok(out_dt) || (bias && !dtype_ok(bias_dt)) ||
        (up && !dtype_ok(up_dt)))
        return fail(W4A4_UNSUPPORTED, "unknown dtype code");
    if (sw_group != 0 && sw_group != 64) return fail(W4A4_INVALID, "w_scale_group must be 0 or 64");
    if (sw_group == 64 && K % 64) return fail(W4A4_INVALID, "K %% 64 != 0 with per-64-group scales");
    if ((lora == nullptr) != (up == nullptr)) return fail(W4A4_INVALID, "lora_act and proj_up go together");
    if (lora && (rank < 1 || rank > 64)) return fail(W4A4_INVALID, "rank=%d outside [1, 64]", rank);
    if (k_chunk < 0 || (k_chunk > 0 && k_chunk % 64))
        return fail(W4A4_INVALID, "k_chunk must be 0 or a positive multiple of 64");
    if (k_chunk > kGemmMaxK) return fail(W4A4_INVALID, "k_chunk exceeds the INT32-safe length");
    if (k_chunk > 0 && sw_group) return fail(W4A4_INVALID, "k_chunk applies to per-channel scales only");
    if (M > 0 && N > 0) {
        if (!scales || !wp || !sw || !out || (K > 0 && !codes))
            return fail(W4A4_INVALID, "a required pointer is NULL");
    }
    return W4A4_OK;
}

}  // namespace

extern "C" {

const char* w4a4_last_error(void) { return g_err; }

int w4a4_device_supported(void) { return device_check(); }

int w4a4_int32_guard(int64_t K, int64_t* k_chunk)
{
    const int64_t c = K > 0 ? guard_chunk(K) : 0;
    if (k_chunk) *k_chunk = c;
    return c > 0 ? 1 : 0;
}

int w4a4_rotate_quant_rowwise(const void* x, int x_dtype, int64_t M, int64_t K, int64_t stride_m,
                              int64_t stride_k, const float* rot, int32_t g, const void* smooth,
                              int8_t* codes, float* scales, void* rotated_out, void* stream)
{
    int rc = rq_validate(x, x_dtype, M, K, stride_m, stride_k, rot, g, codes, scales);
    if (rc) return rc;
    if (M == 0) return W4A4_OK;
    rc = device_check();
    if (rc) return rc;
    RQArgs a{x, x_dtype, M, K, stride_m, stride_k, rot, rot ? g : 0, smooth, codes, scales, rotated_out};
    int path = 0;
    hipError_t e = launch_rotate_quant(a, (hipStream_t)stream, &path);
    if (e == hipErrorNotSupported)
        return fail(W4A4_UNSUPPORTED, "no rotate_quant kernel for this shape (K=%lld)", (long long)K);
    if (e != hipSuccess) return hip_fail(e, "rotate_quant launch");
    return W4A4_OK;
}

int w4a4_lowrank_down(const void* x, int x_dtype, int64_t M, int64_t K, int64_t stride_m,
                      int64_t stride_k, const void* proj_down, int32_t rank, float* lora_act,
                      void* stream)
{
    int rc = check_activation(x, x_dtype, M, K, stride_m, stride_k);
    if (rc) return rc;
    if (rank < 1 || rank > 64) return fail(W4A4_INVALID, "rank=%d outside [1, 64]", rank);
    if (M > 0 && (!proj_down || !lora_act)) return fail(W4A4_INVALID, "proj_down/lora_act is NULL");
    if (M == 0) return W4A4_OK;
    rc = device_check();
    if (rc) return rc;
    LowRankArgs a{x, x_dtype, M, K, stride_m, stride_k, proj_down, rank, lora_act};
    hipError_t e = launch_lowrank_down(a, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "lowrank_down launch");
    return W4A4_OK;
}

size_t w4a4_gemm_workspace_size(int64_t M, int64_t N, int64_t K, int64_t k_chunk)
{
    if (M <= 0 || N <= 0) return 0;
    const int64_t kc = k_chunk > 0 ? k_chunk : guard_chunk(K);
    return kc > 0 ? align256((size_t)M * (size_t)N * 8) : 0;
}

int w4a4_gemm_from_codes(const int8_t* codes, const float* scales, int64_t M, int64_t K,
                         const uint8_t* w_packed, int64_t N, const void* w_scale,
                         int w_scale_dtype, int32_t w_scale_group, const void* bias,
                         int bias_dtype, const float* lora_act, const void* proj_up,
                         int up_dtype, int32_t rank, void* out, int out_dtype,
                         int32_t* acc_out, int64_t k_chunk, void* workspace,
                         size_t workspace_bytes, void* stream)
{
    int rc = gemm_validate(codes, scales, M, K, w_packed, N, w_scale, w_scale_dtype, w_scale_group,
                           bias, bias_dtype, lora_act, proj_up, up_dtype, rank, out, out_dtype,
                           k_chunk);
    if (rc) return rc;
    if (M == 0 || N == 0) return W4A4_OK;
    const int64_t kc = k_chunk > 0 ? k_chunk : (w_scale_group ? 0 : guard_chunk(K));
    const size_t need = kc > 0 ? align256((size_t)M * (size_t)N * 8) : 0;
    if (workspace_bytes < need || (need && !workspace))
        return fail(W4A4_INVALID, "workspace of %zu bytes, need %zu", workspace_bytes, need);
    rc = device_check();
    if (rc) return rc;
    GemmArgs a{codes, scales, M, K, N, w_packed, w_scale, w_scale_dtype, w_scale_group,
               bias, bias_dtype, lora_act, proj_up, up_dtype, lora_act ? rank : 0,
               out, out_dtype, acc_out, kc, (int64_t*)workspace};
    hipError_t e = launch_gemm(a, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "gemm launch");
    return W4A4_OK;
}

size_t w4a4_linear_workspace_size(int64_t M, int64_t K, int64_t N, int32_t rank)
{
    if (M <= 0) return 0;
    size_t s = align256((size_t)M * (size_t)K);            // codes
    s += align256((size_t)M * 4);                          // scales
    if (rank > 0) s += align256((size_t)M * rank * 4);     // lora_act
    const int64_t kc = guard_chunk(K);
    if (kc > 0 && N > 0) s += align256((size_t)M * (size_t)N * 8);
    return s;
}

int w4a4_linear(const void* x, int x_dtype, int64_t M, int64_t K, int64_t stride_m,
                int64_t stride_k, const float* rot, int32_t g, const void* smooth,
                const uint8_t* w_packed, int64_t N, const void* w_scale, int w_scale_dtype,
                int32_t w_scale_group, const void* bias, const void* proj_down,
                const void* proj_up, int32_t rank, void* out, int out_dtype, void* workspace,
                size_t workspace_bytes, void* stream)
{
    // Validate everything before the first launch.
    int8_t* codes = nullptr;
    int rc = rq_validate(x, x_dtype, M, K, stride_m, stride_k, rot, g, (int8_t*)1, (float*)1);
    if (rc) return rc;
    if ((proj_down == nullptr) != (proj_up == nullptr))
        return fail(W4A4_INVALID, "proj_down and proj_up go together");
    const int r = proj_down ? rank : 0;
    if (proj_down && (rank < 1 || rank > 64)) return fail(W4A4_INVALID, "rank=%d outside [1, 64]", rank);
    const float* fake_lora = r ? (const float*)1 : nullptr;
    rc = gemm_validate((const int8_t*)1, (const float*)1, M, K, w_packed, N, w_scale, w_scale_dtype,
                       w_scale_group, bias, x_dtype, fake_lora, proj_up, x_dtype, r, out, out_dtype, 0);
    if (rc) return rc;
    if (M == 0 || N == 0) return W4A4_OK;
    const size_t need = w4a4_linear_workspace_size(M, K, N, r);
    if (!workspace || workspace_bytes < need)
        return fail(W4A4_INVALID, "workspace of %zu bytes, need %zu", workspace_bytes, need);
    rc = device_check();
    if (rc) return rc;

    uint8_t* ws = (uint8_t*)workspace;
    codes = (int8_t*)ws;
    ws += align256((size_t)M * (size_t)K);
    float* scales = (float*)ws;
    ws += align256((size_t)M * 4);
    float* lora = nullptr;
    if (r) {
        lora = (float*)ws;
        ws += align256((size_t)M * r * 4);
    }
    const int64_t kc = w_scale_group ? 0 : guard_chunk(K);
    int64_t* acc64 = kc > 0 ? (int64_t*)ws : nullptr;
    hipStream_t st = (hipStream_t)stream;

    hipError_t e;
    if (r) {
        LowRankArgs la{x, x_dtype, M, K, stride_m, stride_k, proj_down, r, lora};
        e = launch_lowrank_down(la, st);
        if (e != hipSuccess) return hip_fail(e, "lowrank_down launch");
    }
    RQArgs qa{x, x_dtype, M, K, stride_m, stride_k, rot, rot ? g : 0, smooth, codes, scales, nullptr};
    int path = 0;
    e = launch_rotate_quant(qa, st, &path);
    if (e == hipErrorNotSupported)
        return fail(W4A4_UNSUPPORTED, "no rotate_quant kernel for this shape (K=%lld)", (long long)K);
    if (e != hipSuccess) return hip_fail(e, "rotate_quant launch");
    GemmArgs ga{codes, scales, M, K, N, w_packed, w_scale, w_scale_dtype, w_scale_group,
                bias, x_dtype, lora, proj_up, x_dtype, r, out, out_dtype, nullptr, kc, acc64};
    e = launch_gemm(ga, st);
    if (e != hipSuccess) return hip_fail(e, "gemm launch");
    return W4A4_OK;
}

}  // extern "C"
