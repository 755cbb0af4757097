// Host side of the C ABI declared in include/w4a4.h: argument validation,
// status codes, the INT32 overflow guard, workspace layout and kernel
// selection.  No device allocation, no synchronisation.
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

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

int check_activation(const void* x, int dt, int64_t M, int64_t K, int64_t sm, int64_t sk, bool int4 = true)
{
    if (M < 0 || K < 0) return fail(W4A4_INVALID, "negative size M=%lld K=%lld", (long long)M, (long long)K);
    if (sm < 0 || sk < 0) return fail(W4A4_INVALID, "negative stride");
    if (!dtype_ok(dt)) return fail(W4A4_UNSUPPORTED, "unknown activation dtype %d", dt);
    if (int4 && K % 2) return fail(W4A4_INVALID, "K=%lld is odd: INT4 rows need an even width", (long long)K);
    if (M > 0 && K > 0 && !x) return fail(W4A4_INVALID, "x is NULL");
    return W4A4_OK;
}

int rq_validate_g(const void* x, int dt, int64_t M, int64_t K, int64_t sm, int64_t sk, bool rotated,
                  int g, int8_t* codes, float* scales, bool int4)
{
    int rc = check_activation(x, dt, M, K, sm, sk, int4);
    if (rc) return rc;
    if (rotated) {
        if (g <= 0) return fail(W4A4_INVALID, "group size g=%d", g);
        if (K % g) return fail(W4A4_INVALID, "K=%lld is not a multiple of g=%d", (long long)K, g);
        if (!pow2_g(g)) return fail(W4A4_UNSUPPORTED, "g=%d is not a power of two in [16, 256]", g);
    }
    if (M > 0 && (!codes || !scales)) return fail(W4A4_INVALID, "codes/scales is NULL");
    if (M > 0 && K == 0) return fail(W4A4_INVALID, "K=0 with M>0");
    return W4A4_OK;
}

int rq_validate(const void* x, int dt, int64_t M, int64_t K, int64_t sm, int64_t sk, const float* rot,
                int g, int8_t* codes, float* scales, bool int4 = true)
{
    return rq_validate_g(x, dt, M, K, sm, sk, rot != nullptr, g, codes, scales, int4);
}

// the rotate-quant arguments of a structured (Hadamard) rotation
RQArgs hadamard_args(const void* x, int x_dtype, int64_t M, int64_t K, int64_t sm, int64_t sk, int32_t g,
                     const int8_t* sign_in, const int8_t* sign_out, const void* smooth, int qmax,
                     int8_t* codes, float* scales, void* rotated_out)
{
    RQArgs a{x, x_dtype, M, K, sm, sk, nullptr, g, smooth, codes, scales, rotated_out};
    a.qmax = qmax;
    a.hadamard = 1;
    a.sign_in = sign_in;
    a.sign_out = sign_out;
    return a;
}

int64_t guard_chunk(int64_t K) { return K > kGemmMaxK ? kGemmMaxK : 0; }
int64_t guard_chunk8(int64_t K) { return K > kGemmMaxK8 ? kGemmMaxK8 : 0; }

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

// Scratch of w4a4_linear_noalloc: the codes, scales, low-rank activations
// and (for very long K) int64 partial sums of one call.  Each GPU the library
// runs on holds its own copy, allocated with the code object and kept until
// the process ends; host code reaches it only through the device address
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) uint8_t scratch[W4A4_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
void* g_scratch_dev[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of the current device's scratch, looked up once per device
// (with that device current) and kept.
int scratch_address(void** ptr)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(W4A4_UNSUPPORTED, "device index %d", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (!p) return fail(W4A4_HIP_ERROR, "hipGetSymbolAddress(scratch) returned NULL");
        g_scratch_dev[dev] = p;
    }
    *ptr = g_scratch_dev[dev];
    return W4A4_OK;
}

// w4a4_linear given its rotate-quant arguments (x, shape, rotation,
// smoothing; codes and scales are placed in the workspace here)
int linear4_impl(RQArgs qa, bool rotated, const uint8_t* w_packed, int64_t N, const void* w_scale,
                 int w_scale_dtype, int32_t w_scale_group, const void* bias, const void* proj_down,
                 const void* proj_up, int32_t rank, void* out, int out_dtype, void* workspace,
                 size_t workspace_bytes, void* stream)
{
    const int64_t M = qa.M, K = qa.K;
    const int x_dtype = qa.dtype;
    // Validate everything before the first launch.
    int rc = rq_validate_g(qa.x, x_dtype, M, K, qa.sm, qa.sk, rotated, qa.g, (int8_t*)1, (float*)1, true);
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
    int8_t* codes = (int8_t*)ws;
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

    // decide every launch before the first one, so that a call that is
    // refused leaves nothing enqueued
    qa.codes = codes;
    qa.scales = scales;
    qa.yout = nullptr;
    if (rotate_quant_path(qa) < 0)
        return fail(W4A4_UNSUPPORTED, "no rotate_quant kernel for this shape (K=%lld)", (long long)K);
    hipError_t e;
    if (r) {
        LowRankArgs la{qa.x, x_dtype, M, K, qa.sm, qa.sk, proj_down, r, lora};
        e = launch_lowrank_down(la, st);
        if (e != hipSuccess) return hip_fail(e, "lowrank_down launch");
    }
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

size_t w8_workspace(int64_t M, int64_t K, int64_t N)
{
    if (M <= 0) return 0;
    size_t s = align256((size_t)M * (size_t)K) + align256((size_t)M * 4);
    if (N > 0 && guard_chunk8(K) > 0) s += align256((size_t)M * (size_t)N * 8);
    return s;
}

// w8a8_linear given its rotate-quant arguments
int linear8_impl(RQArgs qa, bool rotated, const int8_t* w, int64_t N, const void* w_scale, int w_scale_dtype,
                 const void* bias, void* out, int out_dtype, void* workspace, size_t workspace_bytes,
                 void* stream)
{
    const int64_t M = qa.M, K = qa.K;
    const int x_dtype = qa.dtype;
    int rc = rq_validate_g(qa.x, x_dtype, M, K, qa.sm, qa.sk, rotated, qa.g, (int8_t*)1, (float*)1, false);
    if (rc) return rc;
    if (N < 0) return fail(W4A4_INVALID, "negative size");
    if (!dtype_ok(w_scale_dtype) || !dtype_ok(out_dtype)) return fail(W4A4_UNSUPPORTED, "unknown dtype code");
    if (M > 0 && N > 0 && (!w || !w_scale || !out)) return fail(W4A4_INVALID, "a required pointer is NULL");
    if (M == 0 || N == 0) return W4A4_OK;
    const size_t need = w8_workspace(M, K, N);
    if (!workspace || workspace_bytes < need)
        return fail(W4A4_INVALID, "workspace of %zu bytes, need %zu", workspace_bytes, need);
    rc = device_check();
    if (rc) return rc;
    uint8_t* ws = (uint8_t*)workspace;
    int8_t* codes = (int8_t*)ws;
    ws += align256((size_t)M * (size_t)K);
    float* scales = (float*)ws;
    ws += align256((size_t)M * 4);
    const int64_t kc = guard_chunk8(K);
    hipStream_t st = (hipStream_t)stream;
    qa.codes = codes;
    qa.scales = scales;
    qa.yout = nullptr;
    qa.qmax = 127;
    if (rotate_quant_path(qa) < 0)
        return fail(W4A4_UNSUPPORTED, "no INT8 rotate_quant kernel for this shape (K=%lld)", (long long)K);
    int path = 0;
    hipError_t e = launch_rotate_quant(qa, st, &path);
    if (e != hipSuccess) return hip_fail(e, "rotate_quant launch");
    GemmArgs ga{codes, scales, M, K, N, (const uint8_t*)w, w_scale, w_scale_dtype, 0,
                bias, x_dtype, nullptr, nullptr, 0, 0, out, out_dtype, nullptr, kc, kc > 0 ? (int64_t*)ws : nullptr};
    ga.w8 = 1;
    e = launch_gemm(ga, st);
    if (e != hipSuccess) return hip_fail(e, "gemm launch");
    return W4A4_OK;
}

// ---- SVDQuant variant: validation, K-chunk guard, workspace -------------

int64_t svd_chunk(int64_t K, int act_group, int w_scale_group, int act_unsigned)
{
    // per-group conversions (either side grouped) never overflow INT32
    if (act_group || w_scale_group) return 0;
    const int64_t lim = act_unsigned ? kGemmMaxKU : kGemmMaxK;
    return K > lim ? lim : 0;
}

size_t svd_workspace(int64_t M, int64_t K, int64_t N, int rank, int act_group, int act_unsigned)
{
    if (M <= 0) return 0;
    size_t s = align256((size_t)M * (size_t)K);                                 // codes
    s += align256((size_t)M * (size_t)(act_group ? K / 64 : 1) * 4);            // scales
    if (rank > 0) s += align256((size_t)M * rank * 4);                          // lora_act
    if (N > 0 && svd_chunk(K, act_group, 0, act_unsigned) > 0) s += align256((size_t)M * (size_t)N * 8);
    return s;
}

int svd_act_validate(const void* x, int dt, int64_t M, int64_t K, int64_t sm, int64_t sk, int act_unsigned,
                     int act_group)
{
    int rc = check_activation(x, dt, M, K, sm, sk, true);
    if (rc) return rc;
    if (act_unsigned != 0 && act_unsigned != 1) return fail(W4A4_INVALID, "act_unsigned must be 0 or 1");
    if (act_group != 0 && act_group != 64) return fail(W4A4_INVALID, "act_group must be 0 or 64");
    if (act_group && K % 64) return fail(W4A4_INVALID, "K=%lld is not a multiple of 64", (long long)K);
    if (M > 0 && K == 0) return fail(W4A4_INVALID, "K=0 with M>0");
    return W4A4_OK;
}

// one projection of the SVDQuant layer on prepared codes / scales / lora
int svd_gemm(const int8_t* codes, const float* scales, int act_group, int act_unsigned, int64_t M, int64_t K,
             const uint8_t* w_packed, int64_t N, const void* w_scale, int sw_dt, int sw_group, const void* bias,
             int bias_dt, const float* lora, const void* up, int up_dt, int rank, void* out, int out_dt,
             int64_t* acc64, hipStream_t st)
{
    const int64_t kc = svd_chunk(K, act_group, sw_group, act_unsigned);
    GemmArgs ga{codes, scales, M, K, N, w_packed, w_scale, sw_dt, sw_group, bias, bias_dt, lora, up, up_dt,
                lora ? rank : 0, out, out_dt, nullptr, kc, kc > 0 ? acc64 : nullptr};
    ga.sa_group = act_group;
    const hipError_t e = launch_gemm(ga, st);
    return e == hipSuccess ? W4A4_OK : hip_fail(e, "gemm launch");
}

// rotate-quant entry (both code ranges) given its arguments
int rq_impl(const RQArgs& a, bool rotated, void* stream)
{
    int rc = rq_validate_g(a.x, a.dtype, a.M, a.K, a.sm, a.sk, rotated, a.g, a.codes, a.scales, a.qmax == 7);
    if (rc) return rc;
    if (a.M == 0) return W4A4_OK;
    rc = device_check();
    if (rc) return rc;
    int path = 0;
    hipError_t e = launch_rotate_quant(a, (hipStream_t)stream, &path);
    if (e == hipErrorNotSupported)
        return fail(W4A4_UNSUPPORTED, "no rotate_quant kernel for this shape and layout (K=%lld, g=%d)",
                    (long long)a.K, a.g);
    if (e != hipSuccess) return hip_fail(e, "rotate_quant launch");
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

int w4a4_rotate_quant_plan(const void* x, int x_dtype, int64_t M, int64_t K, int64_t stride_m,
                           int64_t stride_k, const float* rot, int32_t g, const void* smooth,
                           const int8_t* codes, const void* rotated_out, int* kernel)
{
    int rc = rq_validate(x, x_dtype, M, K, stride_m, stride_k, rot, g, (int8_t*)codes, (float*)1);
    if (rc) return rc;
    RQArgs a{x, x_dtype, M, K, stride_m, stride_k, rot, rot ? g : 0, smooth, (int8_t*)codes,
             nullptr, (void*)rotated_out};
    const int p = M > 0 ? rotate_quant_path(a) : -1;
    if (M > 0 && p < 0)
        return fail(W4A4_UNSUPPORTED, "no rotate_quant kernel for this shape (K=%lld)", (long long)K);
    if (kernel) *kernel = p;
    return W4A4_OK;
}

int w4a4_gemm_plan(const int8_t* codes, int64_t M, int64_t K, const uint8_t* w_packed, int64_t N,
                   int32_t w_scale_group, int has_lowrank, const int32_t* acc_out, int64_t k_chunk,
                   const void* out, int* kernel)
{
    const float* fake_lora = has_lowrank ? (const float*)1 : nullptr;
    int rc = gemm_validate(codes, (const float*)1, M, K, w_packed, N, (const void*)1, W4A4_F32,
                           w_scale_group, nullptr, 0, fake_lora, fake_lora, W4A4_F32,
                           has_lowrank ? 1 : 0, (void*)out, W4A4_F32, k_chunk);
    if (rc) return rc;
    const int64_t kc = k_chunk > 0 ? k_chunk : (w_scale_group ? 0 : guard_chunk(K));
    GemmArgs a{codes, nullptr, M, K, N, w_packed, nullptr, W4A4_F32, w_scale_group,
               nullptr, 0, fake_lora, fake_lora, W4A4_F32, has_lowrank ? 1 : 0,
               (void*)out, W4A4_F32, (int32_t*)acc_out, kc, nullptr};
    if (kernel) *kernel = (M > 0 && N > 0) ? gemm_path(a) : -1;
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
    RQArgs qa{x, x_dtype, M, K, stride_m, stride_k, rot, rot ? g : 0, smooth, nullptr, nullptr, nullptr};
    return linear4_impl(qa, rot != nullptr, w_packed, N, w_scale, w_scale_dtype, w_scale_group, bias,
                        proj_down, proj_up, rank, out, out_dtype, workspace, workspace_bytes, stream);
}

// ---- INT8 mode (qmax = 127) and the dynamic INT8 linear ----------------

int w8a8_rotate_quant_rowwise(const void* x, int x_dtype, int64_t M, int64_t K, int64_t stride_m,
                              int64_t stride_k, const float* rot, int32_t g, const void* smooth,
                              int8_t* codes, float* scales, void* rotated_out, void* stream)
{
    int rc = rq_validate(x, x_dtype, M, K, stride_m, stride_k, rot, g, codes, scales, false);
    if (rc) return rc;
    if (M == 0) return W4A4_OK;
    rc = device_check();
    if (rc) return rc;
    RQArgs a{x, x_dtype, M, K, stride_m, stride_k, rot, rot ? g : 0, smooth, codes, scales, rotated_out};
    a.qmax = 127;
    int path = 0;
    hipError_t e = launch_rotate_quant(a, (hipStream_t)stream, &path);
    if (e == hipErrorNotSupported)
        return fail(W4A4_UNSUPPORTED, "no INT8 rotate_quant kernel for this shape (K=%lld)", (long long)K);
    if (e != hipSuccess) return hip_fail(e, "rotate_quant launch");
    return W4A4_OK;
}

int w8a8_rotate_quant_plan(const void* x, int x_dtype, int64_t M, int64_t K, int64_t stride_m,
                           int64_t stride_k, const float* rot, int32_t g, const void* smooth,
                           const int8_t* codes, const void* rotated_out, int* kernel)
{
    int rc = rq_validate(x, x_dtype, M, K, stride_m, stride_k, rot, g, (int8_t*)codes, (float*)1, false);
    if (rc) return rc;
    RQArgs a{x, x_dtype, M, K, stride_m, stride_k, rot, rot ? g : 0, smooth, (int8_t*)codes,
             nullptr, (void*)rotated_out};
    a.qmax = 127;
    const int p = M > 0 ? rotate_quant_path(a) : -1;
    if (M > 0 && p < 0)
        return fail(W4A4_UNSUPPORTED, "no INT8 rotate_quant kernel for this shape (K=%lld)", (long long)K);
    if (kernel) *kernel = p;
    return W4A4_OK;
}

size_t w8a8_gemm_workspace_size(int64_t M, int64_t N, int64_t K)
{
    if (M <= 0 || N <= 0) return 0;
    return guard_chunk8(K) > 0 ? align256((size_t)M * (size_t)N * 8) : 0;
}

int w8a8_gemm_from_codes(const int8_t* codes, const float* scales, int64_t M, int64_t K,
                         const int8_t* w, int64_t N, const void* w_scale, int w_scale_dtype,
                         const void* bias, int bias_dtype, void* out, int out_dtype, void* workspace,
                         size_t workspace_bytes, void* stream)
{
    if (M < 0 || K < 0 || N < 0) return fail(W4A4_INVALID, "negative size");
    if (!dtype_ok(w_scale_dtype) || !dtype_ok(out_dtype) || (bias && !dtype_ok(bias_dtype)))
        return fail(W4A4_UNSUPPORTED, "unknown dtype code");
    if (M > 0 && N > 0 && (!scales || !w || !w_scale || !out || (K > 0 && !codes)))
        return fail(W4A4_INVALID, "a required pointer is NULL");
    if (M == 0 || N == 0) return W4A4_OK;
    const int64_t kc = guard_chunk8(K);
    const size_t need = w8a8_gemm_workspace_size(M, N, K);
    if (workspace_bytes < need || (need && !workspace))
        return fail(W4A4_INVALID, "workspace of %zu bytes, need %zu", workspace_bytes, need);
    int rc = device_check();
    if (rc) return rc;
    GemmArgs a{codes, scales, M, K, N, (const uint8_t*)w, w_scale, w_scale_dtype, 0,
               bias, bias_dtype, nullptr, nullptr, 0, 0, out, out_dtype, nullptr, kc, (int64_t*)workspace};
    a.w8 = 1;
    hipError_t e = launch_gemm(a, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "gemm launch");
    return W4A4_OK;
}

int w8a8_gemm_plan(const int8_t* codes, int64_t M, int64_t K, const int8_t* w, int64_t N,
                   const void* out, int* kernel)
{
    if (M < 0 || K < 0 || N < 0) return fail(W4A4_INVALID, "negative size");
    GemmArgs a{codes, nullptr, M, K, N, (const uint8_t*)w, nullptr, W4A4_F32, 0,
               nullptr, 0, nullptr, nullptr, 0, 0, (void*)out, W4A4_F32, nullptr, guard_chunk8(K), nullptr};
    a.w8 = 1;
    if (kernel) *kernel = (M > 0 && N > 0) ? gemm_path(a) : -1;
    return W4A4_OK;
}

size_t w8a8_linear_workspace_size(int64_t M, int64_t K, int64_t N) { return w8_workspace(M, K, N); }

int w8a8_linear(const void* x, int x_dtype, int64_t M, int64_t K, int64_t stride_m, int64_t stride_k,
                const float* rot, int32_t g, const void* smooth, const int8_t* w, int64_t N,
                const void* w_scale, int w_scale_dtype, const void* bias, void* out, int out_dtype,
                void* workspace, size_t workspace_bytes, void* stream)
{
    RQArgs qa{x, x_dtype, M, K, stride_m, stride_k, rot, rot ? g : 0, smooth, nullptr, nullptr, nullptr};
    return linear8_impl(qa, rot != nullptr, w, N, w_scale, w_scale_dtype, bias, out, out_dtype, workspace,
                        workspace_bytes, stream);
}

// ---- structured (Hadamard) rotation: the fast Walsh-Hadamard kernel ------

int w4a4_rotate_quant_hadamard(const void* x, int x_dtype, int64_t M, int64_t K, int64_t stride_m,
                               int64_t stride_k, int32_t g, const int8_t* sign_in, const int8_t* sign_out,
                               const void* smooth, int32_t qmax, int8_t* codes, float* scales,
                               void* rotated_out, void* stream)
{
    if (qmax != 7 && qmax != 127) return fail(W4A4_INVALID, "qmax=%d is neither 7 nor 127", qmax);
    const RQArgs a = hadamard_args(x, x_dtype, M, K, stride_m, stride_k, g, sign_in, sign_out, smooth, qmax,
                                   codes, scales, rotated_out);
    return rq_impl(a, true, stream);
}

int w4a4_rotate_quant_hadamard_plan(const void* x, int x_dtype, int64_t M, int64_t K, int64_t stride_m,
                                    int64_t stride_k, int32_t g, const void* smooth, int32_t qmax,
                                    const int8_t* codes, const void* rotated_out, int* kernel)
{
    if (qmax != 7 && qmax != 127) return fail(W4A4_INVALID, "qmax=%d is neither 7 nor 127", qmax);
    int rc = rq_validate_g(x, x_dtype, M, K, stride_m, stride_k, true, g, (int8_t*)codes, (float*)1, qmax == 7);
    if (rc) return rc;
    const RQArgs a = hadamard_args(x, x_dtype, M, K, stride_m, stride_k, g, nullptr, nullptr, smooth, qmax,
                                   (int8_t*)codes, nullptr, (void*)rotated_out);
    const int p = M > 0 ? rotate_quant_path(a) : -1;
    if (M > 0 && p < 0)
        return fail(W4A4_UNSUPPORTED, "no Hadamard rotate_quant kernel for this shape and layout (K=%lld, g=%d)",
                    (long long)K, g);
    if (kernel) *kernel = p;
    return W4A4_OK;
}

int w4a4_linear_hadamard(const void* x, int x_dtype, int64_t M, int64_t K, int64_t stride_m,
                         int64_t stride_k, int32_t g, const int8_t* sign_in, const int8_t* sign_out,
                         const void* smooth, const uint8_t* w_packed, int64_t N, const void* w_scale,
                         int w_scale_dtype, int32_t w_scale_group, const void* bias, const void* proj_down,
                         const void* proj_up, int32_t rank, void* out, int out_dtype, void* workspace,
                         size_t workspace_bytes, void* stream)
{
    const RQArgs qa = hadamard_args(x, x_dtype, M, K, stride_m, stride_k, g, sign_in, sign_out, smooth, 7,
                                    nullptr, nullptr, nullptr);
    return linear4_impl(qa, true, w_packed, N, w_scale, w_scale_dtype, w_scale_group, bias, proj_down, proj_up,
                        rank, out, out_dtype, workspace, workspace_bytes, stream);
}

int w8a8_linear_hadamard(const void* x, int x_dtype, int64_t M, int64_t K, int64_t stride_m, int64_t stride_k,
                         int32_t g, const int8_t* sign_in, const int8_t* sign_out, const void* smooth,
                         const int8_t* w, int64_t N, const void* w_scale, int w_scale_dtype, const void* bias,
                         void* out, int out_dtype, void* workspace, size_t workspace_bytes, void* stream)
{
    const RQArgs qa = hadamard_args(x, x_dtype, M, K, stride_m, stride_k, g, sign_in, sign_out, smooth, 127,
                                    nullptr, nullptr, nullptr);
    return linear8_impl(qa, true, w, N, w_scale, w_scale_dtype, bias, out, out_dtype, workspace,
                        workspace_bytes, stream);
}

// ---- the SVDQuant layer: shift, per-group activation scales, grouped ------

size_t w4a4_svdquant_workspace_size(int64_t M, int64_t K, int64_t N, int32_t rank, int32_t act_group,
                                    int32_t act_unsigned)
{
    return svd_workspace(M, K, N, rank, act_group, act_unsigned);
}

int w4a4_quantize_svdquant(const void* x, int x_dtype, int64_t M, int64_t K, int64_t stride_m,
                           int64_t stride_k, const void* smooth, int32_t act_unsigned, int32_t act_group,
                           int8_t* codes, float* scales, void* stream)
{
    int rc = svd_act_validate(x, x_dtype, M, K, stride_m, stride_k, act_unsigned, act_group);
    if (rc) return rc;
    if (M > 0 && (!codes || !scales)) return fail(W4A4_INVALID, "codes/scales is NULL");
    if (M == 0) return W4A4_OK;
    RQArgs a{x, x_dtype, M, K, stride_m, stride_k, nullptr, 0, smooth, codes, scales, nullptr};
    if (!svd_quant_ok(a, act_group))
        return fail(W4A4_UNSUPPORTED, "no SVDQuant quantizer for this dtype, layout or width (K=%lld)", (long long)K);
    rc = device_check();
    if (rc) return rc;
    const hipError_t e = launch_svd_quant(a, act_group, act_unsigned != 0, (hipStream_t)stream);
    return e == hipSuccess ? W4A4_OK : hip_fail(e, "svdquant quantizer launch");
}

int w4a4_gemm_svdquant(const int8_t* codes, const float* scales, int32_t act_group, int32_t act_unsigned,
                       int64_t M, int64_t K, const uint8_t* w_packed, int64_t N, const void* w_scale,
                       int w_scale_dtype, int32_t w_scale_group, const void* bias, int bias_dtype,
                       const float* lora_act, const void* proj_up, int up_dtype, int32_t rank, void* out,
                       int out_dtype, void* workspace, size_t workspace_bytes, void* stream)
{
    int rc = gemm_validate(codes, scales, M, K, w_packed, N, w_scale, w_scale_dtype, w_scale_group, bias,
                           bias_dtype, lora_act, proj_up, up_dtype, rank, out, out_dtype, 0);
    if (rc) return rc;
    if (act_unsigned != 0 && act_unsigned != 1) return fail(W4A4_INVALID, "act_unsigned must be 0 or 1");
    if (act_group != 0 && act_group != 64) return fail(W4A4_INVALID, "act_group must be 0 or 64");
    if (act_group && K % 64) return fail(W4A4_INVALID, "K=%lld is not a multiple of 64", (long long)K);
    if (M == 0 || N == 0) return W4A4_OK;
    const int64_t kc = svd_chunk(K, act_group, w_scale_group, act_unsigned);
    const size_t need = kc > 0 ? align256((size_t)M * (size_t)N * 8) : 0;
    if (workspace_bytes < need || (need && !workspace))
        return fail(W4A4_INVALID, "workspace of %zu bytes, need %zu", workspace_bytes, need);
    rc = device_check();
    if (rc) return rc;
    return svd_gemm(codes, scales, act_group, act_unsigned, M, K, w_packed, N, w_scale, w_scale_dtype,
                    w_scale_group, bias, bias_dtype, lora_act, proj_up, up_dtype, rank, out, out_dtype,
                    (int64_t*)workspace, (hipStream_t)stream);
}

int w4a4_linear_svdquant_grouped(const void* x, int x_dtype, int64_t M, int64_t K, int64_t stride_m,
                                 int64_t stride_k, const void* smooth, int32_t act_unsigned, int32_t act_group,
                                 const void* proj_down, int32_t rank, int32_t nproj,
                                 const uint8_t* const* w_packed, const int64_t* N, const void* const* w_scale,
                                 int w_scale_dtype, int32_t w_scale_group, const void* const* bias,
                                 const void* const* proj_up, void* const* out, int out_dtype, void* workspace,
                                 size_t workspace_bytes, void* stream)
{
    // Validate everything before the first launch.
    int rc = svd_act_validate(x, x_dtype, M, K, stride_m, stride_k, act_unsigned, act_group);
    if (rc) return rc;
    if (nproj < 1) return fail(W4A4_INVALID, "nproj=%d", nproj);
    if (!w_packed || !N || !w_scale || !out) return fail(W4A4_INVALID, "a projection array is NULL");
    const int r = proj_down ? rank : 0;
    if (proj_down && (rank < 1 || rank > 64)) return fail(W4A4_INVALID, "rank=%d outside [1, 64]", rank);
    int64_t maxN = 0;
    for (int i = 0; i < nproj; ++i) {
        const void* up = proj_up ? proj_up[i] : nullptr;
        if ((proj_down == nullptr) != (up == nullptr))
            return fail(W4A4_INVALID, "projection %d: proj_down and proj_up go together", i);
        rc = gemm_validate((const int8_t*)1, (const float*)1, M, K, w_packed[i], N[i], w_scale[i], w_scale_dtype,
                           w_scale_group, bias ? bias[i] : nullptr, x_dtype, r ? (const float*)1 : nullptr, up,
                           x_dtype, r, out[i], out_dtype, 0);
        if (rc) return rc;
        maxN = N[i] > maxN ? N[i] : maxN;
    }
    if (M == 0) return W4A4_OK;
    const size_t need = svd_workspace(M, K, maxN, r, act_group, act_unsigned);
    if (!workspace || workspace_bytes < need)
        return fail(W4A4_INVALID, "workspace of %zu bytes, need %zu", workspace_bytes, need);
    uint8_t* ws = (uint8_t*)workspace;
    int8_t* codes = (int8_t*)ws;
    ws += align256((size_t)M * (size_t)K);
    float* scales = (float*)ws;
    ws += align256((size_t)M * (size_t)(act_group ? K / 64 : 1) * 4);
    float* lora = nullptr;
    if (r) {
        lora = (float*)ws;
        ws += align256((size_t)M * r * 4);
    }
    RQArgs qa{x, x_dtype, M, K, stride_m, stride_k, nullptr, 0, smooth, codes, scales, nullptr};
    if (!svd_quant_ok(qa, act_group))
        return fail(W4A4_UNSUPPORTED, "no SVDQuant quantizer for this dtype, layout or width (K=%lld)", (long long)K);
    rc = device_check();
    if (rc) return rc;
    hipStream_t st = (hipStream_t)stream;
    hipError_t e;
    if (r) {
        // the low-rank branch sees the raw activation (not shifted, not smoothed)
        LowRankArgs la{x, x_dtype, M, K, stride_m, stride_k, proj_down, r, lora};
        e = launch_lowrank_down(la, st);
        if (e != hipSuccess) return hip_fail(e, "lowrank_down launch");
    }
    e = launch_svd_quant(qa, act_group, act_unsigned != 0, st);
    if (e != hipSuccess) return hip_fail(e, "svdquant quantizer launch");
    for (int i = 0; i < nproj; ++i) {
        if (N[i] == 0) continue;
        rc = svd_gemm(codes, scales, act_group, act_unsigned, M, K, w_packed[i], N[i], w_scale[i], w_scale_dtype,
                      w_scale_group, bias ? bias[i] : nullptr, x_dtype, lora, proj_up ? proj_up[i] : nullptr,
                      x_dtype, r, out[i], out_dtype, (int64_t*)ws, st);
        if (rc) return rc;
    }
    return W4A4_OK;
}

int w4a4_linear_svdquant(const void* x, int x_dtype, int64_t M, int64_t K, int64_t stride_m, int64_t stride_k,
                         const void* smooth, int32_t act_unsigned, int32_t act_group, const uint8_t* w_packed,
                         int64_t N, const void* w_scale, int w_scale_dtype, int32_t w_scale_group,
                         const void* bias, const void* proj_down, const void* proj_up, int32_t rank, void* out,
                         int out_dtype, void* workspace, size_t workspace_bytes, void* stream)
{
    if (N < 0) return fail(W4A4_INVALID, "negative size");
    if (N == 0) {
        int rc = svd_act_validate(x, x_dtype, M, K, stride_m, stride_k, act_unsigned, act_group);
        return rc;
    }
    const void* bb[1] = {bias};
    const void* uu[1] = {proj_up};
    void* oo[1] = {out};
    return w4a4_linear_svdquant_grouped(x, x_dtype, M, K, stride_m, stride_k, smooth, act_unsigned, act_group,
                                        proj_down, rank, 1, &w_packed, &N, &w_scale, w_scale_dtype,
                                        w_scale_group, bb, uu, oo, out_dtype, workspace, workspace_bytes, stream);
}

// ---- FP6 (bf6 e3m2) GEMM path -------------------------------------------

int w4a4_codes_to_bf6(const int8_t* codes, int64_t M, int64_t K, uint8_t* out, void* stream)
{
    if (M < 0 || K < 0) return fail(W4A4_INVALID, "negative size");
    if (K % 32) return fail(W4A4_INVALID, "K=%lld is not a multiple of 32", (long long)K);
    if (M > 0 && K > 0 && (!codes || !out)) return fail(W4A4_INVALID, "codes/out is NULL");
    if (((uintptr_t)codes % 16) || ((uintptr_t)out % 16))
        return fail(W4A4_UNSUPPORTED, "codes and out must be 16-byte aligned");
    if (M == 0 || K == 0) return W4A4_OK;
    int rc = device_check();
    if (rc) return rc;
    const hipError_t e = launch_to_bf6(codes, false, M * (K / 32), out, (hipStream_t)stream);
    return e == hipSuccess ? W4A4_OK : hip_fail(e, "bf6 encoder launch");
}

int w4a4_pack_weights_bf6(const uint8_t* w_packed, int64_t N, int64_t K, uint8_t* out, void* stream)
{
    if (N < 0 || K < 0) return fail(W4A4_INVALID, "negative size");
    if (K % 32) return fail(W4A4_INVALID, "K=%lld is not a multiple of 32", (long long)K);
    if (N > 0 && K > 0 && (!w_packed || !out)) return fail(W4A4_INVALID, "w_packed/out is NULL");
    if (((uintptr_t)w_packed % 16) || ((uintptr_t)out % 16))
        return fail(W4A4_UNSUPPORTED, "w_packed and out must be 16-byte aligned");
    if (N == 0 || K == 0) return W4A4_OK;
    int rc = device_check();
    if (rc) return rc;
    const hipError_t e = launch_to_bf6(w_packed, true, N * (K / 32), out, (hipStream_t)stream);
    return e == hipSuccess ? W4A4_OK : hip_fail(e, "bf6 encoder launch");
}

int w4a4_gemm_bf6(const uint8_t* codes6, const float* scales, int64_t M, int64_t K, const uint8_t* w6, int64_t N,
                  const void* w_scale, int w_scale_dtype, const void* bias, int bias_dtype, void* out,
                  int out_dtype, void* stream)
{
    int rc = gemm_validate((const int8_t*)codes6, scales, M, K, w6, N, w_scale, w_scale_dtype, 0, bias,
                           bias_dtype, nullptr, nullptr, 0, 0, out, out_dtype, 0);
    if (rc) return rc;
    if (M == 0 || N == 0) return W4A4_OK;
    GemmArgs a{(const int8_t*)codes6, scales, M, K, N, w6, w_scale, w_scale_dtype, 0, bias, bias_dtype,
               nullptr, nullptr, 0, 0, out, out_dtype, nullptr, 0, nullptr};
    if (!gemm_bf6_ok(a))
        return fail(W4A4_UNSUPPORTED, "bf6 GEMM needs K a multiple of 128 in [256, %lld] and 16-byte aligned "
                    "codes, weights and output", (long long)gemm_bf6_max_k());
    rc = device_check();
    if (rc) return rc;
    const hipError_t e = launch_gemm_bf6(a, (hipStream_t)stream);
    return e == hipSuccess ? W4A4_OK : hip_fail(e, "bf6 gemm launch");
}

size_t w4a4_linear_bf6_workspace_size(int64_t M, int64_t K)
{
    if (M <= 0) return 0;
    return 2 * align256((size_t)M * (size_t)K) + align256((size_t)M * 4);
}

int w4a4_linear_bf6(const void* x, int x_dtype, int64_t M, int64_t K, int64_t stride_m, int64_t stride_k,
                    const float* rot, int32_t g, const void* smooth, const uint8_t* w6, int64_t N,
                    const void* w_scale, int w_scale_dtype, const void* bias, void* out, int out_dtype,
                    void* workspace, size_t workspace_bytes, void* stream)
{
    int rc = rq_validate(x, x_dtype, M, K, stride_m, stride_k, rot, g, (int8_t*)1, (float*)1);
    if (rc) return rc;
    rc = gemm_validate((const int8_t*)1, (const float*)1, M, K, w6, N, w_scale, w_scale_dtype, 0, bias, x_dtype,
                       nullptr, nullptr, 0, 0, out, out_dtype, 0);
    if (rc) return rc;
    if (M == 0 || N == 0) return W4A4_OK;
    const size_t need = w4a4_linear_bf6_workspace_size(M, K);
    if (!workspace || workspace_bytes < need)
        return fail(W4A4_INVALID, "workspace of %zu bytes, need %zu", workspace_bytes, need);
    uint8_t* ws = (uint8_t*)workspace;
    int8_t* codes = (int8_t*)ws;
    ws += align256((size_t)M * (size_t)K);
    uint8_t* codes6 = ws;
    ws += align256((size_t)M * (size_t)K);
    float* scales = (float*)ws;
    RQArgs qa{x, x_dtype, M, K, stride_m, stride_k, rot, rot ? g : 0, smooth, codes, scales, nullptr};
    GemmArgs ga{(const int8_t*)codes6, scales, M, K, N, w6, w_scale, w_scale_dtype, 0, bias, x_dtype,
                nullptr, nullptr, 0, 0, out, out_dtype, nullptr, 0, nullptr};
    if (rotate_quant_path(qa) < 0)
        return fail(W4A4_UNSUPPORTED, "no rotate_quant kernel for this shape (K=%lld)", (long long)K);
    if (!gemm_bf6_ok(ga) || (K % 32))
        return fail(W4A4_UNSUPPORTED, "bf6 GEMM needs K a multiple of 128 in [256, %lld] and 16-byte aligned "
                    "weights and output", (long long)gemm_bf6_max_k());
    rc = device_check();
    if (rc) return rc;
    hipStream_t st = (hipStream_t)stream;
    int path = 0;
    hipError_t e = launch_rotate_quant(qa, st, &path);
    if (e != hipSuccess) return hip_fail(e, "rotate_quant launch");
    e = launch_to_bf6(codes, false, M * (K / 32), codes6, st);
    if (e != hipSuccess) return hip_fail(e, "bf6 encoder launch");
    e = launch_gemm_bf6(ga, st);
    return e == hipSuccess ? W4A4_OK : hip_fail(e, "bf6 gemm launch");
}

int w4a4_linear_noalloc(const void* x, int x_dtype, int64_t M, int64_t K, int64_t stride_m,
                        int64_t stride_k, const float* rot, int32_t g, const void* smooth,
                        const uint8_t* w_packed, int64_t N, const void* w_scale, int w_scale_dtype,
                        int32_t w_scale_group, const void* bias, const void* proj_down,
                        const void* proj_up, int32_t rank, void* out, int out_dtype, void* stream)
{
    if (M < 0 || K < 0 || N < 0) return fail(W4A4_INVALID, "negative size");
    if (proj_down && (rank < 1 || rank > 64)) return fail(W4A4_INVALID, "rank=%d outside [1, 64]", rank);
    const size_t need = w4a4_linear_workspace_size(M, K, N, proj_down ? rank : 0);
    if (need > (size_t)W4A4_NOALLOC_SCRATCH_BYTES)
        return fail(W4A4_INVALID,
                    "this layer needs %zu bytes of scratch, more than the %zu bytes w4a4_linear_noalloc "
                    "holds; call w4a4_linear with a workspace",
                    need, (size_t)W4A4_NOALLOC_SCRATCH_BYTES);
    if (M == 0 || N == 0)
        return w4a4_linear(x, x_dtype, M, K, stride_m, stride_k, rot, g, smooth, w_packed, N, w_scale,
                           w_scale_dtype, w_scale_group, bias, proj_down, proj_up, rank, out, out_dtype,
                           nullptr, 0, stream);
    void* ws = nullptr;
    const int rc = scratch_address(&ws);
    if (rc) return rc;
    return w4a4_linear(x, x_dtype, M, K, stride_m, stride_k, rot, g, smooth, w_packed, N, w_scale,
                       w_scale_dtype, w_scale_group, bias, proj_down, proj_up, rank, out, out_dtype, ws,
                       (size_t)W4A4_NOALLOC_SCRATCH_BYTES, stream);
}

}  // extern "C"
