/*
 * w4a4.h -- C ABI of the MI355X (gfx950) W4A4 rotate/quantize linear layer.
 *
 * The layer (web page "[Feat][Ascend] Consolidate INT8, RotateQuant, RoPE and
 * ConvRot W4A4 backends", section "W4A4 correctness and performance scope";
 * "[Perf][Ascend] Avoid activation pack/unpack in ConvRot W4A4", section
 * "Summary"; "[Feat][Ascend] Add fused RotateQuant backend", section "What this
 * PR does"; SVDQuant extras from the source page
 * comfy_kitchen/tensor/svdquant_w4a4.py, module docstring):
 *
 *   x' = T(fp32(x) / fp32(smooth[k]))                        optional smoothing
 *   y  = T( x'_group . T(R) )  for each group of g entries    block rotation
 *   s  = max(absmax_row(y) / 7, 2^-126)   (fp32, NaN row -> NaN)
 *   c  = clamp(round_half_even(fp32(y) / s), -7, 7)  INT4 codes in int8 storage
 *   acc= sum_k c[m,k] * w[n,k]            exact integer sum (w: packed INT4)
 *   out= O( ((fp32(acc) * s[m]) * s_w[n]) [+ l[m,n]] [+ bias[n]] )
 *   (per-64-group weight scales: ((sum_G fp32(acc_G) * s_w[G,n]) * s[m]) ...)
 *   l  = (x . proj_down) . proj_up^T      optional low-rank term on the raw x
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers (hipMalloc'ed or torch CUDA
 *     memory) unless stated; the caller owns every buffer.  The library never
 *     allocates device memory, never synchronises and keeps no state between
 *     calls.  Work is enqueued on `stream` (a hipStream_t passed as void*,
 *     NULL = the default stream) and completes asynchronously.
 *   - Dtype codes: W4A4_F32 (IEEE binary32), W4A4_F16 (binary16), W4A4_BF16
 *     (bfloat16).  16-bit values are stored as their 2-byte patterns.
 *   - Activations are an (M, K) view with element strides stride_m, stride_k
 *     (a transposed view of a (K, M) buffer has stride_m = 1, stride_k = M).
 *   - Packed weights are (N, K/2) bytes, row-major: byte j of row n holds
 *     k = 2j in its low nibble and k = 2j+1 in its high nibble, each a 4-bit
 *     two's-complement value (0x8 = -8).
 *   - M == 0 is legal and launches nothing.
 *   - Return value: W4A4_OK, or
 *       W4A4_INVALID      bad arguments, detected on the host before any launch
 *                         (odd K, K % g != 0, null required pointer, negative
 *                         size or stride, bad group, workspace too small);
 *       W4A4_UNSUPPORTED  a valid request this build does not serve (dtype
 *                         code unknown, g not a power of two in [16, 256],
 *                         current device not gfx950); the caller may fall back;
 *       W4A4_HIP_ERROR    a HIP call failed (message in w4a4_last_error()).
 *     No exception crosses the ABI.
 */
#ifndef W4A4_H
#define W4A4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { W4A4_OK = 0, W4A4_INVALID = -1, W4A4_UNSUPPORTED = -2, W4A4_HIP_ERROR = -3 };
enum { W4A4_F32 = 0, W4A4_F16 = 1, W4A4_BF16 = 2 };

/*
 * Fused rotate + quantize of activation rows (smoothing, rotation, per-row
 * scale, INT4 codes).  Source: "[Feat][Ascend] Add fused RotateQuant backend",
 * section "What this PR does" (fused rotate+quantize returning codes and
 * positive per-row scales) with the signed-INT4 grid of the W4A4 page, section
 * "W4A4 correctness and performance scope", and the INT8-stored codes of
 * "[Perf][Ascend] Avoid activation pack/unpack in ConvRot W4A4", "Summary".
 *
 *   x          (M, K) activations in x_dtype, strides (stride_m, stride_k)
 *   rot        (g, g) fp32 row-major rotation R (y_j = sum_i x_i R[i][j]), rounded
 *              to x_dtype before use; NULL = no rotation (g ignored)
 *   g          group size: a power of two in [16, 256]; K % g == 0
 *   smooth     (K,) in x_dtype, or NULL (no smoothing)
 *   codes      out (M, K) int8, row-major, values in [-7, 7]
 *   scales     out (M,) fp32, positive for finite rows
 *   rotated_out optional out (M, K) x_dtype row-major: the rotated values y that
 *              the codes were taken from; NULL = not written
 */
int w4a4_rotate_quant_rowwise(const void* x, int x_dtype, int64_t M, int64_t K,
                              int64_t stride_m, int64_t stride_k, const float* rot, int32_t g,
                              const void* smooth, int8_t* codes, float* scales,
                              void* rotated_out, void* stream);

/*
 * Low-rank down projection on the raw activation: lora_act = x . proj_down.
 * Source: comfy_kitchen/tensor/svdquant_w4a4.py, module docstring (proj_down
 * (K, R)) and _w4a4_forward docstring (the low-rank branch sees the raw x).
 *
 *   x          (M, K) in x_dtype, strides as above
 *   proj_down  (K, rank) row-major in x_dtype, rank in [1, 64]
 *   lora_act   out (M, rank) fp32 row-major
 */
int w4a4_lowrank_down(const void* x, int x_dtype, int64_t M, int64_t K, int64_t stride_m,
                      int64_t stride_k, const void* proj_down, int32_t rank, float* lora_act,
                      void* stream);

/*
 * INT8-MFMA GEMM of INT4 codes against packed INT4 weights with the fused
 * epilogue.  Source: "[Feat][Ascend] Consolidate INT8, RotateQuant, RoPE and
 * ConvRot W4A4 backends", section "W4A4 correctness and performance scope"
 * (unpack W4 to INT8, INT32 accumulation with unit scale, then cast, activation
 * scale, weight scale and bias in that order, INT32 overflow guard).
 *
 *   codes      (M, K) int8 row-major, values in [-7, 7]
 *   scales     (M,) fp32 activation scales
 *   w_packed   (N, K/2) packed INT4 weights
 *   w_scale    w_scale_group == 0: (N,) in w_scale_dtype;
 *              w_scale_group == 64: (K/64, N) in w_scale_dtype (K % 64 == 0)
 *   bias       (N,) in bias_dtype, or NULL
 *   lora_act   (M, rank) fp32 and proj_up (N, rank) in up_dtype, or both NULL
 *   out        out (M, N) in out_dtype, row-major
 *   acc_out    optional out (M, N) int32: the exact integer sums (per-channel
 *              mode only; NULL = not written)
 *   k_chunk    0: chunk K only when INT32 could overflow (see w4a4_int32_guard);
 *              > 0 (a multiple of 64): accumulate in K-chunks of this size and
 *              combine them exactly in int64 (per-channel mode only)
 *   workspace  device scratch of w4a4_gemm_workspace_size(M, N, K, k_chunk)
 *              bytes (may be NULL when that size is 0)
 */
int w4a4_gemm_from_codes(const int8_t* codes, const float* scales, int64_t M, int64_t K,
                         const uint8_t* w_packed, int64_t N, const void* w_scale,
                         int w_scale_dtype, int32_t w_scale_group, const void* bias,
                         int bias_dtype, const float* lora_act, const void* proj_up,
                         int up_dtype, int32_t rank, void* out, int out_dtype,
                         int32_t* acc_out, int64_t k_chunk, void* workspace,
                         size_t workspace_bytes, void* stream);

size_t w4a4_gemm_workspace_size(int64_t M, int64_t N, int64_t K, int64_t k_chunk);

/*
 * The whole layer: [lowrank_down] -> rotate_quant_rowwise -> gemm_from_codes,
 * enqueued back to back on `stream`.  proj_down/proj_up/bias are in x_dtype;
 * pass proj_down = proj_up = NULL and rank = 0 for no low-rank term.
 * workspace: w4a4_linear_workspace_size(M, K, N, rank) bytes of device memory
 * (codes, scales, lora_act and, if the guard trips, the int64 accumulator).
 */
int w4a4_linear(const void* x, int x_dtype, int64_t M, int64_t K, int64_t stride_m,
                int64_t stride_k, const float* rot, int32_t g, const void* smooth,
                const uint8_t* w_packed, int64_t N, const void* w_scale, int w_scale_dtype,
                int32_t w_scale_group, const void* bias, const void* proj_down,
                const void* proj_up, int32_t rank, void* out, int out_dtype, void* workspace,
                size_t workspace_bytes, void* stream);

size_t w4a4_linear_workspace_size(int64_t M, int64_t K, int64_t N, int32_t rank);

/*
 * INT32 overflow guard (W4A4 page, section "W4A4 correctness and performance
 * scope").  Returns 1 if a K-long accumulation could overflow the GEMM's INT32
 * registers (which hold 16 * c * w, |c| <= 7, |w| <= 8), else 0; *k_chunk (if
 * non-NULL) receives the chunk length the GEMM then uses (0 when no chunking).
 * Host-only, no device access.
 */
int w4a4_int32_guard(int64_t K, int64_t* k_chunk);

/* Thread-local text for the last non-OK status returned on this thread. */
const char* w4a4_last_error(void);

/* W4A4_OK if the current HIP device is gfx950, else W4A4_UNSUPPORTED. */
int w4a4_device_supported(void);

#ifdef __cplusplus
}
#endif

#endif /* W4A4_H */
