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
 * INT8 mode and the dynamic INT8 ConvRot linear ("[Feat][Ascend] Add fused
 * RotateQuant backend", section "What this PR does / why we need it": the
 * fused block rotation + per-row dynamic INT8 quantization that feeds the
 * ConvRot INT8 linear; positive scales).  Same steps as above with
 * qmax = 127: s = max(absmax / 127, 2^-126), codes clamp(rne(y / s), -127,
 * 127) in int8 (-128 never produced).  K may be odd.
 *
 * w8a8_rotate_quant_rowwise: the arguments of w4a4_rotate_quant_rowwise.
 *   Contiguous 16-bit rows with g = 64 (K <= 4096) or g = 256 (K <= 16384)
 *   take fast kernels; other layouts the exact one-row-per-workgroup kernel
 *   (K <= 40960, else W4A4_UNSUPPORTED).
 * w8a8_gemm_from_codes: exact INT32 product of INT8 codes (M, K) with INT8
 *   weights w (N, K) row-major (any int8 value), then the E-B epilogue with
 *   per-channel weight scales (N,) and optional bias (N,).  When
 *   127 * 128 * K could overflow INT32 the sums are taken in K-chunks and
 *   combined exactly in int64 in a workspace of
 *   w8a8_gemm_workspace_size(M, N, K) bytes (0 otherwise).
 * w8a8_linear: rotate-quant (INT8) then the GEMM, enqueued back to back;
 *   bias in x_dtype; workspace of w8a8_linear_workspace_size(M, K, N) bytes.
 * Return codes and ownership as for the W4A4 calls; nothing is allocated.
 */
int w8a8_rotate_quant_rowwise(const void* x, int x_dtype, int64_t M, int64_t K,
                              int64_t stride_m, int64_t stride_k, const float* rot, int32_t g,
                              const void* smooth, int8_t* codes, float* scales,
                              void* rotated_out, void* stream);
int w8a8_gemm_from_codes(const int8_t* codes, const float* scales, int64_t M, int64_t K,
                         const int8_t* w, int64_t N, const void* w_scale, int w_scale_dtype,
                         const void* bias, int bias_dtype, void* out, int out_dtype,
                         void* workspace, size_t workspace_bytes, void* stream);
size_t w8a8_gemm_workspace_size(int64_t M, int64_t N, int64_t K);
int w8a8_linear(const void* x, int x_dtype, int64_t M, int64_t K, int64_t stride_m,
                int64_t stride_k, const float* rot, int32_t g, const void* smooth,
                const int8_t* w, int64_t N, const void* w_scale, int w_scale_dtype,
                const void* bias, void* out, int out_dtype, void* workspace,
                size_t workspace_bytes, void* stream);
size_t w8a8_linear_workspace_size(int64_t M, int64_t K, int64_t N);
/* host-only: the kernel w8a8_rotate_quant_rowwise would take (ids as for
 * w4a4_rotate_quant_plan below: 0 generic, 5 g = 256, 6 row) */
int w8a8_rotate_quant_plan(const void* x, int x_dtype, int64_t M, int64_t K, int64_t stride_m,
                           int64_t stride_k, const float* rot, int32_t g, const void* smooth,
                           const int8_t* codes, const void* rotated_out, int* kernel);
/* host-only: the kernel w8a8_gemm_from_codes would take for these operand
 * addresses (ids as for w4a4_gemm_plan: 0 128 x 128 tile, 1 the same with
 * int64 K-chunks, 2 three-stage 256 x 256) */
int w8a8_gemm_plan(const int8_t* codes, int64_t M, int64_t K, const int8_t* w, int64_t N,
                   const void* out, int* kernel);

/*
 * Structured rotation (fast Walsh-Hadamard transform).  The rotation is given
 * by its structure instead of its entries:
 *   R = diag(sign_in) . H_g . diag(sign_out) . T(1 / sqrt(g)),
 * H_g the Sylvester Hadamard matrix (H_1 = [1], H_2n = [[H_n, H_n],
 * [H_n, -H_n]]), i.e. the normalized Hadamard rotation with random signs on
 * either side.  Every other step is that of the dense calls above
 * ("[Feat][Ascend] Add fused RotateQuant backend", "What this PR does / why
 * we need it" and "How was this patch tested?": group sizes and asymmetric
 * rotations; "[Feat][Ascend] Consolidate INT8, RotateQuant, RoPE and ConvRot
 * W4A4 backends", "W4A4 correctness and performance scope"); the result equals
 * the dense call's with this R up to the order of the fp32 sum of the same
 * exact products.  At g = 64 on shapes the dense one-wave-per-row kernel takes
 * (16 < K/64 <= 64, M >= 2048) that kernel runs, with R's entries (+-1/8)
 * built from the signs: then the result is the dense call's, bit for bit.
 *   g:        16, 32, 64, 128 or 256; K a multiple of g, K <= 16384.
 *   sign_in, sign_out: device int8 arrays of g entries, 8-byte aligned (a
 *             negative entry is -1, any other +1), or NULL for all +1.  Read
 *             by the kernel.
 *   qmax:     7 (INT4 codes) or 127 (the INT8 mode).
 *   Layout:   16-bit x with contiguous rows (stride_k == 1, stride_m a
 *             multiple of 8, 16-byte aligned); other layouts and fp32 x are
 *             W4A4_UNSUPPORTED (use the dense calls with R written out).
 * w4a4_linear_hadamard / w8a8_linear_hadamard are w4a4_linear / w8a8_linear
 * with this rotation (same workspace sizes).
 */
int w4a4_rotate_quant_hadamard(const void* x, int x_dtype, int64_t M, int64_t K, int64_t stride_m,
                               int64_t stride_k, int32_t g, const int8_t* sign_in,
                               const int8_t* sign_out, const void* smooth, int32_t qmax,
                               int8_t* codes, float* scales, void* rotated_out, void* stream);
/* host-only: which kernel w4a4_rotate_quant_hadamard takes for these
 * arguments (7 the fast Walsh-Hadamard transform, 6 the one-wave-per-row
 * kernel at g = 64), W4A4_UNSUPPORTED when none does */
int w4a4_rotate_quant_hadamard_plan(const void* x, int x_dtype, int64_t M, int64_t K,
                                    int64_t stride_m, int64_t stride_k, int32_t g,
                                    const void* smooth, int32_t qmax, const int8_t* codes,
                                    const void* rotated_out, int* kernel);
int w4a4_linear_hadamard(const void* x, int x_dtype, int64_t M, int64_t K, int64_t stride_m,
                         int64_t stride_k, int32_t g, const int8_t* sign_in,
                         const int8_t* sign_out, const void* smooth, const uint8_t* w_packed,
                         int64_t N, const void* w_scale, int w_scale_dtype,
                         int32_t w_scale_group, const void* bias, const void* proj_down,
                         const void* proj_up, int32_t rank, void* out, int out_dtype,
                         void* workspace, size_t workspace_bytes, void* stream);
int w8a8_linear_hadamard(const void* x, int x_dtype, int64_t M, int64_t K, int64_t stride_m,
                         int64_t stride_k, int32_t g, const int8_t* sign_in,
                         const int8_t* sign_out, const void* smooth, const int8_t* w, int64_t N,
                         const void* w_scale, int w_scale_dtype, const void* bias, void* out,
                         int out_dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * The SVDQuant variant of the layer (source page
 * comfy_kitchen/tensor/svdquant_w4a4.py: module docstring, _w4a4_forward,
 * svdquant_w4a4_grouped_linear): no rotation; optional smoothing; INT4
 * activation codes with one scale per row (act_group 0) or per row and
 * 64-wide K group (act_group 64, scales (M, K/64) row-major); act_unsigned = 1
 * for post-GELU layers: the main path quantizes T(fp32(x) + 0.171875) on the
 * unsigned grid [0, 15] (s = max(absmax / 15, 2^-126)), the low-rank branch
 * sees the raw x.  Epilogue with group activation scales:
 * t = sum_G (fp32(acc_G) * s_a[m][G]) * s_w[G][n] in increasing G (per-channel
 * weights: t = (sum_G fp32(acc_G) * s_a[m][G]) * s_w[n]), then + low-rank term
 * + bias as in w4a4_gemm_from_codes; with act_group 0 it is exactly that call's
 * epilogue.
 *   Layout: 16-bit x with contiguous rows (stride_k == 1, stride_m a multiple
 *   of 8, 16-byte aligned), K <= 16384 (a multiple of 64 with act_group 64,
 *   else of 8); other layouts are W4A4_UNSUPPORTED.
 * w4a4_quantize_svdquant: codes (M, K) int8 (8-byte aligned) and scales.
 * w4a4_gemm_svdquant: the GEMM and epilogue on such codes and scales; a
 *   workspace of M*N*8 bytes only when act_group == 0, w_scale_group == 0 and
 *   K exceeds the INT32-safe length (15 * 8 * 16 per product for unsigned
 *   codes), else none.
 * w4a4_linear_svdquant: the whole layer (low-rank down projection, quantizer,
 *   GEMM), workspace of w4a4_svdquant_workspace_size(M, K, N, rank, act_group,
 *   act_unsigned) bytes.
 * w4a4_linear_svdquant_grouped: nproj projections of the same activation that
 *   share smoothing and proj_down (split Q/K/V): the activation is quantized and
 *   projected down once, then one GEMM per projection; per-projection host
 *   arrays of device pointers w_packed[i] (N[i], K/2), w_scale[i], bias[i] and
 *   proj_up[i] (either array may be NULL) and out[i] (M, N[i]); workspace of
 *   w4a4_svdquant_workspace_size with N the largest N[i].
 */
size_t w4a4_svdquant_workspace_size(int64_t M, int64_t K, int64_t N, int32_t rank, int32_t act_group,
                                    int32_t act_unsigned);
int w4a4_quantize_svdquant(const void* x, int x_dtype, int64_t M, int64_t K, int64_t stride_m,
                           int64_t stride_k, const void* smooth, int32_t act_unsigned,
                           int32_t act_group, int8_t* codes, float* scales, void* stream);
int w4a4_gemm_svdquant(const int8_t* codes, const float* scales, int32_t act_group,
                       int32_t act_unsigned, int64_t M, int64_t K, const uint8_t* w_packed,
                       int64_t N, const void* w_scale, int w_scale_dtype, int32_t w_scale_group,
                       const void* bias, int bias_dtype, const float* lora_act,
                       const void* proj_up, int up_dtype, int32_t rank, void* out, int out_dtype,
                       void* workspace, size_t workspace_bytes, void* stream);
int w4a4_linear_svdquant(const void* x, int x_dtype, int64_t M, int64_t K, int64_t stride_m,
                         int64_t stride_k, const void* smooth, int32_t act_unsigned,
                         int32_t act_group, const uint8_t* w_packed, int64_t N, const void* w_scale,
                         int w_scale_dtype, int32_t w_scale_group, const void* bias,
                         const void* proj_down, const void* proj_up, int32_t rank, void* out,
                         int out_dtype, void* workspace, size_t workspace_bytes, void* stream);
int w4a4_linear_svdquant_grouped(const void* x, int x_dtype, int64_t M, int64_t K,
                                 int64_t stride_m, int64_t stride_k, const void* smooth,
                                 int32_t act_unsigned, int32_t act_group, const void* proj_down,
                                 int32_t rank, int32_t nproj, const uint8_t* const* w_packed,
                                 const int64_t* N, const void* const* w_scale, int w_scale_dtype,
                                 int32_t w_scale_group, const void* const* bias,
                                 const void* const* proj_up, void* const* out, int out_dtype,
                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * FP6 GEMM path ("[Feat][Ascend] Consolidate INT8, RotateQuant, RoPE and
 * ConvRot W4A4 backends", "W4A4 correctness and performance scope": the same
 * exact integer accumulation, evaluated on gfx950's f8f6f4 matrix cores).
 * Codes in [-7, 7] and weights in [-8, 7] are exact in bf6 (e3m2: sign bit 5,
 * exponent bits 4-2 with bias 3, mantissa bits 1-0); the products are small
 * integers and the fp32 accumulator holds every partial sum exactly for
 * K <= 299,520 (56 K < 2^24), so the result is bit-identical to
 * w4a4_gemm_from_codes with per-channel scales.
 *   "bf6 blocks": every 32 consecutive K values of a row take 32 bytes: value
 *   e in bits 6e .. 6e+5 of the first 24 (a little-endian 192-bit block), then
 *   8 bytes written as zero and never read.  A row of K values is K bytes.
 * w4a4_codes_to_bf6: int8 codes (M, K) in [-8, 8] -> bf6 blocks (M, K);
 *   K % 32 == 0, 16-byte aligned buffers.
 * w4a4_pack_weights_bf6: packed INT4 weights (N, K/2) -> bf6 blocks (N, K),
 *   once per layer.
 * w4a4_gemm_bf6: the GEMM and epilogue of w4a4_gemm_from_codes (per-channel
 *   weight scales, optional bias, no low-rank term) on bf6 codes and weights;
 *   K a multiple of 128 in [256, 299520], 16-byte aligned codes, weights and
 *   output, else W4A4_UNSUPPORTED.
 * w4a4_linear_bf6: rotate-quant, bf6 encoding and w4a4_gemm_bf6 back to back;
 *   bias in x_dtype; workspace of w4a4_linear_bf6_workspace_size(M, K) bytes.
 */
int w4a4_codes_to_bf6(const int8_t* codes, int64_t M, int64_t K, uint8_t* out, void* stream);
int w4a4_pack_weights_bf6(const uint8_t* w_packed, int64_t N, int64_t K, uint8_t* out, void* stream);
int w4a4_gemm_bf6(const uint8_t* codes6, const float* scales, int64_t M, int64_t K, const uint8_t* w6,
                  int64_t N, const void* w_scale, int w_scale_dtype, const void* bias, int bias_dtype,
                  void* out, int out_dtype, void* stream);
size_t w4a4_linear_bf6_workspace_size(int64_t M, int64_t K);
int w4a4_linear_bf6(const void* x, int x_dtype, int64_t M, int64_t K, int64_t stride_m,
                    int64_t stride_k, const float* rot, int32_t g, const void* smooth,
                    const uint8_t* w6, int64_t N, const void* w_scale, int w_scale_dtype,
                    const void* bias, void* out, int out_dtype, void* workspace,
                    size_t workspace_bytes, void* stream);

/*
 * w4a4_linear for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same arguments without the workspace, and the same kernels, which work
 * in a scratch array the library holds per GPU (W4A4_NOALLOC_SCRATCH_BYTES,
 * allocated with the code object and kept until the process ends).  The
 * call allocates nothing.  A layer whose w4a4_linear_workspace_size exceeds
 * that size is refused with W4A4_INVALID before anything is enqueued.
 * Every call on a GPU shares that GPU's scratch: calls that overlap on one
 * GPU (other streams, other threads) race and must be serialised by the
 * caller; calls in order on one stream are safe.  The caller still passes x
 * and out.  The first call on a device looks up that device's scratch
 * address (no allocation).
 */
#define W4A4_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
int w4a4_linear_noalloc(const void* x, int x_dtype, int64_t M, int64_t K, int64_t stride_m,
                        int64_t stride_k, const float* rot, int32_t g, const void* smooth,
                        const uint8_t* w_packed, int64_t N, const void* w_scale, int w_scale_dtype,
                        int32_t w_scale_group, const void* bias, const void* proj_down,
                        const void* proj_up, int32_t rank, void* out, int out_dtype, void* stream);

/*
 * INT32 overflow guard (W4A4 page, section "W4A4 correctness and performance
 * scope").  Returns 1 if a K-long accumulation could overflow the GEMM's INT32
 * registers (which hold 16 * c * w, |c| <= 7, |w| <= 8), else 0; *k_chunk (if
 * non-NULL) receives the chunk length the GEMM then uses (0 when no chunking).
 * Host-only, no device access.
 */
int w4a4_int32_guard(int64_t K, int64_t* k_chunk);

/*
 * Host-only plan queries: which kernel the library selects for a call with
 * these arguments.  Same validation and status codes as the call itself
 * (a fused operator that checks dtype, shape and group size and reports when
 * it cannot serve a request: "[Feat][Ascend] Add fused RotateQuant backend",
 * section "What this PR does / why we need it"); no device access, nothing
 * enqueued.  Pointers are only inspected for NULL and alignment.  *kernel
 * receives -1 when M == 0 (nothing would launch).
 *
 * w4a4_rotate_quant_plan, *kernel:
 *   0 generic (exact products summed in fp64, one rounding; fp32 activations)
 *   1 MFMA with an LDS row buffer (other 16-bit layouts)
 *   2 MFMA with the row block's tiles over four waves (few rows, g <= 64)
 *   3 one wave per row block (many contiguous rows, g <= 64)
 *   4 column-major (unit row stride, i.e. a transposed view; M % 8 == 0)
 *   5 g = 256 on contiguous rows
 *   6 one wave per contiguous row, g = 64, 16 < K/64 <= 64 (many rows; also
 *     w4a4_rotate_quant_hadamard_plan at g = 64)
 *   7 fast Walsh-Hadamard transform (w4a4_rotate_quant_hadamard_plan only)
 * w4a4_gemm_plan, *kernel (has_lowrank: a low-rank term will be added):
 *   0 128 x 128 tiles          1 128 x 128 tiles over K chunks (int64 combine)
 *   2 persistent 256 x 256 ring (prefill-sized M)     3 skinny M (M <= 64)
 *   4 persistent 256 x 256 ping-pong (prefill-sized M, N % 16 == 0)
 */
int w4a4_rotate_quant_plan(const void* x, int x_dtype, int64_t M, int64_t K, int64_t stride_m,
                           int64_t stride_k, const float* rot, int32_t g, const void* smooth,
                           const int8_t* codes, const void* rotated_out, int* kernel);
int w4a4_gemm_plan(const int8_t* codes, int64_t M, int64_t K, const uint8_t* w_packed, int64_t N,
                   int32_t w_scale_group, int has_lowrank, const int32_t* acc_out, int64_t k_chunk,
                   const void* out, int* kernel);

/* Thread-local text for the last non-OK status returned on this thread. */
const char* w4a4_last_error(void);

/* W4A4_OK if the current HIP device is gfx950, else W4A4_UNSUPPORTED. */
int w4a4_device_supported(void);

#ifdef __cplusplus
}
#endif

#endif /* W4A4_H */
