// Launch interfaces between the host C-ABI layer and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a4 {

struct RQArgs {
    const void* x;
    int dtype;
    int64_t M, K, sm, sk;   // strides in elements
    const float* rot;       // (g, g) fp32 row-major or nullptr
    int g;
    const void* smooth;     // (K,) in dtype or nullptr
    int8_t* codes;          // (M, K)
    float* scales;          // (M,)
    void* yout;             // (M, K) in dtype or nullptr
    int qmax = 7;           // 7: INT4 codes; 127: the INT8 mode
    // structured rotation (rot unused): R = diag(sign_in) H_g diag(sign_out) / sqrt(g),
    // signs +-1 as int8 (g,) on the device, NULL for all +1
    int hadamard = 0;
    const int8_t* sign_in = nullptr;
    const int8_t* sign_out = nullptr;
};

// The kernel that launch_rotate_quant takes for these arguments (>= 0), or -1
// when no kernel serves them; host-only, no device access.
int rotate_quant_path(const RQArgs& a);
// the row-streaming kernel for many contiguous 16-bit rows with g = 64
bool row_kernel_ok(const RQArgs& a);
hipError_t launch_rotate_quant_row(const RQArgs& a, hipStream_t st);
hipError_t launch_rotate_quant(const RQArgs& a, hipStream_t st, int* path);
// the fast Walsh-Hadamard kernel for a.hadamard (contiguous 16-bit rows)
bool hadamard_kernel_ok(const RQArgs& a);
hipError_t launch_rotate_quant_hadamard(const RQArgs& a, hipStream_t st);

struct GemmArgs {
    const int8_t* codes;    // (M, K) row-major
    const float* sa;        // (M,)
    int64_t M, K, N;
    const uint8_t* wp;      // (N, K/2)
    const void* sw;         // (N,) or (K/64, N)
    int sw_dtype;
    int sw_group;           // 0 or 64
    const void* bias;       // (N,) or nullptr
    int bias_dtype;
    const float* lora;      // (M, R) fp32 or nullptr
    const void* up;         // (N, R) or nullptr
    int up_dtype;
    int rank;
    void* out;              // (M, N)
    int out_dtype;
    int32_t* acc_out;       // optional (M, N) int32
    int64_t k_chunk;        // > 0: accumulate K in chunks of this many (exact int64 combine)
    int64_t* acc64;         // workspace (M, N) int64 when k_chunk > 0
    int w8 = 0;             // 1: wp holds INT8 weights (N, K), codes up to +-127
    int sa_group = 0;       // 64: sa holds (M, K/64) activation scales (K % 64 == 0)
};

// GEMM kernels, as gemm_path names them (host-only choice, no device access)
enum { kGemmTile = 0, kGemmTileSplitK = 1, kGemmRing3 = 2, kGemmSkinny = 3, kGemmPP = 4 };
int gemm_path(const GemmArgs& a);
hipError_t launch_gemm(const GemmArgs& a, hipStream_t st);

struct LowRankArgs {
    const void* x;
    int dtype;
    int64_t M, K, sm, sk;
    const void* down;       // (K, R) in dtype
    int rank;
    float* lora;            // (M, R) fp32
};

hipError_t launch_lowrank_down(const LowRankArgs& a, hipStream_t st);

// SVDQuant activation quantizer (contiguous 16-bit rows, no rotation): shift
// (act_unsigned), smoothing, INT4 codes per row or per 64-wide group
bool svd_quant_ok(const RQArgs& a, int group);
hipError_t launch_svd_quant(const RQArgs& a, int group, bool act_unsigned, hipStream_t st);

// FP6 (bf6 e3m2) GEMM: codes (M, K) and weights (N, K) as bf6 blocks (32
// values in 24 bytes + 8 unused bytes), per-channel scales, optional bias
bool gemm_bf6_ok(const GemmArgs& a);
int64_t gemm_bf6_max_k();
hipError_t launch_gemm_bf6(const GemmArgs& a, hipStream_t st);
// int8 codes (weights = false) or packed INT4 weights -> bf6 blocks
hipError_t launch_to_bf6(const void* src, bool weights, int64_t nblk, uint8_t* out, hipStream_t st);

// Largest K whose accumulation cannot overflow the kernel's INT32 registers.
// The kernel accumulates 16 * c * w (weights are unpacked as 16 * w, which
// needs no per-nibble sign extension), |c| <= 7 and |w| <= 8.
constexpr int64_t kGemmMaxK = (int64_t)2147483647 / (7 * 8 * 16) / 64 * 64;
// The same for INT8 codes (|c| <= 127) and INT8 weights (|w| <= 128), which
// the kernel multiplies as they are.
constexpr int64_t kGemmMaxK8 = (int64_t)2147483647 / (127 * 128) / 64 * 64;
// The same for codes on the unsigned grid [0, 15] with INT4 weights.
constexpr int64_t kGemmMaxKU = (int64_t)2147483647 / (15 * 8 * 16) / 64 * 64;

}  // namespace w4a4
