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
};

hipError_t launch_rotate_quant(const RQArgs& a, hipStream_t st, int* path);

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
};

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

// Largest K whose accumulation cannot overflow the kernel's INT32 registers.
// The kernel accumulates 16 * c * w (weights are unpacked as 16 * w, which
// needs no per-nibble sign extension), |c| <= 7 and |w| <= 8.
constexpr int64_t kGemmMaxK = (int64_t)2147483647 / (7 * 8 * 16) / 64 * 64;

}  // namespace w4a4
