// Streaming-bandwidth probe (measurement only; not part of the layer).
//
// Moves the same bytes as one rotate-quant launch over contiguous 16-bit rows
// -- reads M*K 16-bit values, writes M*K bytes and M fp32 values -- with no
// arithmetic to speak of, so its duration is the practical HBM ceiling for
// that traffic on the device.  Each thread streams 16-byte chunks of x with
// four loads in flight and writes one byte per value (the value's high
// byte), grid-stride over the whole array; the byte stores are ordinary or
// non-temporal (streaming) stores.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <bool NT>
__device__ __forceinline__ void put(u32x2* p, uint32_t lo, uint32_t hi)
{
    const u32x2 v = {lo, hi};
    if constexpr (NT)
        __builtin_nontemporal_store(v, p);
    else
        *p = v;
}

template <bool NT>
__global__ __launch_bounds__(256) void stream_probe_kernel(const uint4* __restrict__ x,
                                                           u32x2* __restrict__ out, float* __restrict__ s,
                                                           int64_t chunks, int64_t M)
{
    constexpr int U = 4;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (; i + (U - 1) * stride < chunks; i += U * stride) {
        uint4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = x[i + u * stride];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t lo = __builtin_amdgcn_perm(v[u].y, v[u].x, 0x07050301u);
            const uint32_t hi = __builtin_amdgcn_perm(v[u].w, v[u].z, 0x07050301u);
            put<NT>(out + i + u * stride, lo, hi);
        }
    }
    for (; i < chunks; i += stride) {
        const uint4 v = x[i];
        put<NT>(out + i, __builtin_amdgcn_perm(v.y, v.x, 0x07050301u),
                __builtin_amdgcn_perm(v.w, v.z, 0x07050301u));
    }
    for (int64_t m = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; m < M; m += stride) s[m] = 0.0f;
}

}  // namespace

extern "C" {

// x: n 16-bit values (n % 8 == 0, 16-byte aligned); out: n bytes (8-byte
// aligned); s: M floats; nt != 0: non-temporal byte stores.  Returns a
// hipError_t value.
int w4a4_stream_probe(const void* x, int64_t n, void* out, float* s, int64_t M, int grid, int nt, void* stream)
{
    if (n % 8 || ((uintptr_t)x % 16) || ((uintptr_t)out % 8) || grid < 1) return (int)hipErrorInvalidValue;
    if (nt)
        hipLaunchKernelGGL(stream_probe_kernel<true>, dim3(grid), dim3(256), 0, (hipStream_t)stream,
                           (const uint4*)x, (u32x2*)out, s, n / 8, M);
    else
        hipLaunchKernelGGL(stream_probe_kernel<false>, dim3(grid), dim3(256), 0, (hipStream_t)stream,
                           (const uint4*)x, (u32x2*)out, s, n / 8, M);
    return (int)hipGetLastError();
}

}  // extern "C"
