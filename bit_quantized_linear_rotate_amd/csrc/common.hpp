// Device-side helpers shared by the W4A4 kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a4 {

enum Dtype : int { F32 = 0, F16 = 1, BF16 = 2 };

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef short v8s __attribute__((ext_vector_type(8)));

// 16-bit storage types carried as raw bits.
struct bf16_t { uint16_t b; };
struct f16_t { uint16_t b; };

__device__ __forceinline__ float bits_to_f32(uint32_t u) { return __uint_as_float(u); }

// bf16 -> f32 is exact: the 16 stored bits are the top half of the fp32 pattern.
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// f32 -> bf16, round to nearest even (gfx950 v_cvt_pk_bf16_f32); NaN stays a
// NaN, overflow gives Inf, bf16 denormals are kept.
__device__ __forceinline__ uint16_t f32_to_bf16(float f)
{
    const __bf16 b = (__bf16)f;
    return __builtin_bit_cast(uint16_t, b);
}

__device__ __forceinline__ float f16_to_f32(uint16_t b)
{
    _Float16 h = __builtin_bit_cast(_Float16, b);
    return (float)h;
}

// f32 -> f16 with the hardware conversion (round to nearest even, IEEE
// overflow to Inf, fp16 denormals kept).
__device__ __forceinline__ uint16_t f32_to_f16(float f)
{
    _Float16 h = (_Float16)f;
    return __builtin_bit_cast(uint16_t, h);
}

template <int DT> __device__ __forceinline__ float load_as_f32(const void* p, int64_t i);
template <> __device__ __forceinline__ float load_as_f32<F32>(const void* p, int64_t i)
{ return ((const float*)p)[i]; }
template <> __device__ __forceinline__ float load_as_f32<F16>(const void* p, int64_t i)
{ return f16_to_f32(((const uint16_t*)p)[i]); }
template <> __device__ __forceinline__ float load_as_f32<BF16>(const void* p, int64_t i)
{ return bf16_to_f32(((const uint16_t*)p)[i]); }

__device__ __forceinline__ float load_any_f32(int dt, const void* p, int64_t i)
{
    if (dt == F32) return ((const float*)p)[i];
    uint16_t b = ((const uint16_t*)p)[i];
    return dt == F16 ? f16_to_f32(b) : bf16_to_f32(b);
}

// 16-bit value -> f32 and f32 -> 16-bit value for the two half formats.
template <int DT> __device__ __forceinline__ float h_to_f32(uint16_t b)
{ return DT == F16 ? f16_to_f32(b) : bf16_to_f32(b); }
template <int DT> __device__ __forceinline__ uint16_t f32_to_h(float f)
{ return DT == F16 ? f32_to_f16(f) : f32_to_bf16(f); }

__device__ __forceinline__ void store_any(int dt, void* p, int64_t i, float v)
{
    if (dt == F32) ((float*)p)[i] = v;
    else if (dt == F16) ((uint16_t*)p)[i] = f32_to_f16(v);
    else ((uint16_t*)p)[i] = f32_to_bf16(v);
}

// Non-temporal (streaming) stores for outputs that no later kernel of the
// same call reads back soon: codes and exported rotated values are written
// once and would otherwise displace the input rows still to be read from the
// caches.  Only for stores that fill whole 64-byte pieces of a line across a
// wave: scattered 4-byte streaming stores measured slower than plain ones.
typedef unsigned v4u_st __attribute__((ext_vector_type(4)));
typedef unsigned v2u_st __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void st_stream16(void* p, uint32_t a, uint32_t b, uint32_t c, uint32_t d)
{
    __builtin_nontemporal_store((v4u_st){a, b, c, d}, (v4u_st*)p);
}
__device__ __forceinline__ void st_stream8(void* p, uint32_t a, uint32_t b)
{
    __builtin_nontemporal_store((v2u_st){a, b}, (v2u_st*)p);
}

// IEEE-exact fp32 multiply and add (never contracted into an FMA).
__device__ __forceinline__ float mul_rn(float a, float b) { return __fmul_rn(a, b); }
__device__ __forceinline__ float add_rn(float a, float b) { return __fadd_rn(a, b); }

}  // namespace w4a4
