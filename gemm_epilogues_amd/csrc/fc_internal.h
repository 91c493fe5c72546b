// Internal helpers shared by the library's translation units (host checks and
// small device utilities).  Not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "../../include/fc.h"

namespace fc {

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// [p, p+bytes) and [q, q+qbytes) intersect
inline bool overlaps(const void *p, size_t bytes, const void *q, size_t qbytes)
{
    if (bytes == 0 || qbytes == 0) return false;
    uintptr_t a = reinterpret_cast<uintptr_t>(p), b = reinterpret_cast<uintptr_t>(q);
    return a < b + qbytes && b < a + bytes;
}

// After a launch: map a launch error to FC_ERR_HIP.
inline int launch_status()
{
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? FC_OK : FC_ERR_HIP;
}

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ---------------------------------------------------------------- device side

// bf16 <-> fp32.  bf16 is the top half of an fp32 word; the narrowing uses the
// hardware round-to-nearest-even conversion.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    f32x2_t v = {lo, hi};
    bf16x2_t r = __builtin_convertvector(v, bf16x2_t);
    return __builtin_bit_cast(uint32_t, r);
}

// fp16 <-> fp32 (hardware conversions, round to nearest even when narrowing).
__device__ __forceinline__ float h2f(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }
__device__ __forceinline__ uint16_t f2h(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }

__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi)
{
    return (uint32_t)f2h(lo) | ((uint32_t)f2h(hi) << 16);
}
// The same rounding (to nearest even) as pack_f16x2, in one gfx950
// v_cvt_pk_f16_f32.
__device__ __forceinline__ uint32_t pack_f16x2_rne(float lo, float hi)
{
    typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
}
__device__ __forceinline__ float f16_lo(uint32_t w) { return h2f((uint16_t)(w & 0xffffu)); }
__device__ __forceinline__ float f16_hi(uint32_t w) { return h2f((uint16_t)(w >> 16)); }

// Wave64 reductions (all lanes end with the result).
__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}
__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

}  // namespace fc
