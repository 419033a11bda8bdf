// kvq_device.hpp -- small device helpers shared by the kvq kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- bit casts
__device__ __forceinline__ half2_t as_h2(uint32_t u) { return __builtin_bit_cast(half2_t, u); }
__device__ __forceinline__ uint32_t as_u32(half2_t h) { return __builtin_bit_cast(uint32_t, h); }

// fp32 -> fp16 bits, round to nearest even (v_cvt_f16_f32 under the default
// round-to-nearest-even mode; fp16 subnormals are produced, overflow gives inf).
__device__ __forceinline__ uint16_t f32_to_f16_bits(float x)
{
    _Float16 h = (_Float16)x;
    return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float f16_bits_to_f32(uint16_t b)
{
    return (float)__builtin_bit_cast(_Float16, b);
}

// -------------------------------------------------------- wave reductions
template <typename T>
__device__ __forceinline__ T shfl_xor(T v, int mask)
{
    return __shfl_xor(v, mask, 64);
}

__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int m = 1; m < 64; m <<= 1)
        v = fmaxf(v, shfl_xor(v, m));
    return v;
}

__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int m = 1; m < 64; m <<= 1)
        v += shfl_xor(v, m);
    return v;
}

// ------------------------------------------------------ vector memory ops
// Loads through the global address space (global_load_*, not flat_load_*).
#define KVQ_GLOBAL __attribute__((address_space(1)))
#define KVQ_CONST __attribute__((address_space(4)))
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 ld_u4(const void *p)
{
    const u32x4_t v = *(const KVQ_GLOBAL u32x4_t *)p;
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 ld_u2(const void *p)
{
    const u32x2_t v = *(const KVQ_GLOBAL u32x2_t *)p;
    return make_uint2(v.x, v.y);
}
__device__ __forceinline__ uint16_t ld_u16(const void *p) { return *(const KVQ_GLOBAL uint16_t *)p; }

} // namespace kvq
