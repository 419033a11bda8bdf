// kvq_device.hpp -- small device helpers shared by the kvq kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <limits.h>

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
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 ld_u4(const void *p)
{
    const u32x4_t v = *(const KVQ_GLOBAL u32x4_t *)p;
    return make_uint4(v.x, v.y, v.z, v.w);
}
// the same load, nontemporal (data streamed once)
__device__ __forceinline__ uint4 ld_u4_nt(const void *p)
{
    const u32x4_t v = __builtin_nontemporal_load((const KVQ_GLOBAL u32x4_t *)p);
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 ld_u2(const void *p)
{
    const u32x2_t v = *(const KVQ_GLOBAL u32x2_t *)p;
    return make_uint2(v.x, v.y);
}
__device__ __forceinline__ uint16_t ld_u16(const void *p) { return *(const KVQ_GLOBAL uint16_t *)p; }

// max of two floats as one v_max_f32 (fmaxf also quiets signalling NaNs
// first, one extra instruction per operand; the values here are never NaN)
__device__ __forceinline__ float fmax_nc(float a, float b)
{
    float r;
    asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}

// ------------------------------------------------------- buffer resources
// Raw buffer (stride 0) over [base, base + n_bytes): loads take a 32-bit
// byte offset, and a load past n_bytes returns zero without touching memory,
// so tails need neither clamping nor branches.  Third descriptor word as
// documented for gfx9-family GPUs.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t n_bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)n_bytes, 0x00020000);
}
// Cache policy of a load (the instruction's cache-policy bits): 0 plain,
// CP_NT nontemporal.  A stream read exactly once, such as the cache codes,
// reaches a markedly higher HBM bandwidth with CP_NT on this device (a plain
// read stream ~79 % of peak, the same stream nontemporal ~88 %).
constexpr int CP_NT = 2;
template <int CP = 0>
__device__ __forceinline__ uint4 bld_u4(rsrc_t r, uint32_t off)
{
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, CP);
    return make_uint4(v.x, v.y, v.z, v.w);
}
template <int CP = 0>
__device__ __forceinline__ uint2 bld_u2(rsrc_t r, uint32_t off)
{
    const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, CP);
    return make_uint2(v.x, v.y);
}
template <int CP = 0>
__device__ __forceinline__ uint32_t bld_u32(rsrc_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, CP);
}
__device__ __forceinline__ uint32_t bld_u16(rsrc_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
}

// ------------------------------------------- DPP wave reductions (uniform)
// In-row steps (quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror,
// row_mirror) leave every lane with its 16-lane row total; row_bcast:15 into
// rows 1 and 3, then row_bcast:31 into rows 2 and 3, leave the wave total in
// lane 63, which is read back as a wave-uniform value.  Rows a broadcast
// does not write keep the operation's identity.  All 64 lanes must be active.
template <int CTRL, int ROWS = 0xF, bool BC = false>
__device__ __forceinline__ int dpp_i(int old, int v)
{
    return __builtin_amdgcn_update_dpp(old, v, CTRL, ROWS, 0xF, BC);
}
__device__ __forceinline__ int wave_max_ui(int v)
{
    v = max(v, dpp_i<0xB1, 0xF, true>(0, v));
    v = max(v, dpp_i<0x4E, 0xF, true>(0, v));
    v = max(v, dpp_i<0x141, 0xF, true>(0, v));
    v = max(v, dpp_i<0x140, 0xF, true>(0, v));
    v = max(v, dpp_i<0x142, 0xA>(INT_MIN, v));
    v = max(v, dpp_i<0x143, 0xC>(INT_MIN, v));
    return __builtin_amdgcn_readlane(v, 63);
}
__device__ __forceinline__ int wave_sum_ui(int v)
{
    v += dpp_i<0xB1, 0xF, true>(0, v);
    v += dpp_i<0x4E, 0xF, true>(0, v);
    v += dpp_i<0x141, 0xF, true>(0, v);
    v += dpp_i<0x140, 0xF, true>(0, v);
    v += dpp_i<0x142, 0xA>(0, v);
    v += dpp_i<0x143, 0xC>(0, v);
    return __builtin_amdgcn_readlane(v, 63);
}
__device__ __forceinline__ float wave_sum_u(float v)
{
    auto f = [](int x) { return __builtin_bit_cast(float, x); };
    auto i = [](float x) { return __builtin_bit_cast(int, x); };
    v += f(dpp_i<0xB1, 0xF, true>(0, i(v)));
    v += f(dpp_i<0x4E, 0xF, true>(0, i(v)));
    v += f(dpp_i<0x141, 0xF, true>(0, i(v)));
    v += f(dpp_i<0x140, 0xF, true>(0, i(v)));
    v += f(dpp_i<0x142, 0xA>(0, i(v)));
    v += f(dpp_i<0x143, 0xC>(0, i(v)));
    return f(__builtin_amdgcn_readlane(i(v), 63));
}
// Order-preserving map of non-NaN floats to int32 (an involution): flips the
// magnitude bits of negative values, so integer max is float max.
__device__ __forceinline__ int f2ord(float x)
{
    const int b = __builtin_bit_cast(int, x);
    return b ^ ((b >> 31) & 0x7FFFFFFF);
}
__device__ __forceinline__ float ord2f(int k) { return __builtin_bit_cast(float, k ^ ((k >> 31) & 0x7FFFFFFF)); }
__device__ __forceinline__ float wave_max_u(float v) { return ord2f(wave_max_ui(f2ord(v))); }
// Maximum over each 16-lane row (the four in-row steps above): every lane
// ends with its row's maximum.  All 64 lanes must be active.
__device__ __forceinline__ float row_max_u(float x)
{
    int v = f2ord(x);
    v = max(v, dpp_i<0xB1, 0xF, true>(0, v));
    v = max(v, dpp_i<0x4E, 0xF, true>(0, v));
    v = max(v, dpp_i<0x141, 0xF, true>(0, v));
    v = max(v, dpp_i<0x140, 0xF, true>(0, v));
    return ord2f(v);
}

// ------------------------------------------------------ matrix cores
// v_mfma_i32_16x16x64_i8: D = A B + C for a 16 x 64 int8 A, a 64 x 16 int8
// B and 16 x 16 int32 C / D.  Lane l holds 16 bytes of row l % 16 of A and
// the same 16 k indices of column l % 16 of B (the k indices depend only on
// l / 16), and D[4 (l / 16) + i][l % 16] in element i of its result.
typedef int i32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4_t mfma_i8(i32x4_t a, i32x4_t b, i32x4_t c)
{
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

} // namespace kvq
