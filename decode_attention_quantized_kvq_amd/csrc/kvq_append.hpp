// kvq_append.hpp -- quantize-and-store kernel for new K/V rows.
//
// Encodings (TinyLoop "KV Cache 模式", five-modes table; mni-ml page,
// symmetric INT8; KVSplit page, separate key / value widths):
//   32-bit side: the float32 value;  16-bit side: fp16 nearest-even;
//   8/4-bit side: per group of g values, amax = max|x|, s32 = amax/qmax in
//   IEEE fp32, stored scale = fp16 nearest-even of s32 (65504 when it would
//   overflow), code = clamp(rint_even(x / stored scale), -qmax, qmax), with
//   the divide correctly rounded (HIP's default fp32 division).
// Slots follow the on-device page's window with anchors (ring storage).
#pragma once

#include "kvq_device.hpp"

namespace kvq {

constexpr int APPEND_THREADS = 256;
constexpr int APPEND_ELEMS = 8;                                   // per thread
constexpr int APPEND_SPAN = APPEND_THREADS * APPEND_ELEMS;        // per block pass

struct AppendParams {
    const float *src[2];      // K, V: [batch][n_kv_heads][n_new][head_dim]
    uint8_t *codes[2];        // float sides: [batch][n_kv_heads][capacity][row bytes]
                              // K (8/4-bit): [batch][n_kv_heads][cap64/64][row bytes/16][64][16]
                              // V (8/4-bit): [batch][n_kv_heads][cap4/4][row bytes][4]
    uint16_t *scales[2];      // see kvq.h
    int bits[2];
    const int32_t *start_pos; // [batch]
    int n_kv_heads, head_dim, capacity, cap4, cap64, n_new, n_anchor, window;
    // storage: cap_u slots per storage unit (a sequence, or a page of
    // 1 << page_shift slots when page_shift > 0, found through block_table)
    int cap_u, page_shift, pages_per_seq, n_pages;
    const int32_t *block_table;
    int group;                // elements per scale
    int per_row;              // 1: one scale per position over all heads
};

// Slot of `pos` for a call whose rows run start .. start+n_new-1, or -1
// when the row is not stored (out of range, or evicted by a later row of
// the same call).
__device__ __forceinline__ int append_slot(const AppendParams &p, int start, int pos)
{
    if (pos < 0)
        return -1;
    if (p.window == 0)
        return pos < p.capacity ? pos : -1;
    if (pos < p.n_anchor)
        return pos;
    const int last = start + p.n_new - 1;
    if (last - pos >= p.window)
        return -1;
    return p.n_anchor + (pos - p.n_anchor) % p.window;
}

__device__ __forceinline__ uint16_t scale_bits_from_amax(float amax, float qmax)
{
    const float s32 = amax / qmax;                 // IEEE fp32 divide
    uint16_t h = f32_to_f16_bits(s32);
    if ((h & 0x7FFFu) == 0x7C00u)                  // would overflow: saturate
        h = 0x7BFFu;
    return h;
}

// 8 values -> 8 codes against stored scale s (s > 0), packed for `bits`.
__device__ __forceinline__ void encode8(const float (&x)[8], float s, float qmax, int bits, uint32_t &w0, uint32_t &w1)
{
    int c[8];
#pragma unroll
    for (int j = 0; j < 8; j++) {
        float r = (s > 0.0f) ? rintf(x[j] / s) : 0.0f;   // IEEE divide, ties to even
        r = fminf(fmaxf(r, -qmax), qmax);
        c[j] = (int)r;
    }
    if (bits == 8) {
        w0 = (uint32_t)(c[0] & 0xFF) | ((uint32_t)(c[1] & 0xFF) << 8) | ((uint32_t)(c[2] & 0xFF) << 16) |
             ((uint32_t)(c[3] & 0xFF) << 24);
        w1 = (uint32_t)(c[4] & 0xFF) | ((uint32_t)(c[5] & 0xFF) << 8) | ((uint32_t)(c[6] & 0xFF) << 16) |
             ((uint32_t)(c[7] & 0xFF) << 24);
    } else {
        uint32_t w = 0;
#pragma unroll
        for (int j = 0; j < 8; j++)
            w |= (uint32_t)(c[j] & 0xF) << (4 * j);   // element j in nibble j
        w0 = w;
        w1 = 0;
    }
}

__device__ __forceinline__ void load8(const float *src, float (&x)[8])
{
    const float4 a = reinterpret_cast<const float4 *>(src)[0];
    const float4 b = reinterpret_cast<const float4 *>(src)[1];
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

// Store 8 encoded values (w0, w1 as packed by encode8) of row `slot`,
// starting at value c0.  8/4-bit keys are stored in tiles of 64 slots,
// slice-major (byte j of the row of slot s at ((s & ~63) * row + (j / 16) *
// 1024 + (s & 63) * 16 + j % 16)), so one 16-byte slice of 64 consecutive
// rows is contiguous; 8/4-bit values are stored offset binary (code + 128
// per byte, code + 8 per nibble) and four positions interleaved per byte
// (byte j of the row of slot s at ((s & ~3) * row + 4 * j + (s & 3))), so a
// 32-bit word holds one byte position of four consecutive positions.
__device__ __forceinline__ void store_codes(uint8_t *codes, size_t unit, int cap4, int cap64, int slot, int row_bytes,
                                            int c0, int bits, bool interleave, uint32_t w0, uint32_t w1)
{
    if (!interleave) {
        const int j0 = bits == 8 ? c0 : c0 / 2;     // first byte (8 or 4 bytes, inside one 16-byte slice)
        uint8_t *dst = codes + (unit * cap64 + (slot & ~63)) * (size_t)row_bytes + (j0 >> 4) * 1024 + (slot & 63) * 16 +
                       (j0 & 15);
        if (bits == 8)
            *reinterpret_cast<uint2 *>(dst) = make_uint2(w0, w1);
        else
            *reinterpret_cast<uint32_t *>(dst) = w0;
        return;
    }
    const uint32_t ob = bits == 8 ? 0x80808080u : 0x88888888u;   // offset binary
    w0 ^= ob;
    w1 ^= ob;
    uint8_t *grp = codes + (unit * cap4 + (slot & ~3)) * (size_t)row_bytes + (slot & 3);
    const int j0 = bits == 8 ? c0 : c0 / 2;
    const int nb = bits == 8 ? 8 : 4;
#pragma unroll
    for (int j = 0; j < 8; j++) {
        if (j < nb) {
            const uint32_t w = j < 4 ? w0 : w1;
            grp[(size_t)(j0 + j) * 4] = (uint8_t)(w >> (8 * (j & 3)));
        }
    }
}

// One block of the append grid: x = batch * n_new rows, y = passes over the
// row (groups inside a head) or 1 (per-row scale), z = side (0 = K, 1 = V).
// 256 threads; block-uniform early exits only.
__device__ __forceinline__ void append_block(const AppendParams &p, int bx, int by, int side)
{
    const int r = bx;
    const int b = r / p.n_new;
    const int i = r - b * p.n_new;
    const int start = p.start_pos[b];
    const int lslot = append_slot(p, start, start + i);
    if (lslot < 0)
        return;                                        // uniform over the block
    // storage unit (sequence or page) and slot inside it
    int ub = b, slot = lslot;
    if (p.page_shift > 0) {
        ub = p.block_table[(size_t)b * p.pages_per_seq + (lslot >> p.page_shift)];
        if (ub < 0 || ub >= p.n_pages)
            return;                                    // no page: not stored
        slot = lslot & ((1 << p.page_shift) - 1);
    }

    const int bits = p.bits[side];
    const int HD = p.head_dim;
    const int R = p.n_kv_heads * HD;
    const float *src = p.src[side];
    uint8_t *codes = p.codes[side];
    uint16_t *scales = p.scales[side];
    const float qmax = bits == 8 ? 127.0f : 7.0f;
    const int tid = threadIdx.x;

    if (p.per_row && bits < 16) {
        // one scale over the whole row of all heads: block-wide amax first
        __shared__ float red[APPEND_THREADS / 64];
        float amax = 0.0f;
        for (int e0 = tid * APPEND_ELEMS; e0 < R; e0 += APPEND_SPAN) {
            const int h = e0 / HD, c0 = e0 - h * HD;
            float x[8];
            load8(src + (((size_t)(b * p.n_kv_heads + h) * p.n_new + i) * HD + c0), x);
#pragma unroll
            for (int j = 0; j < 8; j++)
                amax = fmaxf(amax, fabsf(x[j]));
        }
        amax = wave_max(amax);
        if ((tid & 63) == 0)
            red[tid >> 6] = amax;
        __syncthreads();
        amax = red[0];
#pragma unroll
        for (int w = 1; w < APPEND_THREADS / 64; w++)
            amax = fmaxf(amax, red[w]);
        const uint16_t sh = scale_bits_from_amax(amax, qmax);
        const float s = f16_bits_to_f32(sh);
        if (tid == 0)
            scales[(size_t)ub * p.cap_u + slot] = sh;
        for (int e0 = tid * APPEND_ELEMS; e0 < R; e0 += APPEND_SPAN) {
            const int h = e0 / HD, c0 = e0 - h * HD;
            float x[8];
            load8(src + (((size_t)(b * p.n_kv_heads + h) * p.n_new + i) * HD + c0), x);
            uint32_t w0, w1;
            encode8(x, s, qmax, bits, w0, w1);
            store_codes(codes, (size_t)ub * p.n_kv_heads + h, p.cap4, p.cap64, slot, HD * bits / 8, c0, bits,
                        side == 1, w0, w1);
        }
        return;
    }

    const int e0 = (by * APPEND_THREADS + tid) * APPEND_ELEMS;
    const bool active = e0 < R;
    const int h = active ? e0 / HD : 0;
    const int c0 = active ? e0 - h * HD : 0;
    float x[8];
    if (active)
        load8(src + (((size_t)(b * p.n_kv_heads + h) * p.n_new + i) * HD + c0), x);
    else
#pragma unroll
        for (int j = 0; j < 8; j++) x[j] = 0.0f;
    const size_t row = ((size_t)ub * p.n_kv_heads + h) * p.cap_u + slot;

    if (bits == 32) {
        if (active) {
            float4 *dst = reinterpret_cast<float4 *>(codes + row * (size_t)(HD * 4) + (size_t)c0 * 4);
            dst[0] = make_float4(x[0], x[1], x[2], x[3]);
            dst[1] = make_float4(x[4], x[5], x[6], x[7]);
        }
        return;
    }
    if (bits == 16) {
        if (active) {
            uint32_t w[4];
#pragma unroll
            for (int j = 0; j < 4; j++)
                w[j] = (uint32_t)f32_to_f16_bits(x[2 * j]) | ((uint32_t)f32_to_f16_bits(x[2 * j + 1]) << 16);
            *reinterpret_cast<uint4 *>(codes + row * (size_t)(HD * 2) + (size_t)c0 * 2) = make_uint4(w[0], w[1], w[2], w[3]);
        }
        return;
    }

    // groups of p.group values inside a head: p.group / 8 consecutive lanes
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; j++)
        amax = fmaxf(amax, fabsf(x[j]));
    const int lanes = p.group / APPEND_ELEMS;
    for (int m = 1; m < lanes; m <<= 1)
        amax = fmaxf(amax, shfl_xor(amax, m));
    const uint16_t sh = scale_bits_from_amax(amax, qmax);
    const float s = f16_bits_to_f32(sh);
    uint32_t w0, w1;
    encode8(x, s, qmax, bits, w0, w1);
    if (!active)
        return;
    store_codes(codes, (size_t)ub * p.n_kv_heads + h, p.cap4, p.cap64, slot, HD * bits / 8, c0, bits, side == 1,
                w0, w1);
    if (c0 % p.group == 0)
        scales[row * (size_t)(HD / p.group) + c0 / p.group] = sh;
}

__global__ __launch_bounds__(APPEND_THREADS) void append_kernel(AppendParams p)
{
    append_block(p, blockIdx.x, blockIdx.y, blockIdx.z);
}

} // namespace kvq
