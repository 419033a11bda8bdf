// kvq_append.hpp -- quantize-and-store kernel for new K/V rows.
//
// Encodings (TinyLoop "KV Cache 模式", five-modes table; mni-ml page,
// symmetric INT8; KVSplit page, separate key / value widths):
//   32-bit side: the float32 value;  16-bit side: fp16 nearest-even;
//   8/4-bit side: per group of g values, amax = max|x|, s32 = amax/qmax in
//   IEEE fp32, stored scale = fp16 nearest-even of s32 (65504 when it would
//   overflow), code = clamp(rint_even(x / stored scale), -qmax, qmax), with
//   the divide correctly rounded (HIP's default fp32 division).
//   8/4-bit side with a zero point (the scale/zero-point metadata the
//   mni-ml page names): per group, lo = min(0, min x), hi = max(0, max x),
//   stored scale = fp16(RN((hi - lo) / L)), L = 255 or 15 levels, zero =
//   clamp(rint(-lo / scale), 0, L), code = clamp(rint(x / scale) + zero,
//   0, L); the scale and the zero point share one 32-bit word.
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
    int zp;                   // 1: zero-point codec (scales are 32-bit words: fp16 scale | zero << 16)
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

// One code: clamp(rint_even(x / s), -qmax, qmax), decided by the IEEE fp32
// quotient RN(x / s); a zero scale (an all-zero or vanishing group) gives
// code 0.  rs = v_rcp_f32(s), relative error <= 2^-22, so q = RN(x * rs)
// has relative error <= 2^-22 + 2^-24 < 3e-7 against x / s.  The stored scale
// is the fp16 rounding of amax / qmax, so |x / s| <= 1.5 * qmax < 192 (the
// worst case is an fp16 subnormal rounded down), q is within 5.8e-5 of x / s
// and RN(x / s) within half an ulp (7.6e-6): q and RN(x / s) differ by less
// than 6.6e-5, and unless q is within 1e-4 of a half-integer both round to
// the same integer.  Those rare cases take the IEEE divide itself.  (A scale
// saturated at 65504 allows larger quotients, but beyond 192 the code is
// clamped either way.)
__device__ __forceinline__ int code_of(float x, float s, float rs, float qmax)
{
    const float q = x * rs;
    float r = rintf(q);
    if (fabsf(q - r) > 0.5f - 1.0e-4f) r = rintf(x / (s > 0.0f ? s : 1.0f));
    return (int)(s > 0.0f ? fminf(fmaxf(r, -qmax), qmax) : 0.0f);
}

// the reciprocal code_of takes (1 for a zero scale, whose codes are 0)
__device__ __forceinline__ float code_rcp(float s) { return __builtin_amdgcn_rcpf(s > 0.0f ? s : 1.0f); }

// rint(RN(x / s)) for s > 0, decided as code_of decides it: valid while
// |x / s| < 256 (then q is within 9.2e-5 of RN(x / s), inside the 1e-4 tie
// margin); beyond, only the side of the result matters to the callers,
// which clamp to [0, L] with L <= 255.
__device__ __forceinline__ float rint_quot(float x, float s, float rs)
{
    const float q = x * rs;
    float r = rintf(q);
    if (fabsf(q - r) > 0.5f - 1.0e-4f) r = rintf(x / s);
    return r;
}

// The zero-point codec of one group, given hi = max(0, max x) and m2 =
// max(0, -min x) = -lo over the group: the 32-bit scale word (fp16 scale |
// zero << 16), the scale and the zero point.
__device__ __forceinline__ uint32_t zp_word(float hi, float m2, float L, float &sc, float &zf)
{
    const float s32 = (hi + m2) / L;               // RN(hi - lo) / L, IEEE fp32
    uint16_t sh = f32_to_f16_bits(s32);
    if ((sh & 0x7FFFu) == 0x7C00u) sh = 0x7BFFu;   // would overflow: saturate
    sc = f16_bits_to_f32(sh);
    zf = 0.0f;
    if (sc > 0.0f) zf = fminf(fmaxf(rint_quot(m2, sc, code_rcp(sc)), 0.0f), L);
    return (uint32_t)sh | ((uint32_t)zf << 16);
}

// One zero-point code, less 2^(bits-1) (so it packs like a signed code: the
// keys' stored field is its two's complement, the values' its offset binary,
// which is the code itself).
__device__ __forceinline__ int zp_code(float x, float sc, float rs, float zf, float L, int half)
{
    if (!(sc > 0.0f)) return -half;
    return (int)fminf(fmaxf(rint_quot(x, sc, rs) + zf, 0.0f), L) - half;
}

// 8 values -> 8 zero-point codes (less 2^(bits-1)), packed like encode8.
__device__ __forceinline__ void encode8_zp(const float (&x)[8], float sc, float zf, int bits, uint32_t &w0, uint32_t &w1)
{
    const float L = bits == 8 ? 255.0f : 15.0f;
    const int half = bits == 8 ? 128 : 8;
    const float rs = code_rcp(sc);
    int c[8];
#pragma unroll
    for (int j = 0; j < 8; j++) c[j] = zp_code(x[j], sc, rs, zf, L, half);
    if (bits == 8) {
        w0 = (uint32_t)(c[0] & 0xFF) | ((uint32_t)(c[1] & 0xFF) << 8) | ((uint32_t)(c[2] & 0xFF) << 16) |
             ((uint32_t)(c[3] & 0xFF) << 24);
        w1 = (uint32_t)(c[4] & 0xFF) | ((uint32_t)(c[5] & 0xFF) << 8) | ((uint32_t)(c[6] & 0xFF) << 16) |
             ((uint32_t)(c[7] & 0xFF) << 24);
    } else {
        uint32_t w = 0;
#pragma unroll
        for (int j = 0; j < 8; j++) w |= (uint32_t)(c[j] & 0xF) << (4 * j);
        w0 = w;
        w1 = 0;
    }
}

// 8 values -> 8 codes against stored scale s (s > 0), packed for `bits`.
__device__ __forceinline__ void encode8(const float (&x)[8], float s, float qmax, int bits, uint32_t &w0, uint32_t &w1)
{
    int c[8];
    const float rs = code_rcp(s);
#pragma unroll
    for (int j = 0; j < 8; j++) c[j] = code_of(x[j], s, rs, qmax);
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

// Maximum over aligned groups of `lanes` (1, 2, 4, ..., 32) lanes of values >= 0,
// in every lane of the group.  Non-negative floats order like their bit
// patterns, so an integer max is exact; inside a 16-lane row DPP steps
// (quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror)
// leave each lane with its 2-, 4-, 8- and 16-lane maximum.  For 32 lanes,
// v_permlane16_swap with v as both operands returns (v with its odd rows
// replaced by the even rows below them, v with its even rows replaced by
// the odd rows above them): their max is max(v[i], v[i ^ 16]) in every lane.
// All 64 lanes must be active.
__device__ __forceinline__ float group_max_abs(float a, int lanes)
{
    int v = __float_as_int(a);
    if (lanes >= 2) v = max(v, dpp_i<0xB1, 0xF, true>(0, v));
    if (lanes >= 4) v = max(v, dpp_i<0x4E, 0xF, true>(0, v));
    if (lanes >= 8) v = max(v, dpp_i<0x141, 0xF, true>(0, v));
    if (lanes >= 16) v = max(v, dpp_i<0x140, 0xF, true>(0, v));
    if (lanes >= 32) {
        const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        v = max((int)r[0], (int)r[1]);
    }
    return __int_as_float(v);
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
        // one scale over the whole row of all heads: block-wide maxima first
        // (amax; or, with a zero point, max(0, max x) and max(0, -min x))
        __shared__ float red[2][APPEND_THREADS / 64];
        float amax = 0.0f, m2 = 0.0f;
        for (int e0 = tid * APPEND_ELEMS; e0 < R; e0 += APPEND_SPAN) {
            const int h = e0 / HD, c0 = e0 - h * HD;
            float x[8];
            load8(src + (((size_t)(b * p.n_kv_heads + h) * p.n_new + i) * HD + c0), x);
#pragma unroll
            for (int j = 0; j < 8; j++) {
                amax = fmaxf(amax, p.zp ? x[j] : fabsf(x[j]));
                m2 = fmaxf(m2, -x[j]);
            }
        }
        amax = wave_max(amax);
        m2 = wave_max(m2);
        if ((tid & 63) == 0) {
            red[0][tid >> 6] = amax;
            red[1][tid >> 6] = m2;
        }
        __syncthreads();
        amax = red[0][0];
        m2 = red[1][0];
#pragma unroll
        for (int w = 1; w < APPEND_THREADS / 64; w++) {
            amax = fmaxf(amax, red[0][w]);
            m2 = fmaxf(m2, red[1][w]);
        }
        float s, zf = 0.0f;
        if (p.zp) {
            const uint32_t word = zp_word(amax, m2, bits == 8 ? 255.0f : 15.0f, s, zf);
            if (tid == 0) reinterpret_cast<uint32_t *>(scales)[(size_t)ub * p.cap_u + slot] = word;
        } else {
            const uint16_t sh = scale_bits_from_amax(amax, qmax);
            s = f16_bits_to_f32(sh);
            if (tid == 0) scales[(size_t)ub * p.cap_u + slot] = sh;
        }
        for (int e0 = tid * APPEND_ELEMS; e0 < R; e0 += APPEND_SPAN) {
            const int h = e0 / HD, c0 = e0 - h * HD;
            float x[8];
            load8(src + (((size_t)(b * p.n_kv_heads + h) * p.n_new + i) * HD + c0), x);
            uint32_t w0, w1;
            if (p.zp) encode8_zp(x, s, zf, bits, w0, w1);
            else encode8(x, s, qmax, bits, w0, w1);
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
    uint32_t w0, w1;
    uint32_t word;
    if (p.zp) {
        float hi = 0.0f, m2 = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; j++) {
            hi = fmaxf(hi, x[j]);
            m2 = fmaxf(m2, -x[j]);
        }
        hi = group_max_abs(hi, p.group / APPEND_ELEMS);
        m2 = group_max_abs(m2, p.group / APPEND_ELEMS);
        float s, zf;
        word = zp_word(hi, m2, bits == 8 ? 255.0f : 15.0f, s, zf);
        encode8_zp(x, s, zf, bits, w0, w1);
    } else {
        float amax = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; j++)
            amax = fmaxf(amax, fabsf(x[j]));
        amax = group_max_abs(amax, p.group / APPEND_ELEMS);
        const uint16_t sh = scale_bits_from_amax(amax, qmax);
        word = sh;
        encode8(x, f16_bits_to_f32(sh), qmax, bits, w0, w1);
    }
    if (!active)
        return;
    store_codes(codes, (size_t)ub * p.n_kv_heads + h, p.cap4, p.cap64, slot, HD * bits / 8, c0, bits, side == 1,
                w0, w1);
    if (c0 % p.group == 0) {
        const size_t si = row * (size_t)(HD / p.group) + c0 / p.group;
        if (p.zp) reinterpret_cast<uint32_t *>(scales)[si] = word;
        else scales[si] = (uint16_t)word;
    }
}

// The call's rows of sequence b for KV head kvh whose slots lie in
// [lo, hi), both sides of an 8/4-bit cache, stored by the workgroup that then
// attends over those slots of (b, kvh): wave 0 the keys, wave 1 the values,
// lane l the values 8l .. 8l+7 of the row (waves 2 and 3 store nothing).
// The encoding, slots and layout are append_block's, value for value; with
// one scale per position over all heads each of the n_kv_heads workgroups
// that store a row of sequence b computes that scale from the whole row and
// stores the same bits.
template <int HD>
__device__ __forceinline__ void append_head_rows(const AppendParams &p, int b, int kvh, int lo, int hi)
{
    constexpr int LPH = HD / APPEND_ELEMS;             // lanes holding the head's row
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    if (wave >= 2 || p.n_new <= 0) return;             // wave-uniform
    const int side = wave;
    const int bits = p.bits[side];
    const float qmax = bits == 8 ? 127.0f : 7.0f;
    const int start = p.start_pos[b];
    const float *src = p.src[side];
    const int R = p.n_kv_heads * HD;
    const bool act = lane < LPH;
    const int c0 = act ? lane * APPEND_ELEMS : 0;
    for (int i = 0; i < p.n_new; i++) {
        const int lslot = append_slot(p, start, start + i);
        if (lslot < 0 || lslot < lo || lslot >= hi) continue;   // wave-uniform
        int ub = b, slot = lslot;
        if (p.page_shift > 0) {
            ub = p.block_table[(size_t)b * p.pages_per_seq + (lslot >> p.page_shift)];
            if (ub < 0 || ub >= p.n_pages) continue;   // no page: not stored
            slot = lslot & ((1 << p.page_shift) - 1);
        }
        float x[8];
        if (act)
            load8(src + (((size_t)(b * p.n_kv_heads + kvh) * p.n_new + i) * HD + c0), x);
        else
#pragma unroll
            for (int j = 0; j < 8; j++) x[j] = 0.0f;
        // amax (symmetric), or max(0, max x) and max(0, -min x) (zero point)
        float amax = 0.0f, m2 = 0.0f;
        if (p.per_row) {
            // one scale over the row of all heads
            for (int e0 = lane * APPEND_ELEMS; e0 < R; e0 += 64 * APPEND_ELEMS) {
                const int h = e0 / HD, c = e0 - h * HD;
                float y[8];
                load8(src + (((size_t)(b * p.n_kv_heads + h) * p.n_new + i) * HD + c), y);
#pragma unroll
                for (int j = 0; j < 8; j++) {
                    amax = fmaxf(amax, p.zp ? y[j] : fabsf(y[j]));
                    m2 = fmaxf(m2, -y[j]);
                }
            }
            amax = wave_max(amax);
            m2 = wave_max(m2);
        } else {
#pragma unroll
            for (int j = 0; j < 8; j++) {
                amax = fmaxf(amax, p.zp ? x[j] : fabsf(x[j]));
                m2 = fmaxf(m2, -x[j]);
            }
            amax = group_max_abs(amax, p.group / APPEND_ELEMS);
            m2 = group_max_abs(m2, p.group / APPEND_ELEMS);
        }
        uint32_t w0, w1, word;
        if (p.zp) {
            float sc, zf;
            word = zp_word(amax, m2, bits == 8 ? 255.0f : 15.0f, sc, zf);
            encode8_zp(x, sc, zf, bits, w0, w1);
        } else {
            const uint16_t sh = scale_bits_from_amax(amax, qmax);
            word = sh;
            encode8(x, f16_bits_to_f32(sh), qmax, bits, w0, w1);
        }
        if (!act) continue;
        const size_t unit = (size_t)ub * p.n_kv_heads + kvh;
        store_codes(p.codes[side], unit, p.cap4, p.cap64, slot, HD * bits / 8, c0, bits, side == 1, w0, w1);
        size_t si = SIZE_MAX;
        if (p.per_row) {
            if (lane == 0) si = (size_t)ub * p.cap_u + slot;
        } else if (c0 % p.group == 0) {
            si = (unit * p.cap_u + slot) * (size_t)(HD / p.group) + c0 / p.group;
        }
        if (si != SIZE_MAX) {
            if (p.zp) reinterpret_cast<uint32_t *>(p.scales[side])[si] = word;
            else p.scales[side][si] = (uint16_t)word;
        }
    }
}

// ------------------------------------------------------------------------
// Bulk appends (a prompt's rows in one call) into 8/4-bit caches without a
// window and with scales per head or per group: one workgroup per 64-slot
// tile of one (sequence, KV head, side).  The rows of a tile are contiguous
// in the input and the tile is contiguous in the cache (keys: one tile;
// values: 16 groups of four interleaved slots), so both streams move in
// whole 16-byte pieces; the encoding is the row kernel's, value for value.
// 256 threads = 64 rows x 4 quarters of a row.
// grid: x = tiles (the call's slots from start & ~63), y = batch * n_kv_heads,
// z = side.
// ------------------------------------------------------------------------
constexpr int TILE_ROWS = 64;

template <int HD, int BITS>
__device__ __forceinline__ void append_tile(const AppendParams &p, int tile, int bh, int side)
{
    constexpr int ROWB = HD * BITS / 8;            // code bytes per row
    constexpr int V4 = TILE_ROWS * HD / 4;         // float4 pieces of the tile's input
    constexpr int ROUNDS = V4 / 256;               // per thread
    constexpr int LPR = HD / 4;                    // lanes per row in a round
    static_assert(V4 % 256 == 0 && 64 % LPR == 0, "whole rows per wave and round");
    __shared__ __align__(16) uint8_t tb[TILE_ROWS * ROWB];   // the tile's codes in their cache layout

    const int b = bh / p.n_kv_heads, h = bh - b * p.n_kv_heads;
    const int start = p.start_pos[b];
    const int t0 = (start & ~(TILE_ROWS - 1)) + tile * TILE_ROWS;   // first slot (= position) of the tile
    const int lo = max(max(t0, start), 0), hi = min(min(t0 + TILE_ROWS, start + p.n_new), p.capacity);
    if (lo >= hi) return;                          // block-uniform
    int ub = b, slot0 = t0;                        // storage unit and the tile's first slot in it
    if (p.page_shift > 0) {
        ub = p.block_table[(size_t)b * p.pages_per_seq + (t0 >> p.page_shift)];
        if (ub < 0 || ub >= p.n_pages) return;     // no page: not stored
        slot0 = t0 & ((1 << p.page_shift) - 1);
    }
    const int tid = threadIdx.x;
    const float qmax = BITS == 8 ? 127.0f : 7.0f;
    const int g = p.group;                         // >= 32 values, divides head_dim
    // input rows t0 .. t0 + 63 are contiguous ([n_new][head_dim] per
    // sequence and head): round k, thread tid holds float4 piece k * 256 + tid,
    // row (k * 256 + tid) / LPR, channels 4 * ((k * 256 + tid) % LPR) ..
    const float *src = p.src[side] + (size_t)bh * p.n_new * HD;      // this sequence and head
    uint4 raw[ROUNDS];
#pragma unroll
    for (int k = 0; k < ROUNDS; k++) {
        const int e = k * 256 + tid, t = t0 + e / LPR;
        raw[k] = t >= lo && t < hi ? ld_u4_nt(src + (size_t)(t - start) * HD + 4 * (e % LPR)) : make_uint4(0, 0, 0, 0);
    }
    const uint32_t ob = side == 1 ? (BITS == 8 ? 0x80808080u : 0x88888888u) : 0u;   // values: offset binary
#pragma unroll
    for (int k = 0; k < ROUNDS; k++) {
        const int e = k * 256 + tid, r = e / LPR, c = 4 * (e % LPR);
        const float x[4] = {__uint_as_float(raw[k].x), __uint_as_float(raw[k].y), __uint_as_float(raw[k].z),
                            __uint_as_float(raw[k].w)};
        const float amax = group_max_abs(fmaxf(fmaxf(fabsf(x[0]), fabsf(x[1])), fmaxf(fabsf(x[2]), fabsf(x[3]))),
                                         g / 4);
        const uint16_t sh = scale_bits_from_amax(amax, qmax);
        const float sc = f16_bits_to_f32(sh), rs = code_rcp(sc);
        const int t = t0 + r;
        if (t >= lo && t < hi && c % g == 0)
            p.scales[side][(((size_t)ub * p.n_kv_heads + h) * p.cap_u + slot0 + r) * (size_t)(HD / g) + c / g] = sh;
        const int q0 = code_of(x[0], sc, rs, qmax), q1 = code_of(x[1], sc, rs, qmax);
        const int q2 = code_of(x[2], sc, rs, qmax), q3 = code_of(x[3], sc, rs, qmax);
        uint32_t w;                                // the 2 (int4) or 4 (int8) code bytes of c .. c + 3
        if constexpr (BITS == 8)
            w = (uint32_t)(q0 & 0xFF) | ((uint32_t)(q1 & 0xFF) << 8) | ((uint32_t)(q2 & 0xFF) << 16) |
                ((uint32_t)(q3 & 0xFF) << 24);
        else
            w = (uint32_t)(q0 & 0xF) | ((uint32_t)(q1 & 0xF) << 4) | ((uint32_t)(q2 & 0xF) << 8) |
                ((uint32_t)(q3 & 0xF) << 12);
        w ^= ob;
        const int j = c * BITS / 8;                // first code byte in the row
        if (side == 0) {
            // keys: byte j of row r at (j / 16) * 1024 + r * 16 + j % 16
            uint8_t *d = tb + (j >> 4) * 1024 + r * 16 + (j & 15);
            if constexpr (BITS == 8) *reinterpret_cast<uint32_t *>(d) = w;
            else *reinterpret_cast<uint16_t *>(d) = (uint16_t)w;
        } else {
            // values: byte j of row r at (r & ~3) * ROWB + 4 * j + (r & 3)
            uint8_t *d = tb + (r & ~3) * ROWB + 4 * j + (r & 3);
#pragma unroll
            for (int m = 0; m < BITS / 2; m++) d[4 * m] = (uint8_t)(w >> (8 * m));
        }
    }
    __syncthreads();
    // the tile in the cache: keys one 64-slot tile, values 16 groups of four
    // slots, both contiguous from the tile's first slot; 16-byte pieces
    uint8_t *base = p.codes[side] + ((size_t)ub * p.n_kv_heads + h) * (size_t)(side == 0 ? p.cap64 : p.cap4) * ROWB +
                    (size_t)slot0 * ROWB;
    for (int o = tid * 16; o < TILE_ROWS * ROWB; o += 256 * 16) {
        const uint4 v = *reinterpret_cast<const uint4 *>(tb + o);
        if (side == 0) {
            const int t = t0 + (o & 1023) / 16;    // a key piece is one slot's slice
            if (t >= lo && t < hi) *reinterpret_cast<uint4 *>(base + o) = v;
        } else {
            const int s4 = t0 + 4 * (o / (4 * ROWB));   // a value piece: 4 byte positions of one group
            if (s4 >= lo && s4 + 4 <= hi) {
                *reinterpret_cast<uint4 *>(base + o) = v;
            } else {
                // a group cut by the call's first or last row: its rows only
                const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int m = 0; m < 4; m++)
                    if (s4 + m >= lo && s4 + m < hi)
#pragma unroll
                        for (int e = 0; e < 4; e++) base[o + 4 * e + m] = (uint8_t)(wd[e] >> (8 * m));
            }
        }
    }
}

template <int HD, int KB, int VB>
__global__ __launch_bounds__(256) void append_tile_kernel(AppendParams p)
{
    if (blockIdx.z == 0) append_tile<HD, KB>(p, blockIdx.x, blockIdx.y, 0);
    else append_tile<HD, VB>(p, blockIdx.x, blockIdx.y, 1);
}

} // namespace kvq
