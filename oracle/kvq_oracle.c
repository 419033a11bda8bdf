/*
 * kvq_oracle.c -- plain, slow CPU oracle for the quantized-KV decode path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library calls, links or
 * includes this file.  Only the test suite, the smoke check and the bench's
 * CPU-baseline leg load it.  It shares no code, header, table or constant
 * with the HIP kernels.
 *
 * Everything is written for a reader checking it against the pages by eye:
 * one loop per definition, float64 wherever the pages do not fix a precision,
 * no blocking, no fusion, no reordering.
 *
 * Sources (page, then the part of it followed):
 *   [MNI]  donniechu.com, "KV cache INT8 35x speedup (Rust + CUDA)":
 *          "Cach KV cache tao ra toc do" (one new K and one new V per step,
 *          older K/V reused) and "Tai sao INT8 ma khong mat toc" /
 *          "Limitations" (symmetric INT8 with a scale).
 *   [TL]   TinyLoop docs, "KV Cache 模式": five-modes table (INT8 KV = int8
 *          vectors plus one FP16 scale per head; INT4 symmetric has 15
 *          levels, INT8 255; nibble-packed) and the memory-formula table.
 *   [KVS]  hada.io, "KVSplit": separate key / value bit widths (K8V8, K8V4,
 *          K4V4) and the 8K-token memory comparison.
 *   [OD]   gyaansetu.com, on-device KV-cache quantization: sliding-window
 *          eviction keeping the 1536 most recent tokens plus the first 64 as
 *          anchors.
 *   [AIH]  aihot.vn KV Cache tag page: Q is used only at the current position.
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *   - fp16 encoding is IEEE-754 binary16 round-to-nearest-even with
 *     subnormals; a *scale* that would overflow saturates to 65504.
 *   - scale = fp16(amax / qmax) with the division done in IEEE fp32; codes
 *     are rint_even(x / scale) in IEEE fp32 against the *stored* fp16 scale,
 *     clamped to [-qmax, qmax] (qmax 127 for 255 levels, 7 for 15 levels).
 *   - int4 packing puts the even element in the low nibble, two's complement.
 *   - attention is softmax(scale * q.K^T) V over the attended positions, the
 *     newest position included; default scale 1/sqrt(head_dim).
 *   - query head hq reads KV head hq / (n_q_heads / n_kv_heads).
 *   - the asymmetric (zero-point) codec [MNI: scale/zero-point metadata]:
 *     per group, the range [lo, hi] = [min(0, min x), max(0, max x)] (zero
 *     always representable), scale = fp16(RN((hi - lo) / L)) with L = 255 or
 *     15 levels, zero point z = clamp(rint(-lo / scale), 0, L), code =
 *     clamp(rint(x / scale) + z, 0, L), all quotients IEEE fp32; value =
 *     (code - z) * scale.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ */
/* IEEE-754 binary16, written from the format definition.              */
/* ------------------------------------------------------------------ */

/* Value of a binary16 bit pattern, exactly, as a double. */
double oq_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int m = h & 0x3FF;
    double v;
    if (e == 0x1F)
        v = m ? NAN : INFINITY;
    else if (e == 0)
        v = ldexp((double)m, -24);                 /* subnormal: m * 2^-24 */
    else
        v = ldexp((double)(1024 + m), e - 25);      /* (1.m) * 2^(e-15)    */
    return sign ? -v : v;
}

/*
 * Nearest binary16 to a float32, ties to even, subnormals kept, overflow to
 * +-inf, NaN to a quiet NaN.
 *
 * |x| is an integer significand S times 2^P.  The binary16 grid around |x|
 * has spacing 2^k with k = max(floor(log2|x|) - 10, -24) (10 fraction bits;
 * below 2^-14 the grid is the subnormal spacing 2^-24).  The result is
 * round_even(|x| / 2^k) * 2^k, encoded.  The encoding of M * 2^k is the
 * integer ((k + 24) << 10) + M for every k >= -24: for k = -24 this is the
 * subnormal (or first binade) pattern M, and for larger k the implicit
 * leading 1 of M (= 1024) adds exactly one to the exponent field, which is
 * (k + 10) + 15.  A carry of M to 2048 moves into the exponent the same way.
 */
uint16_t oq_f16_from_f32(float x)
{
    uint32_t u;
    memcpy(&u, &x, 4);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    uint32_t ef = (u >> 23) & 0xFFu;        /* float32 biased exponent */
    uint32_t mf = u & 0x7FFFFFu;            /* float32 fraction        */

    if (ef == 0xFF)                          /* inf or NaN */
        return (uint16_t)(sign | (mf ? 0x7E00u : 0x7C00u));
    if (ef < 102)                            /* |x| < 2^-25: rounds to 0 */
        return sign;

    /* ef >= 102 implies a normal float32: S = 1.mf as an integer, P = ef-150 */
    uint32_t S = 0x800000u | mf;
    int P = (int)ef - 150;
    int floor_log2 = (int)ef - 127;
    int k = floor_log2 - 10;
    if (k < -24)
        k = -24;
    int drop = k - P;                        /* bits of S below the grid: 13..24 */
    uint32_t M = S >> drop;
    uint32_t rem = S & ((1u << drop) - 1u);
    uint32_t half = 1u << (drop - 1);
    if (rem > half || (rem == half && (M & 1u)))
        M += 1;                              /* round to nearest, ties to even */

    uint32_t bits = ((uint32_t)(k + 24) << 10) + M;
    if (bits >= 0x7C00u)                     /* overflow: +-inf */
        bits = 0x7C00u;
    return (uint16_t)(sign | bits);
}

/* fp16 encoding for a scale: as above, but a scale too large for binary16
 * saturates to the largest finite value 65504 (0x7BFF) instead of inf. */
uint16_t oq_f16_scale_from_f32(float s)
{
    uint16_t h = oq_f16_from_f32(s);
    if ((h & 0x7FFFu) == 0x7C00u)
        h = (uint16_t)((h & 0x8000u) | 0x7BFFu);
    return h;
}

/* ------------------------------------------------------------------ */
/* Symmetric quantization of one group [MNI, TL].                      */
/* ------------------------------------------------------------------ */

/* qmax for a code width: 255 levels -> 127, 15 levels -> 7 [TL five-modes
 * table, INT4-h row]. */
int oq_qmax(int bits)
{
    if (bits == 8) return 127;
    if (bits == 4) return 7;
    return 0;
}

/*
 * One group of g float32 values -> g integer codes in [-qmax, qmax] and one
 * fp16 scale (bit pattern).  Dequantized value = code * scale.
 */
void oq_quantize_group(const float *x, int g, int qmax, int8_t *codes, uint16_t *scale_bits)
{
    float amax = 0.0f;
    for (int i = 0; i < g; i++) {
        float a = fabsf(x[i]);
        if (a > amax)
            amax = a;
    }
    float s32 = amax / (float)qmax;                      /* IEEE fp32 divide */
    uint16_t sh = oq_f16_scale_from_f32(s32);
    float s = (float)oq_f16_to_f64(sh);                  /* the stored scale */
    *scale_bits = sh;
    for (int i = 0; i < g; i++) {
        if (s == 0.0f) {                                 /* all-zero group */
            codes[i] = 0;
            continue;
        }
        float r = x[i] / s;                              /* IEEE fp32 divide */
        float c = rintf(r);                              /* ties to even     */
        if (c > (float)qmax) c = (float)qmax;
        if (c < (float)-qmax) c = (float)-qmax;
        codes[i] = (int8_t)c;
    }
}

/* int4 packing: byte j holds element 2j in bits 0-3 and element 2j+1 in
 * bits 4-7, each as a 4-bit two's-complement number [TL: nibble-packed]. */
void oq_pack_int4(const int8_t *codes, int n, uint8_t *out)
{
    for (int j = 0; j < n / 2; j++)
        out[j] = (uint8_t)(((uint8_t)codes[2 * j] & 0x0Fu) | (((uint8_t)codes[2 * j + 1] & 0x0Fu) << 4));
}

void oq_unpack_int4(const uint8_t *in, int n, int8_t *codes)
{
    for (int j = 0; j < n / 2; j++) {
        int lo = in[j] & 0x0F, hi = (in[j] >> 4) & 0x0F;
        codes[2 * j] = (int8_t)(lo >= 8 ? lo - 16 : lo);
        codes[2 * j + 1] = (int8_t)(hi >= 8 ? hi - 16 : hi);
    }
}

/*
 * Encode one stored row of n values (n a multiple of g) the way the cache
 * holds it:
 *   bits 32: float32 copied;   bits 16: fp16 per element;
 *   bits 8 : one code byte per element + one fp16 scale per group of g;
 *   bits 4 : packed nibbles (n/2 bytes) + one fp16 scale per group of g.
 * `payload` receives n*bits/8 bytes; `scales` receives n/g fp16 patterns for
 * 8/4 bits and is untouched otherwise.  Returns 0, or -1 on a bad argument.
 */
int oq_encode_row(const float *x, int n, int g, int bits, uint8_t *payload, uint16_t *scales)
{
    if (bits == 32) {
        memcpy(payload, x, (size_t)n * 4);
        return 0;
    }
    if (bits == 16) {
        for (int i = 0; i < n; i++) {
            uint16_t h = oq_f16_from_f32(x[i]);
            memcpy(payload + 2 * (size_t)i, &h, 2);
        }
        return 0;
    }
    int qmax = oq_qmax(bits);
    if (qmax == 0 || g <= 0 || n % g != 0 || (bits == 4 && g % 2 != 0))
        return -1;
    int8_t *codes = (int8_t *)malloc((size_t)g);
    for (int grp = 0; grp < n / g; grp++) {
        oq_quantize_group(x + (size_t)grp * g, g, qmax, codes, &scales[grp]);
        if (bits == 8)
            memcpy(payload + (size_t)grp * g, codes, (size_t)g);
        else
            oq_pack_int4(codes, g, payload + (size_t)grp * g / 2);
    }
    free(codes);
    return 0;
}

/* Inverse of oq_encode_row: the stored row as exact float64 values. */
int oq_decode_row(const uint8_t *payload, const uint16_t *scales, int n, int g, int bits, double *out)
{
    if (bits == 32) {
        for (int i = 0; i < n; i++) {
            float f;
            memcpy(&f, payload + 4 * (size_t)i, 4);
            out[i] = (double)f;
        }
        return 0;
    }
    if (bits == 16) {
        for (int i = 0; i < n; i++) {
            uint16_t h;
            memcpy(&h, payload + 2 * (size_t)i, 2);
            out[i] = oq_f16_to_f64(h);
        }
        return 0;
    }
    if (oq_qmax(bits) == 0 || g <= 0 || n % g != 0)
        return -1;
    int8_t *codes = (int8_t *)malloc((size_t)n);
    if (bits == 8)
        memcpy(codes, payload, (size_t)n);
    else
        oq_unpack_int4(payload, n, codes);
    for (int i = 0; i < n; i++)
        out[i] = (double)codes[i] * oq_f16_to_f64(scales[i / g]);
    free(codes);
    return 0;
}

/* ------------------------------------------------------------------ */
/* Asymmetric (zero-point) quantization of one group [MNI].            */
/* ------------------------------------------------------------------ */

/* Code levels: 255 for 8 bits, 15 for 4 bits (codes 0 .. L). */
int oq_levels(int bits)
{
    if (bits == 8) return 255;
    if (bits == 4) return 15;
    return 0;
}

/*
 * One group of g float32 values -> g codes in [0, L], one fp16 scale (bit
 * pattern) and one integer zero point in [0, L].  Dequantized value =
 * (code - zero) * scale.  The range is widened to contain 0, so that 0 maps
 * to the zero point exactly.  A zero scale (an all-zero group, or a range
 * below the fp16 grid) gives codes 0 and zero point 0.
 */
void oq_quantize_group_asym(const float *x, int g, int levels, uint8_t *codes, uint16_t *scale_bits, uint8_t *zero)
{
    float lo = 0.0f, hi = 0.0f;
    for (int i = 0; i < g; i++) {
        if (x[i] < lo) lo = x[i];
        if (x[i] > hi) hi = x[i];
    }
    float span = hi - lo;                                /* IEEE fp32 */
    float s32 = span / (float)levels;                    /* IEEE fp32 divide */
    uint16_t sh = oq_f16_scale_from_f32(s32);
    float s = (float)oq_f16_to_f64(sh);                  /* the stored scale */
    *scale_bits = sh;
    if (s == 0.0f) {
        *zero = 0;
        for (int i = 0; i < g; i++) codes[i] = 0;
        return;
    }
    float zf = rintf(-lo / s);                           /* IEEE fp32 divide, ties to even */
    if (zf > (float)levels) zf = (float)levels;
    if (zf < 0.0f) zf = 0.0f;
    *zero = (uint8_t)zf;
    for (int i = 0; i < g; i++) {
        float c = rintf(x[i] / s) + zf;                  /* IEEE fp32 divide, ties to even */
        if (c > (float)levels) c = (float)levels;
        if (c < 0.0f) c = 0.0f;
        codes[i] = (uint8_t)c;
    }
}

/*
 * Encode one stored row of n values (n a multiple of g) with the asymmetric
 * codec: `payload` receives n*bits/8 bytes of codes (8 bits: one unsigned
 * byte per element; 4 bits: element 2j in the low nibble of byte j),
 * `scales` n/g fp16 patterns and `zeros` n/g zero points.  Returns 0, or -1
 * on a bad argument.
 */
int oq_encode_row_asym(const float *x, int n, int g, int bits, uint8_t *payload, uint16_t *scales, uint8_t *zeros)
{
    int L = oq_levels(bits);
    if (L == 0 || g <= 0 || n % g != 0 || (bits == 4 && g % 2 != 0))
        return -1;
    uint8_t *codes = (uint8_t *)malloc((size_t)g);
    for (int grp = 0; grp < n / g; grp++) {
        oq_quantize_group_asym(x + (size_t)grp * g, g, L, codes, &scales[grp], &zeros[grp]);
        if (bits == 8) {
            memcpy(payload + (size_t)grp * g, codes, (size_t)g);
        } else {
            uint8_t *dst = payload + (size_t)grp * g / 2;
            for (int j = 0; j < g / 2; j++)
                dst[j] = (uint8_t)((codes[2 * j] & 0x0Fu) | ((codes[2 * j + 1] & 0x0Fu) << 4));
        }
    }
    free(codes);
    return 0;
}

/* Inverse of oq_encode_row_asym: (code - zero) * scale, exactly in float64. */
int oq_decode_row_asym(const uint8_t *payload, const uint16_t *scales, const uint8_t *zeros, int n, int g, int bits,
                       double *out)
{
    if (oq_levels(bits) == 0 || g <= 0 || n % g != 0)
        return -1;
    for (int i = 0; i < n; i++) {
        int code = bits == 8 ? payload[i] : ((payload[i / 2] >> (4 * (i & 1))) & 0x0F);
        out[i] = (double)(code - (int)zeros[i / g]) * oq_f16_to_f64(scales[i / g]);
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* Cache accounting [TL memory-formula table].                         */
/* ------------------------------------------------------------------ */

/*
 * Bytes one token adds to one layer's cache: the K and V payloads
 * (n_kv_heads * head_dim values each at k_bits / v_bits) plus, for each
 * quantized side, one 2-byte fp16 scale per group of group_size values.
 * With group_size = head_dim this is the INT8-KV row of the table
 * (2*D*1 + 2*n_heads*2); with 16-bit sides it is the FP16-KV row (2*D*2).
 * Returns 0 for an invalid combination.
 */
size_t oq_bytes_per_token(int k_bits, int v_bits, int n_kv_heads, int head_dim, int group_size)
{
    if (n_kv_heads <= 0 || head_dim <= 0)
        return 0;
    size_t D = (size_t)n_kv_heads * (size_t)head_dim;
    int sides[2] = {k_bits, v_bits};
    size_t total = 0;
    for (int i = 0; i < 2; i++) {
        int b = sides[i];
        if (b != 32 && b != 16 && b != 8 && b != 4)
            return 0;
        if ((D * (size_t)b) % 8 != 0)
            return 0;
        total += D * (size_t)b / 8;
        if (b < 16) {
            if (group_size <= 0 || D % (size_t)group_size != 0)
                return 0;
            total += 2 * (D / (size_t)group_size);
        }
    }
    return total;
}

/*
 * The same with the asymmetric codec's metadata as this library stores it:
 * each quantized side keeps, per group, a 32-bit word (the fp16 scale and a
 * 16-bit field holding the zero point), so 4 bytes per group instead of 2.
 * asym == 0 is oq_bytes_per_token.
 */
size_t oq_bytes_per_token_zp(int k_bits, int v_bits, int n_kv_heads, int head_dim, int group_size, int asym)
{
    size_t sym = oq_bytes_per_token(k_bits, v_bits, n_kv_heads, head_dim, group_size);
    if (sym == 0 || !asym)
        return sym;
    size_t D = (size_t)n_kv_heads * (size_t)head_dim;
    size_t extra = 0;
    if (k_bits < 16) extra += 2 * (D / (size_t)group_size);
    if (v_bits < 16) extra += 2 * (D / (size_t)group_size);
    return sym + extra;
}

/* ------------------------------------------------------------------ */
/* Sliding window with anchors [OD], ring storage.                     */
/* ------------------------------------------------------------------ */

/* Storage slot of position pos: anchors keep their own slot; later
 * positions cycle through the `window` recent slots after them.  With
 * window == 0 the cache is linear (slot = pos). */
long oq_slot_of(long pos, int n_anchor, int window)
{
    if (window == 0 || pos < n_anchor)
        return pos;
    return n_anchor + (pos - n_anchor) % window;
}

/*
 * Positions the current query attends to once position t has been written:
 * all of 0..t without a window; with one, the first n_anchor positions and
 * the `window` most recent ones (t included), each counted once.  Writes
 * them in increasing order into `out` and returns how many.
 */
long oq_attended_positions(long t, int n_anchor, int window, long *out)
{
    long n = 0;
    if (window == 0) {
        for (long p = 0; p <= t; p++)
            out[n++] = p;
        return n;
    }
    for (long p = 0; p <= t; p++) {
        int is_anchor = p < n_anchor;
        int is_recent = p > t - window;
        if (is_anchor || is_recent)
            out[n++] = p;
    }
    return n;
}

/* ------------------------------------------------------------------ */
/* Softmax attention for one query head, float64.                      */
/* ------------------------------------------------------------------ */

/*
 * o = sum_t p_t * V[t] / sum_t p_t,  p_t = exp(z_t - max z),
 * z_t = scale * sum_c q[c] * K[t][c], over the n rows given.
 */
void oq_attend(const double *q, const double *K, const double *V, long n, int hd, double scale, double *o)
{
    for (int c = 0; c < hd; c++)
        o[c] = 0.0;
    if (n <= 0)
        return;
    double *z = (double *)malloc((size_t)n * sizeof(double));
    double zmax = -INFINITY;
    for (long t = 0; t < n; t++) {
        double dot = 0.0;
        for (int c = 0; c < hd; c++)
            dot += q[c] * K[(size_t)t * hd + c];
        z[t] = scale * dot;
        if (z[t] > zmax)
            zmax = z[t];
    }
    double denom = 0.0;
    for (long t = 0; t < n; t++) {
        double p = exp(z[t] - zmax);
        denom += p;
        for (int c = 0; c < hd; c++)
            o[c] += p * V[(size_t)t * hd + c];
    }
    for (int c = 0; c < hd; c++)
        o[c] /= denom;
    free(z);
}

/* ------------------------------------------------------------------ */
/* One decode step for one sequence, from the raw float32 K/V rows.    */
/* ------------------------------------------------------------------ */

/*
 * k_src, v_src: float32 [n_kv_heads][n_pos][head_dim], the rows produced at
 *   positions 0..n_pos-1 of one sequence (the newest is n_pos-1).
 * q: float32 [n_q_heads][head_dim], the current query.
 * Scale groups: group_size divides head_dim (groups inside one head), or
 *   group_size == n_kv_heads*head_dim (one scale for the whole row of all
 *   heads at a position).
 * Each attended row is encoded as the cache stores it (oq_encode_row),
 * decoded back exactly, and query heads [hq_begin, hq_end) attend over it.
 * out: float64 [hq_end-hq_begin][head_dim].  Returns 0, or -1 on bad input.
 */
/* One row of n values through the codec of one side and back (float64):
 * the symmetric codec, or the asymmetric one (asym != 0) on 8/4-bit sides. */
static int encode_decode(const float *x, int n, int g, int bits, int asym, uint8_t *payload, uint16_t *scales,
                         uint8_t *zeros, double *out)
{
    if (asym && bits < 16) {
        int rc = oq_encode_row_asym(x, n, g, bits, payload, scales, zeros);
        return rc | oq_decode_row_asym(payload, scales, zeros, n, g, bits, out);
    }
    int rc = oq_encode_row(x, n, g, bits, payload, scales);
    return rc | oq_decode_row(payload, scales, n, g, bits, out);
}

int oq_decode_step_zp(int k_bits, int v_bits, int group_size, int asym, int n_kv_heads, int head_dim,
                      int n_anchor, int window,
                      const float *k_src, const float *v_src, long n_pos,
                      const float *q, int n_q_heads, int hq_begin, int hq_end,
                      double softmax_scale, double *out);

int oq_decode_step(int k_bits, int v_bits, int group_size, int n_kv_heads, int head_dim,
                   int n_anchor, int window,
                   const float *k_src, const float *v_src, long n_pos,
                   const float *q, int n_q_heads, int hq_begin, int hq_end,
                   double softmax_scale, double *out)
{
    return oq_decode_step_zp(k_bits, v_bits, group_size, 0, n_kv_heads, head_dim, n_anchor, window, k_src, v_src,
                             n_pos, q, n_q_heads, hq_begin, hq_end, softmax_scale, out);
}

/* oq_decode_step with the codec chosen: asym != 0 encodes the 8/4-bit sides
 * with the asymmetric (zero-point) codec. */
int oq_decode_step_zp(int k_bits, int v_bits, int group_size, int asym, int n_kv_heads, int head_dim,
                      int n_anchor, int window,
                      const float *k_src, const float *v_src, long n_pos,
                      const float *q, int n_q_heads, int hq_begin, int hq_end,
                      double softmax_scale, double *out)
{
    if (n_kv_heads <= 0 || n_q_heads % n_kv_heads != 0 || hq_begin < 0 || hq_end > n_q_heads)
        return -1;
    if (oq_bytes_per_token(k_bits, v_bits, n_kv_heads, head_dim, group_size) == 0)
        return -1;
    int D = n_kv_heads * head_dim;
    int per_row = (group_size == D && group_size != head_dim);
    if (!per_row && (k_bits < 16 || v_bits < 16) && head_dim % group_size != 0)
        return -1;
    int G = n_q_heads / n_kv_heads;

    long *pos = (long *)malloc((size_t)(n_pos > 0 ? n_pos : 1) * sizeof(long));
    long n_att = n_pos > 0 ? oq_attended_positions(n_pos - 1, n_anchor, window, pos) : 0;

    float *row = (float *)malloc((size_t)D * sizeof(float));
    uint8_t *payload = (uint8_t *)malloc((size_t)D * 4);
    uint16_t *scales = (uint16_t *)malloc((size_t)D * sizeof(uint16_t));
    uint8_t *zeros = (uint8_t *)malloc((size_t)D);
    double *dec = (double *)malloc((size_t)D * sizeof(double));
    double *K = (double *)malloc((size_t)(n_att > 0 ? n_att : 1) * head_dim * sizeof(double));
    double *V = (double *)malloc((size_t)(n_att > 0 ? n_att : 1) * head_dim * sizeof(double));
    double *qd = (double *)malloc((size_t)head_dim * sizeof(double));
    int rc = 0;

    int last_kv = -1;
    for (int hq = hq_begin; hq < hq_end; hq++) {
        int kv = hq / G;
        if (kv != last_kv) {
            /* encode + decode every attended K and V row of this KV head */
            for (int side = 0; side < 2 && rc == 0; side++) {
                const float *src = side == 0 ? k_src : v_src;
                int bits = side == 0 ? k_bits : v_bits;
                double *dst = side == 0 ? K : V;
                for (long i = 0; i < n_att; i++) {
                    long p = pos[i];
                    if (per_row && bits < 16) {
                        /* one scale over the whole position row of all heads */
                        for (int h = 0; h < n_kv_heads; h++)
                            memcpy(row + (size_t)h * head_dim,
                                   src + ((size_t)h * n_pos + p) * head_dim, (size_t)head_dim * 4);
                        rc |= encode_decode(row, D, D, bits, asym, payload, scales, zeros, dec);
                        memcpy(dst + (size_t)i * head_dim, dec + (size_t)kv * head_dim,
                               (size_t)head_dim * sizeof(double));
                    } else {
                        int g = bits < 16 ? group_size : head_dim;
                        const float *r = src + ((size_t)kv * n_pos + p) * head_dim;
                        rc |= encode_decode(r, head_dim, g, bits, asym, payload, scales, zeros,
                                            dst + (size_t)i * head_dim);
                    }
                }
            }
            last_kv = kv;
        }
        for (int c = 0; c < head_dim; c++)
            qd[c] = (double)q[(size_t)hq * head_dim + c];
        oq_attend(qd, K, V, n_att, head_dim, softmax_scale, out + (size_t)(hq - hq_begin) * head_dim);
    }

    free(pos); free(row); free(payload); free(scales); free(zeros); free(dec); free(K); free(V); free(qd);
    return rc ? -1 : 0;
}

/* Bulk forms of the fp16 codec, for exhaustive checks. */
void oq_f16_from_f32_n(const float *x, size_t n, uint16_t *out)
{
    for (size_t i = 0; i < n; i++)
        out[i] = oq_f16_from_f32(x[i]);
}

void oq_f16_to_f64_n(const uint16_t *h, size_t n, double *out)
{
    for (size_t i = 0; i < n; i++)
        out[i] = oq_f16_to_f64(h[i]);
}
