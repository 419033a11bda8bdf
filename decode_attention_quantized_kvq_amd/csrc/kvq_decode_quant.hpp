// kvq_decode_quant.hpp -- split-K decode attention when both K and V are
// stored as integer codes (8- or 4-bit) with fp16 scales.
//
// What is computed (TinyLoop "KV Cache 模式" five-modes table; KVSplit's
// separate key / value widths; the current query against every cached row,
// aihot.vn): for one (sequence, KV head) and the G query heads that read it,
// softmax attention over the rows of a context chunk, each row used as
// code * scale without ever being expanded in memory.  Decode is bound by
// memory bandwidth (mni-ml page, "why INT8 loses no speed"), so every cache
// byte is read once per step and shared by the G query heads.
//
// Arithmetic is integer wherever the data is: exact int32 dot products on
// the stored codes, with the two float quantities held as fixed point:
//  * the query, per head, as q_int = rint(q / s_q), s_q = max|q| / 30000,
//    split into balanced digits (four base-16 digits against int4 keys, two
//    base-256 digits against int8 keys) so v_dot8_i32_i4 / v_dot4_i32_i8
//    take the stored code words unchanged (digit-major Horner: one exact
//    int32 sum per head and position).  When some head of a (sequence, KV
//    head) has a channel beyond 5 times its rms (an outlier channel, which
//    would leave the others few bits), the query also carries one low digit
//    d = rint(14 (int4) or 254 (int8) * (q / s_q - q_int)) whose sum joins
//    the score in float; either way |dq| <= max|q| / 60000 <= |q|_2 / 12000
//    per channel, at most 8.3e-5 of |q|_2 in norm;
//  * the value weights w = 2^(z - max z) * s_v of a sub-chunk, per head and
//    scale group, as w_int = rint(w * 32767 / N), N the sub-chunk's largest
//    w, split into two unsigned bytes, so v_dot4_u32_u8 runs over four
//    positions at once against value codes stored four positions
//    interleaved and offset binary (code + 8 or code + 128, never negative);
//    the offset's share, bias * sum(w), is subtracted once at the end.
// Four or eight query heads at head_dim 128 (the symmetric codec) score
// their keys on the matrix cores instead (the integer dots above take 4 VALU
// instructions per position for the keys alone at G = 4, and the VALU was
// this kernel's busiest unit): per 16 positions two v_mfma_i32_16x16x64_i8
// (four with four scale groups) multiply a 16 x 64 operand holding the
// heads' two base-256 digits of q_int (and, for four heads, the extra low
// digit) with 64 channels of the 16 positions (int4 codes unpacked to bytes
// 16 code, int8 codes as stored), which gives the same exact integer sums;
// the VALU only unpacks nibbles and scales.  With int4 keys and values and
// one scale per head the value sums run there too: the weights as two
// signed bytes (w_int <= 32639), 8 products per 64 positions against the
// unpacked value nibbles.
// Rounding happens only in the query's digits and in w_int
// (|dw| <= N / 65534, or N / 65278, relative to the sub-chunk's own largest
// weight whatever the spread of the value scales or of the softmax);
// accumulation is exact in int32, then fp32.
//
// Workgroup = 4 waves = one context chunk of one (sequence, KV head); each
// wave owns a quarter of the chunk and streams it in sub-chunks of 512
// positions (fewer with many heads or scale groups), the key tiles and the
// value groups loaded ahead without a break between sub-chunks.  Per
// sub-chunk:
//   1. keys, one lane per position: scores -> LDS; the query digits are
//      wave-uniform and come from SGPRs (prepared per (sequence, KV head) by
//      qprep_kernel, or by the workgroup itself in the one-launch step; on
//      the matrix cores one lane per position and head, the digits held in
//      VGPRs as the product's A operand);
//      value scales -> LDS; the sub-chunk's score maxima (DPP).
//   2. weights, one lane per four positions: p = 2^(z - max) and the
//      products p * s_v, whose maximum per head and group (DPP) sets the
//      fixed point; then w_int packed four positions per word -> LDS (over
//      the sub-chunk's scores).
//   3. values: a lane owns fixed byte positions (two channels) of every
//      4-position group and accumulates v_dot4_u32_u8 over the sub-chunk's
//      groups (int4: the even channel's nibbles and the whole bytes, even +
//      16 * odd); the group's weight words are LDS broadcasts.
//   4. the integer sums become floats (byte split and fixed point undone)
//      and are merged into the wave's running (max, sum, acc) with the usual
//      2^(m - M) factors.
// At the end the 4 waves are merged the same way through LDS and the chunk's
// (m, l, acc) written.  LDS use does not depend on the chunk length.
#pragma once

#include <type_traits>

#include "kvq_append.hpp"
#include "kvq_combine.hpp"
#include "kvq_device.hpp"

namespace kvq {

constexpr int QD_THREADS = 256;
constexpr int QD_WAVES = QD_THREADS / 64;
// Positions per wave sub-chunk: 512 while G x vg < 8, else 256 (the maxima,
// merge and prologue then run half as often as at 128, and the compiler keeps
// the G = 4, vg = 4 loop in 156 VGPRs instead of 245); the zero-point codec's
// G x vg >= 16 (whose scale words take twice the LDS) takes 128, as 256
// would not fit the 64 KiB of LDS.  (G = 8 with 2 or 4 scale groups is not
// instantiated: its heads run as two workgroup heads of four.)
// (A sub-chunk's value sums stay exact in uint32: at most
// 512 * 32767 * 255 < 2^32.)
__host__ __device__ constexpr int qd_sub(int G, int vg, bool zp = false)
{
    return zp && G * vg >= 16 ? 128 : G * vg >= 8 ? 256 : 512;
}
constexpr int Q_RANGE = 30000;
// the query's extra low digit: taken when max|q| > Q_OUTLIER * rms(q) for a
// head of the unit; its base keeps |d| within the key width's signed digit
constexpr float Q_OUTLIER = 5.0f;
__host__ __device__ constexpr int qx_base(int KB) { return KB == 4 ? 14 : 254; }
// int32 words between two units' query digit blocks, padded to 256 bytes
// so that no two units share a cache line: the digits [ND + 1][K_COLS][G],
// then (for the zero-point codec) the query's integer sums per scale group,
// [QS_GROUPS][G] for q_int and [QS_GROUPS][G] for the extra low digit
constexpr int QS_GROUPS = 4;
__host__ __device__ constexpr int qd_digits(int KB, int HD, int G) { return ((KB == 4 ? 4 : 2) + 1) * (HD * KB / 32) * G; }
// Four or eight query heads at head_dim 128 score their keys on the matrix
// cores (v_mfma_i32_16x16x64_i8): the sixteen rows of the product are the
// four heads' low and high base-256 digits of q_int, their extra low digits
// and a zero row, or the eight heads' low and high digits.  The digit block
// then also holds that operand, one byte per digit, head and channel
// ([3][G][HD]).
__host__ __device__ constexpr bool qd_mfma(int HD, int G) { return (G == 4 || G == 8) && HD == 128; }
__host__ __device__ constexpr int qd_mf(int KB, int HD, int G) { return qd_digits(KB, HD, G) + 2 * QS_GROUPS * G; }
__host__ __device__ constexpr int qd_mf_words(int HD, int G) { return qd_mfma(HD, G) ? 3 * G * HD / 4 : 0; }
__host__ __device__ constexpr int qd_stride(int KB, int HD, int G)
{
    return (qd_mf(KB, HD, G) + qd_mf_words(HD, G) + 63) / 64 * 64;
}
constexpr int QD_PF = 16;       // value group loads in flight per lane
constexpr int W_RANGE = 32767;

template <int KB, int VB, int HD, int G> struct QT {
    static constexpr int K_ROW = HD * KB / 8;          // bytes per key row
    static constexpr int K_U4 = K_ROW / 16;            // 16-byte loads per key row
    static constexpr int K_COLS = K_ROW / 4;           // dwords per key row
    static constexpr int ND = KB == 4 ? 4 : 2;         // query digits (Horner)
    static constexpr int NDX = ND + 1;                 // digits stored: the Horner ones, then the extra low one
    static constexpr int DBASE = KB == 4 ? 16 : 256;   // digit base
    static constexpr int CPC = KB == 4 ? 8 : 4;        // channels per key dword
    static constexpr int V_ROW = HD * VB / 8;          // bytes per value row
    static constexpr int V_DW = V_ROW;                 // dwords per 4-position group
    static constexpr int V_DPL = V_DW >= 64 ? V_DW / 64 : 1;   // dwords per lane
    static constexpr int V_GPL = V_DW >= 64 ? 1 : 64 / V_DW;   // groups per wave load
    static constexpr int V_LPG = 64 / V_GPL;           // lanes per group
    static constexpr int V_CPD = VB == 4 ? 2 : 1;      // channels per dword
    static constexpr int V_ACC = V_DPL * V_CPD;        // channels per lane
    // cache policy of the code loads: keys always nontemporal; values too,
    // except beside int8 keys with int4 values, where nontemporal value
    // loads measured 2-3 % slower (int4 / int8 keys elsewhere: faster)
    static constexpr int V_CP = (KB == 8 && VB == 4) ? 0 : CP_NT;
};

// (Hkv below: n_kv_heads, the workgroup heads per sequence; the cache
// buffers have n_kv_cache heads)
struct QuantParams {
    const uint8_t *k_codes;    // [B][n_kv_cache][cap64/64][K_ROW/16][64][16]  (tiles of 64 slots, slice-major)
    const uint8_t *v_codes;    // [B][n_kv_cache][cap4/4][V_ROW][4]  (4 positions interleaved per byte)
    const uint16_t *k_scales;
    const uint16_t *v_scales;
    const int32_t *qdig;       // [B*Hkv][qd_stride] packed query digits: [ND + 1][K_COLS][G] (digit-major; digit ND the extra low one);
                               // the one-launch step: [B*Hkv][n_chunks][qd_stride], one slot per workgroup
    const float *qsc;          // [B*Hq]: s_q * softmax_scale * log2(e)
    const int32_t *qflag;      // [B*Hkv]: 1 when the query carries its extra low digit
    const int32_t *seq_len;
    float *ws_ml;
    float *ws_acc;
    int n_kv_heads, capacity, cap4, cap64;   // capacity, cap4, cap64: per storage unit (sequence or page)
    // the cache's KV heads: n_kv_cache = n_kv_heads >> kv_shift.  kv_shift 1:
    // the G query heads of each cache head are split over two workgroup
    // heads (grid.y = n_kv_heads, head kvh reading cache head kvh >> 1),
    // each a unit of its own for the query digits and ticket counters
    int n_kv_cache, kv_shift;
    // paged storage: slot s of sequence b in page block_table[b * pages_per_seq
    // + (s >> page_shift)] (paged kernels only)
    const int32_t *block_table;
    int page_shift, pages_per_seq, n_pages;
    int max_len;
    int chunk, n_chunks;
    // the in-kernel merge: after writing its partials each workgroup takes a
    // ticket on cnt[b * Hkv + kvh] (zero when the launch starts: zeroed by
    // the query preparation of a two-launch step, left zero by the previous
    // one-launch step) and the last one merges the G rows of its unit into
    // out, setting the counter back to zero.  cnt == nullptr: partials only.
    int *cnt;
    float *out;
    // one-launch decode step (step != 0; at most 2 chunks per (sequence, KV
    // head)): each workgroup first stores the step's rows of its head whose
    // slots fall in its chunk (the last chunk also takes those past it) (ap)
    // and prepares its query (q, qk_scale: digits into its own slot of
    // qdig, one per (sequence, KV head) and chunk; scales and flag kept in
    // registers); with one chunk it writes out instead of partials, with
    // more the last workgroup of the (sequence, KV head) merges (cnt)
    int step;
    AppendParams ap;
    const float *q;
    float qk_scale;
    long long k_sc_b, k_sc_h;
    int k_sc_t;
    long long v_sc_b, v_sc_h;
    int v_sc_t;
};

struct QuantSmem {
    int zs, vs, wd, red, misc, total;
    bool wd_alias;             // weight words overwrite each wave's own scores
    bool vs_in_wd;             // value scales sit in the tail of each 4-position block of weight words
};

// Per wave: scores [S][G] fp32, value scales [S][vg] fp16 bits (or 32-bit
// scale | zero words), weight words [S/4][vg][G][lo, hi] (over the scores
// when vg == 1); then the cross-wave merge area (over the scores when it
// fits) and the wave maxima, sums and merge factors.  With several scale groups and the
// symmetric codec the value scales of 4 positions ([4][vg] fp16) occupy the
// last 2 vg words of those positions' block of weight words, which only the
// lane that reads them later overwrites; this keeps the G = 4, vg = 4
// layout at 48 KiB, three workgroups a CU, where its own area (56 KiB) would
// allow two.
__host__ __device__ inline QuantSmem quant_smem(int G, int HD, int vg, bool zp = false)
{
    QuantSmem s;
    const int S = qd_sub(G, vg, zp);
    int off = 0;
    s.zs = off;
    off += QD_WAVES * S * G * 4;
    s.vs_in_wd = vg > 1 && !zp;
    s.vs = off;
    if (!s.vs_in_wd) off += QD_WAVES * S * vg * (zp ? 4 : 2);   // value scale (and zero point) words
    s.wd_alias = vg == 1;
    if (s.wd_alias) {
        s.wd = s.zs;
    } else {
        s.wd = off;
        off += QD_WAVES * vg * (S / 4) * G * 2 * 4;
    }
    const int red = QD_WAVES * G * HD * 4;
    if (QD_WAVES * S * G * 4 >= red) {
        s.red = s.zs;                              // scores and weights are dead by then
    } else {
        s.red = off;
        off += red;
    }
    s.misc = off;
    off += (3 * QD_WAVES + 2) * G * 4;             // wave maxima, sums and merge factors; merged max and sum
    s.total = off;
    return s;
}

// ---------------------------------------------------------------------------
// Query digits: one block per unit (sequence and KV head, or workgroup head
// when a KV head's query heads are split over two).  For head h of the group,
// s_q = max|q| / 30000 and q_int = rint(q / s_q) in [-30000, 30000], split
// into ND balanced digits; digit j of the channels of key dword `col` is
// packed like the codes (int4: channel 8col+i in nibble i; int8: channel
// 4col+i in byte i) at qdig[unit][j][col][h] (digit-major, the order the
// decode kernel reads them in).  When a head of the unit has
// max|q| > 5 rms(q), digit ND holds d = rint(base * (q / s_q - q_int)) for
// every head (base 14 or 254: |d| <= 7 or 127) and qflag[unit] = 1, else
// digit ND is zero and qflag[unit] = 0.
// ---------------------------------------------------------------------------
template <int KB, int HD, int G>
__device__ __forceinline__ void qprep_core(const float *__restrict__ qh, int32_t *__restrict__ qd, float *s_amax,
                                           int *s_xflag, float *s_qv, int kg)
{
    // qh: the unit's G query heads [G][HD]; qd: its digits [ND + 1][K_COLS][G];
    // s_amax [G], s_xflag, s_qv [G][HD]: LDS.  On return (after a barrier)
    // s_amax holds max|q| per head and s_xflag whether the extra digit is on.
    constexpr int K_COLS = HD * KB / 32;
    constexpr int ND = KB == 4 ? 4 : 2;
    constexpr int CPC = KB == 4 ? 8 : 4;
    constexpr int BITS = KB == 4 ? 4 : 8;
    constexpr int XMAX = (1 << (BITS - 1)) - 1;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (tid == 0) *s_xflag = 0;
    __syncthreads();
    for (int h = wave; h < G; h += 4) {
        float a = 0.0f, ss = 0.0f;
        for (int c = lane; c < HD; c += 64) {
            const float v = qh[h * HD + c];
            s_qv[h * HD + c] = v;
            a = fmaxf(a, fabsf(v));
            ss = fmaf(v, v, ss);
        }
        a = wave_max(a);
        ss = wave_sum(ss);
        if (lane == 0) {
            s_amax[h] = a;
            // max|q| > 5 rms(q): the 16-bit form would leave the other
            // channels too few bits
            if (a * a > Q_OUTLIER * Q_OUTLIER * (ss / (float)HD)) atomicOr(s_xflag, 1);
        }
    }
    __syncthreads();
    const bool xq = *s_xflag != 0;
    constexpr float XB = (float)qx_base(KB);
    for (int i = tid; i < K_COLS * G; i += 256) {
        const int col = i / G, h = i - col * G;
        const float sq = s_amax[h] / (float)Q_RANGE;
        const float inv = sq > 0.0f ? 1.0f / sq : 0.0f;
        uint32_t d[ND + 1];
#pragma unroll
        for (int j = 0; j <= ND; j++) d[j] = 0;
#pragma unroll
        for (int e = 0; e < CPC; e++) {
            const float qq = s_qv[h * HD + col * CPC + e];
            int qi = (int)fminf(fmaxf(rintf(qq * inv), -(float)Q_RANGE), (float)Q_RANGE);
            if (xq) {
                // the rest of q / s_q beyond q_int (one rounding), in 1/base units
                const float r = fmaf(qq, inv, -(float)qi);
                const int dx = (int)fminf(fmaxf(rintf(r * XB), -(float)XMAX), (float)XMAX);
                d[ND] |= (uint32_t)(dx & ((1 << BITS) - 1)) << (BITS * e);
            }
#pragma unroll
            for (int j = 0; j < ND; j++) {
                const int half = 1 << (BITS - 1), mask = (1 << BITS) - 1;
                const int dj = j < ND - 1 ? ((qi + half) & mask) - half : qi;   // balanced digit
                d[j] |= (uint32_t)(dj & mask) << (BITS * e);
                qi = (qi - dj) >> BITS;
            }
        }
#pragma unroll
        for (int j = 0; j <= ND; j++) qd[((size_t)j * K_COLS + col) * G + h] = (int32_t)d[j];
    }
    // The query's integer sums over each of the kg scale groups of a head
    // (q_int, and the extra low digit): what the zero-point codec's keys
    // subtract, zero point times sum, from a group's score.
    for (int i = tid; i < kg * G; i += 256) {
        const int g = i / G, h = i - g * G;
        const float sq = s_amax[h] / (float)Q_RANGE;
        const float inv = sq > 0.0f ? 1.0f / sq : 0.0f;
        int sum = 0, sumx = 0;
        for (int c = g * (HD / kg); c < (g + 1) * (HD / kg); c++) {
            const float qq = s_qv[h * HD + c];
            const int qi = (int)fminf(fmaxf(rintf(qq * inv), -(float)Q_RANGE), (float)Q_RANGE);
            sum += qi;
            if (xq) sumx += (int)fminf(fmaxf(rintf(fmaf(qq, inv, -(float)qi) * XB), -(float)XMAX), (float)XMAX);
        }
        qd[qd_digits(KB, HD, G) + g * G + h] = sum;
        qd[qd_digits(KB, HD, G) + (QS_GROUPS + g) * G + h] = sumx;
    }
    // The matrix-core operand: q_int = 256 hi + lo with lo in [-128, 127]
    // (so |hi| <= 118), and the extra low digit d, one byte each.  Against
    // 4-bit keys each 32-channel block holds its 16 even channels, then its
    // 16 odd ones (the order the unpacked nibbles of 16 key bytes arrive in);
    // against 8-bit keys the channels keep their order.
    if constexpr (qd_mfma(HD, G)) {
        int8_t *mf = reinterpret_cast<int8_t *>(qd + qd_mf(KB, HD, G));
        for (int i = tid; i < G * HD; i += 256) {
            const int h = i / HD, c = i - h * HD;
            const float sq = s_amax[h] / (float)Q_RANGE;
            const float inv = sq > 0.0f ? 1.0f / sq : 0.0f;
            const float qq = s_qv[h * HD + c];
            const int qi = (int)fminf(fmaxf(rintf(qq * inv), -(float)Q_RANGE), (float)Q_RANGE);
            const int lo = ((qi + 128) & 255) - 128, hi = (qi - lo) / 256;
            const int dx = xq ? (int)fminf(fmaxf(rintf(fmaf(qq, inv, -(float)qi) * XB), -(float)XMAX), (float)XMAX)
                              : 0;
            const int pos = KB == 4 ? (c & ~31) + 16 * (c & 1) + ((c & 31) >> 1) : c;
            mf[(0 * G + h) * HD + pos] = (int8_t)lo;
            mf[(1 * G + h) * HD + pos] = (int8_t)hi;
            mf[(2 * G + h) * HD + pos] = (int8_t)dx;
        }
    }
    __syncthreads();
}

template <int KB, int HD, int G>
__device__ __forceinline__ void qprep_block(const float *__restrict__ q, int32_t *__restrict__ qdig,
                                            float *__restrict__ qsc, int32_t *__restrict__ qflag, float qk_scale,
                                            int unit, int *cnt, int kg)
{
    // unit = b * Hkv + kvh
    __shared__ float amax[G];
    __shared__ int xflag;
    __shared__ float qv[G * HD];                         // q, read from memory once
    qprep_core<KB, HD, G>(q + (size_t)unit * G * HD, qdig + (size_t)unit * qd_stride(KB, HD, G), amax, &xflag, qv, kg);
    const int tid = threadIdx.x;
    if (tid < G) qsc[unit * G + tid] = amax[tid] / (float)Q_RANGE * qk_scale;
    if (tid == 0) {
        qflag[unit] = xflag;
        if (cnt) cnt[unit] = 0;                      // the fused step's ticket counter
    }
}

template <int KB, int HD, int G>
__global__ __launch_bounds__(256) void qprep_kernel(const float *__restrict__ q, int32_t *__restrict__ qdig,
                                                    float *__restrict__ qsc, int32_t *__restrict__ qflag,
                                                    float qk_scale, int *cnt, int kg)
{
    qprep_block<KB, HD, G>(q, qdig, qsc, qflag, qk_scale, blockIdx.x, cnt, kg);
}

template <int KB>
__device__ __forceinline__ int kdot(int qd, int k, int acc)
{
    if constexpr (KB == 4) return __builtin_amdgcn_sdot8(qd, k, acc, false);
    else return __builtin_amdgcn_sdot4(qd, k, acc, false);
}

// First dot of a sum: the three-operand form with an inline zero accumulator
// (the two-operand form accumulates into its destination, which the compiler
// would first clear with a move).
template <int KB>
__device__ __forceinline__ int kdot0(int qd, int k)
{
    int r;
    if constexpr (KB == 4) asm("v_dot8_i32_i4 %0, %1, %2, 0" : "=v"(r) : "s"(qd), "v"(k));
    else asm("v_dot4_i32_i8 %0, %1, %2, 0" : "=v"(r) : "s"(qd), "v"(k));
    return r;
}

__device__ __forceinline__ uint32_t kword(const uint4 &r, int i)
{
    return (i & 3) == 0 ? r.x : (i & 3) == 1 ? r.y : (i & 3) == 2 ? r.z : r.w;
}

// Pack the low and high bytes of four 16-bit weights (each held as the bits
// of 1.5 * 2^23 + w, i.e. w in the low mantissa bits) into two words, byte k
// of each word belonging to position k.
__device__ __forceinline__ void pack_w(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3, uint32_t &lo, uint32_t &hi)
{
    const uint32_t x01 = __builtin_amdgcn_perm(w1, w0, 0x05010400u);   // w0.b0 w1.b0 w0.b1 w1.b1
    const uint32_t x23 = __builtin_amdgcn_perm(w3, w2, 0x05010400u);   // w2.b0 w3.b0 w2.b1 w3.b1
    lo = __builtin_amdgcn_perm(x23, x01, 0x05040100u);
    hi = __builtin_amdgcn_perm(x23, x01, 0x07060302u);
}

// KG = scale groups per head row for both keys and values (1: groups of
// head_dim, or one scale per position shared by all heads; 2 or 4: groups of
// head_dim / KG channels); key dots are summed per group.
// Instances whose key scores run on the matrix cores: four query heads at
// head_dim 128 with the symmetric codec (1, 2 or 4 scale groups per head),
// and eight with one scale group.
__host__ __device__ constexpr bool qd_mf_keys(int KB, int VB, int HD, int G, int KG, bool zp)
{
    return qd_mfma(HD, G) && !zp && (KG < 4 || (KB == 4 && VB == 4)) && (G == 4 || KG == 1);
}
// waves per SIMD the register allocation must allow: the int4 key and value
// instances with G x KG <= 4 scoring keys on the VALU fit 128 VGPRs (4 waves)
// when asked to (left alone the compiler takes a few more and drops to 3);
// the four-head matrix-core ones are held to 3 (K4V4: 167 VGPRs; with keys
// only on the matrix cores, held to 128 it spilled and ran 212 against 177
// us at 32K); the others take what they need: the zero-point instances would
// spill at 128, the eight-head matrix-core ones at 168 (32-37 registers)
__host__ __device__ constexpr int qd_min_waves(int KB, int VB, int HD, int G, int KG, bool paged, bool zp)
{
    return qd_mf_keys(KB, VB, HD, G, KG, zp) ? (G == 8 ? 1 : 3) : KB == 4 && VB == 4 && G * KG <= 4 && !zp ? 4 : 1;
}

// ZP: the zero-point codec (32-bit scale words: fp16 scale | zero << 16;
// keys stored as code - 2^(KB-1), values as the code).
template <int KB, int VB, int HD, int G, int KG, bool PAGED, bool ZP = false>
__global__ __launch_bounds__(QD_THREADS) __attribute__((amdgpu_waves_per_eu(qd_min_waves(KB, VB, HD, G, KG, PAGED, ZP))))
void decode_quant_kernel(QuantParams p)
{
    using T = QT<KB, VB, HD, G>;
    constexpr int S = qd_sub(G, KG, ZP);
    constexpr bool MF = qd_mf_keys(KB, VB, HD, G, KG, ZP);   // key scores on the matrix cores
    // value sums on the matrix cores too (int4 keys and values, one scale
    // group): the weights become two signed bytes, a low one in [-128, 127]
    // and a high one in [0, 127], so their fixed-point range is 32639
    constexpr bool MV = MF && KB == 4 && VB == 4 && KG == 1;
    constexpr int NHL = G / 4;                       // (MV) heads per lane in the products
    constexpr int WR = MV ? 32639 : W_RANGE;
    extern __shared__ __align__(16) unsigned char smem[];

    const int tid = threadIdx.x, lane = tid & 63;
    // wave index as a wave-uniform (scalar) value, so that everything derived
    // from it (the wave's range, its buffer descriptors) stays in SGPRs
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int chunk_id = blockIdx.x;                 // grid: (chunks, KV heads, sequences)
    const int kvh = blockIdx.y;                      // the unit's head (query heads kvh * G ..)
    const int kvc = kvh >> p.kv_shift;               // the cache's KV head it reads
    const int b = blockIdx.z;
    const int bh = b * p.n_kv_heads + kvh;
    const int Hq = p.n_kv_heads * G;
    const int CH = p.chunk;

    int L = p.seq_len[b];
    L = L < 0 ? 0 : (L > p.max_len ? p.max_len : L);
    const int t0 = chunk_id * CH;
    const int n_tok = min(L - t0, CH);

    const size_t row0 = (size_t)b * Hq + (size_t)kvh * G;
    float *ml0 = p.ws_ml + (row0 * p.n_chunks + chunk_id) * 2;
    float *acc0 = p.ws_acc + (row0 * p.n_chunks + chunk_id) * HD;
    const size_t ml_hs = (size_t)p.n_chunks * 2;
    const size_t acc_hs = (size_t)p.n_chunks * HD;

    // the query digits' slot: per (sequence, KV head), or per chunk too in
    // the one-launch step (each workgroup prepares its own)
    const size_t qslot = p.step ? (size_t)bh * p.n_chunks + chunk_id : (size_t)bh;

    // Query scales (log2 units; floored so that a zero query keeps -inf
    // scores at -inf: 0 * -inf would be NaN) and the extra-digit flag.
    float qs[G];
    bool xq;
    if (p.step) {
        // (block-uniform) this is the only workgroup of its (sequence, KV
        // head): the step's rows of its head, then its query's digits; every
        // store is complete before a wave reads the cache or the digits
        // (with the heads split over two workgroups both store the same
        // rows, byte for byte the same values, each before reading them)
        append_head_rows<HD>(p.ap, b, kvc, t0, chunk_id == p.n_chunks - 1 ? 0x7FFFFFFF : t0 + CH);
        float *s_qv = reinterpret_cast<float *>(smem);
        float *s_amax = s_qv + G * HD;
        int *s_xflag = reinterpret_cast<int *>(s_amax + G);
        qprep_core<KB, HD, G>(p.q + row0 * HD, const_cast<int32_t *>(p.qdig) + qslot * qd_stride(KB, HD, G),
                              s_amax, s_xflag, s_qv, ZP ? KG : 0);
        __builtin_amdgcn_s_waitcnt(WAIT_VMEM_ALL);
        __syncthreads();
#pragma unroll
        for (int h = 0; h < G; h++)                  // (LDS values: made wave-uniform for the compiler)
            qs[h] = __int_as_float(__builtin_amdgcn_readfirstlane(
                __float_as_int(fmaxf(s_amax[h] / (float)Q_RANGE * p.qk_scale, 1e-30f))));
        xq = __builtin_amdgcn_readfirstlane(*s_xflag) != 0;
        __syncthreads();                             // the LDS is reused below
    } else {
#pragma unroll
        for (int h = 0; h < G; h++) qs[h] = fmaxf(p.qsc[row0 + h], 1e-30f);
        xq = ((const KVQ_CONST int32_t *)p.qflag)[bh] != 0;
    }

    // (block-uniform; the ticket needs one int of LDS, free by then)
    auto finish = [&]() {
        if (p.cnt)
            combine_if_last<HD, G, QD_THREADS>(p.ws_ml, p.ws_acc, p.out, p.cnt + bh, p.n_chunks, row0,
                                               reinterpret_cast<int *>(smem));
    };

    if (n_tok <= 0) {
        if (p.step && p.n_chunks == 1) {             // nothing attended: out = 0
            for (int i = tid; i < G * HD; i += QD_THREADS) p.out[row0 * HD + i] = 0.0f;
            return;
        }
        for (int i = tid; i < G * HD; i += QD_THREADS) store_partial(&acc0[(i / HD) * acc_hs + (i % HD)], 0.0f);
        if (tid < G) {
            store_partial(&ml0[tid * ml_hs], -INFINITY);
            store_partial(&ml0[tid * ml_hs + 1], 0.0f);
        }
        finish();
        return;
    }

    const QuantSmem lay = quant_smem(G, HD, KG, ZP);
    constexpr int SCB = ZP ? 4 : 2;                  // bytes per scale entry
    constexpr int SW = (KG * SCB + 3) / 4;           // 32-bit words of one position's scales (one tensor)
    constexpr bool VS_IN_WD = KG > 1 && !ZP;         // value scales inside the weight words' area
    constexpr int WBLK = KG * G * 2;                 // weight words of one 4-position group
    float *zs = reinterpret_cast<float *>(smem + lay.zs) + wave * S * G;       // this wave's scores
    uint32_t *wdw = lay.wd_alias ? reinterpret_cast<uint32_t *>(zs)
                                 : reinterpret_cast<uint32_t *>(smem + lay.wd) + wave * KG * (S / 4) * G * 2;
    // value scale words of position pos (within the sub-chunk): one fp16 (one
    // scale group), 2 fp16 a word (several groups: the last 2 KG words of the
    // position's 4-group block of weight words), or 32-bit scale | zero words
    uint16_t *vs16 = reinterpret_cast<uint16_t *>(smem + lay.vs) + wave * S;
    uint32_t *vsw = VS_IN_WD ? wdw : reinterpret_cast<uint32_t *>(smem + lay.vs) + wave * S * KG;
    auto vs_word = [&](int pos) -> int {
        if constexpr (VS_IN_WD) return (pos >> 2) * WBLK + (WBLK - 2 * KG) + (pos & 3) * (KG / 2);
        else return pos * KG;
    };
    auto vs_rd = [&](int pos, uint32_t (&w)[SW]) {
        if constexpr (!ZP && KG == 1) {
            w[0] = vs16[pos];
        } else if constexpr (SW == 1) {
            w[0] = vsw[vs_word(pos)];
        } else if constexpr (SW == 2) {
            const uint2 v = *reinterpret_cast<const uint2 *>(vsw + vs_word(pos));
            w[0] = v.x; w[1] = v.y;
        } else {
            const uint4 v = *reinterpret_cast<const uint4 *>(vsw + vs_word(pos));
            w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
        }
    };
    auto vs_wr = [&](int pos, const uint32_t (&w)[SW]) {
        if constexpr (!ZP && KG == 1) {
            vs16[pos] = (uint16_t)w[0];
        } else if constexpr (SW == 1) {
            vsw[vs_word(pos)] = w[0];
        } else if constexpr (SW == 2) {
            *reinterpret_cast<uint2 *>(vsw + vs_word(pos)) = make_uint2(w[0], w[1]);
        } else {
            *reinterpret_cast<uint4 *>(vsw + vs_word(pos)) = make_uint4(w[0], w[1], w[2], w[3]);
        }
    };
    // scale word of group g (fp16 bits, or fp16 | zero << 16)
    auto sc_of = [](const uint32_t (&w)[SW], int g) -> uint32_t {
        if constexpr (ZP) return w[g];
        else if constexpr (KG == 1) return w[0];
        else return (w[g >> 1] >> (16 * (g & 1))) & 0xFFFFu;
    };
    float *red = reinterpret_cast<float *>(smem + lay.red);
    float *misc = reinterpret_cast<float *>(smem + lay.misc);

    const int sub = CH / QD_WAVES;                   // positions per wave (multiple of 64)
    const int s0 = wave * sub;
    const int nw = max(min(sub, n_tok - s0), 0);     // positions of this wave


    // ---- key stream: tiles of 64 positions, one lane per position, loaded
    // one tile ahead into the other of two register sets; the descriptors
    // move with the tile.  A tile is stored slice-major, so load u (16 bytes
    // per lane) reads 1 KiB of contiguous memory.  A tile with any position
    // of the wave is read whole (lanes past the range see other rows and are
    // masked); tiles past the range read zeros.  Scales past the range read
    // zeros.
    // Storage unit (the sequence, or with paged storage the page) of the
    // wave-relative position tw, and tw's slot inside it.  Paged: lane i holds
    // the page of the wave's i-th logical page (a wave's range touches at most
    // 2048 / 64 + 1 pages); -1 marks a missing page, whose slots read as zero.
    const int w0 = t0 + s0;                          // a multiple of 64
    int pg_lane = -1, pg_first = 0;
    if constexpr (PAGED) {
        pg_first = w0 >> p.page_shift;
        const int npg = nw > 0 ? ((w0 + nw - 1) >> p.page_shift) - pg_first + 1 : 0;
        if (lane < npg) {
            const int e = p.block_table[(size_t)b * p.pages_per_seq + pg_first + lane];
            pg_lane = (e >= 0 && e < p.n_pages) ? e : -1;
        }
    }
    auto unit_of = [&](int tw) -> int {
        if constexpr (PAGED) {
            const int i = min(((w0 + tw) >> p.page_shift) - pg_first, 63);
            return __builtin_amdgcn_readlane(pg_lane, i);
        } else {
            return b;
        }
    };
    auto slot_of = [&](int tw) -> int {
        if constexpr (PAGED) return (w0 + tw) & ((1 << p.page_shift) - 1);
        else return w0 + tw;
    };
    const KVQ_CONST int32_t *qd = (const KVQ_CONST int32_t *)(p.qdig + qslot * qd_stride(KB, HD, G));
    constexpr float XINV = 1.0f / (float)qx_base(KB);
    const uint32_t ko = lane * 16;
    const uint32_t mko = (lane >> 4) * 1024 + (lane & 15) * 16;
    const uint32_t kso = lane * p.k_sc_t * SCB, vso = lane * p.v_sc_t * SCB;
    struct Tile {
        uint4 k[T::K_U4];
        uint32_t ks[SW], vs[SW];                     // the position's scale words (sc_of)
    };
    auto load = [&](int tb, Tile &d) {
        const int u = unit_of(tb);
        const int sl = slot_of(tb);
        const uint32_t rem = u < 0 ? 0u : (uint32_t)max(nw - tb, 0);
        const uint32_t kbytes = rem > 0 ? 64 * T::K_ROW : 0;
        const int uu = u < 0 ? 0 : u;
        const uint8_t *kb = p.k_codes + (((size_t)uu * p.n_kv_cache + kvc) * p.cap64 + sl) * T::K_ROW;
        const rsrc_t krs = make_rsrc(kb, kbytes);
        const rsrc_t ksrs = make_rsrc(reinterpret_cast<const char *>(p.k_scales) +
                                          (uu * p.k_sc_b + kvc * p.k_sc_h + (size_t)sl * p.k_sc_t) * SCB,
                                      rem * p.k_sc_t * SCB);
        const rsrc_t vsrs = make_rsrc(reinterpret_cast<const char *>(p.v_scales) +
                                          (uu * p.v_sc_b + kvc * p.v_sc_h + (size_t)sl * p.v_sc_t) * SCB,
                                      rem * p.v_sc_t * SCB);
        // (immediate offsets reach 4 KiB: int8 rows use a second descriptor
        // for slices 4..7)
        const rsrc_t krs2 = make_rsrc(kb + 4096, kbytes > 4096 ? kbytes - 4096 : 0);
        if constexpr (MF) {
            // the matrix-core layout: for each 16-position block t of the
            // tile, lane l reads 16 bytes of position 16 t + l % 16, slice
            // l / 16 (int4) or slices l / 16 and 4 + l / 16 (int8)
#pragma unroll
            for (int t = 0; t < 4; t++) {
                if constexpr (KB == 4) {
                    d.k[t] = bld_u4<CP_NT>(krs, mko + t * 256);
                } else {
                    d.k[2 * t] = bld_u4<CP_NT>(krs, mko + t * 256);
                    d.k[2 * t + 1] = bld_u4<CP_NT>(krs2, mko + t * 256);
                }
            }
        } else {
#pragma unroll
            for (int u4 = 0; u4 < T::K_U4; u4++) d.k[u4] = bld_u4<CP_NT>(u4 < 4 ? krs : krs2, ko + (u4 % 4) * 1024);
        }
        // (a position's scale words are contiguous: one load each)
        if constexpr (SW == 1 && SCB * KG == 2) {
            d.ks[0] = bld_u16(ksrs, kso);
            d.vs[0] = bld_u16(vsrs, vso);
        } else if constexpr (SW == 1) {
            d.ks[0] = bld_u32<0>(ksrs, kso);
            d.vs[0] = bld_u32<0>(vsrs, vso);
        } else if constexpr (SW == 2) {
            const uint2 a = bld_u2(ksrs, kso), v = bld_u2(vsrs, vso);
            d.ks[0] = a.x; d.ks[1] = a.y;
            d.vs[0] = v.x; d.vs[1] = v.y;
        } else {
            const uint4 a = bld_u4<0>(ksrs, kso), v = bld_u4<0>(vsrs, vso);
            d.ks[0] = a.x; d.ks[1] = a.y; d.ks[2] = a.z; d.ks[3] = a.w;
            d.vs[0] = v.x; d.vs[1] = v.y; d.vs[2] = v.z; d.vs[3] = v.w;
        }
    };
    float mloc[G];                                   // per-lane score maxima of the current sub-chunk
    float mown[2] = {-INFINITY, -INFINITY};          // (matrix cores) the same for the lane's own head(s)
    // The matrix-core query operands, one per row set and MFMA m = 0, 1 of a
    // 16-position block (m: int4 keys, even / odd channels; int8 keys,
    // slices 0-3 / 4-7).  Lane l supplies row l % 16 of A over k-block
    // (m, l / 16): channels 32 (l / 16) .. + 31 (int4) or slice 4 m + l / 16
    // (int8), scale group mf_grp(m, l / 16).  Rows 4 h + i belong to head h
    // (so that lane l of the product holds head l / 16):
    //   one scale group: one set, i = low, high and extra digit, zero;
    //   2 or 4 groups: sets P = 0 .. KG / 2 - 1, i = 2 p + d for digit d
    //   (low, high) of group 2 P + p, the A bytes zero in k-blocks of other
    //   groups; then the extra digit's set, i = the group.
    // Eight heads (one scale group): rows 2 h + d, digit d (low, high) of
    // head h, so lane l holds heads 2 (l / 16) and + 1; then the extra
    // digit's set, rows 2 h.
    // A set whose every k-block of some m lies outside its groups skips that
    // MFMA (int8 keys with 4 groups: each set sees one m).
    constexpr int MF_NP = KG == 1 ? 1 : KG / 2;      // sets of low and high digits
    constexpr int MF_NS = KG == 1 && G == 4 ? 1 : MF_NP + 1;   // + the extra digit's set
    auto mf_grp = [](int m, int L) { return KB == 4 ? L * KG / 4 : (4 * m + L) * KG / 8; };
    auto mf_live = [&](int P, int m) {
        bool any = false;
        for (int L = 0; L < 4; L++) any |= KG == 1 || mf_grp(m, L) / 2 == P;
        return any;
    };
    // (the extra digit's set of 2 or 4 groups or 8 heads is loaded per
    // block, and only when the query carries that digit: held throughout,
    // its registers would cost a wave per SIMD)
    i32x4_t mfa[MF_NP][2];
#pragma unroll
    for (int st = 0; st < MF_NP; st++) mfa[st][0] = mfa[st][1] = i32x4_t{0, 0, 0, 0};
    const uint8_t *mfq = nullptr;                    // this lane's extra-digit bytes (2 or 4 groups, 8 heads)
    if constexpr (MF) {
        const uint8_t *qm = reinterpret_cast<const uint8_t *>(p.qdig + qslot * qd_stride(KB, HD, G) + qd_mf(KB, HD, G));
        const int r = lane & 15, hh = G == 8 ? r >> 1 : r >> 2, i = r & 3, L = lane >> 4;
        auto digits = [&](int d, int m) {            // 16 bytes of digit plane d, head hh, k-block (m, L)
            const uint4 a = ld_u4(qm + (d * G + hh) * HD + (KB == 4 ? 32 * L + 16 * m : 16 * (4 * m + L)));
            return i32x4_t{(int)a.x, (int)a.y, (int)a.z, (int)a.w};
        };
        mfq = qm + (2 * G + hh) * HD + (KB == 4 ? 32 * L : 16 * L);
#pragma unroll
        for (int m = 0; m < 2; m++) {
            if constexpr (G == 8) {
                mfa[0][m] = digits(r & 1, m);
            } else if constexpr (KG == 1) {
                if (i < 3) mfa[0][m] = digits(i, m);
            } else {
                const int grp = mf_grp(m, L);
#pragma unroll
                for (int P = 0; P < MF_NP; P++)
                    if (mf_live(P, m) && grp == 2 * P + (i >> 1)) mfa[P][m] = digits(i & 1, m);
            }
        }
    }
    // scores of one tile (tb: first position of the tile within the wave;
    // sc0: first position of the sub-chunk)
    auto compute = [&](int tb, int sc0, const Tile &c) {
        const int t = tb + lane;
        const bool valid = t < nw;
        // (zero past the wave's range: the load returned zero; every tile of
        // the sub-chunk lies inside its S rows of LDS)
        vs_wr(t - sc0, c.vs);
        if constexpr (MF) {
            // Per 16-position block: D = A B, A the query's digit rows, B 64
            // channels of the block's 16 positions: int4 keys unpacked to
            // bytes 16 code (each nibble moved to the top of its byte keeps
            // its sign: even channels from the low nibbles, odd from the high
            // ones), int8 codes as stored.  Lane l ends with head l / 16's
            // sums for position l % 16 over its low, high and extra digits
            // (per scale group): Σ q_int code = (256 hi + lo) / KS exactly,
            // KS = 16 for int4 keys; each group's score then as on the VALU.
            constexpr float KSI = KB == 4 ? 0.0625f : 1.0f;
            const int n = lane & 15, hq = lane >> 4;
#pragma unroll
            for (int tt = 0; tt < 4; tt++) {
                i32x4_t bk[2];
                if constexpr (KB == 4) {
                    const uint4 w = c.k[tt];
                    bk[0] = i32x4_t{(int)((w.x << 4) & 0xF0F0F0F0u), (int)((w.y << 4) & 0xF0F0F0F0u),
                                    (int)((w.z << 4) & 0xF0F0F0F0u), (int)((w.w << 4) & 0xF0F0F0F0u)};
                    bk[1] = i32x4_t{(int)(w.x & 0xF0F0F0F0u), (int)(w.y & 0xF0F0F0F0u), (int)(w.z & 0xF0F0F0F0u),
                                    (int)(w.w & 0xF0F0F0F0u)};
                } else {
                    const uint4 w0 = c.k[2 * tt], w1 = c.k[2 * tt + 1];
                    bk[0] = i32x4_t{(int)w0.x, (int)w0.y, (int)w0.z, (int)w0.w};
                    bk[1] = i32x4_t{(int)w1.x, (int)w1.y, (int)w1.z, (int)w1.w};
                }
                i32x4_t acc[MF_NS];
#pragma unroll
                for (int st = 0; st < MF_NP; st++) {
                    acc[st] = i32x4_t{0, 0, 0, 0};
#pragma unroll
                    for (int m = 0; m < 2; m++)
                        if (mf_live(st, m)) acc[st] = mfma_i8(mfa[st][m], bk[m], acc[st]);
                }
                if ((KG > 1 || G == 8) && xq) {
                    // rows 4 h + g: the extra digit of group g, zero in other
                    // groups' k-blocks (eight heads: rows 2 h)
                    acc[MF_NS - 1] = i32x4_t{0, 0, 0, 0};
#pragma unroll
                    for (int m = 0; m < 2; m++) {
                        const uint4 a = ld_u4(mfq + (KB == 4 ? 16 * m : 64 * m));
                        const bool on = G == 8 ? (lane & 1) == 0 : mf_grp(m, lane >> 4) == (lane & 3);
                        const i32x4_t ax = i32x4_t{on ? (int)a.x : 0, on ? (int)a.y : 0, on ? (int)a.z : 0,
                                                   on ? (int)a.w : 0};
                        acc[MF_NS - 1] = mfma_i8(ax, bk[m], acc[MF_NS - 1]);
                    }
                }
                const int pos = 16 * tt + n;         // within the tile
                // the key scale words of the position, from the lane that loaded them
                uint32_t ksw[SW];
#pragma unroll
                for (int w = 0; w < SW; w++) ksw[w] = (uint32_t)__builtin_amdgcn_ds_bpermute(pos * 4, (int)c.ks[w]);
                if constexpr (G == 8) {
                    // heads 2 hq and 2 hq + 1: rows 4 hq .. + 3 = their low and high sums
                    const float sk = f16_bits_to_f32((uint16_t)sc_of(ksw, 0)) * KSI;
                    float z2[2];
#pragma unroll
                    for (int e = 0; e < 2; e++) {
                        float z = (float)(acc[0][2 * e + 1] * 256 + acc[0][2 * e]) * sk;
                        if (xq) z = fmaf((float)acc[1][2 * e], sk * XINV, z);
                        z2[e] = tb + pos < nw ? z : -INFINITY;
                        mown[e] = fmax_nc(mown[e], z2[e]);
                    }
                    *reinterpret_cast<float2 *>(zs + (size_t)(tb + pos - sc0) * G + 2 * hq) = make_float2(z2[0], z2[1]);
                    __builtin_amdgcn_sched_barrier(0);
                    continue;
                }
                float z = 0.0f;
#pragma unroll
                for (int g = 0; g < KG; g++) {
                    const float sk = f16_bits_to_f32((uint16_t)sc_of(ksw, g)) * KSI;
                    const int e = KG == 1 ? 0 : 2 * (g & 1);
                    const float sg = (float)(acc[g >> 1][e + 1] * 256 + acc[g >> 1][e]);
                    z = g == 0 ? sg * sk : fmaf(sg, sk, z);
                    if (xq) z = fmaf((float)(KG == 1 ? acc[0][2] : acc[MF_NS - 1][g]), sk * XINV, z);
                }
                z = tb + pos < nw ? z : -INFINITY;   // past the wave's range: -inf
                mown[0] = fmax_nc(mown[0], z);
                zs[(size_t)(tb + pos - sc0) * G + hq] = z;
                // (blocks in order: a block's operands are dead before the
                // next block's are made)
                __builtin_amdgcn_sched_barrier(0);
            }
            return;
        }
        // an opaque zero offset, redefined every tile, keeps the digit loads
        // inside the loop (hoisted, they would need hundreds of SGPRs)
        int qz;
        asm volatile("s_mov_b32 %0, 0" : "=s"(qz));
        const KVQ_CONST int32_t *qdl = qd + qz;
        // int4 keys: the digits of a quad of columns come through a pointer
        // that depends on the sums after the quad LAG quads earlier, which
        // bounds the digit words held in SGPRs (the scheduler would otherwise
        // load them all early and spill); a quad's 4G words are one scalar
        // load per digit.  int8 keys (twice the columns) run faster with the
        // scheduler's own deeper prefetch, spills included.
        constexpr int LAG = 48 / (4 * G) > 2 ? 48 / (4 * G) : 2;
        const KVQ_CONST int32_t *ring[LAG];
#pragma unroll
        for (int i = 0; i < LAG; i++) ring[i] = qdl;
        constexpr int CPB = T::K_COLS / KG;          // key dwords per scale group (a multiple of 4)
        static_assert(CPB % 4 == 0, "scale groups hold whole quads of key dwords");
        float z[G];
#pragma unroll
        for (int blk = 0; blk < KG; blk++) {
            // digit-major Horner: acc = sum_j DBASE^j sum_col digit_j * code,
            // the exact int32 sum of q_int * code over the group's channels
            int acc[G];
#pragma unroll
            for (int j = T::ND - 1; j >= 0; j--) {
                if (j < T::ND - 1) {
#pragma unroll
                    for (int h = 0; h < G; h++) acc[h] *= T::DBASE;
                }
                const KVQ_CONST int32_t *qp = qdl;
#pragma unroll
                for (int cc = 0; cc < CPB; cc++) {
                    const int col = blk * CPB + cc;
                    if ((cc & 3) == 0) qp = ring[0];
                    const int kw = (int)kword(c.k[col / 4], col);
                    const KVQ_CONST int32_t *qc = qp + (j * T::K_COLS + col) * G;
#pragma unroll
                    for (int h = 0; h < G; h++)
                        acc[h] = (j == T::ND - 1 && cc == 0) ? kdot0<KB>(qc[h], kw) : kdot<KB>(qc[h], kw, acc[h]);
                    if ((cc & 3) == 3) {
#pragma unroll
                        for (int i = 0; i + 1 < LAG; i++) ring[i] = ring[i + 1];
                        const KVQ_CONST int32_t *qn = qdl;
#pragma unroll
                        for (int h = 0; h < G; h++)
                            if constexpr (KB == 4) asm("" : "+s"(qn) : "v"(acc[h]));
                        ring[LAG - 1] = qn;
                    }
                }
            }
            const float sk = f16_bits_to_f32((uint16_t)sc_of(c.ks, blk));
            // zero-point codec: the stored code is code - 2^(KB-1), so the
            // group's score is sk * (acc - (zero - 2^(KB-1)) * sum q_int)
            int zk = 0;
            if constexpr (ZP) {
                zk = (int)(sc_of(c.ks, blk) >> 16) - (1 << (KB - 1));
                const KVQ_CONST int32_t *qsum = qdl + qd_digits(KB, HD, G) + blk * G;
#pragma unroll
                for (int h = 0; h < G; h++) acc[h] -= __mul24(zk, qsum[h]);
            }
#pragma unroll
            for (int h = 0; h < G; h++) z[h] = blk == 0 ? (float)acc[h] * sk : fmaf((float)acc[h], sk, z[h]);
            if (xq) {
                // the extra low digit: its exact int32 sum, 1/base of a unit
                const KVQ_CONST int32_t *qx = qdl + T::ND * T::K_COLS * G;
#pragma unroll
                for (int cc = 0; cc < CPB; cc++) {
                    const int col = blk * CPB + cc;
                    const int kw = (int)kword(c.k[col / 4], col);
#pragma unroll
                    for (int h = 0; h < G; h++)
                        acc[h] = cc == 0 ? kdot0<KB>(qx[col * G + h], kw) : kdot<KB>(qx[col * G + h], kw, acc[h]);
                }
                if constexpr (ZP) {
                    const KVQ_CONST int32_t *qsx = qdl + qd_digits(KB, HD, G) + (QS_GROUPS + blk) * G;
#pragma unroll
                    for (int h = 0; h < G; h++) acc[h] -= __mul24(zk, qsx[h]);
                }
                const float skx = sk * XINV;
#pragma unroll
                for (int h = 0; h < G; h++) z[h] = fmaf((float)acc[h], skx, z[h]);
            }
        }
        {
            // positions past the wave's range score -inf (their p is then 0)
#pragma unroll
            for (int h = 0; h < G; h++) {
                z[h] = valid ? z[h] : -INFINITY;
                mloc[h] = fmax_nc(mloc[h], z[h]);
            }
            float *dst = zs + (size_t)(t - sc0) * G;
            if constexpr (G % 4 == 0) {
#pragma unroll
                for (int h = 0; h < G; h += 4)
                    *reinterpret_cast<float4 *>(dst + h) = make_float4(z[h], z[h + 1], z[h + 2], z[h + 3]);
            } else if constexpr (G == 2) {
                *reinterpret_cast<float2 *>(dst) = make_float2(z[0], z[1]);
            } else {
                dst[0] = z[0];
            }
        }
    };

    // ---- value stream: 4-position groups, a lane owns fixed byte positions
    // of each group; rotating buffer, slot f consumed then reloaded one batch
    // (PF loads) ahead, the descriptors moving with the batch
    const int gi = lane / T::V_LPG;                  // group slot of a wave load
    const int qsl = lane % T::V_LPG;                 // dword slice of the group
    constexpr uint32_t GSTEP = T::V_GPL * 4 * T::V_ROW;   // bytes per wave-wide group load
    // group loads in flight per lane (at most one sub-chunk's groups; paged
    // storage keeps a batch to 64 positions, so that it lies in one page)
    constexpr int PF_WANT = PAGED && QD_PF * T::V_GPL > 16 ? 16 / T::V_GPL : QD_PF;
    constexpr int PF = PF_WANT < (S / 4) / T::V_GPL ? PF_WANT : (S / 4) / T::V_GPL;
    constexpr int NPF = PF < 4096 / (int)GSTEP ? PF : 4096 / (int)GSTEP;   // loads per descriptor (offsets < 4 KiB)
    constexpr int NR = PF / NPF;                     // descriptors per batch
    static_assert(PF % NPF == 0, "whole descriptors per batch");
    constexpr int PB = PF * T::V_GPL;                // groups per batch (divides S / 4)
    static_assert((S / 4) % PB == 0, "a sub-chunk holds whole batches");
    static_assert(!PAGED || PB <= 16, "a paged batch lies in one 64-slot block");
    const int ngw = (nw + 3) >> 2;                   // groups of this wave
    const uint32_t vo = gi * 4 * T::V_ROW + qsl * T::V_DPL * 4;
    struct VRs {
        rsrc_t r[NR];
    };
    // descriptors of the batch starting at group g0 (paged storage: a batch
    // is at most 64 positions, aligned to its size within the 64-aligned
    // range of the wave, so it lies in one page)
    auto vrsrc = [&](int g0) {
        VRs d;
        const int u = unit_of(4 * g0);
        const int uu = u < 0 ? 0 : u;
        const uint8_t *vb = p.v_codes + (((size_t)uu * p.n_kv_cache + kvc) * p.cap4 + slot_of(4 * g0)) * T::V_ROW;
        const int left = u < 0 ? 0 : (ngw - g0) * 4 * T::V_ROW;   // bytes of the wave's range from the batch on
#pragma unroll
        for (int r = 0; r < NR; r++) {
            const int b0 = r * NPF * (int)GSTEP;
            d.r[r] = make_rsrc(vb + b0, (uint32_t)max(left - b0, 0));
        }
        return d;
    };
    uint32_t buf[PF][T::V_DPL];
    auto vload = [&](int f, const VRs &rs) {
#pragma unroll
        for (int d = 0; d < T::V_DPL; d++) buf[f][d] = bld_u32<T::V_CP>(rs.r[f / NPF], vo + (f % NPF) * GSTEP + d * 4);
    };
    const int vgrp = (qsl * T::V_DPL * T::V_CPD) / (HD / KG);   // value scale group of the lane
    const uint32_t *wdg = wdw + (size_t)vgrp * G * 2;
    uint32_t accl[G][T::V_ACC], acch[G][T::V_ACC];
    // one 4-position group: weight words of local group rg (LDS broadcast)
    // times the value codes this lane holds for it
    auto group = [&](int rg, const uint32_t (&x)[T::V_DPL]) {
        uint32_t wl[G], wh[G];
        const uint32_t *src = wdg + (size_t)rg * WBLK;
#pragma unroll
        for (int h = 0; h < G; h++) {
            wl[h] = src[2 * h];
            wh[h] = src[2 * h + 1];
        }
#pragma unroll
        for (int d = 0; d < T::V_DPL; d++) {
            if constexpr (VB == 4) {
                // (codes are stored offset binary) the even channel's nibbles,
                // and whole bytes: even + 16 * odd channel
                const uint32_t u = x[d];
                const uint32_t ulo = u & 0x0F0F0F0Fu;
#pragma unroll
                for (int h = 0; h < G; h++) {
                    accl[h][2 * d] = __builtin_amdgcn_udot4(wl[h], ulo, accl[h][2 * d], false);
                    acch[h][2 * d] = __builtin_amdgcn_udot4(wh[h], ulo, acch[h][2 * d], false);
                    accl[h][2 * d + 1] = __builtin_amdgcn_udot4(wl[h], u, accl[h][2 * d + 1], false);
                    acch[h][2 * d + 1] = __builtin_amdgcn_udot4(wh[h], u, acch[h][2 * d + 1], false);
                }
            } else {
                const uint32_t u = x[d];                       // offset binary per byte
#pragma unroll
                for (int h = 0; h < G; h++) {
                    accl[h][d] = __builtin_amdgcn_udot4(wl[h], u, accl[h][d], false);
                    acch[h][d] = __builtin_amdgcn_udot4(wh[h], u, acch[h][d], false);
                }
            }
        }
    };

    // ---- values on the matrix cores (MV): per 64-position block of the
    // sub-chunk, 8 products D += A B over 16 channels each.  A: lane l holds
    // row l % 16 = 4 h + b (b = 0, 1: head h's signed low and high weight
    // bytes; b = 2, 3 zero; eight heads: row 2 h + b) over the block's groups
    // 4 (l / 16) .. + 3 (16 positions, the block's weight words in LDS).  B: column n = l % 16 of
    // product 4 t + q holds channel 64 t + 4 n + q of those 16 positions, the
    // stored nibbles (code + 8) as bytes; lane l loads bytes 32 t + 2 n and
    // + 1 of its four groups, one 8-byte load per group and t (16 lanes read
    // 128 contiguous bytes).  D: lane l holds head l / 16's two sums for
    // channel 64 t + 4 (l % 16) + q (eight heads: heads 2 (l / 16) + e, e =
    // 0, 1, in elements 2 e and 2 e + 1).
    uint32_t vx[8][2];                               // the next block's value words, [t][group][byte]
    auto vload_mv = [&](int gb) {                    // gb: the block's first group (within the wave)
        const int u = unit_of(4 * gb);
        const int uu = u < 0 ? 0 : u;
        const uint8_t *vb = p.v_codes + (((size_t)uu * p.n_kv_cache + kvc) * p.cap4 + slot_of(4 * gb)) * T::V_ROW;
        const int left = u < 0 ? 0 : (ngw - gb) * 4 * T::V_ROW;   // bytes of the wave's range from the block on
        const rsrc_t rs = make_rsrc(vb, (uint32_t)max(left, 0));
        const uint32_t o = (lane >> 4) * 16 * T::V_ROW + (lane & 15) * 8;
#pragma unroll
        for (int t = 0; t < 2; t++)
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const uint2 v = bld_u2<T::V_CP>(rs, o + i * 4 * T::V_ROW + t * 128);
                vx[4 * t + i][0] = v.x;
                vx[4 * t + i][1] = v.y;
            }
    };
    i32x4_t vacc[8];
    float afm[NHL > 0 ? NHL : 1][8];                  // (MV) the lane's channels 64 t + 4 n + q of its head(s)

    // ---- the wave's running result: max M (unscaled score units), per-lane
    // partial sum of p, and the lane's output channels, all relative to M
    float M[G], lsum[G], af[G][T::V_ACC], bsum[KG][G];
#pragma unroll
    for (int h = 0; h < G; h++) {
        M[h] = -INFINITY;
        lsum[h] = 0.0f;
#pragma unroll
        for (int g = 0; g < KG; g++) bsum[g][h] = 0.0f;
#pragma unroll
        for (int c = 0; c < T::V_ACC; c++) af[h][c] = 0.0f;
    }
#pragma unroll
    for (int t = 0; t < 8; t++) afm[0][t] = afm[NHL > 1 ? 1 : 0][t] = 0.0f;

    Tile ta, tb_;
    load(0, ta);
    for (int sc0 = 0; sc0 < nw; sc0 += S) {
        const int ns = min(S, nw - sc0);             // positions of this sub-chunk
        // ---------------- pass 1: scores of the sub-chunk ----------------------
#pragma unroll
        for (int h = 0; h < G; h++) mloc[h] = -INFINITY;
        mown[0] = mown[1] = -INFINITY;
        // (tiles run in pairs, both halves unconditionally: a half past the
        // end sees only invalid lanes and zero rows, and the code stays free
        // of a merge point that would send the two register sets through
        // memory; the last pair is peeled to start the value loads early)
        int tb = sc0;
        for (; tb + 128 < sc0 + ns; tb += 128) {
            load(tb + 64, tb_);
            compute(tb, sc0, ta);
            load(tb + 128, ta);
            compute(tb + 64, sc0, tb_);
        }
        load(tb + 64, tb_);
        compute(tb, sc0, ta);
        // the sub-chunk's first batch of value loads, in flight during the
        // last key tile and the weights pass
        if constexpr (MV) {
            vload_mv(sc0 >> 2);
        } else {
            const VRs rs = vrsrc(sc0 >> 2);
#pragma unroll
            for (int f = 0; f < PF; f++) vload(f, rs);
        }
        compute(tb + 64, sc0, tb_);
        float ms[G];                                 // sub-chunk score maxima, wave-uniform
        if constexpr (MF) {
            // lanes 16 h .. 16 h + 15 hold head h (eight heads: heads 2 h
            // and 2 h + 1, in mown[0] and mown[1])
            const float mr0 = row_max_u(mown[0]);
            const float mr1 = G == 8 ? row_max_u(mown[1]) : mr0;
#pragma unroll
            for (int h = 0; h < G; h++) {
                const float mr = G == 8 && (h & 1) ? mr1 : mr0;
                ms[h] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, mr),
                                                                            16 * (G == 8 ? h >> 1 : h)));
            }
        } else {
#pragma unroll
            for (int h = 0; h < G; h++) ms[h] = wave_max_u(mloc[h]);
        }

        // ---------------- pass 2: weights, one lane per 4 positions ---------------
        // (a) p = 2^(qs * (z - ms)) <= 1, written over its score, and the
        // largest product p * s_v per head and scale group, N (DPP; the
        // products are >= 0, so their bits compare as integers); (b) w_int =
        // rint(p * s_v * 32767 / N), rounded by one fma onto 1.5 * 2^23 (the
        // integer lands in the low mantissa bits), bytes packed four positions
        // per word.  One lane per group of 4 positions and turn; a lane only
        // rewrites the scores it has read, and the weight words go over
        // positions whose p every lane has already read.
        float lloc[G];
        int wsl[KG][G];                              // sum of w_int (symmetric: the offset binary's share)
        uint32_t wzl[KG][G], wzh[KG][G];             // zero point: sum of w_int * zero, low / high weight bytes
        float nrm[KG][G];                            // N per scale group and head, wave-uniform
        {
            constexpr float MAGIC = 12582912.0f;     // 1.5 * 2^23
            constexpr int TURNS = (S / 4 + 63) / 64;
            auto rd = [&](const float *src, float (&zz)[G]) {
                if constexpr (G % 4 == 0) {
#pragma unroll
                    for (int h = 0; h < G; h += 4) {
                        const float4 v = *reinterpret_cast<const float4 *>(src + h);
                        zz[h] = v.x; zz[h + 1] = v.y; zz[h + 2] = v.z; zz[h + 3] = v.w;
                    }
                } else if constexpr (G == 2) {
                    const float2 v = *reinterpret_cast<const float2 *>(src);
                    zz[0] = v.x; zz[1] = v.y;
                } else {
                    zz[0] = src[0];
                }
            };
            auto wr = [&](float *dst, const float (&zz)[G]) {
                if constexpr (G % 4 == 0) {
#pragma unroll
                    for (int h = 0; h < G; h += 4)
                        *reinterpret_cast<float4 *>(dst + h) = make_float4(zz[h], zz[h + 1], zz[h + 2], zz[h + 3]);
                } else if constexpr (G == 2) {
                    *reinterpret_cast<float2 *>(dst) = make_float2(zz[0], zz[1]);
                } else {
                    dst[0] = zz[0];
                }
            };
            float nqm[G];
            int pmx[KG][G];
#pragma unroll
            for (int h = 0; h < G; h++) {
                nqm[h] = -ms[h] * qs[h];
                lloc[h] = 0.0f;
#pragma unroll
                for (int g = 0; g < KG; g++) {
                    wsl[g][h] = 0;
                    wzl[g][h] = wzh[g][h] = 0u;
                    pmx[g][h] = 0;
                }
            }
#pragma unroll
            for (int t = 0; t < TURNS; t++) {
                const int tq = 4 * (t * 64 + lane);  // first position of the group (within the sub-chunk)
                if (tq < ns) {
#pragma unroll
                    for (int k = 0; k < 4; k++) {
                        // (positions past the range hold score -inf, scale 0)
                        float *src = zs + (size_t)(tq + k) * G;
                        float pr[G];
                        rd(src, pr);
#pragma unroll
                        for (int h = 0; h < G; h++) {
                            pr[h] = __builtin_amdgcn_exp2f(fmaf(pr[h], qs[h], nqm[h]));
                            lloc[h] += pr[h];
                        }
                        float prod[KG][G];
                        uint32_t vw[SW];
                        vs_rd(tq + k, vw);
#pragma unroll
                        for (int g = 0; g < KG; g++) {
                            const float sv = f16_bits_to_f32((uint16_t)sc_of(vw, g));
#pragma unroll
                            for (int h = 0; h < G; h++) {
                                prod[g][h] = pr[h] * sv;
                                pmx[g][h] = max(pmx[g][h], __builtin_bit_cast(int, prod[g][h]));
                            }
                        }
                        // one scale group: p * s_v goes back, the weight needs
                        // one fma; more: p goes back
                        if constexpr (KG == 1) wr(src, prod[0]);
                        else wr(src, pr);
                    }
                }
            }
            float fsc[KG][G];
#pragma unroll
            for (int g = 0; g < KG; g++)
#pragma unroll
                for (int h = 0; h < G; h++) {
                    nrm[g][h] = __builtin_bit_cast(float, wave_max_ui(pmx[g][h]));
                    fsc[g][h] = nrm[g][h] > 0.0f ? (float)WR * __builtin_amdgcn_rcpf(nrm[g][h]) : 0.0f;
                }
#pragma unroll
            for (int t = 0; t < TURNS; t++) {
                const int grp = t * 64 + lane;
                const int tq = 4 * grp;
                if (tq < ns) {
                    float pr[4][G];                  // p * s_v (one group) or p
#pragma unroll
                    for (int k = 0; k < 4; k++) rd(zs + (size_t)(tq + k) * G, pr[k]);
                    // the 4 positions' value scale words, all read before the
                    // first weight word goes out (they may share its block)
                    uint32_t vw[4][SW];
                    if constexpr (KG > 1 || ZP) {
#pragma unroll
                        for (int k = 0; k < 4; k++) vs_rd(tq + k, vw[k]);
                    }
#pragma unroll
                    for (int g = 0; g < KG; g++) {
                        float sv[4];
                        if constexpr (KG > 1) {
#pragma unroll
                            for (int k = 0; k < 4; k++) sv[k] = f16_bits_to_f32((uint16_t)sc_of(vw[k], g));
                        }
                        // zero point: the four positions' zero points, one byte each
                        uint32_t zb = 0;
                        if constexpr (ZP) {
                            const uint32_t a0 = sc_of(vw[0], g), a1 = sc_of(vw[1], g);
                            const uint32_t a2 = sc_of(vw[2], g), a3 = sc_of(vw[3], g);
                            const uint32_t z01 = __builtin_amdgcn_perm(a1, a0, 0x0c0c0602u);   // a0.b2 a1.b2
                            const uint32_t z23 = __builtin_amdgcn_perm(a3, a2, 0x0c0c0602u);
                            zb = __builtin_amdgcn_perm(z23, z01, 0x05040100u);
                        }
                        uint32_t *dst = wdw + ((size_t)grp * KG + g) * G * 2;
#pragma unroll
                        for (int h = 0; h < G; h++) {
                            uint32_t wb[4];
#pragma unroll
                            for (int k = 0; k < 4; k++)
                                wb[k] = __builtin_bit_cast(uint32_t, KG == 1 ? fmaf(pr[k][h], fsc[g][h], MV ? MAGIC + 128.0f : MAGIC)
                                                                             : fmaf(pr[k][h] * fsc[g][h], sv[k], MAGIC));
                            uint32_t lo, hi;
                            pack_w(wb[0], wb[1], wb[2], wb[3], lo, hi);
                            if constexpr (MV) {
                                // the bytes of w + 128: the high byte is w's
                                // signed high digit, the low byte less 128
                                // its signed low digit (the same bits as w's
                                // low byte with the top one flipped);
                                // block-major words, [64 positions][head]
                                // [low, high][16 groups]
                                wsl[g][h] += (int)__builtin_amdgcn_udot4(lo, 0x01010101u, 0u, false)
                                           + 256 * (int)__builtin_amdgcn_udot4(hi, 0x01010101u, 0u, false) - 512;
                                uint32_t *dm = wdw + (size_t)((grp >> 4) * G + h) * 32 + (grp & 15);
                                dm[0] = lo ^ 0x80808080u;
                                dm[16] = hi;
                                continue;
                            }
                            if constexpr (ZP) {
                                wzl[g][h] = __builtin_amdgcn_udot4(lo, zb, wzl[g][h], false);
                                wzh[g][h] = __builtin_amdgcn_udot4(hi, zb, wzh[g][h], false);
                            } else {
                                wsl[g][h] += (int)__builtin_amdgcn_udot4(lo, 0x01010101u, 0u, false)
                                           + 256 * (int)__builtin_amdgcn_udot4(hi, 0x01010101u, 0u, false);
                            }
                            dst[2 * h] = lo;
                            dst[2 * h + 1] = hi;
                        }
                    }
                }
            }
        }

        // ---------------- pass 3: values of the sub-chunk ------------------------
        if constexpr (MV) {
#pragma unroll
            for (int t = 0; t < 8; t++) vacc[t] = i32x4_t{0, 0, 0, 0};
            const int g0 = sc0 >> 2;                 // first group of the sub-chunk (within the wave)
            const int nblk = (ns + 63) >> 6;         // its 64-position blocks
            const int r = lane & 15, L = lane >> 4;
            for (int bb = 0; bb < nblk; bb++) {
                // the block's weight bytes (rows with b >= 2: zero); groups
                // past the sub-chunk's positions meet zero value bytes
                i32x4_t a = {0, 0, 0, 0};
                const int ha = G == 8 ? r >> 1 : r >> 2, ba = G == 8 ? r & 1 : r & 3;
                if (ba < 2) {
                    const uint4 w = *reinterpret_cast<const uint4 *>(wdw + (size_t)((bb * G + ha) * 2 + ba) * 16 + 4 * L);
                    a = i32x4_t{(int)w.x, (int)w.y, (int)w.z, (int)w.w};
                }
#pragma unroll
                for (int t = 0; t < 2; t++) {
                    i32x4_t bv[4];                   // channels 64 t + 4 n + q
#pragma unroll
                    for (int i = 0; i < 4; i++) {
                        bv[0][i] = (int)(vx[4 * t + i][0] & 0x0F0F0F0Fu);
                        bv[1][i] = (int)((vx[4 * t + i][0] >> 4) & 0x0F0F0F0Fu);
                        bv[2][i] = (int)(vx[4 * t + i][1] & 0x0F0F0F0Fu);
                        bv[3][i] = (int)((vx[4 * t + i][1] >> 4) & 0x0F0F0F0Fu);
                    }
                    if (t == 1 && bb + 1 < nblk) vload_mv(g0 + 16 * (bb + 1));
#pragma unroll
                    for (int q = 0; q < 4; q++) vacc[4 * t + q] = mfma_i8(a, bv[q], vacc[4 * t + q]);
                }
            }
            // the next sub-chunk's first key tile
            load(sc0 + S, ta);
        } else {
#pragma unroll
            for (int h = 0; h < G; h++)
#pragma unroll
                for (int c = 0; c < T::V_ACC; c++) accl[h][c] = acch[h][c] = 0u;
            // Full batches are straight-line code (the weight reads of later
            // groups are issued early); a partial last batch checks each group.
            const int g0 = sc0 >> 2;                 // first group of the sub-chunk (within the wave)
            const int ngs = (ns + 3) >> 2;           // its groups
            // (the last batch reloads nothing: the next sub-chunk starts its own)
            const int nfull = (ngs - 1) / PB * PB;
            int rb = 0;
            for (; rb < nfull; rb += PB) {
                const int nb = g0 + rb + PB;         // first group of the next batch
                const VRs rs = vrsrc(nb);
#pragma unroll
                for (int f = 0; f < PF; f++) {
                    group(rb + f * T::V_GPL + gi, buf[f]);
                    vload(f, rs);
                }
            }
#pragma unroll
            for (int f = 0; f < PF; f++) {
                const int rg = rb + f * T::V_GPL + gi;
                if (rg < ngs) group(rg, buf[f]);
            }
            // the next sub-chunk's first key tile (unconditional: past the end
            // it reads zeros, and the old tile is then visibly dead)
            load(sc0 + S, ta);
        }

        // ---------------- merge the sub-chunk into the wave's running result -----
        // integer sums -> floats: undo the byte split and (int4) the even
        // channel inside the whole-byte sums, then the fixed point; scale both
        // parts to the new max.  The offset binary's share (bias * sum of
        // w_int, the same for every channel) is kept as per-lane partial sums
        // and taken out once at the end.
        {
            float fo_h[G], cs_h[G];                  // (MV) per head: the old part's factor, the new sums' scale
#pragma unroll
            for (int h = 0; h < G; h++) {
                const float Mn = fmaxf(M[h], ms[h]);
                const float fo = M[h] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(qs[h] * (M[h] - Mn));
                const float fn = __builtin_amdgcn_exp2f(qs[h] * (ms[h] - Mn));
                M[h] = Mn;
                lsum[h] = fmaf(lsum[h], fo, lloc[h] * fn);
                float cg[KG];                        // c = fn * N / 32767 per scale group
#pragma unroll
                for (int g = 0; g < KG; g++) {
                    cg[g] = fn * nrm[g][h] * (1.0f / (float)WR);
                    // the stored values' offset, in w_int units: bias * sum w
                    // (offset binary), or sum w * zero (zero point)
                    const float woff = ZP ? fmaf(256.0f, (float)wzh[g][h], (float)wzl[g][h])
                                          : (float)wsl[g][h] * (VB == 4 ? 8.0f : 128.0f);
                    bsum[g][h] = fmaf(bsum[g][h], fo, woff * cg[g]);
                }
                fo_h[h] = fo;
                cs_h[h] = cg[0];
                if constexpr (MV) continue;
                // 256 * hi + lo is exact in uint32 (hi bytes <= 127, at most
                // 128 groups a sub-chunk: <= 512 * 32767 * 255 < 2^32)
                uint32_t vi[T::V_ACC];
#pragma unroll
                for (int c = 0; c < T::V_ACC; c++) vi[c] = (acch[h][c] << 8) + accl[h][c];
                if constexpr (VB == 4) {
#pragma unroll
                    for (int c = 1; c < T::V_ACC; c += 2) vi[c] -= vi[c - 1];   // 16 * odd channel
                }
#pragma unroll
                for (int c = 0; c < T::V_ACC; c++) {
                    const int g = ((qsl * T::V_ACC + c) / (HD / KG));   // scale group of the channel
                    const float cs = (VB == 4 && (c & 1)) ? cg[g] * 0.0625f : cg[g];
                    af[h][c] = fmaf(af[h][c], fo, (float)vi[c] * cs);
                }
            }
            if constexpr (MV) {
                // the lane's head(s) NHL (l / 16) + e; 256 hi + lo = sum of
                // w_int (code + 8), exact in int32 (|hi| sums <= 512 * 127 * 15)
#pragma unroll
                for (int e = 0; e < NHL; e++) {
                    const int hl = NHL * (lane >> 4) + e;
                    float fol = fo_h[0], csl = cs_h[0];
#pragma unroll
                    for (int h = 1; h < G; h++) {
                        fol = hl == h ? fo_h[h] : fol;
                        csl = hl == h ? cs_h[h] : csl;
                    }
#pragma unroll
                    for (int t = 0; t < 8; t++)
                        afm[e][t] = fmaf(afm[e][t], fol, (float)(vacc[t][2 * e + 1] * 256 + vacc[t][2 * e]) * csl);
                }
            }
        }
    }

    // ---------------- merge the 4 waves, write --------------------------------
    float lw[G];
#pragma unroll
    for (int h = 0; h < G; h++) lw[h] = wave_sum_u(lsum[h]);
    if constexpr (T::V_GPL > 1) {
        // lanes holding the same channels for different group slots
#pragma unroll
        for (int m = T::V_LPG; m < 64; m <<= 1)
#pragma unroll
            for (int h = 0; h < G; h++)
#pragma unroll
                for (int c = 0; c < T::V_ACC; c++) af[h][c] += __shfl_xor(af[h][c], m, 64);
    }
    {
        // the stored value is code + bias (offset binary) or code + zero (zero
        // point): subtract the offset's share, bias * sum w or sum w * zero,
        // which bsum holds in the accumulators' units, from every channel
#pragma unroll
        for (int g = 0; g < KG; g++)
#pragma unroll
            for (int h = 0; h < G; h++) {
                const float ob = wave_sum_u(bsum[g][h]);
                if constexpr (MV) {
#pragma unroll
                    for (int e = 0; e < NHL; e++)
#pragma unroll
                        for (int t = 0; t < 8; t++) afm[e][t] -= NHL * (lane >> 4) + e == h ? ob : 0.0f;
                    continue;
                }
#pragma unroll
                for (int c = 0; c < T::V_ACC; c++)
                    if ((qsl * T::V_ACC + c) / (HD / KG) == g) af[h][c] -= ob;
            }
    }
    __syncthreads();                                 // every wave is done with scores and weights
    float *pm = misc;                                // [QD_WAVES][G] wave maxima (log2 units)
    float *pl = pm + QD_WAVES * G;                   // [QD_WAVES][G] wave sums of p
    if constexpr (MV) {
#pragma unroll
        for (int e = 0; e < NHL; e++)
#pragma unroll
            for (int t = 0; t < 8; t++)
                red[(wave * G + NHL * (lane >> 4) + e) * HD + 64 * (t >> 2) + 4 * (lane & 15) + (t & 3)] = afm[e][t];
    } else if (gi == 0) {
#pragma unroll
        for (int c = 0; c < T::V_ACC; c++)
#pragma unroll
            for (int h = 0; h < G; h++) red[(wave * G + h) * HD + qsl * T::V_ACC + c] = af[h][c];
    }
    if (lane == 0) {
#pragma unroll
        for (int h = 0; h < G; h++) {
            pm[wave * G + h] = nw > 0 ? M[h] * qs[h] : -INFINITY;
            pl[wave * G + h] = lw[h];
        }
    }
    __syncthreads();
    // per head, once: the merged max m, the waves' factors 2^(m_w - m) (0 for
    // a wave that saw nothing) and the merged sum l
    float *pf = pl + QD_WAVES * G;                   // [QD_WAVES][G] factors, then [G] m, [G] l
    if (tid < G) {
        float m = pm[tid];
#pragma unroll
        for (int w = 1; w < QD_WAVES; w++) m = fmaxf(m, pm[w * G + tid]);
        float l = 0.0f;
#pragma unroll
        for (int w = 0; w < QD_WAVES; w++) {
            const float mv = pm[w * G + tid];
            const float f = mv != -INFINITY ? __builtin_amdgcn_exp2f(mv - m) : 0.0f;
            pf[w * G + tid] = f;
            l = fmaf(f, pl[w * G + tid], l);
        }
        pf[QD_WAVES * G + tid] = m;
        pf[QD_WAVES * G + G + tid] = l;
    }
    __syncthreads();
    const bool write_out = p.step && p.n_chunks == 1;   // the only chunk: out = acc / l
    for (int i = tid; i < G * HD; i += QD_THREADS) {
        const int h = i / HD, c = i - h * HD;
        float s = 0.0f;
#pragma unroll
        for (int w = 0; w < QD_WAVES; w++) s = fmaf(pf[w * G + h], red[(w * G + h) * HD + c], s);
        if (write_out) {
            const float m = pf[QD_WAVES * G + h], l = pf[QD_WAVES * G + G + h];
            p.out[(row0 + h) * HD + c] = m != -INFINITY && l > 0.0f ? s / l : 0.0f;
        } else {
            store_partial(&acc0[h * acc_hs + c], s);
        }
    }
    if (write_out) return;
    if (tid < G) {
        store_partial(&ml0[tid * ml_hs], pf[QD_WAVES * G + tid]);
        store_partial(&ml0[tid * ml_hs + 1], pf[QD_WAVES * G + G + tid]);
    }
    finish();
}

// Every (head_dim, query heads per KV head, scale groups per head)
// instance of one (key width, value width, paged, zero point) family of the
// split kernel: head_dim 64 with 1 or 2 scale groups, head_dim 128 with 1, 2
// or 4; G in {1, 2, 4, 8}, G = 8 with one scale group only (with more, the
// eight heads run as two workgroup heads of four, kv_shift 1).
// X(KB, VB, HD, G, KG, PG, ZP) is applied to each.
#define KVQ_QUANT_FAMILY(X, KB, VB, PG, ZP)                                                     \
    X(KB, VB, 64, 1, 1, PG, ZP) X(KB, VB, 64, 2, 1, PG, ZP) X(KB, VB, 64, 4, 1, PG, ZP)          \
    X(KB, VB, 64, 8, 1, PG, ZP) X(KB, VB, 64, 1, 2, PG, ZP) X(KB, VB, 64, 2, 2, PG, ZP)          \
    X(KB, VB, 64, 4, 2, PG, ZP) X(KB, VB, 128, 1, 1, PG, ZP)                                     \
    X(KB, VB, 128, 2, 1, PG, ZP) X(KB, VB, 128, 4, 1, PG, ZP) X(KB, VB, 128, 8, 1, PG, ZP)       \
    X(KB, VB, 128, 1, 2, PG, ZP) X(KB, VB, 128, 2, 2, PG, ZP) X(KB, VB, 128, 4, 2, PG, ZP)       \
    X(KB, VB, 128, 1, 4, PG, ZP) X(KB, VB, 128, 2, 4, PG, ZP) X(KB, VB, 128, 4, 4, PG, ZP)

// all families the library dispatches to: four width pairs, each contiguous
// and paged, with the symmetric and the zero-point codec
#define KVQ_QUANT_ALL(X)                                                                        \
    KVQ_QUANT_FAMILY(X, 8, 8, false, false) KVQ_QUANT_FAMILY(X, 8, 4, false, false)              \
    KVQ_QUANT_FAMILY(X, 4, 4, false, false) KVQ_QUANT_FAMILY(X, 4, 8, false, false)              \
    KVQ_QUANT_FAMILY(X, 8, 8, true, false) KVQ_QUANT_FAMILY(X, 8, 4, true, false)                \
    KVQ_QUANT_FAMILY(X, 4, 4, true, false) KVQ_QUANT_FAMILY(X, 4, 8, true, false)                \
    KVQ_QUANT_FAMILY(X, 8, 8, false, true) KVQ_QUANT_FAMILY(X, 8, 4, false, true)                \
    KVQ_QUANT_FAMILY(X, 4, 4, false, true) KVQ_QUANT_FAMILY(X, 4, 8, false, true)                \
    KVQ_QUANT_FAMILY(X, 8, 8, true, true) KVQ_QUANT_FAMILY(X, 8, 4, true, true)                  \
    KVQ_QUANT_FAMILY(X, 4, 4, true, true) KVQ_QUANT_FAMILY(X, 4, 8, true, true)

#define KVQ_QUANT_DECLARE(KB, VB, HD, G, KG, PG, ZP) \
    extern template __global__ void decode_quant_kernel<KB, VB, HD, G, KG, PG, ZP>(QuantParams);
#define KVQ_QUANT_DEFINE(KB, VB, HD, G, KG, PG, ZP) \
    template __global__ void decode_quant_kernel<KB, VB, HD, G, KG, PG, ZP>(QuantParams);

} // namespace kvq
