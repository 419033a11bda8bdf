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
//    int32 sum per head and position);
//  * the value weights w = 2^(z - max z) * s_v, per chunk, as
//    w_int = rint(w * 32767 / max s_v) split into two unsigned bytes, so
//    v_dot4_u32_u8 runs over four positions at once against value codes
//    stored four positions interleaved and offset binary (code + 8 or
//    code + 128, never negative); the offset's share, bias * sum(w), is
//    subtracted once at the end.
// Rounding happens only in q_int (|dq| <= s_q / 2) and in w_int
// (|dw| <= max s_v / 65534); accumulation is exact in int32, then fp32.
//
// Workgroup = 4 waves = one context chunk of one (sequence, KV head); each
// wave owns a quarter of the chunk and streams it in sub-chunks of 512
// positions (fewer with many heads or scale groups), the key tiles and the
// value groups loaded ahead without a break between sub-chunks.  Per
// sub-chunk:
//   1. keys, one lane per position: scores -> LDS; the query digits are
//      wave-uniform and come from SGPRs (prepared per (sequence, KV head) by
//      qprep_kernel); value scales -> LDS; the sub-chunk's maxima (DPP).
//   2. weights, one lane per four positions: p = 2^(z - max), w_int packed
//      four positions per word -> LDS (over the sub-chunk's scores).
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

#include "kvq_combine.hpp"
#include "kvq_device.hpp"

namespace kvq {

constexpr int QD_THREADS = 256;
constexpr int QD_WAVES = QD_THREADS / 64;
// Positions per wave sub-chunk: 512 while G x vg < 8, else 256 (the maxima,
// merge and prologue then run half as often as at 128, and the compiler keeps
// the G = 4, vg = 4 loop in 156 VGPRs instead of 245); G = 8 with 2 or 4
// scale groups takes 128, as 256 would not fit the LDS.  (A sub-chunk's value
// sums stay exact in uint32: at most 512 * 32767 * 255 < 2^32.)
__host__ __device__ constexpr int qd_sub(int G, int vg)
{
    return G == 8 && vg >= 2 ? 128 : G * vg >= 8 ? 256 : 512;
}
constexpr int Q_RANGE = 30000;
constexpr int QD_PF = 16;       // value group loads in flight per lane
constexpr int W_RANGE = 32767;

template <int KB, int VB, int HD, int G> struct QT {
    static constexpr int K_ROW = HD * KB / 8;          // bytes per key row
    static constexpr int K_U4 = K_ROW / 16;            // 16-byte loads per key row
    static constexpr int K_COLS = K_ROW / 4;           // dwords per key row
    static constexpr int ND = KB == 4 ? 4 : 2;         // query digits
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

struct QuantParams {
    const uint8_t *k_codes;    // [B][Hkv][cap64/64][K_ROW/16][64][16]  (tiles of 64 slots, slice-major)
    const uint8_t *v_codes;    // [B][Hkv][cap4/4][V_ROW][4]  (4 positions interleaved per byte)
    const uint16_t *k_scales;
    const uint16_t *v_scales;
    const int32_t *qdig;       // [B*Hkv][ND][K_COLS][G] packed query digits (digit-major)
    const float *qsc;          // [B*Hq]: s_q * softmax_scale * log2(e)
    const int32_t *seq_len;
    float *ws_ml;
    float *ws_acc;
    int n_kv_heads, capacity, cap4, cap64;   // capacity, cap4, cap64: per storage unit (sequence or page)
    // paged storage: slot s of sequence b in page block_table[b * pages_per_seq
    // + (s >> page_shift)] (paged kernels only)
    const int32_t *block_table;
    int page_shift, pages_per_seq, n_pages;
    int max_len;
    int chunk, n_chunks;
    // one decode step in one launch pair: after writing its partials each
    // workgroup takes a ticket on cnt[b * Hkv + kvh] (zeroed by the query
    // preparation before the launch) and the last one merges the G rows of
    // its (sequence, KV head) into out.  cnt == nullptr: partials only.
    int *cnt;
    float *out;
    long long k_sc_b, k_sc_h;
    int k_sc_t;
    long long v_sc_b, v_sc_h;
    int v_sc_t;
};

struct QuantSmem {
    int zs, vs, wd, red, misc, total;
    bool wd_alias;             // weight words overwrite each wave's own scores
};

// Per wave: scores [S][G] fp32, value scales [S][vg] fp16 bits, weight words
// [vg][S/4][G][lo, hi] (over the scores when vg == 1); then the
// cross-wave merge area (over the scores when it fits) and the wave maxima
// and sums.
__host__ __device__ inline QuantSmem quant_smem(int G, int HD, int vg)
{
    QuantSmem s;
    const int S = qd_sub(G, vg);
    int off = 0;
    s.zs = off;
    off += QD_WAVES * S * G * 4;
    s.vs = off;
    off += QD_WAVES * S * vg * 2;
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
    off += 2 * QD_WAVES * G * 4;                   // wave maxima and sums
    s.total = off;
    return s;
}

// ---------------------------------------------------------------------------
// Query digits: one block per (sequence, KV head).  For head h of the group,
// s_q = max|q| / 30000 and q_int = rint(q / s_q) in [-30000, 30000], split
// into ND balanced digits; digit j of the channels of key dword `col` is
// packed like the codes (int4: channel 8col+i in nibble i; int8: channel
// 4col+i in byte i) at qdig[unit][j][col][h] (digit-major, the order the
// decode kernel reads them in).
// ---------------------------------------------------------------------------
template <int KB, int HD, int G>
__device__ __forceinline__ void qprep_block(const float *__restrict__ q, int32_t *__restrict__ qdig,
                                            float *__restrict__ qsc, float qk_scale, int unit, int *cnt)
{
    constexpr int K_COLS = HD * KB / 32;
    constexpr int ND = KB == 4 ? 4 : 2;
    constexpr int CPC = KB == 4 ? 8 : 4;
    constexpr int BITS = KB == 4 ? 4 : 8;
    // unit = b * Hkv + kvh
    const float *qh = q + (size_t)unit * G * HD;         // query heads unit*G .. unit*G+G-1
    __shared__ float amax[G];
    __shared__ float qv[G * HD];                         // q, read from memory once
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int h = wave; h < G; h += 4) {
        float a = 0.0f;
        for (int c = lane; c < HD; c += 64) {
            const float v = qh[h * HD + c];
            qv[h * HD + c] = v;
            a = fmaxf(a, fabsf(v));
        }
        a = wave_max(a);
        if (lane == 0) amax[h] = a;
    }
    __syncthreads();
    for (int i = tid; i < K_COLS * G; i += 256) {
        const int col = i / G, h = i - col * G;
        const float sq = amax[h] / (float)Q_RANGE;
        const float inv = sq > 0.0f ? 1.0f / sq : 0.0f;
        uint32_t d[ND];
#pragma unroll
        for (int j = 0; j < ND; j++) d[j] = 0;
#pragma unroll
        for (int e = 0; e < CPC; e++) {
            int qi = (int)fminf(fmaxf(rintf(qv[h * HD + col * CPC + e] * inv), -(float)Q_RANGE), (float)Q_RANGE);
#pragma unroll
            for (int j = 0; j < ND; j++) {
                const int half = 1 << (BITS - 1), mask = (1 << BITS) - 1;
                const int dj = j < ND - 1 ? ((qi + half) & mask) - half : qi;   // balanced digit
                d[j] |= (uint32_t)(dj & mask) << (BITS * e);
                qi = (qi - dj) >> BITS;
            }
        }
#pragma unroll
        for (int j = 0; j < ND; j++) qdig[(((size_t)unit * ND + j) * K_COLS + col) * G + h] = (int32_t)d[j];
    }
    if (tid < G) qsc[unit * G + tid] = amax[tid] / (float)Q_RANGE * qk_scale;
    if (cnt && tid == 0) cnt[unit] = 0;              // the fused step's ticket counter
}

template <int KB, int HD, int G>
__global__ __launch_bounds__(256) void qprep_kernel(const float *__restrict__ q, int32_t *__restrict__ qdig,
                                                    float *__restrict__ qsc, float qk_scale, int *cnt)
{
    qprep_block<KB, HD, G>(q, qdig, qsc, qk_scale, blockIdx.x, cnt);
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
// waves per SIMD the register allocation must allow: the contiguous int4
// key and value instances with G x KG <= 4 fit 128 VGPRs (4 waves) by
// themselves; their paged instances would miss it by a register or two, so
// they ask for it (the others take what they need)
__host__ __device__ constexpr int qd_min_waves(int KB, int VB, int G, int KG, bool paged)
{
    return paged && KB == 4 && VB == 4 && G * KG <= 4 ? 4 : 1;
}

template <int KB, int VB, int HD, int G, int KG, bool PAGED>
__global__ __launch_bounds__(QD_THREADS) __attribute__((amdgpu_waves_per_eu(qd_min_waves(KB, VB, G, KG, PAGED))))
void decode_quant_kernel(QuantParams p)
{
    using T = QT<KB, VB, HD, G>;
    constexpr int S = qd_sub(G, KG);
    extern __shared__ __align__(16) unsigned char smem[];

    const int tid = threadIdx.x, lane = tid & 63;
    // wave index as a wave-uniform (scalar) value, so that everything derived
    // from it (the wave's range, its buffer descriptors) stays in SGPRs
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int chunk_id = blockIdx.x;
    const int bh = blockIdx.y;
    const int b = bh / p.n_kv_heads;
    const int kvh = bh - b * p.n_kv_heads;
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

    // (block-uniform; the ticket needs one int of LDS, free by then)
    auto finish = [&]() {
        if (p.cnt)
            combine_if_last<HD, G, QD_THREADS>(p.ws_ml, p.ws_acc, p.out, p.cnt + bh, p.n_chunks, row0,
                                               reinterpret_cast<int *>(smem));
    };

    if (n_tok <= 0) {
        for (int i = tid; i < G * HD; i += QD_THREADS) store_partial(&acc0[(i / HD) * acc_hs + (i % HD)], 0.0f);
        if (tid < G) {
            store_partial(&ml0[tid * ml_hs], -INFINITY);
            store_partial(&ml0[tid * ml_hs + 1], 0.0f);
        }
        finish();
        return;
    }

    const QuantSmem lay = quant_smem(G, HD, KG);
    float *zs = reinterpret_cast<float *>(smem + lay.zs) + wave * S * G;       // this wave's scores
    uint16_t *vsl = reinterpret_cast<uint16_t *>(smem + lay.vs) + wave * S * KG;   // and value scales
    uint32_t *wdw = lay.wd_alias ? reinterpret_cast<uint32_t *>(zs)
                                 : reinterpret_cast<uint32_t *>(smem + lay.wd) + wave * KG * (S / 4) * G * 2;
    float *red = reinterpret_cast<float *>(smem + lay.red);
    float *misc = reinterpret_cast<float *>(smem + lay.misc);

    const int sub = CH / QD_WAVES;                   // positions per wave (multiple of 64)
    const int s0 = wave * sub;
    const int nw = max(min(sub, n_tok - s0), 0);     // positions of this wave

    float qs[G];
#pragma unroll
    for (int h = 0; h < G; h++) qs[h] = p.qsc[row0 + h];

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
    const KVQ_CONST int32_t *qd = (const KVQ_CONST int32_t *)(p.qdig + (size_t)bh * T::ND * T::K_COLS * G);
    const uint32_t ko = lane * 16;
    const uint32_t kso = lane * p.k_sc_t * 2, vso = lane * p.v_sc_t * 2;
    struct Tile {
        uint4 k[T::K_U4];
        uint32_t ks[KG], vs[KG];
    };
    auto load = [&](int tb, Tile &d) {
        const int u = unit_of(tb);
        const int sl = slot_of(tb);
        const uint32_t rem = u < 0 ? 0u : (uint32_t)max(nw - tb, 0);
        const uint32_t kbytes = rem > 0 ? 64 * T::K_ROW : 0;
        const int uu = u < 0 ? 0 : u;
        const uint8_t *kb = p.k_codes + (((size_t)uu * p.n_kv_heads + kvh) * p.cap64 + sl) * T::K_ROW;
        const rsrc_t krs = make_rsrc(kb, kbytes);
        const rsrc_t ksrs = make_rsrc(p.k_scales + uu * p.k_sc_b + kvh * p.k_sc_h + (size_t)sl * p.k_sc_t,
                                      rem * p.k_sc_t * 2);
        const rsrc_t vsrs = make_rsrc(p.v_scales + uu * p.v_sc_b + kvh * p.v_sc_h + (size_t)sl * p.v_sc_t,
                                      rem * p.v_sc_t * 2);
        // (immediate offsets reach 4 KiB: int8 rows use a second descriptor
        // for slices 4..7)
        const rsrc_t krs2 = make_rsrc(kb + 4096, kbytes > 4096 ? kbytes - 4096 : 0);
#pragma unroll
        for (int u4 = 0; u4 < T::K_U4; u4++) d.k[u4] = bld_u4<CP_NT>(u4 < 4 ? krs : krs2, ko + (u4 % 4) * 1024);
#pragma unroll
        for (int g = 0; g < KG; g++) {
            d.ks[g] = bld_u16(ksrs, kso + 2 * g);
            d.vs[g] = bld_u16(vsrs, vso + 2 * g);
        }
    };
    float mloc[G];                                   // per-lane maxima of the current sub-chunk:
    uint32_t vmloc[KG];                              // scores; value scales as fp16 bits (>= 0, so
                                                     // the largest bits are the largest value)
    // scores of one tile (tb: first position of the tile within the wave;
    // sc0: first position of the sub-chunk)
    auto compute = [&](int tb, int sc0, const Tile &c) {
        const int t = tb + lane;
        const bool valid = t < nw;
#pragma unroll
        for (int g = 0; g < KG; g++) {
            // (zero past the wave's range: the load returned zero)
            if (valid) vsl[(t - sc0) * KG + g] = (uint16_t)c.vs[g];
            vmloc[g] = max(vmloc[g], c.vs[g]);
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
            const float sk = f16_bits_to_f32((uint16_t)c.ks[blk]);
#pragma unroll
            for (int h = 0; h < G; h++) z[h] = blk == 0 ? (float)acc[h] * sk : fmaf((float)acc[h], sk, z[h]);
        }
        if (valid) {
#pragma unroll
            for (int h = 0; h < G; h++) mloc[h] = fmax_nc(mloc[h], z[h]);
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
        const uint8_t *vb = p.v_codes + (((size_t)uu * p.n_kv_heads + kvh) * p.cap4 + slot_of(4 * g0)) * T::V_ROW;
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
    const uint32_t *wdg = wdw + (size_t)vgrp * (S / 4) * G * 2;
    uint32_t accl[G][T::V_ACC], acch[G][T::V_ACC];
    // one 4-position group: weight words of local group rg (LDS broadcast)
    // times the value codes this lane holds for it
    auto group = [&](int rg, const uint32_t (&x)[T::V_DPL]) {
        uint32_t wl[G], wh[G];
        const uint32_t *src = wdg + (size_t)rg * G * 2;
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

    Tile ta, tb_;
    load(0, ta);
    for (int sc0 = 0; sc0 < nw; sc0 += S) {
        const int ns = min(S, nw - sc0);             // positions of this sub-chunk
        // ---------------- pass 1: scores of the sub-chunk ----------------------
#pragma unroll
        for (int h = 0; h < G; h++) mloc[h] = -INFINITY;
#pragma unroll
        for (int g = 0; g < KG; g++) vmloc[g] = 0u;
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
        {
            const VRs rs = vrsrc(sc0 >> 2);
#pragma unroll
            for (int f = 0; f < PF; f++) vload(f, rs);
        }
        compute(tb + 64, sc0, tb_);
        float ms[G], vms[KG];                        // sub-chunk maxima, wave-uniform
#pragma unroll
        for (int h = 0; h < G; h++) ms[h] = wave_max_u(mloc[h]);
#pragma unroll
        for (int g = 0; g < KG; g++) vms[g] = f16_bits_to_f32((uint16_t)wave_max_ui((int)vmloc[g]));

        // ---------------- pass 2: weights, one lane per 4 positions ---------------
        // p = 2^(qs * (z - ms)) <= 1; w_int = rint(p * s_v * 32767 / vms),
        // rounded by one fma onto 1.5 * 2^23 (the integer lands in the low
        // mantissa bits); bytes packed four positions per word.
        float lloc[G];
        int wsl[KG][G];
        {
            constexpr float MAGIC = 12582912.0f;     // 1.5 * 2^23
            float nqm[G];
#pragma unroll
            for (int h = 0; h < G; h++) {
                nqm[h] = -ms[h] * qs[h];
                lloc[h] = 0.0f;
            }
#pragma unroll
            for (int g = 0; g < KG; g++)
#pragma unroll
                for (int h = 0; h < G; h++) wsl[g][h] = 0;
            float fsc[KG];
#pragma unroll
            for (int g = 0; g < KG; g++) fsc[g] = vms[g] > 0.0f ? (float)W_RANGE * __builtin_amdgcn_rcpf(vms[g]) : 0.0f;
            // S / 4 groups of 4 positions, one per lane and turn (the weight
            // words go over the scores: a turn writes only rows it or an
            // earlier turn has read)
#pragma unroll
            for (int gq = 0; gq < S / 4; gq += 64) {
            const int grp = gq + lane;
            const int tq = 4 * grp;                  // first position of the group (within the sub-chunk)
            if (tq < ns) {
                float pr[4][G];
#pragma unroll
                for (int k = 0; k < 4; k++) {
                    const bool valid = tq + k < ns;
                    const float *src = zs + (size_t)(tq + k) * G;
                    float zz[G];
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
#pragma unroll
                    for (int h = 0; h < G; h++) {
                        pr[k][h] = valid ? __builtin_amdgcn_exp2f(fmaf(zz[h], qs[h], nqm[h])) : 0.0f;
                        lloc[h] += pr[k][h];
                    }
                }
#pragma unroll
                for (int g = 0; g < KG; g++) {
                    float sv[4];
#pragma unroll
                    for (int k = 0; k < 4; k++)
                        sv[k] = tq + k < ns ? f16_bits_to_f32(vsl[(tq + k) * KG + g]) * fsc[g] : 0.0f;
                    uint32_t *dst = wdw + ((size_t)g * (S / 4) + grp) * G * 2;
#pragma unroll
                    for (int h = 0; h < G; h++) {
                        uint32_t wb[4];
#pragma unroll
                        for (int k = 0; k < 4; k++) wb[k] = __builtin_bit_cast(uint32_t, fmaf(pr[k][h], sv[k], MAGIC));
                        uint32_t lo, hi;
                        pack_w(wb[0], wb[1], wb[2], wb[3], lo, hi);
                        wsl[g][h] += (int)__builtin_amdgcn_udot4(lo, 0x01010101u, 0u, false)
                                   + 256 * (int)__builtin_amdgcn_udot4(hi, 0x01010101u, 0u, false);
                        dst[2 * h] = lo;
                        dst[2 * h + 1] = hi;
                    }
                }
            }
            }
        }

        // ---------------- pass 3: values of the sub-chunk ------------------------
#pragma unroll
        for (int h = 0; h < G; h++)
#pragma unroll
            for (int c = 0; c < T::V_ACC; c++) accl[h][c] = acch[h][c] = 0u;
        {
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
#pragma unroll
            for (int h = 0; h < G; h++) {
                const float Mn = fmaxf(M[h], ms[h]);
                const float fo = M[h] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(qs[h] * (M[h] - Mn));
                const float fn = __builtin_amdgcn_exp2f(qs[h] * (ms[h] - Mn));
                M[h] = Mn;
                lsum[h] = fmaf(lsum[h], fo, lloc[h] * fn);
                float cg[KG];                        // c = fn * vms / 32767 per scale group
#pragma unroll
                for (int g = 0; g < KG; g++) {
                    cg[g] = fn * vms[g] * (1.0f / (float)W_RANGE);
                    bsum[g][h] = fmaf(bsum[g][h], fo, (float)wsl[g][h] * cg[g]);
                }
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
        // the offset binary: code = stored - bias, so subtract bias * sum(w)
        // (in the same fixed-point units) from every channel
        const float bias = VB == 4 ? 8.0f : 128.0f;
#pragma unroll
        for (int g = 0; g < KG; g++)
#pragma unroll
            for (int h = 0; h < G; h++) {
                const float ob = bias * wave_sum_u(bsum[g][h]);
#pragma unroll
                for (int c = 0; c < T::V_ACC; c++)
                    if ((qsl * T::V_ACC + c) / (HD / KG) == g) af[h][c] -= ob;
            }
    }
    __syncthreads();                                 // every wave is done with scores and weights
    float *pm = misc;                                // [QD_WAVES][G] wave maxima (log2 units)
    float *pl = pm + QD_WAVES * G;                   // [QD_WAVES][G] wave sums of p
    if (gi == 0) {
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
    for (int i = tid; i < G * HD; i += QD_THREADS) {
        const int h = i / HD, c = i - h * HD;
        float m = pm[h];
#pragma unroll
        for (int w = 1; w < QD_WAVES; w++) m = fmaxf(m, pm[w * G + h]);
        float s = 0.0f;
#pragma unroll
        for (int w = 0; w < QD_WAVES; w++) {
            const float mv = pm[w * G + h];
            if (mv != -INFINITY) s = fmaf(__builtin_amdgcn_exp2f(mv - m), red[(w * G + h) * HD + c], s);
        }
        store_partial(&acc0[h * acc_hs + c], s);
    }
    if (tid < G) {
        float m = pm[tid];
#pragma unroll
        for (int w = 1; w < QD_WAVES; w++) m = fmaxf(m, pm[w * G + tid]);
        float l = 0.0f;
#pragma unroll
        for (int w = 0; w < QD_WAVES; w++) {
            const float mv = pm[w * G + tid];
            if (mv != -INFINITY) l = fmaf(__builtin_amdgcn_exp2f(mv - m), pl[w * G + tid], l);
        }
        store_partial(&ml0[tid * ml_hs], m);
        store_partial(&ml0[tid * ml_hs + 1], l);
    }
    finish();
}

} // namespace kvq
