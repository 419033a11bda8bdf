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
//    stored four positions interleaved (offset binary after one XOR).
// Rounding happens only in q_int (|dq| <= s_q / 2) and in w_int
// (|dw| <= max s_v / 65534); accumulation is exact in int32, then fp32.
//
// Workgroup = 4 waves = one context chunk of one (sequence, KV head); each
// wave owns a quarter of the chunk.
//   1. keys, one lane per position: scores (log2 units) -> LDS; the query
//      digits are wave-uniform and come from SGPRs (prepared per (sequence,
//      KV head) by qprep_kernel); value scales -> LDS; running maxima.
//   -- workgroup barrier: chunk max of the scores and of the value scales --
//   2. weights, one lane per four positions: p = 2^(z - max), l += p,
//      w_int digits packed four positions per word -> LDS (over the wave's
//      own scores).
//   3. values: a lane owns fixed byte positions (two channels) of every
//      4-position group and accumulates v_dot4_u32_u8 over the wave's groups;
//      the group's weight words are LDS broadcasts.
//   -- workgroup barrier --
//   4. sum the 4 waves, undo the offset binary and the fixed point, write the
//      chunk's (m, l, acc).
#pragma once

#include "kvq_device.hpp"

namespace kvq {

constexpr int QD_THREADS = 256;
constexpr int QD_WAVES = QD_THREADS / 64;
constexpr int Q_RANGE = 30000;
constexpr int W_RANGE = 32767;

template <int KB, int VB, int HD, int G> struct QT {
    static constexpr int K_ROW = HD * KB / 8;          // bytes per key row
    static constexpr int K_U4 = K_ROW / 16;            // 16-byte loads per key row
    static constexpr int K_COLS = K_ROW / 4;           // dwords per key row
    static constexpr int ND = KB == 4 ? 4 : 2;         // query digits
    static constexpr int DBASE = KB == 4 ? 16 : 256;   // digit base
    static constexpr int CPC = KB == 4 ? 8 : 4;        // channels per key dword
    static constexpr int BLK_COLS = 32 / CPC;          // key dwords per 32-channel block
    static constexpr int V_ROW = HD * VB / 8;          // bytes per value row
    static constexpr int V_DW = V_ROW;                 // dwords per 4-position group
    static constexpr int V_DPL = V_DW >= 64 ? V_DW / 64 : 1;   // dwords per lane
    static constexpr int V_GPL = V_DW >= 64 ? 1 : 64 / V_DW;   // groups per wave load
    static constexpr int V_LPG = 64 / V_GPL;           // lanes per group
    static constexpr int V_CPD = VB == 4 ? 2 : 1;      // channels per dword
    static constexpr int V_ACC = V_DPL * V_CPD;        // channels per lane
};

struct QuantParams {
    const uint8_t *k_codes;    // [B][Hkv][cap][K_ROW]
    const uint8_t *v_codes;    // [B][Hkv][cap4/4][V_ROW][4]  (4 positions interleaved per byte)
    const uint16_t *k_scales;
    const uint16_t *v_scales;
    const int32_t *qdig;       // [B*Hkv][ND][K_COLS][G] packed query digits
    const float *qsc;          // [B*Hq]: s_q * softmax_scale * log2(e)
    const int32_t *seq_len;
    float *ws_ml;
    float *ws_acc;
    int n_kv_heads, capacity, cap4;
    int max_len;
    int chunk, n_chunks;
    int kg, vg;                // scale groups per head row
    int k_group, v_group;      // values per scale
    long long k_sc_b, k_sc_h;
    int k_sc_t;
    long long v_sc_b, v_sc_h;
    int v_sc_t;
};

struct QuantSmem {
    int zs, vs, wd, red, misc, total;
    bool wd_alias;             // weight words overwrite each wave's own scores
};

__host__ __device__ inline QuantSmem quant_smem(int G, int HD, int chunk, int vg)
{
    QuantSmem s;
    int off = 0;
    s.zs = off;
    off += chunk * G * 4;                          // scores [chunk][G]
    s.vs = off;
    off += chunk * vg * 4;                         // value scales [chunk][vg]
    s.wd_alias = vg == 1;
    if (s.wd_alias) {
        s.wd = s.zs;
    } else {
        s.wd = off;
        off += vg * (chunk / 4) * G * 2 * 4;       // weight words [vg][chunk/4][G][lo, hi]
    }
    const int red = QD_WAVES * G * HD * 4;
    if (chunk * G * 4 >= red) {
        s.red = s.zs;                              // scores and weights are dead in pass 4
    } else {
        s.red = off;
        off += red;
    }
    s.misc = off;
    off += (2 * G + 8 + QD_WAVES * G + QD_WAVES * 4 + QD_WAVES * G + QD_WAVES * 4 * G) * 4;
    s.total = off;
    return s;
}

// ---------------------------------------------------------------------------
// Query digits: one block per (sequence, KV head).  For head h of the group,
// s_q = max|q| / 30000 and q_int = rint(q / s_q) in [-30000, 30000], split
// into ND balanced digits; digit j of the channels of key dword `col` is
// packed like the codes (int4: channel 8col+i in nibble i; int8: channel
// 4col+i in byte i) at qdig[unit][j][col][h].
// ---------------------------------------------------------------------------
template <int KB, int HD, int G>
__global__ __launch_bounds__(256) void qprep_kernel(const float *__restrict__ q, int32_t *__restrict__ qdig,
                                                    float *__restrict__ qsc, float qk_scale)
{
    constexpr int K_COLS = HD * KB / 32;
    constexpr int ND = KB == 4 ? 4 : 2;
    constexpr int CPC = KB == 4 ? 8 : 4;
    constexpr int BITS = KB == 4 ? 4 : 8;
    const int unit = blockIdx.x;                         // b * Hkv + kvh
    const float *qh = q + (size_t)unit * G * HD;         // query heads unit*G .. unit*G+G-1
    __shared__ float amax[G];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int h = wave; h < G; h += 4) {
        float a = 0.0f;
        for (int c = lane; c < HD; c += 64) a = fmaxf(a, fabsf(qh[h * HD + c]));
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
            int qi = (int)fminf(fmaxf(rintf(qh[h * HD + col * CPC + e] * inv), -(float)Q_RANGE), (float)Q_RANGE);
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
}

template <int KB>
__device__ __forceinline__ int kdot(int qd, int k, int acc)
{
    if constexpr (KB == 4) return __builtin_amdgcn_sdot8(qd, k, acc, false);
    else return __builtin_amdgcn_sdot4(qd, k, acc, false);
}

__device__ __forceinline__ uint32_t kword(const uint4 &r, int i)
{
    return (i & 3) == 0 ? r.x : (i & 3) == 1 ? r.y : (i & 3) == 2 ? r.z : r.w;
}

// Exact sum_c q_int[h][c] * code[c] over key dwords [c0, c1) of one row,
// digit-major Horner (highest digit first, acc *= base between digits).
// c0, c1 are compile-time constants after unrolling at every call.
template <int KB, int VB, int HD, int G>
__device__ __forceinline__ void key_dots(const uint4 (&kr)[QT<KB, VB, HD, G>::K_U4], const KVQ_CONST int32_t *qd,
                                         int c0, int c1, int (&acc)[G])
{
    using T = QT<KB, VB, HD, G>;
#pragma unroll
    for (int h = 0; h < G; h++) acc[h] = 0;
#pragma unroll
    for (int j = T::ND - 1; j >= 0; j--) {
        if (j < T::ND - 1) {
#pragma unroll
            for (int h = 0; h < G; h++) acc[h] *= T::DBASE;
        }
#pragma unroll
        for (int col = 0; col < T::K_COLS; col++) {
            if (col < c0 || col >= c1) continue;
            if (((col - c0) & 1) == 0)
                asm volatile("" : "+s"(qd));         // at most two digit columns in SGPRs at once
            const int kw = (int)kword(kr[col / 4], col);
#pragma unroll
            for (int h = 0; h < G; h++) acc[h] = kdot<KB>(qd[(j * T::K_COLS + col) * G + h], kw, acc[h]);
        }
    }
}

// KGM = 1: one key scale per row (groups of head_dim or per-position scales);
// KGM = 4: up to 4 scale groups per row, summed per 32-channel block.
template <int KB, int VB, int HD, int G, int KGM>
__global__ __launch_bounds__(QD_THREADS) void decode_quant_kernel(QuantParams p)
{
    using T = QT<KB, VB, HD, G>;
    extern __shared__ __align__(16) unsigned char smem[];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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

    if (n_tok <= 0) {
        for (int i = tid; i < G * HD; i += QD_THREADS) acc0[(i / HD) * acc_hs + (i % HD)] = 0.0f;
        if (tid < G) {
            ml0[tid * ml_hs] = -INFINITY;
            ml0[tid * ml_hs + 1] = 0.0f;
        }
        return;
    }

    const QuantSmem lay = quant_smem(G, HD, CH, p.vg);
    float *zs = reinterpret_cast<float *>(smem + lay.zs);
    float *vs = reinterpret_cast<float *>(smem + lay.vs);
    float *red = reinterpret_cast<float *>(smem + lay.red);
    float *misc = reinterpret_cast<float *>(smem + lay.misc);
    float *m_sh = misc;                              // [G]
    float *l_sh = m_sh + G;                          // [G]
    float *vmax_sh = l_sh + G;                       // [4] (8 reserved)
    float *part = vmax_sh + 8;                       // [QD_WAVES][G]
    float *vpart = part + QD_WAVES * G;              // [QD_WAVES][4]
    float *lpart = vpart + QD_WAVES * 4;             // [QD_WAVES][G]
    float *wsum = lpart + QD_WAVES * G;              // [QD_WAVES][4][G]

    const int sub = CH / QD_WAVES;                   // positions per wave (multiple of 16)
    const int s0 = wave * sub;
    const int s1 = min(s0 + sub, n_tok);             // may be <= s0
    // this wave's weight words: over its own scores when there is one value group
    uint32_t *wdw = lay.wd_alias ? reinterpret_cast<uint32_t *>(zs + (size_t)s0 * G)
                                 : reinterpret_cast<uint32_t *>(smem + lay.wd) + (size_t)wave * p.vg * (sub / 4) * G * 2;

    float qs[G];
#pragma unroll
    for (int h = 0; h < G; h++) qs[h] = p.qsc[row0 + h];

    // ---------------- pass 1: scores ------------------------------------
    float mloc[G];
#pragma unroll
    for (int h = 0; h < G; h++) mloc[h] = -INFINITY;
    float vmloc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    {
        const uint8_t *kbase = p.k_codes + ((size_t)bh * p.capacity + t0) * T::K_ROW;
        const uint16_t *ksrc = p.k_scales + b * p.k_sc_b + kvh * p.k_sc_h + (size_t)t0 * p.k_sc_t;
        const uint16_t *vsrc = p.v_scales + b * p.v_sc_b + kvh * p.v_sc_h + (size_t)t0 * p.v_sc_t;
        const KVQ_CONST int32_t *qd = (const KVQ_CONST int32_t *)(p.qdig + (size_t)bh * T::ND * T::K_COLS * G);
        // Everything a tile needs (key row, key scales, value scales) is
        // loaded one tile ahead, so the loads of tile i+1 are in flight while
        // tile i computes: the vector-memory counter retires loads in order,
        // and consuming a load issued in the same iteration would wait for
        // the prefetch too.
        constexpr int NKS = KGM;                     // key scales per row loaded
        uint4 kr[T::K_U4];
        // (scales kept one per 32-bit register: packing two 16-bit loads into
        // one register would make the compiler wait for them at once)
        uint32_t ksr[NKS], vsr[4];
        // Loads are unconditional (positions past the end read the last
        // valid row and are ignored), so the code stays straight-line and the
        // compiler can wait for exactly the previous tile's loads.
        const int t_last = s1 - 1;                   // >= 0: the chunk has a position
        auto load_tile = [&](int t, uint4 (&k)[T::K_U4], uint32_t (&ks)[NKS], uint32_t (&vv)[4]) {
            const int ts = min(t, t_last);
#pragma unroll
            for (int u = 0; u < T::K_U4; u++) k[u] = ld_u4(kbase + (size_t)ts * T::K_ROW + u * 16);
#pragma unroll
            for (int g = 0; g < NKS; g++) ks[g] = ld_u16(ksrc + (size_t)ts * p.k_sc_t + min(g, p.kg - 1));
#pragma unroll
            for (int g = 0; g < 4; g++) vv[g] = ld_u16(vsrc + (size_t)ts * p.v_sc_t + min(g, p.vg - 1));
        };
        load_tile(s0 + lane, kr, ksr, vsr);
        for (int tb = s0; tb < s1; tb += 64) {
            const int t = tb + lane;
            const bool valid = t < s1;
            uint4 kn[T::K_U4];
            uint32_t ksn[NKS], vsn[4];
            load_tile(t + 64, kn, ksn, vsn);
            // value scales of this position -> LDS, running max per group
#pragma unroll
            for (int g = 0; g < 4; g++) {
                if (g < p.vg) {
                    const float sv = valid ? f16_bits_to_f32((uint16_t)vsr[g]) : 0.0f;
                    if (valid) vs[t * p.vg + g] = sv;
                    vmloc[g] = fmaxf(vmloc[g], sv);
                }
            }
            const KVQ_CONST int32_t *qdl = qd;
            asm volatile("" : "+s"(qdl));            // keep the digit loads inside the loop
            float z[G];
            if constexpr (KGM == 1) {
                int acc[G];
                key_dots<KB, VB, HD, G>(kr, qdl, 0, T::K_COLS, acc);
                const float sk = f16_bits_to_f32((uint16_t)ksr[0]);
#pragma unroll
                for (int h = 0; h < G; h++) z[h] = (float)acc[h] * sk;
            } else {
#pragma unroll
                for (int h = 0; h < G; h++) z[h] = 0.0f;
#pragma unroll
                for (int blk = 0; blk < HD / 32; blk++) {
                    int acc[G];
                    key_dots<KB, VB, HD, G>(kr, qdl, blk * T::BLK_COLS, (blk + 1) * T::BLK_COLS, acc);
                    const int grp = (blk * 32) / p.k_group;
                    const float sk = f16_bits_to_f32((uint16_t)(grp == 0 ? ksr[0] : grp == 1 ? ksr[NKS > 1 ? 1 : 0]
                                                     : grp == 2 ? ksr[NKS > 2 ? 2 : 0] : ksr[NKS > 3 ? 3 : 0]));
#pragma unroll
                    for (int h = 0; h < G; h++) z[h] = fmaf((float)acc[h], sk, z[h]);
                }
            }
            if (valid) {
#pragma unroll
                for (int h = 0; h < G; h++) {
                    z[h] *= qs[h];
                    mloc[h] = fmaxf(mloc[h], z[h]);
                }
                float *dst = zs + (size_t)t * G;
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
#pragma unroll
            for (int u = 0; u < T::K_U4; u++) kr[u] = kn[u];
#pragma unroll
            for (int g = 0; g < NKS; g++) ksr[g] = ksn[g];
#pragma unroll
            for (int g = 0; g < 4; g++) vsr[g] = vsn[g];
        }
    }
    // chunk maxima of the scores (per head) and of the value scales (per group)
#pragma unroll
    for (int h = 0; h < G; h++) {
        const float v = wave_max(mloc[h]);
        if (lane == 0) part[wave * G + h] = v;
    }
#pragma unroll
    for (int g = 0; g < 4; g++) {
        if (g < p.vg) {
            const float v = wave_max(vmloc[g]);
            if (lane == 0) vpart[wave * 4 + g] = v;
        }
    }
    __syncthreads();
    if (tid < G) {
        float v = part[tid];
#pragma unroll
        for (int w = 1; w < QD_WAVES; w++) v = fmaxf(v, part[w * G + tid]);
        m_sh[tid] = v;
    } else if (tid >= 64 && tid < 64 + p.vg) {
        const int g = tid - 64;
        float v = vpart[g];
#pragma unroll
        for (int w = 1; w < QD_WAVES; w++) v = fmaxf(v, vpart[w * 4 + g]);
        vmax_sh[g] = v;
    }
    __syncthreads();

    // ---------------- pass 2: weights, one lane per 4 positions ---------------
    {
        float mh[G], lloc[G];
#pragma unroll
        for (int h = 0; h < G; h++) {
            mh[h] = m_sh[h];
            lloc[h] = 0.0f;
        }
        int wsl[4][G];
#pragma unroll
        for (int g = 0; g < 4; g++)
#pragma unroll
            for (int h = 0; h < G; h++) wsl[g][h] = 0;
        float fsc[4];
#pragma unroll
        for (int g = 0; g < 4; g++) {
            const float vmax = g < p.vg ? vmax_sh[g] : 0.0f;
            fsc[g] = vmax > 0.0f ? (float)W_RANGE / vmax : 0.0f;
        }
        for (int tb = s0; tb < s1; tb += 256) {
            const int tq = tb + 4 * lane;                // first position of this lane's group
            if (tq < s1) {
                float pr[4][G];
#pragma unroll
                for (int k = 0; k < 4; k++) {
                    const bool valid = tq + k < s1;
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
                        pr[k][h] = valid ? __builtin_amdgcn_exp2f(zz[h] - mh[h]) : 0.0f;
                        lloc[h] += pr[k][h];
                    }
                }
                const int rg = (tq - s0) >> 2;           // group index within the wave
#pragma unroll
                for (int g = 0; g < 4; g++) {
                    if (g < p.vg) {
                        float sv[4];
#pragma unroll
                        for (int k = 0; k < 4; k++) sv[k] = tq + k < s1 ? vs[(tq + k) * p.vg + g] * fsc[g] : 0.0f;
                        uint32_t *dst = wdw + ((size_t)g * (sub / 4) + rg) * G * 2;
#pragma unroll
                        for (int h = 0; h < G; h++) {
                            uint32_t lo = 0, hi = 0;
#pragma unroll
                            for (int k = 0; k < 4; k++) {
                                const int wi = (int)rintf(fminf(pr[k][h] * sv[k], (float)W_RANGE));
                                wsl[g][h] += wi;
                                lo |= (uint32_t)(wi & 0xFF) << (8 * k);
                                hi |= (uint32_t)(wi >> 8) << (8 * k);
                            }
                            dst[2 * h] = lo;
                            dst[2 * h + 1] = hi;
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int h = 0; h < G; h++) {
            const float v = wave_sum(lloc[h]);
            if (lane == 0) lpart[wave * G + h] = v;
        }
#pragma unroll
        for (int g = 0; g < 4; g++) {
            if (g < p.vg) {
#pragma unroll
                for (int h = 0; h < G; h++) {
                    int v = wsl[g][h];
#pragma unroll
                    for (int m = 1; m < 64; m <<= 1) v += __shfl_xor(v, m, 64);
                    if (lane == 0) wsum[(wave * 4 + g) * G + h] = (float)v;
                }
            }
        }
    }

    // ---------------- pass 3: values ---------------------------------------
    // lane -> (group slot gi of the load, dword slice qsl of the group)
    const int gi = lane / T::V_LPG;
    const int qsl = lane % T::V_LPG;
    uint32_t accl[G][T::V_ACC], acch[G][T::V_ACC];
#pragma unroll
    for (int h = 0; h < G; h++)
#pragma unroll
        for (int c = 0; c < T::V_ACC; c++) accl[h][c] = acch[h][c] = 0u;
    {
        constexpr int PF = 8;                        // group loads per lane in flight
        const int ng = (s1 - s0 + 3) >> 2;           // groups of this wave with a valid position
        const int vgrp = (qsl * T::V_DPL * T::V_CPD) / p.v_group;
        const uint32_t *wdg = wdw + (size_t)vgrp * (sub / 4) * G * 2;
        const uint8_t *vbase = p.v_codes + ((size_t)bh * p.cap4 + t0 + s0) * T::V_ROW + qsl * T::V_DPL * 4;
        // unconditional loads (groups past the end re-read the last one and
        // are skipped), one batch of PF groups ahead
        const int g_last = ng - 1;
        uint32_t cur[PF][T::V_DPL];
#pragma unroll
        for (int f = 0; f < PF; f++) {
            const int rg = max(min(f * T::V_GPL + gi, g_last), 0);
#pragma unroll
            for (int d = 0; d < T::V_DPL; d++)
                cur[f][d] = *(const KVQ_GLOBAL uint32_t *)(vbase + (size_t)rg * 4 * T::V_ROW + d * 4);
        }
        for (int rb = 0; rb < ng; rb += PF * T::V_GPL) {
            uint32_t nxt[PF][T::V_DPL];
#pragma unroll
            for (int f = 0; f < PF; f++) {
                const int rg = min(rb + (PF + f) * T::V_GPL + gi, g_last);
#pragma unroll
                for (int d = 0; d < T::V_DPL; d++)
                    nxt[f][d] = *(const KVQ_GLOBAL uint32_t *)(vbase + (size_t)rg * 4 * T::V_ROW + d * 4);
            }
#pragma unroll
            for (int f = 0; f < PF; f++) {
                const int rg = rb + f * T::V_GPL + gi;
                if (rg < ng) {
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
                            const uint32_t u = cur[f][d] ^ 0x88888888u;   // offset binary per nibble
                            const uint32_t ulo = u & 0x0F0F0F0Fu;          // even channel, 4 positions
                            const uint32_t uhi = u & 0xF0F0F0F0u;          // odd channel, x16
#pragma unroll
                            for (int h = 0; h < G; h++) {
                                accl[h][2 * d] = __builtin_amdgcn_udot4(wl[h], ulo, accl[h][2 * d], false);
                                acch[h][2 * d] = __builtin_amdgcn_udot4(wh[h], ulo, acch[h][2 * d], false);
                                accl[h][2 * d + 1] = __builtin_amdgcn_udot4(wl[h], uhi, accl[h][2 * d + 1], false);
                                acch[h][2 * d + 1] = __builtin_amdgcn_udot4(wh[h], uhi, acch[h][2 * d + 1], false);
                            }
                        } else {
                            const uint32_t u = cur[f][d] ^ 0x80808080u;   // offset binary per byte
#pragma unroll
                            for (int h = 0; h < G; h++) {
                                accl[h][d] = __builtin_amdgcn_udot4(wl[h], u, accl[h][d], false);
                                acch[h][d] = __builtin_amdgcn_udot4(wh[h], u, acch[h][d], false);
                            }
                        }
                    }
                }
            }
#pragma unroll
            for (int f = 0; f < PF; f++)
#pragma unroll
                for (int d = 0; d < T::V_DPL; d++) cur[f][d] = nxt[f][d];
        }
    }

    // ---------------- pass 4: reduce, undo offsets, write ------------------
    float af[G][T::V_ACC];
#pragma unroll
    for (int h = 0; h < G; h++)
#pragma unroll
        for (int c = 0; c < T::V_ACC; c++) af[h][c] = 256.0f * (float)acch[h][c] + (float)accl[h][c];
    if constexpr (T::V_GPL > 1) {
        // lanes holding the same channels for different group slots
#pragma unroll
        for (int m = T::V_LPG; m < 64; m <<= 1)
#pragma unroll
            for (int h = 0; h < G; h++)
#pragma unroll
                for (int c = 0; c < T::V_ACC; c++) af[h][c] += __shfl_xor(af[h][c], m, 64);
    }
    __syncthreads();                                 // every wave is done with scores and weights
    if (gi == 0) {
        // lane's channels: byte positions qsl*V_DPL + d -> V4: channels 2(...), 2(...)+1; V8: (...)
#pragma unroll
        for (int h = 0; h < G; h++)
#pragma unroll
            for (int c = 0; c < T::V_ACC; c++) red[(wave * G + h) * HD + qsl * T::V_ACC + c] = af[h][c];
    }
    __syncthreads();
    for (int i = tid; i < G * HD; i += QD_THREADS) {
        const int h = i / HD, c = i - h * HD;
        float s = 0.0f, wtot = 0.0f;
#pragma unroll
        for (int w = 0; w < QD_WAVES; w++) s += red[(w * G + h) * HD + c];
        const int g = p.vg == 1 ? 0 : c / p.v_group;  // scale group of channel c
#pragma unroll
        for (int w = 0; w < QD_WAVES; w++) wtot += wsum[(w * 4 + g) * G + h];
        // V4 odd channels accumulated 16u; the codes are u - 8 (V4) or u - 128 (V8)
        const float su = (VB == 4 && (c & 1)) ? s * 0.0625f : s;
        const float bias = VB == 4 ? 8.0f : 128.0f;
        acc0[h * acc_hs + c] = (su - bias * wtot) * (vmax_sh[g] / (float)W_RANGE);
    }
    if (tid < G) {
        float lt = 0.0f;
#pragma unroll
        for (int w = 0; w < QD_WAVES; w++) lt += lpart[w * G + tid];
        ml0[tid * ml_hs] = m_sh[tid];
        ml0[tid * ml_hs + 1] = lt;
    }
}

} // namespace kvq
