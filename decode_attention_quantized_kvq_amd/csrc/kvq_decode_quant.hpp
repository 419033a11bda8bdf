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
    off += 2 * QD_WAVES * G * 4;                   // wave maxima and sums
    s.total = off;
    return s;
}

// ---------------------------------------------------------------------------
// Query digits: one block per (sequence, KV head).  For head h of the group,
// s_q = max|q| / 30000 and q_int = rint(q / s_q) in [-30000, 30000], split
// into ND balanced digits; digit j of the channels of key dword `col` is
// packed like the codes (int4: channel 8col+i in nibble i; int8: channel
// 4col+i in byte i) at qdig[unit][col][j][h], so the ND * G digit words of
// one key dword are contiguous (one scalar load).
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
        for (int j = 0; j < ND; j++) qdig[(((size_t)unit * K_COLS + col) * ND + j) * G + h] = (int32_t)d[j];
    }
    if (tid < G) qsc[unit * G + tid] = amax[tid] / (float)Q_RANGE * qk_scale;
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
// per 32-channel block.
template <int KB, int VB, int HD, int G, int KG>
__global__ __launch_bounds__(QD_THREADS) void decode_quant_kernel(QuantParams p)
{
    using T = QT<KB, VB, HD, G>;
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

    if (n_tok <= 0) {
        for (int i = tid; i < G * HD; i += QD_THREADS) acc0[(i / HD) * acc_hs + (i % HD)] = 0.0f;
        if (tid < G) {
            ml0[tid * ml_hs] = -INFINITY;
            ml0[tid * ml_hs + 1] = 0.0f;
        }
        return;
    }

    const QuantSmem lay = quant_smem(G, HD, CH, KG);
    float *zs = reinterpret_cast<float *>(smem + lay.zs);
    float *vs = reinterpret_cast<float *>(smem + lay.vs);
    float *red = reinterpret_cast<float *>(smem + lay.red);
    float *misc = reinterpret_cast<float *>(smem + lay.misc);

    const int sub = CH / QD_WAVES;                   // positions per wave (multiple of 16)
    const int s0 = wave * sub;
    const int nw = max(min(sub, n_tok - s0), 0);     // positions of this wave
    // this wave's weight words: over its own scores when there is one value group
    uint32_t *wdw = lay.wd_alias ? reinterpret_cast<uint32_t *>(zs + (size_t)s0 * G)
                                 : reinterpret_cast<uint32_t *>(smem + lay.wd) + (size_t)wave * KG * (sub / 4) * G * 2;

    float qs[G];
#pragma unroll
    for (int h = 0; h < G; h++) qs[h] = p.qsc[row0 + h];

    // ---------------- pass 1: scores (unscaled: z = sum q_int * code * s_k) ----
    float mloc[G];
#pragma unroll
    for (int h = 0; h < G; h++) mloc[h] = -INFINITY;
    float vmloc[KG];
#pragma unroll
    for (int g = 0; g < KG; g++) vmloc[g] = 0.0f;
    {
        const uint8_t *kb0 = p.k_codes + ((size_t)bh * p.capacity + t0 + s0) * T::K_ROW;
        const uint16_t *ks0 = p.k_scales + b * p.k_sc_b + kvh * p.k_sc_h + (size_t)(t0 + s0) * p.k_sc_t;
        const uint16_t *vs0 = p.v_scales + b * p.v_sc_b + kvh * p.v_sc_h + (size_t)(t0 + s0) * p.v_sc_t;
        const KVQ_CONST int32_t *qd = (const KVQ_CONST int32_t *)(p.qdig + (size_t)bh * T::K_COLS * T::ND * G);
        const uint32_t ko = lane * T::K_ROW;         // this lane's row within a tile
        const uint32_t kso = lane * p.k_sc_t * 2, vso = lane * p.v_sc_t * 2;
        constexpr int CPB = T::K_COLS / KG;                    // key dwords per scale group
        struct Tile {
            uint4 k[T::K_U4];
            uint32_t ks[KG], vs[KG];
        };
        // Everything a tile needs is loaded one tile ahead into the other of
        // two register sets (the loop is unrolled twice, so no copies and no
        // waits on the newer loads); past the wave's range the buffer loads
        // return zeros.
        // (the descriptors move with the tile, so the per-lane offsets are
        // loop-invariant and the pieces of a row use immediate offsets)
        auto load = [&](int tb, Tile &d) {
            const uint32_t rem = (uint32_t)max(nw - tb, 0);
            const rsrc_t krs = make_rsrc(kb0 + (size_t)tb * T::K_ROW, rem * T::K_ROW);
            const rsrc_t ksrs = make_rsrc(ks0 + (size_t)tb * p.k_sc_t, rem * p.k_sc_t * 2);
            const rsrc_t vsrs = make_rsrc(vs0 + (size_t)tb * p.v_sc_t, rem * p.v_sc_t * 2);
#pragma unroll
            for (int u = 0; u < T::K_U4; u++) d.k[u] = bld_u4(krs, ko + u * 16);
#pragma unroll
            for (int g = 0; g < KG; g++) {
                d.ks[g] = bld_u16(ksrs, kso + 2 * g);
                d.vs[g] = bld_u16(vsrs, vso + 2 * g);
            }
        };
        auto compute = [&](int tb, const Tile &c) {
            const int t = tb + lane;                           // position within the wave
            const bool valid = t < nw;
            // value scales of this position -> LDS, running max per group
#pragma unroll
            for (int g = 0; g < KG; g++) {
                // (zero past the wave's range: the load returned zero)
                const float sv = f16_bits_to_f32((uint16_t)c.vs[g]);
                if (valid) vs[(s0 + t) * KG + g] = sv;
                vmloc[g] = fmax_nc(vmloc[g], sv);
            }
            // an opaque zero offset, redefined every tile, keeps the digit
            // loads inside the loop (hoisted, they would need 256 SGPRs)
            int qz;
            asm volatile("s_mov_b32 %0, 0" : "=s"(qz));
            const KVQ_CONST int32_t *qdl = qd + qz;
            float z[G];
            // int4 keys: the digits of column c come through a pointer that
            // depends on every sum after column c - LAG, so about 96 digit
            // words are in SGPRs at once (the scheduler would otherwise load
            // them all early and spill).  int8 keys (twice the columns, half
            // the digits each) run faster with the scheduler's own deeper
            // prefetch, spills included.
            constexpr int LAG = 96 / (T::ND * G) > 2 ? 96 / (T::ND * G) : 2;
            const KVQ_CONST int32_t *ring[LAG];
#pragma unroll
            for (int i = 0; i < LAG; i++) ring[i] = qdl;
#pragma unroll
            for (int blk = 0; blk < KG; blk++) {
                int acc[T::ND][G];
#pragma unroll
                for (int cc = 0; cc < CPB; cc++) {
                    const int col = blk * CPB + cc;
                    const int kw = (int)kword(c.k[col / 4], col);
                    const KVQ_CONST int32_t *qc = ring[0] + col * T::ND * G;
#pragma unroll
                    for (int j = 0; j < T::ND; j++)
#pragma unroll
                        for (int h = 0; h < G; h++)
                            acc[j][h] = cc == 0 ? kdot0<KB>(qc[j * G + h], kw) : kdot<KB>(qc[j * G + h], kw, acc[j][h]);
#pragma unroll
                    for (int i = 0; i + 1 < LAG; i++) ring[i] = ring[i + 1];
                    const KVQ_CONST int32_t *qn = qdl;
#pragma unroll
                    for (int j = 0; j < T::ND; j++)
#pragma unroll
                        for (int h = 0; h < G; h++)
                            if constexpr (KB == 4) asm("" : "+s"(qn) : "v"(acc[j][h]));
                    ring[LAG - 1] = qn;
                }
                // Horner over the digits: exact int32 sum of q_int * code
                int tot[G];
#pragma unroll
                for (int h = 0; h < G; h++) {
                    tot[h] = acc[T::ND - 1][h];
#pragma unroll
                    for (int j = T::ND - 2; j >= 0; j--) tot[h] = tot[h] * T::DBASE + acc[j][h];
                }
                const float sk = f16_bits_to_f32((uint16_t)c.ks[blk]);
#pragma unroll
                for (int h = 0; h < G; h++) z[h] = blk == 0 ? (float)tot[h] * sk : fmaf((float)tot[h], sk, z[h]);
            }
            if (valid) {
#pragma unroll
                for (int h = 0; h < G; h++) mloc[h] = fmax_nc(mloc[h], z[h]);
                float *dst = zs + (size_t)(s0 + t) * G;
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
        // (both halves run unconditionally: a half past the end sees only
        // invalid lanes and zero rows, and the code stays free of a merge
        // point that would send the two register sets through memory)
        Tile ta, tb_;
        load(0, ta);
        for (int tb = 0; tb < nw; tb += 128) {
            load(tb + 64, tb_);
            compute(tb, ta);
            load(tb + 128, ta);
            compute(tb + 64, tb_);
        }
    }
    // ---------------- value prefetch ----------------------------------------
    // The first batch of value loads is issued here, so that it is in flight
    // during the reductions, the barrier and the weights pass.
    // lane -> (group slot gi of a load, dword slice qsl of the group)
    const int gi = lane / T::V_LPG;
    const int qsl = lane % T::V_LPG;
    constexpr uint32_t GSTEP = T::V_GPL * 4 * T::V_ROW;   // bytes per wave-wide group load
    constexpr int PFH = GSTEP * 8 <= 4096 ? 8 : 4096 / GSTEP;     // loads per descriptor (offsets < 4 KiB)
    constexpr int PF = 2 * PFH;                            // group loads in flight per lane
    const int ng = (nw + 3) >> 2;                          // groups of this wave with a valid position
    const uint8_t *vb0 = p.v_codes + ((size_t)bh * p.cap4 + t0 + s0) * T::V_ROW;
    const uint32_t vo = gi * 4 * T::V_ROW + qsl * T::V_DPL * 4;   // loop-invariant lane offset
    // descriptor half `hf` of the batch starting at group g0 (zero past the
    // wave's groups)
    auto vrsrc = [&](int g0, int hf) {
        const int b0 = g0 * 4 * T::V_ROW + hf * PFH * (int)GSTEP;
        return make_rsrc(vb0 + b0, (uint32_t)max(ng * 4 * T::V_ROW - b0, 0));
    };
    // rotating buffer: slot f is consumed, then reloaded one batch (PF loads)
    // ahead; the descriptors move with the batch
    uint32_t buf[PF][T::V_DPL];
    {
        const rsrc_t vra = vrsrc(0, 0), vrb = vrsrc(0, 1);
#pragma unroll
        for (int f = 0; f < PF; f++)
#pragma unroll
            for (int d = 0; d < T::V_DPL; d++) buf[f][d] = bld_u32(f < PFH ? vra : vrb, vo + (f % PFH) * GSTEP + d * 4);
    }

    // this wave's maxima of the scores (per head) and of the value scales
    // (per group), wave-uniform; each wave weights its own positions against
    // them and the waves are merged once, at the end
    float mw[G], vmw[KG];
#pragma unroll
    for (int h = 0; h < G; h++) mw[h] = wave_max_u(mloc[h]);
#pragma unroll
    for (int g = 0; g < KG; g++) vmw[g] = wave_max_u(vmloc[g]);

    // ---------------- pass 2: weights, one lane per 4 positions ---------------
    float lw[G], wsw[KG][G];                         // this wave's sum of p and of w_int
    // p = 2^(qs * (z - m)) <= 1; w_int = rint(p * s_v * 32767 / max s_v),
    // rounded by one fma onto 1.5 * 2^23 (the integer lands in the low
    // mantissa bits); bytes packed four positions per word.
    {
        constexpr float MAGIC = 12582912.0f;         // 1.5 * 2^23
        float nqm[G], lloc[G];
#pragma unroll
        for (int h = 0; h < G; h++) {
            nqm[h] = nw > 0 ? -mw[h] * qs[h] : 0.0f;
            lloc[h] = 0.0f;
        }
        int wsl[KG][G];
#pragma unroll
        for (int g = 0; g < KG; g++)
#pragma unroll
            for (int h = 0; h < G; h++) wsl[g][h] = 0;
        float fsc[KG];
#pragma unroll
        for (int g = 0; g < KG; g++) {
            const float vmax = vmw[g];
            fsc[g] = vmax > 0.0f ? (float)W_RANGE * __builtin_amdgcn_rcpf(vmax) : 0.0f;
        }
        const int ngw = (nw + 3) >> 2;               // groups of 4 positions
        for (int gb = 0; gb < ngw; gb += 64) {
            const int grp = gb + lane;
            if (grp < ngw) {
                const int tq = 4 * grp;              // first position of the group (within the wave)
                float pr[4][G];
#pragma unroll
                for (int k = 0; k < 4; k++) {
                    const bool valid = tq + k < nw;
                    const float *src = zs + (size_t)(s0 + tq + k) * G;
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
                    {
                        float sv[4];
#pragma unroll
                        for (int k = 0; k < 4; k++) sv[k] = tq + k < nw ? vs[(s0 + tq + k) * KG + g] * fsc[g] : 0.0f;
                        uint32_t *dst = wdw + ((size_t)g * (sub / 4) + grp) * G * 2;
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
#pragma unroll
        for (int h = 0; h < G; h++) lw[h] = wave_sum_u(lloc[h]);
#pragma unroll
        for (int g = 0; g < KG; g++)
#pragma unroll
            for (int h = 0; h < G; h++) wsw[g][h] = (float)wave_sum_ui(wsl[g][h]);
    }

    // ---------------- pass 3: values ---------------------------------------
    uint32_t accl[G][T::V_ACC], acch[G][T::V_ACC];
#pragma unroll
    for (int h = 0; h < G; h++)
#pragma unroll
        for (int c = 0; c < T::V_ACC; c++) accl[h][c] = acch[h][c] = 0u;
    {
        const int vgrp = (qsl * T::V_DPL * T::V_CPD) / (HD / KG);   // value scale group of the lane
        const uint32_t *wdg = wdw + (size_t)vgrp * (sub / 4) * G * 2;
        // one 4-position group: weight words of group rg (LDS broadcast) times
        // the value codes this lane holds for it
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
                    const uint32_t u = x[d] ^ 0x88888888u;        // offset binary per nibble
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
                    const uint32_t u = x[d] ^ 0x80808080u;        // offset binary per byte
#pragma unroll
                    for (int h = 0; h < G; h++) {
                        accl[h][d] = __builtin_amdgcn_udot4(wl[h], u, accl[h][d], false);
                        acch[h][d] = __builtin_amdgcn_udot4(wh[h], u, acch[h][d], false);
                    }
                }
            }
        };
        // Full batches are straight-line code (the weight reads of later
        // groups are issued early); the last, partial batch checks each group.
        constexpr int PB = PF * T::V_GPL;                  // groups per batch
        const int nfull = ng / PB * PB;
        int rb = 0;
        for (; rb < nfull; rb += PB) {
            const int nb = rb + PB;                        // first group of the next batch
            const rsrc_t vra = vrsrc(nb, 0), vrb = vrsrc(nb, 1);
#pragma unroll
            for (int f = 0; f < PF; f++) {
                group(rb + f * T::V_GPL + gi, buf[f]);
#pragma unroll
                for (int d = 0; d < T::V_DPL; d++)
                    buf[f][d] = bld_u32(f < PFH ? vra : vrb, vo + (f % PFH) * GSTEP + d * 4);
            }
        }
        if (rb < ng) {
#pragma unroll
            for (int f = 0; f < PF; f++) {
                const int rg = rb + f * T::V_GPL + gi;
                if (rg < ng) group(rg, buf[f]);
            }
        }
    }

    // ---------------- pass 4: per-wave values, merge the waves, write -------
    // This wave's output (relative to its own maxima): undo the byte split,
    // the x16 of odd V4 channels and the offset binary, then the fixed point.
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
    float *pm = misc;                                // [QD_WAVES][G] wave maxima
    float *pl = pm + QD_WAVES * G;                   // [QD_WAVES][G] wave sums of p
    if (gi == 0) {
        const float bias = VB == 4 ? 8.0f : 128.0f;
#pragma unroll
        for (int c = 0; c < T::V_ACC; c++) {
            const int ch = qsl * T::V_ACC + c;       // channel
            const int g = ch / (HD / KG);             // its scale group
#pragma unroll
            for (int h = 0; h < G; h++) {
                const float su = (VB == 4 && (c & 1)) ? af[h][c] * 0.0625f : af[h][c];
                red[(wave * G + h) * HD + ch] = (su - bias * wsw[g][h]) * (vmw[g] * (1.0f / (float)W_RANGE));
            }
        }
    }
    if (lane == 0) {
#pragma unroll
        for (int h = 0; h < G; h++) {
            pm[wave * G + h] = nw > 0 ? mw[h] * qs[h] : -INFINITY;   // log2 units
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
        acc0[h * acc_hs + c] = s;
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
        ml0[tid * ml_hs] = m;
        ml0[tid * ml_hs + 1] = l;
    }
}

} // namespace kvq
