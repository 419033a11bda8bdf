// kvq_decode.hpp -- split-K decode attention over the quantized cache, and
// the kernel that merges the per-chunk partial results.
//
// What is computed: for one (sequence, KV head) and the G query heads that
// read it, softmax attention of the current query over the cached rows,
// each row dequantized in registers as code * scale (TinyLoop "KV Cache 模式"
// five-modes table; KVSplit key/value widths).  Memory bandwidth bounds the
// work (mni-ml page, "why INT8 loses no speed"), so the kernel reads every
// cache byte exactly once, with the G query heads of a KV head sharing it.
//
// One workgroup = one context chunk of one (sequence, KV head):
//   A. stream the chunk's K rows; score z[h][t] for all G heads (log2 units)
//   B. per-head max over the chunk, p = 2^(z - max), l = sum p, and the value
//      weights w = p * value scale (fp16 pairs) in LDS
//   C. stream the chunk's V rows; acc[h][c] += w[h][t] * code[t][c]
//   D. reduce acc across lanes and waves; write (m, l, acc) for the chunk.
//
// Key side, quantized: the query is held as a 16-bit fixed-point integer per
// head (q ~ s_q * q_int, |q_int| <= 30000, s_q = max|q| / 30000), split into
// balanced digits (two base-256 digits for int8 keys, four base-16 digits for
// int4 keys) so that the integer dot-product units take the stored codes as
// they are (v_dot4_i32_i8 / v_dot8_i32_i4), with exact integer accumulation.
// The only rounding is q's own, |dq| <= s_q / 2.
// Value side, quantized: codes of two consecutive positions are turned into
// fp16 pairs with exact integer arithmetic and accumulated with
// v_dot2_f32_f16 against fp16 weight pairs (relative rounding of each
// weight <= 2^-11); accumulation is fp32.
// Float sides (fp16 / fp32 rows) use fp32 FMAs throughout.
#pragma once

#include <type_traits>

#include "kvq_device.hpp"

namespace kvq {

constexpr int DEC_THREADS = 256;
constexpr int DEC_WAVES = DEC_THREADS / 64;
constexpr int QRANGE = 30000;

struct DecodeParams {
    const uint8_t *k_codes;
    const uint8_t *v_codes;
    const uint16_t *k_scales;
    const uint16_t *v_scales;
    const float *q;            // [batch][n_q_heads][head_dim]
    const int32_t *seq_len;    // [batch]
    float *ws_ml;              // [batch*n_q_heads][n_chunks][2]
    float *ws_acc;             // [batch*n_q_heads][n_chunks][head_dim]
    int n_kv_heads, capacity;
    int max_len;               // min(max_seq_len, capacity)
    int chunk, n_chunks;
    int kg, vg;                // scale groups per head row (1 for per-position scales)
    int k_group, v_group;      // values per scale (a large value for per-position)
    long long k_sc_b, k_sc_h;  // scale index = b*sc_b + h*sc_h + t*sc_t + group
    int k_sc_t;
    long long v_sc_b, v_sc_h;
    int v_sc_t;
    float qk_scale;            // softmax_scale * log2(e)
};

// LDS layout (byte offsets), shared by the host (launch size) and the kernel.
struct DecodeSmem {
    int zs, ks, vs, wv, red, misc, total;
};

__host__ __device__ inline DecodeSmem decode_smem(int G, int HD, int KB, int VB, int chunk, int kg, int vg)
{
    DecodeSmem s;
    int off = 0;
    s.zs = off;
    off += G * chunk * 4;                       // scores, then p
    s.ks = off;
    if (KB < 16) off += chunk * kg * 4;          // key scales (float)
    s.vs = off;
    if (VB < 16) off += chunk * vg * 4;          // value scales (float)
    s.wv = off;
    if (VB < 16) off += vg * (chunk / 2) * G * 4; // fp16 weight pairs
    const int red_bytes = DEC_WAVES * G * HD * 4;
    if (VB < 16 && G * chunk * 4 >= red_bytes) {
        s.red = s.zs;                            // scores are dead in step C
    } else {
        s.red = off;
        off += red_bytes;
    }
    s.misc = off;
    off += (2 * G + 2 * DEC_WAVES * G + G) * 4;  // m, l, wave partials, q amax
    s.total = off;
    return s;
}

// ------------------------------------------------------------------------
// Key side.  One lane holds 16 bytes of a row (a "slice"); LPT lanes cover a
// row.  dot() returns, per head, the slice's share of sum_c q[c] * K[t][c]
// in units of the group scale (quantized) or exactly (float).
// ------------------------------------------------------------------------
template <int KB, int HD, int G> struct KSide;

// balanced base-2^bits digits of q_int, lowest first
__device__ __forceinline__ int digit_lo(int v, int bits)
{
    const int half = 1 << (bits - 1), mask = (1 << bits) - 1;
    return ((v + half) & mask) - half;
}

template <int HD, int G> struct KSide<4, HD, G> {
    static constexpr int LPT = HD / 32;   // 32 int4 codes per 16-byte slice
    static constexpr int CPL = 32;
    static constexpr bool QUANT = true;
    int qd[G][4][4];                      // [head][digit][dword]: 8 nibbles each

    __device__ void init(const float *qh, const float *qscale, int sl)
    {
#pragma unroll
        for (int h = 0; h < G; h++) {
            const float inv = qscale[h] > 0.0f ? 1.0f / qscale[h] : 0.0f;
#pragma unroll
            for (int w = 0; w < 4; w++) {
                uint32_t d[4] = {0, 0, 0, 0};
#pragma unroll
                for (int i = 0; i < 8; i++) {
                    const float qv = qh[h * HD + sl * CPL + w * 8 + i];
                    int qi = (int)fminf(fmaxf(rintf(qv * inv), -(float)QRANGE), (float)QRANGE);
#pragma unroll
                    for (int j = 0; j < 4; j++) {
                        const int dj = j < 3 ? digit_lo(qi, 4) : qi;
                        d[j] |= (uint32_t)(dj & 0xF) << (4 * i);
                        qi = (qi - dj) >> 4;
                    }
                }
#pragma unroll
                for (int j = 0; j < 4; j++) qd[h][j][w] = (int)d[j];
            }
        }
    }

    __device__ __forceinline__ void dot(const uint4 &r, float (&out)[G]) const
    {
        const int k[4] = {(int)r.x, (int)r.y, (int)r.z, (int)r.w};
#pragma unroll
        for (int h = 0; h < G; h++) {
            int a[4];
#pragma unroll
            for (int j = 0; j < 4; j++) {
                int s = 0;
#pragma unroll
                for (int w = 0; w < 4; w++) s = __builtin_amdgcn_sdot8(qd[h][j][w], k[w], s, false);
                a[j] = s;
            }
            out[h] = (float)(a[0] + a[1] * 16 + a[2] * 256 + a[3] * 4096);
        }
    }
};

template <int HD, int G> struct KSide<8, HD, G> {
    static constexpr int LPT = HD / 16;   // 16 int8 codes per slice
    static constexpr int CPL = 16;
    static constexpr bool QUANT = true;
    int qd[G][2][4];                      // [head][lo, hi][dword]: 4 bytes each

    __device__ void init(const float *qh, const float *qscale, int sl)
    {
#pragma unroll
        for (int h = 0; h < G; h++) {
            const float inv = qscale[h] > 0.0f ? 1.0f / qscale[h] : 0.0f;
#pragma unroll
            for (int w = 0; w < 4; w++) {
                uint32_t lo = 0, hi = 0;
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const float qv = qh[h * HD + sl * CPL + w * 4 + i];
                    const int qi = (int)fminf(fmaxf(rintf(qv * inv), -(float)QRANGE), (float)QRANGE);
                    const int d0 = digit_lo(qi, 8);
                    const int d1 = (qi - d0) >> 8;
                    lo |= (uint32_t)(d0 & 0xFF) << (8 * i);
                    hi |= (uint32_t)(d1 & 0xFF) << (8 * i);
                }
                qd[h][0][w] = (int)lo;
                qd[h][1][w] = (int)hi;
            }
        }
    }

    __device__ __forceinline__ void dot(const uint4 &r, float (&out)[G]) const
    {
        const int k[4] = {(int)r.x, (int)r.y, (int)r.z, (int)r.w};
#pragma unroll
        for (int h = 0; h < G; h++) {
            int lo = 0, hi = 0;
#pragma unroll
            for (int w = 0; w < 4; w++) {
                lo = __builtin_amdgcn_sdot4(qd[h][0][w], k[w], lo, false);
                hi = __builtin_amdgcn_sdot4(qd[h][1][w], k[w], hi, false);
            }
            out[h] = (float)(lo + hi * 256);
        }
    }
};

template <int HD, int G> struct KSide<16, HD, G> {
    static constexpr int LPT = HD / 8;    // 8 fp16 values per slice
    static constexpr int CPL = 8;
    static constexpr bool QUANT = false;
    float qf[G][8];

    __device__ void init(const float *qh, const float *, int sl)
    {
#pragma unroll
        for (int h = 0; h < G; h++)
#pragma unroll
            for (int i = 0; i < 8; i++) qf[h][i] = qh[h * HD + sl * CPL + i];
    }

    __device__ __forceinline__ void dot(const uint4 &r, float (&out)[G]) const
    {
        const uint32_t u[4] = {r.x, r.y, r.z, r.w};
        float k[8];
#pragma unroll
        for (int w = 0; w < 4; w++) {
            const half2_t hv = as_h2(u[w]);
            k[2 * w] = (float)hv.x;
            k[2 * w + 1] = (float)hv.y;
        }
#pragma unroll
        for (int h = 0; h < G; h++) {
            float s = 0.0f;
#pragma unroll
            for (int i = 0; i < 8; i++) s = fmaf(qf[h][i], k[i], s);
            out[h] = s;
        }
    }
};

template <int HD, int G> struct KSide<32, HD, G> {
    static constexpr int LPT = HD / 4;    // 4 fp32 values per slice
    static constexpr int CPL = 4;
    static constexpr bool QUANT = false;
    float qf[G][4];

    __device__ void init(const float *qh, const float *, int sl)
    {
#pragma unroll
        for (int h = 0; h < G; h++)
#pragma unroll
            for (int i = 0; i < 4; i++) qf[h][i] = qh[h * HD + sl * CPL + i];
    }

    __device__ __forceinline__ void dot(const uint4 &r, float (&out)[G]) const
    {
        const float k[4] = {__uint_as_float(r.x), __uint_as_float(r.y), __uint_as_float(r.z), __uint_as_float(r.w)};
#pragma unroll
        for (int h = 0; h < G; h++) {
            float s = 0.0f;
#pragma unroll
            for (int i = 0; i < 4; i++) s = fmaf(qf[h][i], k[i], s);
            out[h] = s;
        }
    }
};

// ------------------------------------------------------------------------
// Value side, quantized: one lane holds 8 bytes of two consecutive rows.
// accum() adds w[h] . (code[t][c], code[t+1][c]) into acc[h][c].
// ------------------------------------------------------------------------
template <int VB, int HD, int G> struct VSideQ;

template <int HD, int G> struct VSideQ<4, HD, G> {
    static constexpr int LPT = HD / 16;   // 16 int4 codes per 8-byte slice
    static constexpr int CPL = 16;

    __device__ __forceinline__ static void accum(float (&acc)[G][CPL], uint2 ra, uint2 rb, const half2_t (&w)[G])
    {
        const uint32_t xa[2] = {ra.x ^ 0x88888888u, ra.y ^ 0x88888888u};   // offset binary u = code + 8
        const uint32_t xb[2] = {rb.x ^ 0x88888888u, rb.y ^ 0x88888888u};
        const half2_t lo_bias = {(_Float16)-1032.0f, (_Float16)-1032.0f};
        const half2_t hi_mul = {(_Float16)0.0625f, (_Float16)0.0625f};
        const half2_t hi_bias = {(_Float16)-72.0f, (_Float16)-72.0f};
#pragma unroll
        for (int d = 0; d < 2; d++) {
#pragma unroll
            for (int i = 0; i < 4; i++) {
                // bytes [a.byte_i, 0, b.byte_i, 0]
                const uint32_t sel = 0x0c000c00u | ((uint32_t)(4 + i) << 16) | (uint32_t)i;
                const uint32_t rr = __builtin_amdgcn_perm(xb[d], xa[d], sel);
                // low nibbles -> fp16 1024 + u; high nibbles -> fp16 1024 + 16 u
                const half2_t flo = as_h2((rr & 0x000F000Fu) | 0x64006400u);
                const half2_t fhi = as_h2((rr & 0x00F000F0u) | 0x64006400u);
                const half2_t clo = flo + lo_bias;                 // exact: u - 8
                const half2_t chi = fhi * hi_mul + hi_bias;        // exact: u - 8
                const int c = d * 8 + 2 * i;
#pragma unroll
                for (int h = 0; h < G; h++) {
                    acc[h][c] = __builtin_amdgcn_fdot2(clo, w[h], acc[h][c], false);
                    acc[h][c + 1] = __builtin_amdgcn_fdot2(chi, w[h], acc[h][c + 1], false);
                }
            }
        }
    }
};

template <int HD, int G> struct VSideQ<8, HD, G> {
    static constexpr int LPT = HD / 8;    // 8 int8 codes per 8-byte slice
    static constexpr int CPL = 8;

    __device__ __forceinline__ static void accum(float (&acc)[G][CPL], uint2 ra, uint2 rb, const half2_t (&w)[G])
    {
        const uint32_t xa[2] = {ra.x ^ 0x80808080u, ra.y ^ 0x80808080u};   // u = code + 128
        const uint32_t xb[2] = {rb.x ^ 0x80808080u, rb.y ^ 0x80808080u};
        const half2_t bias = {(_Float16)-1152.0f, (_Float16)-1152.0f};
#pragma unroll
        for (int d = 0; d < 2; d++) {
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const uint32_t sel = 0x0c000c00u | ((uint32_t)(4 + i) << 16) | (uint32_t)i;
                const uint32_t rr = __builtin_amdgcn_perm(xb[d], xa[d], sel);
                const half2_t f = as_h2(rr | 0x64006400u);         // 1024 + u
                const half2_t cv = f + bias;                       // exact: u - 128
                const int c = d * 4 + i;
#pragma unroll
                for (int h = 0; h < G; h++) acc[h][c] = __builtin_amdgcn_fdot2(cv, w[h], acc[h][c], false);
            }
        }
    }
};

// Value side, float rows: one lane holds 16 bytes of one row.
template <int VB, int HD, int G> struct VSideF;

template <int HD, int G> struct VSideF<16, HD, G> {
    static constexpr int LPT = HD / 8;
    static constexpr int CPL = 8;
    __device__ __forceinline__ static void accum(float (&acc)[G][CPL], uint4 r, const float (&w)[G])
    {
        const uint32_t u[4] = {r.x, r.y, r.z, r.w};
        float v[8];
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const half2_t hv = as_h2(u[j]);
            v[2 * j] = (float)hv.x;
            v[2 * j + 1] = (float)hv.y;
        }
#pragma unroll
        for (int h = 0; h < G; h++)
#pragma unroll
            for (int c = 0; c < 8; c++) acc[h][c] = fmaf(w[h], v[c], acc[h][c]);
    }
};

template <int HD, int G> struct VSideF<32, HD, G> {
    static constexpr int LPT = HD / 4;
    static constexpr int CPL = 4;
    __device__ __forceinline__ static void accum(float (&acc)[G][CPL], uint4 r, const float (&w)[G])
    {
        const float v[4] = {__uint_as_float(r.x), __uint_as_float(r.y), __uint_as_float(r.z), __uint_as_float(r.w)};
#pragma unroll
        for (int h = 0; h < G; h++)
#pragma unroll
            for (int c = 0; c < 4; c++) acc[h][c] = fmaf(w[h], v[c], acc[h][c]);
    }
};

template <int VB, int HD, int G>
using VSide = typename std::conditional<(VB < 16), VSideQ<VB, HD, G>, VSideF<VB, HD, G>>::type;

// Sum acc over the lanes of a wave that hold the same slice (lane % LPT),
// then over the waves through LDS; write the chunk's partial accumulator.
template <int G, int CPL, int LPT, int HD>
__device__ __forceinline__ void reduce_and_store(float (&acc)[G][CPL], float *red, float *dst_acc0, size_t head_stride)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
#pragma unroll
    for (int m = LPT; m < 64; m <<= 1)
#pragma unroll
        for (int h = 0; h < G; h++)
#pragma unroll
            for (int c = 0; c < CPL; c++) acc[h][c] += shfl_xor(acc[h][c], m);
    if (lane < LPT) {
#pragma unroll
        for (int h = 0; h < G; h++)
#pragma unroll
            for (int c = 0; c < CPL; c++) red[(wave * G + h) * HD + lane * CPL + c] = acc[h][c];
    }
    __syncthreads();
    for (int i = tid; i < G * HD; i += DEC_THREADS) {
        const int h = i / HD, c = i - h * HD;
        float s = 0.0f;
#pragma unroll
        for (int w = 0; w < DEC_WAVES; w++) s += red[(w * G + h) * HD + c];
        dst_acc0[h * head_stride + c] = s;
    }
}

template <int KB, int VB, int HD, int G, int UA, int UC>
__global__ __launch_bounds__(DEC_THREADS) void decode_split_kernel(DecodeParams p)
{
    extern __shared__ __align__(16) unsigned char smem[];
    using KS = KSide<KB, HD, G>;
    constexpr int K_ROW = HD * KB / 8;
    constexpr int V_ROW = HD * VB / 8;
    constexpr int VCPL = VSide<VB, HD, G>::CPL;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int chunk_id = blockIdx.x;
    const int bh = blockIdx.y;
    const int b = bh / p.n_kv_heads;
    const int kvh = bh - b * p.n_kv_heads;
    const int Hq = p.n_kv_heads * G;
    const int hq0 = kvh * G;
    const int CH = p.chunk;

    int L = p.seq_len[b];
    L = L < 0 ? 0 : (L > p.max_len ? p.max_len : L);
    const int t0 = chunk_id * CH;
    const int n_tok = min(L - t0, CH);

    // partial-result addresses of query head hq0 + h: row (b*Hq + hq0 + h)
    const size_t row0 = (size_t)b * Hq + hq0;
    float *ml0 = p.ws_ml + (row0 * p.n_chunks + chunk_id) * 2;
    float *acc0 = p.ws_acc + (row0 * p.n_chunks + chunk_id) * HD;
    const size_t ml_hstride = (size_t)p.n_chunks * 2;
    const size_t acc_hstride = (size_t)p.n_chunks * HD;

    if (n_tok <= 0) {                       // chunk past the sequence: empty partial
        for (int i = tid; i < G * HD; i += DEC_THREADS)
            acc0[(i / HD) * acc_hstride + (i % HD)] = 0.0f;
        if (tid < G) {
            ml0[tid * ml_hstride] = -INFINITY;
            ml0[tid * ml_hstride + 1] = 0.0f;
        }
        return;
    }

    const DecodeSmem lay = decode_smem(G, HD, KB, VB, CH, p.kg, p.vg);
    float *zs = reinterpret_cast<float *>(smem + lay.zs);
    float *ks = reinterpret_cast<float *>(smem + lay.ks);
    float *vs = reinterpret_cast<float *>(smem + lay.vs);
    uint32_t *wv = reinterpret_cast<uint32_t *>(smem + lay.wv);
    float *red = reinterpret_cast<float *>(smem + lay.red);
    float *m_sh = reinterpret_cast<float *>(smem + lay.misc);
    float *l_sh = m_sh + G;
    float *part = l_sh + G;                 // [DEC_WAVES][G] x 2
    float *qamax = part + 2 * DEC_WAVES * G;

    const float *qh = p.q + row0 * HD;      // the G query heads of this KV head

    // ---- 0. scales of the chunk into LDS; query scale per head ----------
    if (KB < 16) {
        const uint16_t *src = p.k_scales + b * p.k_sc_b + kvh * p.k_sc_h;
        for (int i = tid; i < n_tok * p.kg; i += DEC_THREADS) {
            const int t = i / p.kg, g = i - t * p.kg;
            ks[i] = f16_bits_to_f32(src[(size_t)(t0 + t) * p.k_sc_t + g]);
        }
    }
    if (VB < 16) {
        const uint16_t *src = p.v_scales + b * p.v_sc_b + kvh * p.v_sc_h;
        for (int i = tid; i < n_tok * p.vg; i += DEC_THREADS) {
            const int t = i / p.vg, g = i - t * p.vg;
            vs[i] = f16_bits_to_f32(src[(size_t)(t0 + t) * p.v_sc_t + g]);
        }
    }
    float qsc[G];                           // per-head factor turning a key dot into z (log2 units)
    if (KS::QUANT) {
        for (int h = wave; h < G; h += DEC_WAVES) {
            float a = 0.0f;
            for (int c = lane; c < HD; c += 64) a = fmaxf(a, fabsf(qh[h * HD + c]));
            a = wave_max(a);
            if (lane == 0) qamax[h] = a / (float)QRANGE;
        }
        __syncthreads();
#pragma unroll
        for (int h = 0; h < G; h++) qsc[h] = qamax[h];
    } else {
        __syncthreads();
#pragma unroll
        for (int h = 0; h < G; h++) qsc[h] = 1.0f;
    }

    // ---- A. scores ------------------------------------------------------
    {
        constexpr int LPT = KS::LPT;
        constexpr int TPP = DEC_THREADS / LPT;
        const int sl = tid % LPT, tr = tid / LPT;
        KS kside;
        kside.init(qh, qsc, sl);
        float zmul[G];
#pragma unroll
        for (int h = 0; h < G; h++) zmul[h] = qsc[h] * p.qk_scale;
        const int kgrp = KS::QUANT ? (sl * KS::CPL) / p.k_group : 0;
        const uint8_t *kbase = p.k_codes + ((size_t)bh * p.capacity + t0) * K_ROW + sl * 16;
        for (int base = 0; base < n_tok; base += TPP * UA) {
            uint4 raw[UA];
#pragma unroll
            for (int u = 0; u < UA; u++) {
                const int t = base + u * TPP + tr;
                raw[u] = t < n_tok ? ld_u4(kbase + (size_t)t * K_ROW) : make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int u = 0; u < UA; u++) {
                const int t = base + u * TPP + tr;
                float d[G];
                kside.dot(raw[u], d);
                if (KS::QUANT) {
                    const float s = t < n_tok ? ks[t * p.kg + kgrp] : 0.0f;
#pragma unroll
                    for (int h = 0; h < G; h++) d[h] *= s;
                }
#pragma unroll
                for (int m = 1; m < LPT; m <<= 1)
#pragma unroll
                    for (int h = 0; h < G; h++) d[h] += shfl_xor(d[h], m);
                if (t < n_tok) {
#pragma unroll
                    for (int h = 0; h < G; h++)
                        if (h % LPT == sl) zs[h * CH + t] = d[h] * zmul[h];
                }
            }
        }
    }
    __syncthreads();

    // ---- B. softmax statistics and value weights -------------------------
    {
        float mloc[G];
#pragma unroll
        for (int h = 0; h < G; h++) mloc[h] = -INFINITY;
        for (int t = tid; t < n_tok; t += DEC_THREADS)
#pragma unroll
            for (int h = 0; h < G; h++) mloc[h] = fmaxf(mloc[h], zs[h * CH + t]);
#pragma unroll
        for (int h = 0; h < G; h++) {
            const float v = wave_max(mloc[h]);
            if (lane == 0) part[wave * G + h] = v;
        }
        __syncthreads();
        if (tid < G) {
            float v = part[tid];
#pragma unroll
            for (int w = 1; w < DEC_WAVES; w++) v = fmaxf(v, part[w * G + tid]);
            m_sh[tid] = v;
        }
        __syncthreads();
        float mh[G], lloc[G];
#pragma unroll
        for (int h = 0; h < G; h++) {
            mh[h] = m_sh[h];
            lloc[h] = 0.0f;
        }
        for (int t = tid; t < n_tok; t += DEC_THREADS)
#pragma unroll
            for (int h = 0; h < G; h++) {
                const float e = exp2f(zs[h * CH + t] - mh[h]);
                zs[h * CH + t] = e;
                lloc[h] += e;
            }
#pragma unroll
        for (int h = 0; h < G; h++) {
            const float v = wave_sum(lloc[h]);
            if (lane == 0) part[DEC_WAVES * G + wave * G + h] = v;
        }
        __syncthreads();
        if (tid < G) {
            float v = 0.0f;
#pragma unroll
            for (int w = 0; w < DEC_WAVES; w++) v += part[DEC_WAVES * G + w * G + tid];
            l_sh[tid] = v;
        }
        if (VB < 16) {
            const int npairs = (n_tok + 1) >> 1;
            const int half_ch = CH >> 1;
            for (int i = tid; i < p.vg * npairs * G; i += DEC_THREADS) {
                const int h = i % G;
                const int pi = (i / G) % npairs;
                const int g = i / (G * npairs);
                const int t = 2 * pi;
                const float w0 = zs[h * CH + t] * vs[t * p.vg + g];
                const float w1 = (t + 1 < n_tok) ? zs[h * CH + t + 1] * vs[(t + 1) * p.vg + g] : 0.0f;
                wv[(g * half_ch + pi) * G + h] = (uint32_t)f32_to_f16_bits(w0) | ((uint32_t)f32_to_f16_bits(w1) << 16);
            }
        }
        __syncthreads();
    }

    // ---- C. values --------------------------------------------------------
    float acc[G][VCPL];
#pragma unroll
    for (int h = 0; h < G; h++)
#pragma unroll
        for (int c = 0; c < VCPL; c++) acc[h][c] = 0.0f;

    if constexpr (VB < 16) {
        using VS = VSideQ<VB, HD, G>;
        constexpr int LPT = VS::LPT;
        constexpr int PPP = DEC_THREADS / LPT;              // position pairs per pass
        const int sl = tid % LPT, tr = tid / LPT;
        const int vgrp = (sl * VS::CPL) / p.v_group;
        const int npairs = (n_tok + 1) >> 1;
        const uint32_t *wrow = wv + (size_t)vgrp * (CH >> 1) * G;
        const uint8_t *vbase = p.v_codes + ((size_t)bh * p.capacity + t0) * V_ROW + sl * 8;
        for (int base = 0; base < npairs; base += PPP * UC) {
            uint2 ra[UC], rb[UC];
#pragma unroll
            for (int u = 0; u < UC; u++) {
                const int t = 2 * (base + u * PPP + tr);
                ra[u] = t < n_tok ? ld_u2(vbase + (size_t)t * V_ROW) : make_uint2(0, 0);
                rb[u] = t + 1 < n_tok ? ld_u2(vbase + (size_t)(t + 1) * V_ROW) : make_uint2(0, 0);
            }
#pragma unroll
            for (int u = 0; u < UC; u++) {
                const int pi = base + u * PPP + tr;
                half2_t w[G];
#pragma unroll
                for (int h = 0; h < G; h++) w[h] = as_h2(pi < npairs ? wrow[pi * G + h] : 0u);
                VS::accum(acc, ra[u], rb[u], w);
            }
        }
        reduce_and_store<G, VCPL, LPT, HD>(acc, red, acc0, acc_hstride);
    } else {
        using VS = VSideF<VB, HD, G>;
        constexpr int LPT = VS::LPT;
        constexpr int TPP = DEC_THREADS / LPT;
        const int sl = tid % LPT, tr = tid / LPT;
        const uint8_t *vbase = p.v_codes + ((size_t)bh * p.capacity + t0) * V_ROW + sl * 16;
        for (int base = 0; base < n_tok; base += TPP * UC) {
            uint4 raw[UC];
#pragma unroll
            for (int u = 0; u < UC; u++) {
                const int t = base + u * TPP + tr;
                raw[u] = t < n_tok ? ld_u4(vbase + (size_t)t * V_ROW) : make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int u = 0; u < UC; u++) {
                const int t = base + u * TPP + tr;
                float w[G];
#pragma unroll
                for (int h = 0; h < G; h++) w[h] = t < n_tok ? zs[h * CH + t] : 0.0f;
                VS::accum(acc, raw[u], w);
            }
        }
        __syncthreads();   // zs may alias nothing here, but keep step D ordered
        reduce_and_store<G, VCPL, LPT, HD>(acc, red, acc0, acc_hstride);
    }
    if (tid < G) {
        ml0[tid * ml_hstride] = m_sh[tid];
        ml0[tid * ml_hstride + 1] = l_sh[tid];
    }
}

// ------------------------------------------------------------------------
// Merge: for each (sequence, query head) row, M = max m_i,
// out = sum acc_i 2^(m_i - M) / sum l_i 2^(m_i - M); 0 if every chunk is empty.
// grid: rows; block: head_dim threads.
// ------------------------------------------------------------------------
__global__ __launch_bounds__(256) void combine_kernel(const float *__restrict__ ml, const float *__restrict__ acc,
                                                      float *__restrict__ out, int n_chunks, int head_dim)
{
    const size_t row = blockIdx.x;
    const int c = threadIdx.x;
    const float *mr = ml + row * (size_t)n_chunks * 2;
    float M = -INFINITY;
    for (int i = 0; i < n_chunks; i++) M = fmaxf(M, mr[2 * i]);
    float Ls = 0.0f, o = 0.0f;
    if (M != -INFINITY) {
        for (int i = 0; i < n_chunks; i++) {
            const float m = mr[2 * i];
            if (m == -INFINITY) continue;
            const float e = exp2f(m - M);
            Ls = fmaf(mr[2 * i + 1], e, Ls);
            o = fmaf(acc[(row * n_chunks + i) * head_dim + c], e, o);
        }
    }
    out[row * head_dim + c] = Ls > 0.0f ? o / Ls : 0.0f;
}

} // namespace kvq
