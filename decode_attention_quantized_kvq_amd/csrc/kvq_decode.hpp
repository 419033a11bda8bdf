// kvq_decode.hpp -- split-K decode attention over float rows (fp16 or fp32
// cache), the kernel that merges per-chunk partial results, and the
// parameters shared by the decode kernels.
//
// What is computed: for one (sequence, KV head) and the G query heads that
// read it, softmax attention of the current query over the cached rows of a
// context chunk (TinyLoop "KV Cache 模式": FP16 KV is the reference mode;
// mni-ml page: the FP32 cache it compares INT8 against).  Memory bandwidth
// bounds the work, so every cache byte is read once and shared by the G
// query heads.
//
// One workgroup = one context chunk of one (sequence, KV head):
//   A. stream the chunk's K rows; score z[h][t] for all G heads (log2 units)
//   B. per-head max over the chunk, p = 2^(z - max), l = sum p
//   C. stream the chunk's V rows; acc[h][c] += p[h][t] * V[t][c]
//   D. reduce acc across lanes and waves; write (m, l, acc) for the chunk.
// All arithmetic is fp32 (fp16 rows are widened exactly).
#pragma once

#include <type_traits>

#include "kvq_combine.hpp"

#include "kvq_device.hpp"

namespace kvq {

constexpr int DEC_THREADS = 256;
constexpr int DEC_WAVES = DEC_THREADS / 64;

struct FloatParams {
    const uint8_t *k_codes;    // [batch][n_kv_heads][capacity][head_dim * bytes]
    const uint8_t *v_codes;
    const float *q;            // [batch][n_q_heads][head_dim]
    const int32_t *seq_len;    // [batch]
    float *ws_ml;              // [batch*n_q_heads][n_chunks][2]
    float *ws_acc;             // [batch*n_q_heads][n_chunks][head_dim]
    int n_kv_heads, capacity;  // capacity: slots per storage unit (a sequence, or a page)
    int max_len;               // min(max_seq_len, logical capacity)
    int chunk, n_chunks;
    float qk_scale;            // softmax_scale * log2(e)
    // paged storage: slot s of sequence b in page block_table[b * pages_per_seq
    // + (s >> page_shift)] (paged kernels only)
    const int32_t *block_table;
    int page_shift, pages_per_seq, n_pages;
};

// LDS layout (byte offsets), shared by the host (launch size) and the kernel.
struct FloatSmem {
    int zs, red, misc, total;
};

__host__ __device__ inline FloatSmem float_smem(int G, int HD, int chunk)
{
    FloatSmem s;
    int off = 0;
    s.zs = off;
    off += G * chunk * 4;                        // scores, then p
    s.red = off;
    off += DEC_WAVES * G * HD * 4;               // cross-wave reduction of acc
    s.misc = off;
    off += (2 * G + 2 * DEC_WAVES * G) * 4;      // m, l, wave partials
    s.total = off;
    return s;
}

// ------------------------------------------------------------------------
// Key side.  One lane holds 16 bytes of a row (a "slice"); LPT lanes cover a
// row.  dot() returns, per head, the slice's share of sum_c q[c] * K[t][c].
// ------------------------------------------------------------------------
template <int KB, int HD, int G> struct KSide;

template <int HD, int G> struct KSide<16, HD, G> {
    static constexpr int LPT = HD / 8;    // 8 fp16 values per slice
    static constexpr int CPL = 8;
    float qf[G][8];

    __device__ void init(const float *qh, int sl)
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
    float qf[G][4];

    __device__ void init(const float *qh, int sl)
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

template <int KB, int VB, int HD, int G, int UA, int UC, bool PAGED>
__global__ __launch_bounds__(DEC_THREADS) void decode_float_kernel(FloatParams p)
{
    extern __shared__ __align__(16) unsigned char smem[];
    using KS = KSide<KB, HD, G>;
    using VS = VSideF<VB, HD, G>;
    constexpr int K_ROW = HD * KB / 8;
    constexpr int V_ROW = HD * VB / 8;

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

    const FloatSmem lay = float_smem(G, HD, CH);
    float *zs = reinterpret_cast<float *>(smem + lay.zs);
    // paged storage: the pages of the chunk's slots (-1: none, read as zero),
    // entry i in lane i % 64 of pgv[i / 64] of every wave.  A chunk (at most
    // 8192 slots, a multiple of 64 from a multiple of 64) touches at most 128
    // pages of at least 64 slots.
    const int pg0 = PAGED ? (t0 >> p.page_shift) : 0;
    int pgv[2] = {-1, -1};
    if constexpr (PAGED) {
        const int npg = ((t0 + n_tok - 1) >> p.page_shift) - pg0 + 1;
        const int lane = tid & 63;
#pragma unroll
        for (int k = 0; k < 2; k++) {
            const int i = k * 64 + lane;
            if (i < npg) {
                const int e = p.block_table[(size_t)b * p.pages_per_seq + pg0 + i];
                pgv[k] = (e >= 0 && e < p.n_pages) ? e : -1;
            }
        }
    }
    // block-uniform address of row t0 + t1 of this KV head, t1 a multiple of
    // 64 or the first row of a load batch inside one 64-row block (nullptr:
    // no page).  A page holds whole 64-row blocks, so the rows of the block
    // from t1 on follow at row_bytes each; the lookup is a readlane.
    auto block_ptr = [&](const uint8_t *base, int t1, int row_bytes) -> const uint8_t * {
        if constexpr (PAGED) {
            const int pos = t0 + t1;
            const int i = (pos >> p.page_shift) - pg0;
            const int lo = __builtin_amdgcn_readlane(pgv[0], i & 63), hi = __builtin_amdgcn_readlane(pgv[1], i & 63);
            const int u = i < 64 ? lo : hi;
            if (u < 0) return nullptr;
            return base + (((size_t)u * p.n_kv_heads + kvh) * p.capacity + (pos & ((1 << p.page_shift) - 1))) *
                              (size_t)row_bytes;
        } else {
            return base + ((size_t)bh * p.capacity + t0 + t1) * (size_t)row_bytes;
        }
    };
    float *red = reinterpret_cast<float *>(smem + lay.red);
    float *m_sh = reinterpret_cast<float *>(smem + lay.misc);
    float *l_sh = m_sh + G;
    float *part = l_sh + G;                 // [DEC_WAVES][G] x 2

    const float *qh = p.q + row0 * HD;      // the G query heads of this KV head

    // ---- A. scores ------------------------------------------------------
    {
        constexpr int LPT = KS::LPT;
        constexpr int TPP = DEC_THREADS / LPT;
        constexpr int S64 = 64 / TPP;           // load steps per 64-row block
        static_assert(TPP <= 64 && 64 % TPP == 0, "a load step lies in one 64-row block");
        const int sl = tid % LPT, tr = tid / LPT;
        KS kside;
        kside.init(qh, sl);
        for (int base = 0; base < n_tok; base += TPP * UA) {
            uint4 raw[UA];
            // one address per 64 rows (S64 steps of TPP rows), then 32-bit offsets
            const uint8_t *blk = nullptr;
#pragma unroll
            for (int u = 0; u < UA; u++) {
                const int t = base + u * TPP + tr;
                if (u % S64 == 0) blk = block_ptr(p.k_codes, base + u * TPP, K_ROW);
                const uint32_t off = (uint32_t)(((u % S64) * TPP + tr) * K_ROW + sl * 16);
                raw[u] = blk && t < n_tok ? ld_u4_nt(blk + off) : make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int u = 0; u < UA; u++) {
                const int t = base + u * TPP + tr;
                float d[G];
                kside.dot(raw[u], d);
#pragma unroll
                for (int m = 1; m < LPT; m <<= 1)
#pragma unroll
                    for (int h = 0; h < G; h++) d[h] += shfl_xor(d[h], m);
                if (t < n_tok) {
#pragma unroll
                    for (int h = 0; h < G; h++)
                        if (h % LPT == sl) zs[h * CH + t] = d[h] * p.qk_scale;
                }
            }
        }
    }
    __syncthreads();

    // ---- B. softmax statistics -------------------------------------------
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
    }

    // ---- C. values --------------------------------------------------------
    float acc[G][VS::CPL];
#pragma unroll
    for (int h = 0; h < G; h++)
#pragma unroll
        for (int c = 0; c < VS::CPL; c++) acc[h][c] = 0.0f;
    {
        constexpr int LPT = VS::LPT;
        constexpr int TPP = DEC_THREADS / LPT;
        constexpr int S64 = 64 / TPP;           // load steps per 64-row block
        static_assert(TPP <= 64 && 64 % TPP == 0, "a load step lies in one 64-row block");
        const int sl = tid % LPT, tr = tid / LPT;
        for (int base = 0; base < n_tok; base += TPP * UC) {
            uint4 raw[UC];
            // one address per 64 rows (S64 steps of TPP rows), then 32-bit offsets
            const uint8_t *blk = nullptr;
#pragma unroll
            for (int u = 0; u < UC; u++) {
                const int t = base + u * TPP + tr;
                if (u % S64 == 0) blk = block_ptr(p.v_codes, base + u * TPP, V_ROW);
                const uint32_t off = (uint32_t)(((u % S64) * TPP + tr) * V_ROW + sl * 16);
                raw[u] = blk && t < n_tok ? ld_u4_nt(blk + off) : make_uint4(0, 0, 0, 0);
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
        reduce_and_store<G, VS::CPL, LPT, HD>(acc, red, acc0, acc_hstride);
    }
    if (tid < G) {
        ml0[tid * ml_hstride] = m_sh[tid];
        ml0[tid * ml_hstride + 1] = l_sh[tid];
    }
}

} // namespace kvq
