// kvq.hip -- the C ABI of libkvq.so: host-side validation, dispatch and
// launches of the append, split-K decode and combine kernels (gfx950).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/kvq.h"
#include "kvq_append.hpp"
#include "kvq_decode.hpp"
#include "kvq_decode_quant.hpp"
#include "kvq_step.hpp"
#include "kvq_probe.hpp"

using namespace kvq;

// The split kernel's instances are compiled in their own translation units
// (kvq_inst.hip, one per family), in parallel.
namespace kvq {
KVQ_QUANT_ALL(KVQ_QUANT_DECLARE)

// the row append: grid (batch * n_new rows, passes over the row, side)
__global__ __launch_bounds__(APPEND_THREADS) void append_kernel(AppendParams p)
{
    append_block(p, blockIdx.x, blockIdx.y, blockIdx.z);
}
}

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return code;
}

int ok()
{
    g_err[0] = 0;
    return KVQ_OK;
}

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool quantized(int bits) { return bits == 8 || bits == 4; }

bool bits_pair_ok(int kb, int vb)
{
    if (kb == 32 || vb == 32) return kb == 32 && vb == 32;
    if (kb == 16 || vb == 16) return kb == 16 && vb == 16;
    return quantized(kb) && quantized(vb);
}

bool per_row(const kvq_cache *c) { return c->group_size == c->n_kv_heads * c->head_dim && c->group_size != c->head_dim; }

constexpr size_t kMaxLds = 64 * 1024;    // largest workgroup LDS accepted
constexpr size_t kAutoLds = 48 * 1024;   // the library's choice keeps 3 workgroups per CU

// Geometry checks shared by every entry point (no pointer is read).
int check_geometry(const kvq_cache *c)
{
    if (!c) return fail(KVQ_ERR_NULL, "cache descriptor is NULL");
    if (c->batch < 1 || c->n_kv_heads < 1 || c->capacity < 1)
        return fail(KVQ_ERR_SHAPE, "batch (%d), n_kv_heads (%d) and capacity (%d) must be >= 1", c->batch,
                    c->n_kv_heads, c->capacity);
    if (c->head_dim != 64 && c->head_dim != 128)
        return fail(KVQ_ERR_SHAPE, "head_dim %d unsupported (64 or 128)", c->head_dim);
    if ((long long)c->batch * c->n_kv_heads > 65535)
        return fail(KVQ_ERR_SHAPE, "batch * n_kv_heads = %lld exceeds 65535", (long long)c->batch * c->n_kv_heads);
    if (!bits_pair_ok(c->k_bits, c->v_bits))
        return fail(KVQ_ERR_BITS, "unsupported widths k_bits=%d v_bits=%d", c->k_bits, c->v_bits);
    if (quantized(c->k_bits)) {
        const int g = c->group_size;
        const bool in_head = g >= 32 && g % 32 == 0 && c->head_dim % g == 0;
        if (!in_head && !(g == c->n_kv_heads * c->head_dim))
            return fail(KVQ_ERR_GROUP, "group_size %d must divide head_dim %d (multiple of 32) or equal n_kv_heads*head_dim",
                        g, c->head_dim);
    }
    if (c->zero_point != 0 && c->zero_point != 1)
        return fail(KVQ_ERR_ARG, "zero_point %d must be 0 or 1", c->zero_point);
    if (c->zero_point && !quantized(c->k_bits))
        return fail(KVQ_ERR_BITS, "the zero-point codec needs 8/4-bit sides (k_bits=%d)", c->k_bits);
    if (c->n_anchor < 0 || c->window < 0)
        return fail(KVQ_ERR_WINDOW, "n_anchor (%d) and window (%d) must be >= 0", c->n_anchor, c->window);
    if (c->window == 0 && c->n_anchor != 0)
        return fail(KVQ_ERR_WINDOW, "n_anchor %d without a window", c->n_anchor);
    if (c->window > 0 && (long long)c->n_anchor + c->window != c->capacity)
        return fail(KVQ_ERR_WINDOW, "capacity %d != n_anchor %d + window %d", c->capacity, c->n_anchor, c->window);
    if (c->page_size != 0) {
        const int P = c->page_size;
        if (P < 64 || P > 4096 || (P & (P - 1)) != 0)
            return fail(KVQ_ERR_SHAPE, "page_size %d must be a power of two in [64, 4096] (or 0)", P);
        if (c->capacity % P != 0)
            return fail(KVQ_ERR_SHAPE, "capacity %d is not a multiple of page_size %d", c->capacity, P);
        if (c->n_pages < 1) return fail(KVQ_ERR_SHAPE, "n_pages %d must be >= 1", c->n_pages);
        if ((long long)c->n_pages * c->n_kv_heads * P > 0x7FFFFFFFLL)
            return fail(KVQ_ERR_SHAPE, "n_pages * n_kv_heads * page_size exceeds 2^31 - 1 slots");
    }
    return KVQ_OK;
}

int check_pointers(const kvq_cache *c)
{
    if (!c->k_codes || !c->v_codes) return fail(KVQ_ERR_NULL, "k_codes / v_codes is NULL");
    if (!aligned(c->k_codes, 16) || !aligned(c->v_codes, 16))
        return fail(KVQ_ERR_ALIGN, "k_codes / v_codes must be 16-byte aligned");
    if (quantized(c->k_bits) && !c->k_scales) return fail(KVQ_ERR_NULL, "k_scales is NULL for a quantized key side");
    if (quantized(c->v_bits) && !c->v_scales) return fail(KVQ_ERR_NULL, "v_scales is NULL for a quantized value side");
    const int sa = c->zero_point ? 4 : 2;            // fp16 scales, or 32-bit scale | zero point words
    if ((c->k_scales && !aligned(c->k_scales, sa)) || (c->v_scales && !aligned(c->v_scales, sa)))
        return fail(KVQ_ERR_ALIGN, "scale buffers must be %d-byte aligned", sa);
    if (c->page_size != 0) {
        if (!c->block_table) return fail(KVQ_ERR_NULL, "block_table is NULL for paged storage");
        if (!aligned(c->block_table, 4)) return fail(KVQ_ERR_ALIGN, "block_table must be 4-byte aligned");
    }
    return KVQ_OK;
}

int groups_per_head(const kvq_cache *c) { return per_row(c) ? 1 : c->head_dim / c->group_size; }

int check_heads(const kvq_cache *c, int n_q_heads)
{
    if (n_q_heads < 1 || n_q_heads % c->n_kv_heads != 0)
        return fail(KVQ_ERR_SHAPE, "n_q_heads %d must be a positive multiple of n_kv_heads %d", n_q_heads, c->n_kv_heads);
    const int G = n_q_heads / c->n_kv_heads;
    if (G != 1 && G != 2 && G != 4 && G != 8)
        return fail(KVQ_ERR_SHAPE, "query heads per KV head %d unsupported (1, 2, 4, 8)", G);
    return KVQ_OK;
}

bool quant_modes(const kvq_cache *c) { return quantized(c->k_bits); }   // both sides quantized (bits_pair_ok)

// storage units (sequences, or pages) and the slots each holds
bool paged(const kvq_cache *c) { return c->page_size != 0; }
int units_of(const kvq_cache *c) { return paged(c) ? c->n_pages : c->batch; }
int cap_u(const kvq_cache *c) { return paged(c) ? c->page_size : c->capacity; }
int cap4_of(const kvq_cache *c) { return (cap_u(c) + 3) & ~3; }
int cap64_of(const kvq_cache *c) { return (cap_u(c) + 63) & ~63; }
int log2i(int x)
{
    int r = 0;
    while ((1 << r) < x) r++;
    return r;
}

// G = 8 query heads per KV head with scale groups inside the head run as
// two workgroup heads of four per cache head (kv_shift 1): eight heads with
// 2 or 4 groups keep too many per-head, per-group sums live (236-256 VGPRs,
// one or two waves per SIMD), four run at the G = 4 rate, and reading each
// cache byte twice costs less than that
bool split_heads(const kvq_cache *c, int G) { return quant_modes(c) && G == 8 && groups_per_head(c) > 1; }

// the query heads one workgroup handles, and the (sequence, KV head) units
// (per workgroup head) of the split kernel's grid
int unit_g(const kvq_cache *c, int G) { return split_heads(c, G) ? 4 : G; }
int unit_kv(const kvq_cache *c, int G) { return split_heads(c, G) ? 2 * c->n_kv_heads : c->n_kv_heads; }

size_t lds_bytes(const kvq_cache *c, int G, int chunk)
{
    G = unit_g(c, G);
    if (quant_modes(c)) {
        const int vg = groups_per_head(c);
        return (size_t)quant_smem(G, c->head_dim, vg, c->zero_point != 0).total;
    }
    return (size_t)float_smem(G, c->head_dim, chunk).total;
}

int max_len_of(const kvq_cache *c, int max_seq_len) { return max_seq_len < c->capacity ? max_seq_len : c->capacity; }

// kvq_decode_step runs as one launch up to kStepMaxChunks chunks per
// (sequence, KV head), the last workgroup of each merging, and as two
// launches (append with query preparation, then the split kernel whose last
// workgroups merge) up to kFusedMaxChunks
constexpr int kStepMaxChunks = 2;
constexpr int kFusedMaxChunks = 4;

int auto_chunk(const kvq_cache *c, int n_q_heads, int max_seq_len)
{
    const int G = n_q_heads / c->n_kv_heads;
    const long long units = (long long)c->batch * c->n_kv_heads;
    const int L = max_len_of(c, max_seq_len);
    // The largest chunk of at most 2048 slots (1024 for float caches) that
    // fits the LDS budget and still gives enough workgroups; when no chunk
    // does, the smallest one.
    // Float caches: >= 8 workgroups per CU over 256 CUs, at least 64 slots;
    // at most 1024, where a chunk's scores take 16 KB of LDS at G = 4 and 6
    // workgroups fit a CU (2048: 4; FP16 at 32K ran 701 us at 1024 against
    // 777 us at 2048).
    // Integer caches: >= one round of 4 workgroups per CU (1024), at least
    // 512 slots: their workgroups carry a fixed start (query digits, first
    // tile) and final merge, so fewer, longer ones win once the chip holds
    // them all.  (Measured: at 32K contexts 4096-slot chunks leave a longer
    // ragged last round and 1024-slot ones pay the start and merge twice as
    // often.)
    const bool q = quant_modes(c);
    const int smallest = q ? 512 : 64;
    const long long want = q ? 1024 : 2048;
    int pick = smallest;
    for (int ch = q ? 2048 : 1024; ch >= smallest; ch >>= 1) {
        // (an integer cache's LDS does not depend on the chunk)
        if (!q && lds_bytes(c, G, ch) > kAutoLds) continue;
        if (units * ((L + ch - 1) / ch) >= want) {
            pick = ch;
            break;
        }
    }
    // Integer caches with short contexts (<= 2048 slots) that this rule would
    // split in more than two chunks: two chunks at most, so that a decode step
    // is one launch (measured: the 1600-slot window over 256 units, cold,
    // 36.3 us a step in two 1024-slot chunks against 38.4 in four 512-slot
    // ones in one launch and ≈ 36.5 in two launches; a 34-layer 1K-context
    // step 503 us in two 512-slot chunks against 548 in one of 1024).
    if (q && L <= 2048 && (L + pick - 1) / pick > kStepMaxChunks) pick = L > 1024 ? 1024 : 512;
    return pick;
}

using FloatFn = void (*)(FloatParams);
using QuantFn = void (*)(QuantParams);
using PrepFn = void (*)(const float *, int32_t *, float *, int32_t *, float, int *, int);

template <int B, int HD, bool PG>
FloatFn pick_float_g(int G)
{
    switch (G) {
    case 1: return decode_float_kernel<B, B, HD, 1, 4, 4, PG>;
    case 2: return decode_float_kernel<B, B, HD, 2, 4, 4, PG>;
    case 4: return decode_float_kernel<B, B, HD, 4, 4, 4, PG>;
    case 8: return decode_float_kernel<B, B, HD, 8, 4, 4, PG>;
    }
    return nullptr;
}

template <bool PG>
FloatFn pick_float_p(int bits, int hd, int G)
{
    if (bits == 32) return hd == 64 ? pick_float_g<32, 64, PG>(G) : pick_float_g<32, 128, PG>(G);
    return hd == 64 ? pick_float_g<16, 64, PG>(G) : pick_float_g<16, 128, PG>(G);
}

FloatFn pick_float(int bits, int hd, int G, bool pg)
{
    return pg ? pick_float_p<true>(bits, hd, G) : pick_float_p<false>(bits, hd, G);
}

template <int KB, int VB, int HD, int KG, bool PG, bool ZP>
QuantFn pick_quant_g(int G)
{
    switch (G) {
    case 1: return decode_quant_kernel<KB, VB, HD, 1, KG, PG, ZP>;
    case 2: return decode_quant_kernel<KB, VB, HD, 2, KG, PG, ZP>;
    case 4: return decode_quant_kernel<KB, VB, HD, 4, KG, PG, ZP>;
    case 8:
        if constexpr (KG == 1) return decode_quant_kernel<KB, VB, HD, 8, KG, PG, ZP>;
        return nullptr;                              // split into two heads of four
    }
    return nullptr;
}

template <int KB, int VB, bool PG, bool ZP>
QuantFn pick_quant_hd(int hd, int G, int kg)
{
    if (hd == 64)
        return kg == 2 ? pick_quant_g<KB, VB, 64, 2, PG, ZP>(G) : kg == 1 ? pick_quant_g<KB, VB, 64, 1, PG, ZP>(G) : nullptr;
    switch (kg) {
    case 1: return pick_quant_g<KB, VB, 128, 1, PG, ZP>(G);
    case 2: return pick_quant_g<KB, VB, 128, 2, PG, ZP>(G);
    case 4: return pick_quant_g<KB, VB, 128, 4, PG, ZP>(G);
    }
    return nullptr;
}

template <bool PG, bool ZP>
QuantFn pick_quant_p(int kb, int vb, int hd, int G, int kg)
{
    if (kb == 8 && vb == 8) return pick_quant_hd<8, 8, PG, ZP>(hd, G, kg);
    if (kb == 8 && vb == 4) return pick_quant_hd<8, 4, PG, ZP>(hd, G, kg);
    if (kb == 4 && vb == 4) return pick_quant_hd<4, 4, PG, ZP>(hd, G, kg);
    if (kb == 4 && vb == 8) return pick_quant_hd<4, 8, PG, ZP>(hd, G, kg);
    return nullptr;
}

// kg: scale groups per head row (head_dim / group_size; 1 for one scale per
// position shared by all heads); pg: paged storage; zp: the zero-point codec
QuantFn pick_quant(int kb, int vb, int hd, int G, int kg, bool pg, bool zp)
{
    if (zp) return pg ? pick_quant_p<true, true>(kb, vb, hd, G, kg) : pick_quant_p<false, true>(kb, vb, hd, G, kg);
    return pg ? pick_quant_p<true, false>(kb, vb, hd, G, kg) : pick_quant_p<false, false>(kb, vb, hd, G, kg);
}

template <int KB, int HD>
PrepFn pick_prep_g(int G)
{
    switch (G) {
    case 1: return qprep_kernel<KB, HD, 1>;
    case 2: return qprep_kernel<KB, HD, 2>;
    case 4: return qprep_kernel<KB, HD, 4>;
    case 8: return qprep_kernel<KB, HD, 8>;
    }
    return nullptr;
}

PrepFn pick_prep(int kb, int hd, int G)
{
    if (kb == 4) return hd == 64 ? pick_prep_g<4, 64>(G) : pick_prep_g<4, 128>(G);
    return hd == 64 ? pick_prep_g<8, 64>(G) : pick_prep_g<8, 128>(G);
}

using StepPrepFn = void (*)(AppendParams, int, int, const float *, int32_t *, float *, int32_t *, float, int *, int);

template <int KB, int HD>
StepPrepFn pick_step_g(int G)
{
    switch (G) {
    case 1: return step_prep_kernel<KB, HD, 1>;
    case 2: return step_prep_kernel<KB, HD, 2>;
    case 4: return step_prep_kernel<KB, HD, 4>;
    case 8: return step_prep_kernel<KB, HD, 8>;
    }
    return nullptr;
}

StepPrepFn pick_step(int kb, int hd, int G)
{
    if (kb == 4) return hd == 64 ? pick_step_g<4, 64>(G) : pick_step_g<4, 128>(G);
    return hd == 64 ? pick_step_g<8, 64>(G) : pick_step_g<8, 128>(G);
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// the ticket-counter zone at the end of a workspace, for `pairs` (sequence,
// cache KV head) pairs: two int32 counters each
size_t cnt_zone_bytes(size_t pairs) { return align256(pairs * 2 * sizeof(int)); }

// Workspace (U = B * the split kernel's heads per sequence, unit_kv): ml
// [P][C][2] | acc [P][C][HD] | (quantized keys) query digits
// [U][S][qd_stride] int32 (each slot's [ND+1][K_COLS][G] padded to 256
// bytes; S = C slots, one per chunk for the one-launch step, when
// C <= kStepMaxChunks, else 1) | query scales [P] float | extra-digit flags
// [U] int32 | the ticket counters' zone (the counters [U] int32, zero between
// calls, sit in the last bytes of the caller's extent, see cnt_offset).
struct WsLayout {
    size_t ml, acc, qdig, qsc, qflag, cnt, total;
};

// n_kv_heads: the split kernel's heads per sequence (twice the cache's when
// its heads are split, unit_kv).  cnt_zone: a cache's workspace
// (kvq_workspace_bytes) ends with the zone of the step's ticket counters,
// round_up(8 batch n_kv_cache, 256) bytes (room for two per (sequence, cache
// KV head), as a split-head step takes), on 16/32-bit caches too (whose calls
// leave it untouched), so that the data of no call reaches the counters of an
// 8/4-bit cache of as many (sequence, KV head) pairs sharing the workspace;
// kvq_combine's partials alone have none.
WsLayout ws_layout(int batch, int n_q_heads, int head_dim, int n_chunks, int n_kv_heads, int k_bits,
                   bool cnt_zone = true, int n_kv_cache = 0)
{
    const size_t P = (size_t)batch * n_q_heads;
    const size_t units = (size_t)batch * n_kv_heads;
    WsLayout w;
    w.ml = 0;
    w.acc = align256(P * n_chunks * 2 * sizeof(float));
    size_t off = w.acc + P * n_chunks * head_dim * sizeof(float);
    w.qdig = w.qsc = w.qflag = w.cnt = 0;
    if (quantized(k_bits)) {
        const size_t slots = n_chunks <= kStepMaxChunks ? (size_t)n_chunks : 1;
        w.qdig = align256(off);
        off = w.qdig + units * slots * (size_t)qd_stride(k_bits, head_dim, n_q_heads / n_kv_heads) * 4;
        w.qsc = align256(off);
        off = w.qsc + P * sizeof(float);
        w.qflag = align256(off);
        off = w.qflag + units * sizeof(int32_t);
    }
    if (cnt_zone) {
        // the step's ticket counters: within the last round_up(8 (sequence,
        // cache KV head) pairs, 256) bytes (cnt_offset places them by the
        // caller's workspace_bytes)
        w.cnt = align256(off);
        off = w.cnt + cnt_zone_bytes((size_t)batch * (n_kv_cache ? n_kv_cache : n_kv_heads));
    }
    w.total = off;
    return w;
}

// Offset of the ticket counters in a workspace of `bytes` bytes: the last
// round_up(4 units, 256) bytes, aligned down to 256, units being the split
// kernel's (sequence, workgroup head) pairs (one or two per (sequence, KV
// head)).  It depends only on the extent the caller hands over and on the
// geometry's units, and it lies inside the counter zone that ends every
// cache's workspace, so calls of other geometries sharing that workspace
// (passing the same extent, with as many (sequence, KV head) pairs) never
// write over them: their own data ends before the zone.
size_t cnt_offset(size_t bytes, size_t units)
{
    return (bytes - align256(units * sizeof(int))) & ~(size_t)255;
}

// kvq_combine's workspace: the partials only
size_t ws_bytes(int batch, int n_q_heads, int head_dim, int n_chunks)
{
    return ws_layout(batch, n_q_heads, head_dim, n_chunks, 1, 32, false).total;
}

int hip_status(const char *what)
{
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(KVQ_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

} // namespace

extern "C" {

size_t kvq_bytes_per_token(int k_bits, int v_bits, int n_kv_heads, int head_dim, int group_size)
{
    if (n_kv_heads <= 0 || head_dim <= 0) return 0;
    const size_t D = (size_t)n_kv_heads * head_dim;
    size_t total = 0;
    const int sides[2] = {k_bits, v_bits};
    for (int s : sides) {
        if (s != 32 && s != 16 && s != 8 && s != 4) return 0;
        if ((D * s) % 8) return 0;
        total += D * s / 8;
        if (s < 16) {
            if (group_size <= 0 || D % (size_t)group_size) return 0;
            total += 2 * (D / group_size);
        }
    }
    return total;
}

int kvq_cache_sizes(const kvq_cache *c, size_t *kc, size_t *vc, size_t *ksb, size_t *vsb)
{
    int st = check_geometry(c);
    if (st) return st;
    const size_t U = (size_t)units_of(c);
    const size_t rows = U * c->n_kv_heads * cap_u(c);
    const size_t sc = per_row(c) ? U * cap_u(c) : rows * groups_per_head(c);
    if (kc) {
        const size_t krows = quantized(c->k_bits) ? U * c->n_kv_heads * cap64_of(c) : rows;
        *kc = krows * c->head_dim * c->k_bits / 8;
    }
    if (vc) {
        const size_t vrows = quantized(c->v_bits) ? U * c->n_kv_heads * cap4_of(c) : rows;
        *vc = vrows * c->head_dim * c->v_bits / 8;
    }
    const size_t scb = c->zero_point ? 4 : 2;       // fp16 scale, or scale | zero point word
    if (ksb) *ksb = quantized(c->k_bits) ? sc * scb : 0;
    if (vsb) *vsb = quantized(c->v_bits) ? sc * scb : 0;
    return ok();
}

} // extern "C"

// Validates an append and fills its parameters and grid (grid.x == 0: nothing
// to store).  Launches nothing.
static int prepare_append(const kvq_cache *c, const float *k_new, const float *v_new, int n_new,
                          const int32_t *start_pos, AppendParams *p, dim3 *grid)
{
    int st = check_geometry(c);
    if (st) return st;
    if (n_new < 0) return fail(KVQ_ERR_SHAPE, "n_new %d < 0", n_new);
    *grid = dim3(0, 1, 1);
    if (n_new == 0) return ok();
    if ((st = check_pointers(c))) return st;
    if (!k_new || !v_new || !start_pos) return fail(KVQ_ERR_NULL, "k_new / v_new / start_pos is NULL");
    if (!aligned(k_new, 16) || !aligned(v_new, 16)) return fail(KVQ_ERR_ALIGN, "k_new / v_new must be 16-byte aligned");
    if (!aligned(start_pos, 4)) return fail(KVQ_ERR_ALIGN, "start_pos must be 4-byte aligned");
    const long long rows = (long long)c->batch * n_new;
    if (rows > 0x7FFFFFFFLL) return fail(KVQ_ERR_SHAPE, "batch * n_new too large");

    p->src[0] = k_new;
    p->src[1] = v_new;
    p->codes[0] = static_cast<uint8_t *>(c->k_codes);
    p->codes[1] = static_cast<uint8_t *>(c->v_codes);
    p->scales[0] = static_cast<uint16_t *>(c->k_scales);
    p->scales[1] = static_cast<uint16_t *>(c->v_scales);
    p->bits[0] = c->k_bits;
    p->bits[1] = c->v_bits;
    p->start_pos = start_pos;
    p->n_kv_heads = c->n_kv_heads;
    p->head_dim = c->head_dim;
    p->capacity = c->capacity;
    p->cap4 = cap4_of(c);
    p->cap64 = cap64_of(c);
    p->cap_u = cap_u(c);
    p->page_shift = paged(c) ? log2i(c->page_size) : 0;
    p->pages_per_seq = paged(c) ? c->capacity / c->page_size : 0;
    p->n_pages = c->n_pages;
    p->block_table = c->block_table;
    p->n_new = n_new;
    p->n_anchor = c->n_anchor;
    p->window = c->window;
    p->per_row = per_row(c) && quantized(c->k_bits) ? 1 : 0;
    p->zp = c->zero_point && quantized(c->k_bits) ? 1 : 0;
    p->group = p->per_row ? c->n_kv_heads * c->head_dim : (quantized(c->k_bits) ? c->group_size : c->head_dim);
    const int R = c->n_kv_heads * c->head_dim;
    const int passes = p->per_row ? 1 : (R + APPEND_SPAN - 1) / APPEND_SPAN;
    *grid = dim3((unsigned)rows, (unsigned)passes, 2);
    return KVQ_OK;
}

// Bulk appends (n_new >= this) into 8/4-bit caches without a window and with
// scales per head or group go through the 64-slot tile kernel.
constexpr int APPEND_TILE_MIN_ROWS = 64;

using AppendTileFn = void (*)(AppendParams);

template <int HD>
AppendTileFn pick_append_tile_hd(int kb, int vb)
{
    if (kb == 8) return vb == 8 ? append_tile_kernel<HD, 8, 8> : append_tile_kernel<HD, 8, 4>;
    return vb == 8 ? append_tile_kernel<HD, 4, 8> : append_tile_kernel<HD, 4, 4>;
}

AppendTileFn pick_append_tile(const kvq_cache *c, int n_new)
{
    if (n_new < APPEND_TILE_MIN_ROWS || !quantized(c->k_bits) || c->window != 0 || per_row(c) || c->zero_point)
        return nullptr;
    if ((long long)c->batch * c->n_kv_heads > 65535) return nullptr;   // grid y: the row kernel takes these
    return c->head_dim == 64 ? pick_append_tile_hd<64>(c->k_bits, c->v_bits)
                             : pick_append_tile_hd<128>(c->k_bits, c->v_bits);
}

extern "C" {

int kvq_append(const kvq_cache *c, const float *k_new, const float *v_new, int n_new, const int32_t *start_pos,
               void *stream)
{
    AppendParams p;
    dim3 grid;
    int st = prepare_append(c, k_new, v_new, n_new, start_pos, &p, &grid);
    if (st || grid.x == 0) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (AppendTileFn tile = pick_append_tile(c, n_new)) {
        // tiles of 64 slots from start & ~63 (start is read on the device)
        const unsigned tiles = (unsigned)((n_new + 2 * TILE_ROWS - 2) / TILE_ROWS);
        hipLaunchKernelGGL(tile, dim3(tiles, (unsigned)(c->batch * c->n_kv_heads), 2), dim3(256), 0, s, p);
        return hip_status("append_tile_kernel launch");
    }
    hipLaunchKernelGGL(append_kernel, grid, dim3(APPEND_THREADS), 0, s, p);
    return hip_status("append_kernel launch");
}

int kvq_chunk_tokens(const kvq_cache *c, int n_q_heads, int max_seq_len)
{
    int st = check_geometry(c);
    if (st) return st;
    if ((st = check_heads(c, n_q_heads))) return st;
    if (max_seq_len < 1) return fail(KVQ_ERR_ARG, "max_seq_len %d < 1", max_seq_len);
    ok();
    return auto_chunk(c, n_q_heads, max_seq_len);
}

static int resolve_chunk(const kvq_cache *c, int n_q_heads, int max_seq_len, int chunk_tokens, int *chunk, int *n_chunks)
{
    int st = check_geometry(c);
    if (st) return st;
    if ((st = check_heads(c, n_q_heads))) return st;
    if (unit_kv(c, n_q_heads / c->n_kv_heads) > 65535)   // the split kernel's grid y
        return fail(KVQ_ERR_SHAPE, "n_kv_heads %d: G = 8 with scale groups runs two workgroup heads per KV head, "
                    "at most 65535", c->n_kv_heads);
    if (max_seq_len < 1) return fail(KVQ_ERR_ARG, "max_seq_len %d < 1", max_seq_len);
    int ch = chunk_tokens;
    if (ch == 0) ch = auto_chunk(c, n_q_heads, max_seq_len);
    if (ch < 64 || ch > 8192 || ch % 64 != 0)
        return fail(KVQ_ERR_ARG, "chunk_tokens %d must be a multiple of 64 in [64, 8192]", ch);
    if (quant_modes(c) && ch % 256 != 0)
        return fail(KVQ_ERR_ARG, "chunk_tokens %d must be a multiple of 256 for 8/4-bit caches", ch);
    const int G = n_q_heads / c->n_kv_heads;
    if (lds_bytes(c, G, ch) > kMaxLds)
        return fail(KVQ_ERR_ARG, "chunk_tokens %d needs %zu bytes of LDS (limit %zu)", ch, lds_bytes(c, G, ch), kMaxLds);
    const int L = max_len_of(c, max_seq_len);
    *chunk = ch;
    *n_chunks = (L + ch - 1) / ch;
    return KVQ_OK;
}

static WsLayout cache_ws_layout(const kvq_cache *c, int n_q_heads, int n_chunks)
{
    const int G = n_q_heads / c->n_kv_heads;
    return ws_layout(c->batch, n_q_heads, c->head_dim, n_chunks, unit_kv(c, G), c->k_bits, true, c->n_kv_heads);
}

static size_t cache_ws_bytes(const kvq_cache *c, int n_q_heads, int n_chunks)
{
    return cache_ws_layout(c, n_q_heads, n_chunks).total;
}

int kvq_chunk_count(const kvq_cache *c, int n_q_heads, int max_seq_len, int chunk_tokens)
{
    int ch, nc;
    const int st = resolve_chunk(c, n_q_heads, max_seq_len, chunk_tokens, &ch, &nc);
    if (st) return st;
    ok();
    return nc;
}

size_t kvq_workspace_bytes(const kvq_cache *c, int n_q_heads, int max_seq_len, int chunk_tokens)
{
    int ch, nc;
    if (resolve_chunk(c, n_q_heads, max_seq_len, chunk_tokens, &ch, &nc)) return 0;
    ok();
    return cache_ws_bytes(c, n_q_heads, nc);
}

} // extern "C"

// Query prep + split kernel (the float path: the split kernel alone).  With
// `ap` (a decode step), the step's append runs first: in the same launch as
// the query prep on an integer cache, as its own launch otherwise.  Every
// check runs before anything is enqueued.
enum { PHASE_PREP = 1, PHASE_SPLIT = 2, PHASE_STEP = 4 };

// PHASE_STEP (integer caches, at most kStepMaxChunks chunks): the one-launch
// decode step, writing out.  out with both other phases (integer caches, at
// most kFusedMaxChunks chunks): the split kernel's last workgroup per
// (sequence, KV head) also merges the partials into out.
static int enqueue_partials(const kvq_cache *c, const float *q, int n_q_heads, const int32_t *seq_len,
                            int max_seq_len, float softmax_scale, int chunk_tokens, void *workspace,
                            size_t workspace_bytes, void *stream, const AppendParams *ap, dim3 ap_grid,
                            int phases = PHASE_PREP | PHASE_SPLIT, float *out = nullptr)
{
    int ch, nc;
    int st = resolve_chunk(c, n_q_heads, max_seq_len, chunk_tokens, &ch, &nc);
    if (st) return st;
    if ((st = check_pointers(c))) return st;
    if (phases != (PHASE_PREP | PHASE_SPLIT) && !quant_modes(c))
        return fail(KVQ_ERR_BITS, "only 8/4-bit caches have a separate query preparation");
    if ((phases & PHASE_STEP) && (nc > kStepMaxChunks || !out || !ap))
        return fail(KVQ_ERR_ARG, "a one-launch step needs at most %d chunks, the output and the step's rows",
                    kStepMaxChunks);
    const bool uses_q = (phases & (PHASE_PREP | PHASE_STEP)) != 0;
    const bool uses_len = (phases & (PHASE_SPLIT | PHASE_STEP)) != 0;
    if ((uses_q && !q) || (uses_len && !seq_len) || !workspace)
        return fail(KVQ_ERR_NULL, "q / seq_len / workspace is NULL");
    if (uses_q && !aligned(q, 16)) return fail(KVQ_ERR_ALIGN, "q must be 16-byte aligned");
    if (uses_len && !aligned(seq_len, 4)) return fail(KVQ_ERR_ALIGN, "seq_len must be 4-byte aligned");
    if (!aligned(workspace, 256)) return fail(KVQ_ERR_ALIGN, "workspace must be 256-byte aligned");
    const size_t need = cache_ws_bytes(c, n_q_heads, nc);
    if (workspace_bytes < need) return fail(KVQ_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, need);
    if (!std::isfinite(softmax_scale) || softmax_scale < 0.0f)
        return fail(KVQ_ERR_ARG, "softmax_scale must be finite and >= 0");
    const float scale = softmax_scale == 0.0f ? 1.0f / std::sqrt((float)c->head_dim) : softmax_scale;
    const float qk_scale = scale * 1.4426950408889634f;   // log2(e): scores kept in log2 units
    const int G = n_q_heads / c->n_kv_heads;
    const WsLayout wl = cache_ws_layout(c, n_q_heads, nc);
    char *ws = static_cast<char *>(workspace);
    hipStream_t st_ = static_cast<hipStream_t>(stream);
    const dim3 grid((unsigned)nc, (unsigned)(c->batch * c->n_kv_heads));
    const size_t lds = lds_bytes(c, G, ch);

    if (!quant_modes(c)) {
        FloatFn fn = pick_float(c->k_bits, c->head_dim, G, paged(c));
        if (!fn) return fail(KVQ_ERR_BITS, "no kernel for k_bits=%d", c->k_bits);
        FloatParams p;
        p.k_codes = static_cast<const uint8_t *>(c->k_codes);
        p.v_codes = static_cast<const uint8_t *>(c->v_codes);
        p.q = q;
        p.seq_len = seq_len;
        p.ws_ml = reinterpret_cast<float *>(ws + wl.ml);
        p.ws_acc = reinterpret_cast<float *>(ws + wl.acc);
        p.n_kv_heads = c->n_kv_heads;
        p.capacity = cap_u(c);
        p.max_len = max_len_of(c, max_seq_len);
        p.block_table = c->block_table;
        p.page_shift = paged(c) ? log2i(c->page_size) : 0;
        p.pages_per_seq = paged(c) ? c->capacity / c->page_size : 0;
        p.n_pages = c->n_pages;
        p.chunk = ch;
        p.n_chunks = nc;
        p.qk_scale = qk_scale;
        if (ap && ap_grid.x > 0) {
            hipLaunchKernelGGL(append_kernel, ap_grid, dim3(APPEND_THREADS), 0, st_, *ap);
            const int hs = hip_status("append_kernel launch");
            if (hs) return hs;
        }
        hipLaunchKernelGGL(fn, grid, dim3(DEC_THREADS), lds, st_, p);
        return hip_status("decode_float_kernel launch");
    }

    // the split kernel's units: (sequence, workgroup head) pairs of Gu query
    // heads each (two per cache KV head when its heads are split)
    const int Gu = unit_g(c, G), Hu = unit_kv(c, G);
    QuantFn fn = pick_quant(c->k_bits, c->v_bits, c->head_dim, Gu, groups_per_head(c), paged(c), c->zero_point != 0);
    const int kg = c->zero_point ? groups_per_head(c) : 0;   // per-group query sums for the zero-point codec
    PrepFn prep = pick_prep(c->k_bits, c->head_dim, Gu);
    StepPrepFn sprep = pick_step(c->k_bits, c->head_dim, Gu);
    if (!fn || !prep || !sprep) return fail(KVQ_ERR_BITS, "no kernel for k_bits=%d v_bits=%d", c->k_bits, c->v_bits);
    int32_t *qdig = reinterpret_cast<int32_t *>(ws + wl.qdig);
    float *qsc = reinterpret_cast<float *>(ws + wl.qsc);
    int32_t *qflag = reinterpret_cast<int32_t *>(ws + wl.qflag);
    const bool one_launch = (phases & PHASE_STEP) != 0;
    if (out && !one_launch && phases != (PHASE_PREP | PHASE_SPLIT))
        return fail(KVQ_ERR_ARG, "a merge inside the split kernel needs both phases");
    // the split kernel's last workgroups merge through the ticket counters:
    // in the one-launch step with several chunks, and in the two-launch one
    // (whose query preparation also zeroes them)
    int *cnt = (one_launch && nc > 1) || (out && !one_launch)
                   ? reinterpret_cast<int *>(ws + cnt_offset(workspace_bytes, (size_t)c->batch * Hu))
                   : nullptr;
    const unsigned units = (unsigned)(c->batch * Hu);
    if (ap && ap_grid.x > 0 && (unsigned long long)ap_grid.x * ap_grid.y * 2 + units > 0x7FFFFFFFull)
        return fail(KVQ_ERR_SHAPE, "batch * n_new too large for a fused step");
    if ((phases & PHASE_PREP) && !one_launch) {
        if (ap && ap_grid.x > 0) {
            const unsigned n_app = ap_grid.x * ap_grid.y * 2;
            hipLaunchKernelGGL(sprep, dim3(n_app + units), dim3(256), 0, st_, *ap, (int)ap_grid.x, (int)ap_grid.y, q,
                               qdig, qsc, qflag, qk_scale, cnt, kg);
        } else {
            hipLaunchKernelGGL(prep, dim3(units), dim3(256), 0, st_, q, qdig, qsc, qflag, qk_scale, cnt, kg);
        }
        const int hs = hip_status("query prep launch");
        if (hs) return hs;
    }
    if (!(phases & (PHASE_SPLIT | PHASE_STEP))) return KVQ_OK;

    QuantParams p;
    p.k_codes = static_cast<const uint8_t *>(c->k_codes);
    p.v_codes = static_cast<const uint8_t *>(c->v_codes);
    p.k_scales = static_cast<const uint16_t *>(c->k_scales);
    p.v_scales = static_cast<const uint16_t *>(c->v_scales);
    p.qdig = qdig;
    p.qsc = qsc;
    p.qflag = qflag;
    p.seq_len = seq_len;
    p.ws_ml = reinterpret_cast<float *>(ws + wl.ml);
    p.ws_acc = reinterpret_cast<float *>(ws + wl.acc);
    p.n_kv_heads = Hu;
    p.n_kv_cache = c->n_kv_heads;
    p.kv_shift = Hu == c->n_kv_heads ? 0 : 1;
    p.capacity = cap_u(c);
    p.cap4 = cap4_of(c);
    p.cap64 = cap64_of(c);
    p.block_table = c->block_table;
    p.page_shift = paged(c) ? log2i(c->page_size) : 0;
    p.pages_per_seq = paged(c) ? c->capacity / c->page_size : 0;
    p.n_pages = c->n_pages;
    p.max_len = max_len_of(c, max_seq_len);
    p.chunk = ch;
    p.n_chunks = nc;
    p.cnt = cnt;
    p.out = out;
    p.step = one_launch ? 1 : 0;
    if (one_launch) {
        if (ap_grid.x > 0) {
            p.ap = *ap;
        } else {
            std::memset(&p.ap, 0, sizeof(p.ap));     // no rows to store (n_new == 0)
        }
        p.q = q;
        p.qk_scale = qk_scale;
    } else {
        std::memset(&p.ap, 0, sizeof(p.ap));
        p.q = nullptr;
        p.qk_scale = 0.0f;
    }
    const bool pr = per_row(c);
    const int gph = groups_per_head(c);
    if (pr) {                                        // strides per storage unit (sequence or page)
        p.k_sc_b = p.v_sc_b = cap_u(c);
        p.k_sc_h = p.v_sc_h = 0;
        p.k_sc_t = p.v_sc_t = 1;
    } else {
        p.k_sc_b = p.v_sc_b = (long long)c->n_kv_heads * cap_u(c) * gph;
        p.k_sc_h = p.v_sc_h = (long long)cap_u(c) * gph;
        p.k_sc_t = p.v_sc_t = gph;
    }
    hipLaunchKernelGGL(fn, dim3((unsigned)nc, (unsigned)Hu, (unsigned)c->batch), dim3(QD_THREADS), lds, st_, p);
    return hip_status("decode_quant_kernel launch");
}

extern "C" {

int kvq_decode_partials(const kvq_cache *c, const float *q, int n_q_heads, const int32_t *seq_len, int max_seq_len,
                        float softmax_scale, int chunk_tokens, void *workspace, size_t workspace_bytes, void *stream)
{
    return enqueue_partials(c, q, n_q_heads, seq_len, max_seq_len, softmax_scale, chunk_tokens, workspace,
                            workspace_bytes, stream, nullptr, dim3(0, 1, 1));
}

int kvq_prepare_query(const kvq_cache *c, const float *q, int n_q_heads, int max_seq_len, float softmax_scale,
                      int chunk_tokens, void *workspace, size_t workspace_bytes, void *stream)
{
    return enqueue_partials(c, q, n_q_heads, nullptr, max_seq_len, softmax_scale, chunk_tokens, workspace,
                            workspace_bytes, stream, nullptr, dim3(0, 1, 1), PHASE_PREP);
}

int kvq_decode_partials_prepared(const kvq_cache *c, int n_q_heads, const int32_t *seq_len, int max_seq_len,
                                 int chunk_tokens, void *workspace, size_t workspace_bytes, void *stream)
{
    return enqueue_partials(c, nullptr, n_q_heads, seq_len, max_seq_len, 0.0f, chunk_tokens, workspace,
                            workspace_bytes, stream, nullptr, dim3(0, 1, 1), PHASE_SPLIT);
}

int kvq_combine(int batch, int n_q_heads, int head_dim, int n_chunks, const void *workspace, size_t workspace_bytes,
                float *out, void *stream)
{
    if (batch < 1 || n_q_heads < 1 || n_chunks < 1) return fail(KVQ_ERR_SHAPE, "batch, n_q_heads, n_chunks must be >= 1");
    if (head_dim != 64 && head_dim != 128) return fail(KVQ_ERR_SHAPE, "head_dim %d unsupported", head_dim);
    if (!workspace || !out) return fail(KVQ_ERR_NULL, "workspace / out is NULL");
    if (!aligned(workspace, 256)) return fail(KVQ_ERR_ALIGN, "workspace must be 256-byte aligned");
    if (!aligned(out, 16)) return fail(KVQ_ERR_ALIGN, "out must be 16-byte aligned");
    const size_t need = ws_bytes(batch, n_q_heads, head_dim, n_chunks);
    if (workspace_bytes < need) return fail(KVQ_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, need);
    const size_t P = (size_t)batch * n_q_heads;
    if (P > 0x7FFFFFFFull) return fail(KVQ_ERR_SHAPE, "too many rows");
    const float *ml = static_cast<const float *>(workspace);
    const float *acc = reinterpret_cast<const float *>(static_cast<const char *>(workspace) + align256(P * n_chunks * 2 * sizeof(float)));
    const int rpb = 256 / head_dim;
    const dim3 grid((unsigned)((P + rpb - 1) / rpb));
    if (head_dim == 64)
        hipLaunchKernelGGL(combine_kernel<64>, grid, dim3(256), 0, static_cast<hipStream_t>(stream), ml, acc, out, n_chunks,
                           (int)P);
    else
        hipLaunchKernelGGL(combine_kernel<128>, grid, dim3(256), 0, static_cast<hipStream_t>(stream), ml, acc, out, n_chunks,
                           (int)P);
    return hip_status("combine_kernel launch");
}

int kvq_decode_attn(const kvq_cache *c, const float *q, int n_q_heads, const int32_t *seq_len, int max_seq_len,
                    float softmax_scale, int chunk_tokens, float *out, void *workspace, size_t workspace_bytes,
                    void *stream)
{
    int ch, nc;
    int st = resolve_chunk(c, n_q_heads, max_seq_len, chunk_tokens, &ch, &nc);
    if (st) return st;
    if (!out) return fail(KVQ_ERR_NULL, "out is NULL");
    if (!aligned(out, 16)) return fail(KVQ_ERR_ALIGN, "out must be 16-byte aligned");
    st = kvq_decode_partials(c, q, n_q_heads, seq_len, max_seq_len, softmax_scale, ch, workspace, workspace_bytes, stream);
    if (st) return st;
    return kvq_combine(c->batch, n_q_heads, c->head_dim, nc, workspace, workspace_bytes, out, stream);
}

int kvq_decode_step(const kvq_cache *c, const float *k_new, const float *v_new, int n_new, const int32_t *start_pos,
                    const float *q, int n_q_heads, const int32_t *seq_len, int max_seq_len, float softmax_scale,
                    int chunk_tokens, float *out, void *workspace, size_t workspace_bytes, void *stream)
{
    int ch, nc;
    int st = resolve_chunk(c, n_q_heads, max_seq_len, chunk_tokens, &ch, &nc);
    if (st) return st;
    if (!out) return fail(KVQ_ERR_NULL, "out is NULL");
    if (!aligned(out, 16)) return fail(KVQ_ERR_ALIGN, "out must be 16-byte aligned");
    AppendParams ap;
    dim3 ag;
    if ((st = prepare_append(c, k_new, v_new, n_new, start_pos, &ap, &ag))) return st;
    // One or two chunks per (sequence, KV head) on an integer cache: one
    // launch, each workgroup storing the step's rows of its chunk, preparing
    // its query and, with one chunk, writing out; with two the last
    // workgroup of each (sequence, KV head) merges the partials and sets its
    // ticket counter back to zero.  Three or four: the append with the query
    // preparation, then the split kernel merging in its last workgroups (each
    // workgroup preparing its own query costs more there than the launch).
    // More chunks: the merge as a launch of its own (the in-kernel merge adds
    // a store wait to every workgroup and a serial merge at the end).
    if (quant_modes(c) && nc <= kStepMaxChunks)
        return enqueue_partials(c, q, n_q_heads, seq_len, max_seq_len, softmax_scale, ch, workspace, workspace_bytes,
                                stream, &ap, ag, PHASE_STEP, out);
    if (quant_modes(c) && nc <= kFusedMaxChunks)
        return enqueue_partials(c, q, n_q_heads, seq_len, max_seq_len, softmax_scale, ch, workspace, workspace_bytes,
                                stream, &ap, ag, PHASE_PREP | PHASE_SPLIT, out);
    st = enqueue_partials(c, q, n_q_heads, seq_len, max_seq_len, softmax_scale, ch, workspace, workspace_bytes, stream,
                          &ap, ag);
    if (st) return st;
    return kvq_combine(c->batch, n_q_heads, c->head_dim, nc, workspace, workspace_bytes, out, stream);
}

} // extern "C"

// ---------------------------------------------------------------------------
// The library's own workspace for kvq_decode_step_static: one array per
// device, held until the process ends.  In host code `scratch` names a
// host-side stand-in, never the device memory: kernels get the address that
// hipGetSymbolAddress returns for the current device, looked up once per
// device.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[KVQ_STATIC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
// the static scratch's counter zone: room for the two counters of each of
// the 65535 (sequence, KV head) pairs a cache may have
constexpr size_t kStaticCntZone = 512 * 1024;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up on the first
// call per device), or an error status.
int static_scratch(void **out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(KVQ_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(KVQ_ERR_HIP, "device %d beyond the %d the library tracks", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr)
            return fail(KVQ_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return KVQ_OK;
}

} // namespace

extern "C" {

int kvq_decode_step_static(const kvq_cache *c, const float *k_new, const float *v_new, int n_new,
                           const int32_t *start_pos, const float *q, int n_q_heads, const int32_t *seq_len,
                           int max_seq_len, float softmax_scale, int chunk_tokens, float *out, void *stream)
{
    int ch, nc;
    int st = resolve_chunk(c, n_q_heads, max_seq_len, chunk_tokens, &ch, &nc);
    if (st) return st;
    // The last kStaticCntZone bytes of the array hold the ticket counters of
    // every geometry (each within the last round_up(8 (sequence, KV head)
    // pairs, 256) bytes); every step's other data stays below them, so no
    // call writes over the counters of another, whatever their geometries.
    const size_t zone = cnt_zone_bytes((size_t)c->batch * c->n_kv_heads);
    const size_t need = cache_ws_bytes(c, n_q_heads, nc);
    if (zone > kStaticCntZone || need - zone > (size_t)KVQ_STATIC_SCRATCH_BYTES - kStaticCntZone)
        return fail(KVQ_ERR_WORKSPACE,
                    "this step needs %zu bytes of workspace, beyond the static scratch's %zu bytes (its last %zu "
                    "for ticket counters)",
                    need, (size_t)KVQ_STATIC_SCRATCH_BYTES, kStaticCntZone);
    void *ws = nullptr;
    if ((st = static_scratch(&ws))) return st;
    return kvq_decode_step(c, k_new, v_new, n_new, start_pos, q, n_q_heads, seq_len, max_seq_len, softmax_scale, ch,
                           out, ws, (size_t)KVQ_STATIC_SCRATCH_BYTES, stream);
}

int kvq_read_probe(const void *buf, size_t bytes, void *sink, size_t sink_bytes, void *stream)
{
    const size_t blk = (size_t)PROBE_THREADS * PROBE_UNROLL * 16;
    if (!buf || !sink) return fail(KVQ_ERR_NULL, "buf / sink is NULL");
    if (!aligned(buf, 16) || !aligned(sink, 4)) return fail(KVQ_ERR_ALIGN, "buf must be 16-byte, sink 4-byte aligned");
    if (bytes < blk || bytes % blk != 0) return fail(KVQ_ERR_ARG, "bytes must be a positive multiple of %zu", blk);
    const size_t grid = sink_bytes / 4 < 8192 ? sink_bytes / 4 : 8192;
    if (grid < 1) return fail(KVQ_ERR_ARG, "sink must hold at least one 4-byte word");
    hipLaunchKernelGGL(read_probe_kernel, dim3((unsigned)grid), dim3(PROBE_THREADS), 0, static_cast<hipStream_t>(stream),
                       static_cast<const probe_u4 *>(buf), (long long)(bytes / blk), static_cast<uint32_t *>(sink));
    return hip_status("read_probe_kernel launch");
}

const char *kvq_status_str(int status)
{
    switch (status) {
    case KVQ_OK: return "ok";
    case KVQ_ERR_NULL: return "required pointer is NULL";
    case KVQ_ERR_BITS: return "unsupported k_bits / v_bits";
    case KVQ_ERR_SHAPE: return "invalid shape";
    case KVQ_ERR_GROUP: return "invalid group_size";
    case KVQ_ERR_WINDOW: return "invalid n_anchor / window";
    case KVQ_ERR_WORKSPACE: return "workspace too small";
    case KVQ_ERR_ALIGN: return "misaligned pointer";
    case KVQ_ERR_HIP: return "HIP launch failed";
    case KVQ_ERR_ARG: return "argument out of range";
    }
    return "unknown status";
}

const char *kvq_last_error(void) { return g_err; }

} // extern "C"
