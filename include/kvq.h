/*
 * kvq.h -- quantized KV cache for single-query decode attention on AMD
 * Instinct MI355X (gfx950).
 *
 * The library stores, for every sequence and KV head, the K and V rows of
 * each position either as float32 / fp16 values or as symmetric integer
 * codes (8-bit, or 4-bit packed two per byte) with one fp16 scale per group
 * of values, and runs decode attention over that cache without ever
 * expanding it in memory.
 *
 * Sources for the operations (page, then the part of it):
 *   - mni-ml page (donniechu.com), "how the KV cache creates speed": each
 *     decode step computes one new K and one new V row per head and reuses
 *     the cached rows; "why INT8 loses no speed": 1 byte per element instead
 *     of 4, symmetric scaling, decode limited by memory bandwidth.
 *   - TinyLoop "KV Cache 模式": five-modes table (FP16 KV; INT8 KV = int8
 *     vectors + one FP16 scale per head; INT4 symmetric with 15 levels,
 *     nibble-packed) and the memory-formula table (bytes per token).
 *   - KVSplit page (hada.io): key and value bit widths chosen separately
 *     (K8V8, K8V4, K4V4; K4V8 as a demo).
 *   - on-device page (gyaansetu.com): sliding-window eviction keeping the
 *     first 64 tokens as anchors and the 1536 most recent ones.
 *   - aihot.vn KV Cache page: Q is only used at the current position.
 *
 * Conventions for every entry point:
 *   - All buffer pointers are DEVICE pointers owned by the caller.  The
 *     library never allocates, frees or synchronizes; every call only
 *     enqueues kernels on `stream` (a hipStream_t passed as void*, NULL for
 *     the default stream) and returns.  Its only device memory of its own is
 *     the static workspace of kvq_decode_step_static(), part of the loaded
 *     code object.
 *   - Return value: KVQ_OK when the work was enqueued; a negative KVQ_ERR_*
 *     when a host-side check failed (then nothing was launched), or
 *     KVQ_ERR_HIP when HIP refused the launch.  kvq_last_error() describes
 *     the most recent failure of the calling thread.
 *   - Values that live in device memory (start positions, sequence lengths)
 *     cannot be checked on the host; their preconditions are stated per call
 *     and out-of-range values are clamped or skipped, never read or written
 *     outside the buffers.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---------------------------------------------------- */
#define KVQ_OK             0
#define KVQ_ERR_NULL      -1  /* a required pointer is NULL                         */
#define KVQ_ERR_BITS      -2  /* unsupported k_bits / v_bits combination             */
#define KVQ_ERR_SHAPE     -3  /* batch, heads, head_dim, capacity or count invalid  */
#define KVQ_ERR_GROUP     -4  /* group_size invalid for the widths and head_dim      */
#define KVQ_ERR_WINDOW    -5  /* n_anchor / window inconsistent with capacity        */
#define KVQ_ERR_WORKSPACE -6  /* workspace smaller than kvq_workspace_bytes()        */
#define KVQ_ERR_ALIGN     -7  /* a pointer is not aligned as documented              */
#define KVQ_ERR_HIP       -8  /* the HIP runtime refused the launch                  */
#define KVQ_ERR_ARG       -9  /* another argument out of range (scale, chunk, ...)   */

/* ---- the cache descriptor -------------------------------------------- */
/*
 * Geometry and storage of one layer's cache.  The struct is read during the
 * call only; the buffers it points to must stay allocated while kernels
 * enqueued with it may still run.
 *
 * Widths (k_bits, v_bits), per side:
 *   32 = float32 rows, 16 = fp16 rows (round to nearest even),
 *    8 = int8 codes in [-127, 127], 4 = int4 codes in [-7, 7], two per byte,
 *        element 2j in the low nibble of byte j.  Key codes are stored two's
 *        complement; value codes offset binary (code + 128 per byte, code + 8
 *        per nibble, so the stored field is never negative).
 *   Supported pairs: (32,32), (16,16) and any pair from {8,4} x {8,4}.
 *
 * group_size: values per fp16 scale on the quantized sides.  Either a
 *   divisor of head_dim that is a multiple of 32 (one scale per group inside
 *   a head; head_dim itself is one scale per head and position, the TinyLoop
 *   INT8-KV layout), or n_kv_heads * head_dim (one scale per position over
 *   all heads).  Ignored when both sides are 16/32-bit.
 *
 * Window (on-device page): n_anchor = window = 0 stores position p in slot
 *   p (capacity = largest position + 1).  Otherwise capacity must equal
 *   n_anchor + window; position p < n_anchor lives in slot p and later
 *   positions cycle through slots n_anchor .. capacity-1
 *   (slot = n_anchor + (p - n_anchor) % window), so the cache always holds
 *   the anchors and the `window` most recent positions.
 *
 * Layouts (row-major, innermost last; R = head_dim * bits / 8 bytes):
 *   k_codes and v_codes of a 16/32-bit side:
 *       [batch][n_kv_heads][capacity][R] bytes, 16-byte aligned
 *   k_codes of an 8/4-bit key side, tiles of 64 slots stored slice-major:
 *       [batch][n_kv_heads][cap64 / 64][R / 16][64][16] bytes, cap64 =
 *       capacity rounded up to a multiple of 64: byte j of the row of slot s
 *       sits at ((s & ~63) * R + (j / 16) * 1024 + (s & 63) * 16 + j % 16)
 *       within its (sequence, head), so the same 16-byte slice of 64
 *       consecutive rows is 1 KiB of contiguous memory.
 *   v_codes of an 8/4-bit value side, four positions interleaved per byte:
 *       [batch][n_kv_heads][cap4 / 4][R][4] bytes, cap4 = capacity rounded up
 *       to a multiple of 4: byte j of the row of slot s sits at
 *       ((s & ~3) * R + 4 * j + (s & 3)) within its (sequence, head), so one
 *       32-bit word holds byte j of four consecutive slots.
 *   k_scales / v_scales (quantized sides only, NULL otherwise), fp16 bits:
 *       groups inside a head : [batch][n_kv_heads][capacity][head_dim/group_size]
 *       one scale per position: [batch][capacity]
 *     2-byte aligned.
 * kvq_cache_sizes() returns the byte size of each buffer.
 *
 * Paged storage (page_size != 0): the four buffers are pools of n_pages
 * pages, each holding page_size consecutive slots of every KV head, laid out
 * exactly as above with [batch] replaced by [n_pages] and capacity by
 * page_size (so cap4 = cap64 = page_size).  Slot s of sequence b lives in
 * page block_table[b * (capacity / page_size) + s / page_size], at slot
 * s % page_size of that page.  page_size is a power of two in [64, 4096]
 * that divides capacity; block_table is device memory, int32 [batch]
 * [capacity / page_size], 4-byte aligned, read by the kernels.  Pages may be
 * shared, reordered or reused between sequences as the caller manages them;
 * an entry outside [0, n_pages) is never written (the append skips the row)
 * and its slots read as zero codes.  page_size == 0: contiguous storage,
 * n_pages and block_table ignored.
 *
 * Zero-point codec (zero_point = 1; the scale / zero-point metadata of the
 * mni-ml page, "why INT8 loses no speed"; 8/4-bit pairs only, contiguous or
 * paged): per group of g values, lo = min(0, min x), hi = max(0, max x),
 * scale = fp16(RN((hi - lo) / L)) with L = 255 or 15 levels (65504 when it
 * would overflow), zero = clamp(rint(-lo / scale), 0, L), code =
 * clamp(rint(x / scale) + zero, 0, L) in [0, L], decoded as
 * (code - zero) * scale; an all-zero group stores scale 0, zero 0, codes 0.
 * Codes are stored less 2^(bits-1) in the fields above (keys: the two's
 * complement of code - 128 or code - 8; values: the offset binary of the
 * same, which is the code itself).  The scale buffers then hold one 32-bit
 * word per scale entry, fp16 scale bits in the low half and the zero point
 * in the high half, 4-byte aligned: twice the symmetric codec's bytes.
 */
typedef struct kvq_cache {
    int32_t batch;        /* batch * n_kv_heads <= 65535 */
    int32_t n_kv_heads;
    int32_t head_dim;     /* 64 or 128 */
    int32_t capacity;     /* slots per (sequence, KV head) */
    int32_t k_bits;
    int32_t v_bits;
    int32_t group_size;
    int32_t n_anchor;
    int32_t window;
    void *k_codes;
    void *v_codes;
    void *k_scales;
    void *v_scales;
    int32_t page_size;    /* 0 = contiguous */
    int32_t n_pages;
    const int32_t *block_table;
    int32_t zero_point;   /* 0 = symmetric codes; 1 = zero-point codec (8/4-bit sides) */
} kvq_cache;

/* ---- accounting ------------------------------------------------------ */
/*
 * Bytes one position adds to one layer's cache for one sequence: the K and
 * V payloads of n_kv_heads * head_dim values plus 2 bytes per fp16 scale on
 * each quantized side (TinyLoop memory-formula table: FP16 KV = 2*D*2,
 * INT8 KV = 2*D*1 + 2*n_heads*2; with D = 2048 and 16 heads these are 8192
 * and 4160).  group_size as in kvq_cache.  Host-only, pure arithmetic.
 * Returns 0 for an invalid combination.
 */
size_t kvq_bytes_per_token(int k_bits, int v_bits, int n_kv_heads, int head_dim, int group_size);

/*
 * Byte sizes of the four buffers of `c` (pointers in `c` are not read).
 * Any output pointer may be NULL.  Returns KVQ_OK or a KVQ_ERR_* for an
 * invalid geometry.  Host-only.
 */
int kvq_cache_sizes(const kvq_cache *c, size_t *k_codes_bytes, size_t *v_codes_bytes,
                    size_t *k_scales_bytes, size_t *v_scales_bytes);

/* ---- append (quantize the new rows into the cache) -------------------- */
/*
 * Encode n_new new K rows and V rows per sequence and KV head and store
 * them at their slots (mni-ml page: one new K and V per step; TinyLoop
 * five-modes table for the encodings).
 *
 * Encoding of one group of g values x (quantized sides):
 *   amax = max |x|;  s32 = amax / qmax in IEEE float32 (qmax 127 or 7);
 *   stored scale = fp16(s32) rounded to nearest even, 65504 if it would
 *   overflow;  s = that stored value;  code = clamp(round_half_even(x / s)
 *   in float32, -qmax, qmax);  an all-zero group stores scale 0, codes 0.
 * 16-bit sides store fp16(x) (nearest even); 32-bit sides store x.
 *
 * k_new, v_new : float32 [batch][n_kv_heads][n_new][head_dim], 16-byte aligned.
 * start_pos    : int32 [batch] in device memory; row i of sequence b is
 *                position start_pos[b] + i.
 * Device-side rules: a row whose position is negative, or >= capacity with
 * no window, is not stored.  With a window, a row that a later row of the
 * same call would evict (position >= n_anchor and at least `window`
 * positions older than the call's last row) is not stored, so one call with
 * n_new rows leaves the cache exactly as n_new single-row calls would.
 * n_new == 0 is a no-op.  Rows written by one call must not be read by
 * kernels running concurrently on another stream.  One launch: a row-wise
 * kernel, or, for n_new >= 64 rows into an 8/4-bit cache without a window
 * and with per-head or group scales (a prompt's prefill), a kernel over
 * 64-slot tiles that stores the same bytes.
 */
int kvq_append(const kvq_cache *c, const float *k_new, const float *v_new, int n_new,
               const int32_t *start_pos, void *stream);

/* ---- decode attention --------------------------------------------------- */
/*
 * The attention computed (the current query against every cached row,
 * aihot.vn page: Q only at the current position):
 *   for each sequence b and query head hq, with KV head kv = hq / (n_q_heads
 *   / n_kv_heads) and L = min(seq_len[b], capacity, max_seq_len) slots:
 *     z_t = softmax_scale * sum_c q[b][hq][c] * Khat[t][c]
 *     out[b][hq][c] = sum_t exp(z_t - max z) * Vhat[t][c] / sum_t exp(z_t - max z)
 *   over slots t = 0 .. L-1, where Khat/Vhat = code * scale (or the stored
 *   float value).  With a window the slots hold exactly the anchors and the
 *   most recent positions, so slot order differs from position order, which
 *   softmax does not see.  L == 0 gives out = 0.
 *
 * The work is split along the context into chunks of `chunk_tokens` slots
 * (C = kvq_chunk_count() of them): kvq_decode_partials() writes per-chunk
 * partial results (running max m in log2 units, sum l, and unnormalized
 * accumulator) into the workspace; kvq_combine() merges them;
 * kvq_decode_attn() does both.  Splitting the two lets the partials of
 * several devices be merged by one kvq_combine().
 *
 * q, out       : float32 [batch][n_q_heads][head_dim], 16-byte aligned.
 *                n_q_heads must be n_kv_heads * G with G in {1, 2, 4, 8}
 *                (G = 8 on an 8/4-bit cache with scale groups inside the
 *                head, which runs as two workgroup heads per KV head:
 *                n_kv_heads <= 32767).
 * seq_len      : int32 [batch] in device memory, positions written so far
 *                (the newest included).
 * max_seq_len  : host upper bound on seq_len[]; sizes the grid.  Slots at or
 *                beyond it are not attended.
 * softmax_scale: > 0, or 0 for 1/sqrt(head_dim).
 * chunk_tokens : 0 for the library's choice (kvq_chunk_tokens()), or a
 *                multiple of 64 (of 256 for 8/4-bit caches) in [64, 8192]
 *                whose working set fits the device's LDS (else KVQ_ERR_ARG).
 * workspace    : device memory of at least kvq_workspace_bytes(...) bytes,
 *                256-byte aligned.  Layout, for P = batch * n_q_heads rows
 *                and C = kvq_chunk_count(...) chunks: float ml[P][C][2] = (m, l) at offset 0, then
 *                float acc[P][C][head_dim] at offset round_up(8*P*C, 256);
 *                with 8/4-bit keys, scratch for the query's fixed-point form
 *                and one int32 ticket counter per (sequence, KV head) for
 *                kvq_decode_step follow.  An empty chunk has m = -inf, l = 0,
 *                acc = 0.  kvq_decode_step's ticket counters (8/4-bit
 *                caches): one int32 per (sequence, KV head), two when the
 *                eight query heads of a KV head with scale groups inside
 *                the head are split over two workgroups, within the last
 *                round_up(8 * batch * n_kv_heads, 256) bytes of the
 *                workspace_bytes given (the counters at its end, their
 *                start aligned down to 256 bytes); a step needs them zero
 *                when it starts and leaves them zero.  kvq_workspace_bytes()
 *                of every cache, 16/32-bit ones too, ends with that zone,
 *                which no call's other data reaches.  Hand a workspace over zero-filled before its
 *                first kvq_decode_step; calls that share it pass the same
 *                workspace_bytes (then no call of the same batch *
 *                n_kv_heads writes over the counters, whatever its widths,
 *                heads or chunks); a call with another batch * n_kv_heads
 *                on it needs them zeroed again.
 * Results are deterministic: the chunk partition and the merge order are
 * fixed (kvq_decode_step's in-kernel merge takes an atomic ticket only to
 * decide which workgroup merges, not in what order).
 *
 * kvq_chunk_tokens() returns the library's chunk: for 8/4-bit caches the
 * largest power of two <= 2048 slots that still gives >= 1024 workgroups
 * (sequences x KV heads x chunks), at least 512, except that a context of at
 * most 2048 slots which that would split in more than two chunks takes 512
 * (<= 1024 slots) or 1024 (so that its decode step is one launch); for
 * 16/32-bit caches at most 1024, >= 2048 workgroups, at least 64 slots and
 * within the LDS budget.
 *
 * kvq_chunk_count() returns C, the chunks per (sequence, KV head) for these
 * arguments: ceil(L / chunk) for L = min(max_seq_len, capacity) and the
 * chunk of chunk_tokens (or of kvq_chunk_tokens() when it is 0), or a
 * negative status.  kvq_combine() takes it as n_chunks.
 */
int kvq_chunk_tokens(const kvq_cache *c, int n_q_heads, int max_seq_len);

int kvq_chunk_count(const kvq_cache *c, int n_q_heads, int max_seq_len, int chunk_tokens);

size_t kvq_workspace_bytes(const kvq_cache *c, int n_q_heads, int max_seq_len, int chunk_tokens);

int kvq_decode_partials(const kvq_cache *c, const float *q, int n_q_heads, const int32_t *seq_len,
                        int max_seq_len, float softmax_scale, int chunk_tokens,
                        void *workspace, size_t workspace_bytes, void *stream);

/*
 * The two halves of kvq_decode_partials() on an 8/4-bit cache (KVQ_ERR_BITS
 * on a 16/32-bit one), same arguments: kvq_prepare_query() writes the
 * query's fixed-point form (per head a scale and the integer digits the
 * split kernel multiplies the codes with) into the workspace;
 * kvq_decode_partials_prepared() runs the split kernel on it and writes the
 * partials.  The prepared form stays valid until the workspace is written
 * again, so one preparation can serve several split launches for the same
 * query, n_q_heads, max_seq_len and chunk_tokens (e.g. to time the split
 * kernel alone).  kvq_decode_partials() = both, in order.
 */
int kvq_prepare_query(const kvq_cache *c, const float *q, int n_q_heads, int max_seq_len,
                      float softmax_scale, int chunk_tokens, void *workspace,
                      size_t workspace_bytes, void *stream);

int kvq_decode_partials_prepared(const kvq_cache *c, int n_q_heads, const int32_t *seq_len,
                                 int max_seq_len, int chunk_tokens, void *workspace,
                                 size_t workspace_bytes, void *stream);

/*
 * Merge the partials of `n_chunks` chunks for P = batch * n_q_heads rows
 * (layout as above) into out[P][head_dim]:
 *   M = max_i m_i,  out = sum_i acc_i * 2^(m_i - M) / sum_i l_i * 2^(m_i - M),
 * or 0 when every chunk is empty.
 */
int kvq_combine(int batch, int n_q_heads, int head_dim, int n_chunks, const void *workspace,
                size_t workspace_bytes, float *out, void *stream);

int kvq_decode_attn(const kvq_cache *c, const float *q, int n_q_heads, const int32_t *seq_len,
                    int max_seq_len, float softmax_scale, int chunk_tokens, float *out,
                    void *workspace, size_t workspace_bytes, void *stream);

/*
 * One decode step (mni-ml page, how the KV cache gives its speed: a step
 * adds only the new token's K and V to the cache, then attends over it):
 * exactly kvq_append(c, k_new, v_new, n_new, start_pos, stream) followed by
 * kvq_decode_attn(c, q, ..., stream), with the same arguments, rules and
 * results, bit for bit.  On an 8/4-bit cache whose max_seq_len (capped at
 * the capacity) spans one or two chunks: one launch, each workgroup storing
 * the step's rows whose slots fall in its chunk (the last chunk also those
 * past it), preparing its query and, with one chunk, writing out; with two,
 * the last workgroup of each (sequence, KV head) to finish merges the
 * partials (the combine's arithmetic) and sets the workspace's ticket
 * counter of that (sequence, KV head) back to zero.  The counters must
 * therefore be zero when a step starts: a workspace is handed over
 * zero-filled before its first kvq_decode_step, and every step leaves them
 * zero (no memset, so the step can be captured in a graph and replayed).
 * With more chunks the append and the query's fixed-point preparation share
 * the first launch, then the split kernel, then (beyond 4 chunks) the
 * combine; up to 4 chunks the split kernel's last workgroups merge.  On a
 * 16/32-bit cache: append, split, combine.
 * Every argument is checked before anything is enqueued; on an error
 * nothing is.
 */
int kvq_decode_step(const kvq_cache *c, const float *k_new, const float *v_new, int n_new,
                    const int32_t *start_pos, const float *q, int n_q_heads, const int32_t *seq_len,
                    int max_seq_len, float softmax_scale, int chunk_tokens, float *out,
                    void *workspace, size_t workspace_bytes, void *stream);

/* ---- a decode step that allocates nothing ----------------------------- */
/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * kvq_decode_step() with the same arguments, rules and results (bit for bit
 * the same output and cache), minus workspace and workspace_bytes, using a
 * workspace of KVQ_STATIC_SCRATCH_BYTES that the library keeps in a static
 * device array, one per device, held until the process ends.  The first
 * call on a device looks that array's address up (no allocation); no call
 * allocates or frees memory.  The step needs kvq_workspace_bytes(c,
 * n_q_heads, max_seq_len, chunk_tokens) bytes of it; a step needing more is
 * rejected with KVQ_ERR_WORKSPACE before anything is enqueued.  Every call
 * on one device shares that device's array, and each call leaves its
 * contents there: two calls that may run at the same time on one device
 * (different streams, or host threads) race on it and must be ordered by
 * the caller.  Nothing in it must be cleared: the array starts zero-filled,
 * every call passes its whole extent as workspace_bytes (so the ticket
 * counters sit in its last bytes), and each step leaves them zero.  The
 * last 512 KiB of the array are kept for those counters, whatever the
 * geometry (room for two counters for each of the 65535 (sequence, KV head)
 * pairs a cache may have): a step whose other workspace data would not fit
 * below them is rejected with KVQ_ERR_WORKSPACE.
 */
#define KVQ_STATIC_SCRATCH_BYTES (32u << 20)

int kvq_decode_step_static(const kvq_cache *c, const float *k_new, const float *v_new, int n_new,
                           const int32_t *start_pos, const float *q, int n_q_heads, const int32_t *seq_len,
                           int max_seq_len, float softmax_scale, int chunk_tokens, float *out, void *stream);

/* ---- diagnostics ------------------------------------------------------- */
/*
 * Not part of the attention path: stream `bytes` of device memory at `buf`
 * once with 16-byte loads (a grid of min(sink_bytes / 4, 8192) workgroups,
 * each writing one word to `sink`), so that a caller timing it learns the
 * read bandwidth this device reaches in practice.  bytes must be a positive
 * multiple of 32768; buf 16-byte aligned, sink 4-byte aligned.  Asynchronous
 * on `stream`.
 */
int kvq_read_probe(const void *buf, size_t bytes, void *sink, size_t sink_bytes, void *stream);

/* Static text for a status code. */
const char *kvq_status_str(int status);

/* Text describing the calling thread's most recent failure (or ""). */
const char *kvq_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
