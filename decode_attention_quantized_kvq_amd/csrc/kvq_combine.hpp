// kvq_combine.hpp -- merging the per-chunk partial results of split-K decode
// into the attention output.  For each (sequence, query head) row the chunks
// hold (m_i, l_i, acc_i): their maximum score in log2 units, their sum of
// 2^(z - m_i) and their unnormalized value accumulator.  The output is
//   M = max m_i,  out = sum_i acc_i 2^(m_i - M) / sum_i l_i 2^(m_i - M),
// and 0 when every chunk is empty.  (The split itself is this library's; the
// pages describe the softmax over the whole context only.)
#pragma once

#include <hip/hip_runtime.h>

namespace kvq {

// One output element (row, channel c).  LD loads a float from the partials;
// the combine kernel reads them plainly, the fused step's last workgroup
// through agent-scope loads, with the same arithmetic in the same order.
template <int HD, typename LD>
__device__ __forceinline__ float combine_one(const float *ml, const float *acc, int n_chunks, size_t row, int c,
                                             LD ld)
{
    const float *mr = ml + row * (size_t)n_chunks * 2;
    float M = -INFINITY;
#pragma unroll 8
    for (int i = 0; i < n_chunks; i++) M = fmaxf(M, ld(mr + 2 * i));
    float L = 0.0f, o = 0.0f;
    if (M != -INFINITY) {
        const float *ac = acc + row * (size_t)n_chunks * HD + c;
#pragma unroll 8
        for (int i = 0; i < n_chunks; i++) {
            const float m = ld(mr + 2 * i), l = ld(mr + 2 * i + 1);
            const float e = m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m - M);
            L = fmaf(l, e, L);
            o = fmaf(ld(ac + (size_t)i * HD), e, o);
        }
    }
    return L > 0.0f ? o / L : 0.0f;
}

struct PlainLoad {
    __device__ __forceinline__ float operator()(const float *p) const { return *p; }
};

// partials written by other workgroups of the same launch: relaxed
// device-scope loads, which read the device-coherent copy (never the scalar
// cache, never a stale line of this XCD's L2).  No acquire fence precedes
// them: the ordering they rely on is the hardware's, stated at
// combine_if_last.
struct AgentLoad {
    __device__ __forceinline__ float operator()(const float *p) const
    {
        return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
};

// A block holds 256 / HD rows, one thread per output channel; the chunk loop
// is unrolled so several partial loads are in flight per thread.
template <int HD>
__global__ __launch_bounds__(256) void combine_kernel(const float *__restrict__ ml, const float *__restrict__ acc,
                                                      float *__restrict__ out, int n_chunks, int n_rows)
{
    constexpr int RPB = 256 / HD;
    const int r = threadIdx.x / HD, c = threadIdx.x - r * HD;
    const size_t row = (size_t)blockIdx.x * RPB + r;
    if (row >= (size_t)n_rows) return;
    out[row * HD + c] = combine_one<HD>(ml, acc, n_chunks, row, c, PlainLoad{});
}

// Partials that a workgroup of the same launch may merge are written with
// device-scope stores (coherent across the XCDs' L2 caches without any
// cache-wide write-back or invalidation).
__device__ __forceinline__ void store_partial(float *p, float v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// s_waitcnt vmcnt(0) (expcnt and lgkmcnt left at their maxima): every vector
// memory access of this thread, stores included, has completed
constexpr int WAIT_VMEM_ALL = 0x0F70;

// The fused step's ending, run by every workgroup of the split kernel after
// it has written its chunk's partials with store_partial: each thread waits
// for its own stores, then one ticket per workgroup on the counter of its
// (sequence, KV head); the workgroup that draws the last ticket merges the G
// rows row0 .. row0 + G - 1 into out, reading the partials with device-scope
// loads, and sets the counter back to zero: every other workgroup of the
// (sequence, KV head) has taken its ticket by then, so the counter is zero
// for the next launch (the first launch on a workspace needs it zero: the
// workspace is handed over zero-filled).  No workgroup waits for another.
// flag: one int of LDS.
// Memory ordering: there is no release/acquire pair (a __threadfence()
// before the ticket made the fused step several times slower).  The merge
// relies on this gfx9-family behaviour: a device-scope store has reached
// the device-coherent level shared by all XCDs once the storing thread's
// vmcnt is 0; the ticket is a device-scope atomic performed there after
// every thread of the workgroup has passed that wait (the barrier); the
// merging workgroup's device-scope loads are issued after it draws the
// last ticket and read that level.  So every partial is visible to the
// merge, by hardware behaviour rather than by the HIP memory model.
template <int HD, int G, int THREADS>
__device__ __forceinline__ void combine_if_last(const float *ml, const float *acc, float *out, int *cnt,
                                                int n_chunks, size_t row0, int *flag)
{
    const int tid = threadIdx.x;
    __builtin_amdgcn_s_waitcnt(WAIT_VMEM_ALL);       // this thread's partials are device-visible
    __syncthreads();
    if (tid == 0) *flag = atomicAdd(cnt, 1) == n_chunks - 1;
    __syncthreads();
    if (!*flag) return;                              // block-uniform
    for (int i = tid; i < G * HD; i += THREADS) {
        const int h = i / HD, c = i - h * HD;
        out[(row0 + h) * HD + c] = combine_one<HD>(ml, acc, n_chunks, row0 + h, c, AgentLoad{});
    }
    if (tid == 0) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

} // namespace kvq
