// kvq_probe.hpp -- a plain HBM read stream, to measure the bandwidth a
// read-only kernel actually reaches on this device (the ceiling the decode
// kernels are compared with, beside the published peak).  Not part of the
// attention path.
#pragma once

#include "kvq_device.hpp"

namespace kvq {

constexpr int PROBE_THREADS = 256;
constexpr int PROBE_UNROLL = 8;   // 16-byte loads in flight per thread

// Each workgroup reads whole 32 KiB blocks (256 threads x 8 x 16 B) in a
// grid-stride loop over n_blocks of them, folds the words with xor and
// writes one word to sink[blockIdx.x] so the loads are not removed.
typedef uint32_t probe_u4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(PROBE_THREADS) void read_probe_kernel(const probe_u4 *__restrict__ src, long long n_blocks,
                                                                   uint32_t *__restrict__ sink)
{
    uint32_t acc = 0;
    for (long long blk = blockIdx.x; blk < n_blocks; blk += gridDim.x) {
        const probe_u4 *p = src + blk * (PROBE_THREADS * PROBE_UNROLL) + threadIdx.x;
        probe_u4 v[PROBE_UNROLL];
#pragma unroll
        for (int i = 0; i < PROBE_UNROLL; i++) v[i] = __builtin_nontemporal_load(p + i * PROBE_THREADS);
#pragma unroll
        for (int i = 0; i < PROBE_UNROLL; i++) acc ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
    }
    acc = (uint32_t)wave_max_ui((int)(acc & 0x7FFFFFFF));
    if (threadIdx.x == 0) sink[blockIdx.x] = acc;
}

} // namespace kvq
