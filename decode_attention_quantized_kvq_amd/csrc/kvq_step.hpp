// kvq_step.hpp -- the first launch of a fused decode step on an integer
// cache: the blocks that quantize and store the step's new K/V rows and the
// blocks that prepare the query digits run in one grid.  Neither part reads
// what the other writes, so one launch replaces two; the split kernel that
// follows sees both.
#pragma once

#include "kvq_append.hpp"
#include "kvq_decode_quant.hpp"

namespace kvq {

// grid.x = app_x * app_y * 2 append blocks (row, pass, side), then one query
// block per (sequence, KV head), which also zeroes that unit's ticket counter
// when cnt is not null.  256 threads.
template <int KB, int HD, int G>
__global__ __launch_bounds__(256) void step_prep_kernel(AppendParams ap, int app_x, int app_y, const float *q,
                                                        int32_t *qdig, float *qsc, int32_t *qflag, float qk_scale,
                                                        int *cnt, int kg)
{
    const int n_app = app_x * app_y * 2;
    const int bid = blockIdx.x;
    if (bid < n_app) {                                 // block-uniform
        const int xy = app_x * app_y;
        const int side = bid / xy;
        const int r = bid - side * xy;
        append_block(ap, r % app_x, r / app_x, side);
        return;
    }
    qprep_block<KB, HD, G>(q, qdig, qsc, qflag, qk_scale, bid - n_app, cnt, kg);
}

} // namespace kvq
