// rest_draw.hip -- early exit, second round: the remaining rows of the
// undecided sequences and the draw chunks of the sequences the leading
// positions already settled, in one launch.
//
// The two kinds of work are independent (a settled sequence's draw reads
// only its own rows, read in the first round, and its DrawTask), so they
// share a grid without any hand-off between workgroups: the row segments
// keep HBM busy while the draw chunks, bound by fp64 vector arithmetic, fill
// the ALUs the streaming leaves idle.  Both lists are built by the lead
// accept scan; their lengths are known only on the device, so the grid is
// sized for the largest case and block w maps to the w-th item of an even
// interleave of the two lists (workgroups past their ends return at once).
#include "draw_pass.h"
#include "row_pass.h"

namespace sv {
namespace {

template <int DT>
__global__ __launch_bounds__(kThreads) void rest_and_early_draws_kernel(Problem p, Plan plan) {
    const int64_t nr = *plan.rest_n;
    const int64_t nd = static_cast<int64_t>(*plan.early_n) * plan.nchunk;
    const int64_t w = blockIdx.x, all = nr + nd;
    if (w >= all) return;
    // Even interleave: item w is a draw chunk iff the count of draw items
    // among the first w+1 items, floor((w+1) nd / all), steps up at w.
    const int64_t d0 = (w * nd) / all, d1 = ((w + 1) * nd) / all;
    __shared__ union {
        RowLds row;
        struct {
            drawpass::TabEntry tbl[256];
            DrawLds draw;
        } d;
    } lds;
    if (d1 == d0) {
        const RestItem it = plan.rest[w - d0];
        row_segment<DT, false>(p, plan, it.b, it.is_target != 0, it.row, it.seg, lds.row);
        return;
    }
    const int32_t b = plan.early[d0 / plan.nchunk];
    const int32_t c = static_cast<int32_t>(d0 % plan.nchunk);
    load_exp2_table(lds.d.tbl, kThreads);
    const DrawTask task = load_task<false>(p, plan, b);
    __syncthreads();
    draw_chunk<DT, false>(p, plan, task, b, c, lds.d.tbl, lds.d.draw);
}

}  // namespace

hipError_t launch_rest_and_early_draws(const Problem& p, const Plan& plan, hipStream_t s) {
    const int64_t blocks = (2 * p.total + p.B) * static_cast<int64_t>(plan.nseg) +
                           static_cast<int64_t>(p.B) * plan.nchunk;
    if (blocks == 0) return hipSuccess;
    if (p.dtype == SV_BF16)
        rest_and_early_draws_kernel<SV_BF16><<<dim3(static_cast<uint32_t>(blocks)), dim3(kThreads), 0, s>>>(p, plan);
    else
        rest_and_early_draws_kernel<SV_F32><<<dim3(static_cast<uint32_t>(blocks)), dim3(kThreads), 0, s>>>(p, plan);
    return hipGetLastError();
}

}  // namespace sv
