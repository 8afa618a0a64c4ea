// row_stats.hip -- pass 1 of the staged verify step: one streaming read of
// every needed logit row (the per-segment work is in row_pass.h).
//
// The grid is (rows x segments), rows enumerated target rows first, then
// draft rows; each 256-thread workgroup streams one contiguous segment of
// one row and writes its SegStat.  The kernel boundary publishes the
// statistics to the accept scan.
#include "row_pass.h"

namespace sv {
namespace {

template <int DT>
__global__ __launch_bounds__(kThreads) void row_stats_kernel(Problem p, Plan plan) {
    const int64_t w = blockIdx.x;
    const int64_t row_all = w / plan.nseg;
    const int64_t seg = w - row_all * plan.nseg;
    const int64_t ntarget = p.total + p.B;
    const bool is_target = row_all < ntarget;
    const int64_t r = is_target ? row_all : row_all - ntarget;
    const int32_t b = is_target ? seq_of_target_row(p, r) : seq_of_draft_row(p, r);
    __shared__ RowLds lds;
    row_segment<DT, false>(p, plan, b, is_target, r, seg, lds);
}

}  // namespace

hipError_t launch_row_stats(const Problem& p, const Plan& plan, hipStream_t s) {
    const int64_t blocks = (2 * p.total + p.B) * static_cast<int64_t>(plan.nseg);
    if (blocks == 0) return hipSuccess;
    if (p.dtype == SV_BF16)
        row_stats_kernel<SV_BF16><<<dim3(static_cast<uint32_t>(blocks)), dim3(kThreads), 0, s>>>(p, plan);
    else
        row_stats_kernel<SV_F32><<<dim3(static_cast<uint32_t>(blocks)), dim3(kThreads), 0, s>>>(p, plan);
    return hipGetLastError();
}

}  // namespace sv
