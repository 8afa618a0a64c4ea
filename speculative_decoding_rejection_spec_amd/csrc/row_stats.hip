// row_stats.hip -- pass 1 of the staged verify step: one streaming read of
// every needed logit row (the per-segment work is in row_pass.h).
//
// The grid is (rows x segments), rows enumerated target rows first, then
// draft rows; each 256-thread workgroup streams one contiguous segment of
// one row and writes its SegStat.  The kernel boundary publishes the
// statistics to the accept scan.
//
// Early exit (lead_pass.h): row_lead reads the leading positions of every
// sequence and runs their accept scans; row_list then reads the rest only
// for sequences still undecided.
//
// Gathered form (the drafter hands over q_i(x_i), page
// "大模型推理无损加速:投机采样..." section 三): the accept tests need no draft
// rows, so the passes above read target rows only, and row_list then reads
// the one draft row at each rejection, for the residual.
#include "lead_pass.h"

namespace sv {
namespace {

// Every needed row in one pass (draft rows only when the accept tests need
// their softmax, i.e. not in the gathered form).
template <int DT>
__global__ __launch_bounds__(kThreads) void row_stats_kernel(Problem p, Plan plan) {
    plan.epoch = begin_epoch(plan);                // (the call's first kernel)
    const int64_t w = blockIdx.x;
    if (w == 0 && threadIdx.x == 0) *plan.dlist_n = 0;   // the accept scan fills the draft list
    if (w < p.B && threadIdx.x == 0) plan.picked[w] = 0u;   // (the grid has at least B blocks)
    __shared__ RowLds lds;
    const int64_t row_all = w / plan.nseg;
    const int64_t seg = w - row_all * plan.nseg;
    const int64_t ntarget = p.total + p.B;
    const bool is_target = row_all < ntarget;
    const int64_t r = is_target ? row_all : row_all - ntarget;
    if (!is_target && p.draft_probs) return;
    const int32_t b = is_target ? seq_of_target_row(p, r) : seq_of_draft_row(p, r);
    row_segment<DT, false>(p, plan, b, is_target, r, seg, lds);
}

// The row segments of a list built by an accept scan: with early exit the
// rows the leading positions left to read, in the gathered form the draft
// rows at rejections.  Workgroups past the end of the list return at once.
template <int DT>
__global__ __launch_bounds__(kThreads) void row_list_kernel(Problem p, Plan plan, const RestItem* list,
                                                            const uint32_t* count) {
    plan.epoch = call_epoch(plan);
    const int64_t w = blockIdx.x;
    if (w >= *count) return;
    const RestItem it = list[w];
    __shared__ RowLds lds;
    row_segment<DT, false>(p, plan, it.b, item_kind(it) == kItemTarget, it.row, item_seg(it), lds, it.x);
}

// The row segments early exit's first round listed in its schedule (the
// gathered form, whose schedule holds row segments only).
template <int DT>
__global__ __launch_bounds__(kThreads) void sched_rows_kernel(Problem p, Plan plan, const uint32_t* count) {
    plan.epoch = call_epoch(plan);
    const int64_t w = blockIdx.x;
    if (w >= *count) return;
    RestItem it;
    (void)load_entry<false>(plan.sched + w, plan.epoch, &it);   // (the kernel boundary published it)
    __shared__ RowLds lds;
    row_segment<DT, false>(p, plan, it.b, item_kind(it) == kItemTarget, it.row, item_seg(it), lds, it.x);
}

// Early exit, first round, as its own launch (the gathered form; the
// other forms run it inside the second round's launch): lead_pass.h.
template <int DT>
__global__ __launch_bounds__(kThreads) void row_lead_kernel(Problem p, Plan plan) {
    plan.epoch = begin_epoch(plan);                // (the call's first kernel)
    __shared__ RowLds lds;
    __shared__ int32_t s_last;
    lead_workgroup<DT>(p, plan, blockIdx.x, lds, s_last);
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

hipError_t launch_row_list(const Problem& p, const Plan& plan, const RestItem* list, const uint32_t* count,
                           int64_t max_items, hipStream_t s) {
    if (max_items == 0) return hipSuccess;
    if (p.dtype == SV_BF16)
        row_list_kernel<SV_BF16><<<dim3(static_cast<uint32_t>(max_items)), dim3(kThreads), 0, s>>>(p, plan, list, count);
    else
        row_list_kernel<SV_F32><<<dim3(static_cast<uint32_t>(max_items)), dim3(kThreads), 0, s>>>(p, plan, list, count);
    return hipGetLastError();
}

hipError_t launch_sched_rows(const Problem& p, const Plan& plan, const uint32_t* count, int64_t max_items,
                             hipStream_t s) {
    if (max_items == 0) return hipSuccess;
    if (p.dtype == SV_BF16)
        sched_rows_kernel<SV_BF16><<<dim3(static_cast<uint32_t>(max_items)), dim3(kThreads), 0, s>>>(p, plan, count);
    else
        sched_rows_kernel<SV_F32><<<dim3(static_cast<uint32_t>(max_items)), dim3(kThreads), 0, s>>>(p, plan, count);
    return hipGetLastError();
}

hipError_t launch_row_lead(const Problem& p, const Plan& plan, hipStream_t s) {
    const int64_t blocks = static_cast<int64_t>(p.B) * plan.lead * 2 * plan.nseg;
    if (blocks == 0) return hipSuccess;
    if (p.dtype == SV_BF16)
        row_lead_kernel<SV_BF16><<<dim3(static_cast<uint32_t>(blocks)), dim3(kThreads), 0, s>>>(p, plan);
    else
        row_lead_kernel<SV_F32><<<dim3(static_cast<uint32_t>(blocks)), dim3(kThreads), 0, s>>>(p, plan);
    return hipGetLastError();
}

}  // namespace sv
