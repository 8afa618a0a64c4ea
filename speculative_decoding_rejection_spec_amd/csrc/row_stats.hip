// row_stats.hip -- pass 1 of the staged verify step: one streaming read of
// every needed logit row (the per-segment work is in row_pass.h).
//
// The grid is (rows x segments), rows enumerated target rows first, then
// draft rows; each 256-thread workgroup streams one contiguous segment of
// one row and writes its SegStat.  The kernel boundary publishes the
// statistics to the accept scan.
//
// Early exit: the pages verify one position at a time and stop at the first
// rejection, so rows after it are never needed (page "投机解码", section
// 投机解码的三步流程, step 3; page "大模型推理无损加速:投机采样...", section 三).
// row_lead reads the leading positions of every sequence and runs their
// accept scans; row_list (or the second round) then reads the rest only for
// sequences still undecided.
//
// Gathered form (the drafter hands over q_i(x_i), page
// "大模型推理无损加速:投机采样..." section 三): the accept tests need no draft
// rows, so the passes above read target rows only, and row_list then reads
// the one draft row at each rejection, for the residual.
#include "accept_scan.h"
#include "row_pass.h"

namespace sv {
namespace {

// First drafted slot of sequence b.
__device__ __forceinline__ int64_t first_slot(const Problem& p, int32_t b) {
    return p.offsets ? static_cast<int64_t>(p.offsets[b]) : static_cast<int64_t>(b) * p.k_uniform;
}

// Every needed row in one pass (draft rows only when the accept tests need
// their softmax, i.e. not in the gathered form).
template <int DT>
__global__ __launch_bounds__(kThreads) void row_stats_kernel(Problem p, Plan plan) {
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
    const int64_t w = blockIdx.x;
    if (w >= *count) return;
    const RestItem it = list[w];
    __shared__ RowLds lds;
    row_segment<DT, false>(p, plan, it.b, item_kind(it) == kItemTarget, it.row, item_seg(it), lds, it.x);
}

// Early exit, first round: the rows of positions < lead of every sequence,
// and their accept scans.  Grid (sequence, position, target/draft,
// segment); a workgroup whose row does not exist (position past k_b, a
// draft row the scan does not use, or a sequence whose offsets describe no
// usable range) streams nothing.  Every workgroup then counts itself on its
// sequence's counter, its statistics written through first; the one that
// completes the count (all lead x 2 x nseg workgroups of the sequence) runs
// the accept scan over the leading positions, which settles the sequence or
// lists the rows it still needs.  The scans thus run beside the streaming
// of other sequences' rows, with no launch of their own.
constexpr uint32_t kClearPolls = 1u << 22;   // bound of the wait for block 0's clearing

template <int DT>
__global__ __launch_bounds__(kThreads) void row_lead_kernel(Problem p, Plan plan) {
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        // The accept scans below fill these lists: cleared (written through)
        // before the epoch that lets a scan use them.
        st_co<true>(plan.blk_ctr, uint64_t{0});
        st_co<true>(plan.dlist_n, 0u);
        st_co<true>(plan.early_n, 0u);
        wait_stores();
        st_co<true>(plan.lead_clr, plan.epoch);
    }
    if (blockIdx.x < static_cast<uint32_t>(p.B) && threadIdx.x == 0)   // (the grid has at least 2B blocks)
        plan.aband[blockIdx.x] = 0;
    int64_t q = blockIdx.x;
    const int64_t seg = q % plan.nseg;
    q /= plan.nseg;
    const bool is_target = (q & 1) == 0;
    q >>= 1;
    const int32_t i = static_cast<int32_t>(q % plan.lead);
    const int32_t b = static_cast<int32_t>(q / plan.lead);
    const int64_t o = first_slot(p, b);
    const int64_t o1 = p.offsets ? static_cast<int64_t>(p.offsets[b + 1]) : o + p.k_uniform;
    const int64_t k = o1 - o;
    const bool usable = o >= 0 && o1 >= o && k <= kKMax && o1 <= p.total;
    const bool exists = usable && (is_target ? i <= k : (i < k && !p.draft_probs));
    __shared__ RowLds lds;
    __shared__ int32_t s_last;
    if (exists) row_segment<DT, true>(p, plan, b, is_target, is_target ? o + b + i : o + i, seg, lds);
    if (threadIdx.x == 0) {
        wait_stores();
        s_last = arrive(plan.lead_ctr + b, plan.epoch) == static_cast<uint32_t>(plan.lead * 2 * plan.nseg);
    }
    __syncthreads();
    if (!s_last || threadIdx.x >= 64) return;
    bool cleared = false;
    for (uint32_t polls = 0; polls < kClearPolls && !cleared; ++polls) {
        cleared = ld_co<true>(plan.lead_clr) == plan.epoch;
        if (!cleared) __builtin_amdgcn_s_sleep(2);
    }
    if (!cleared) {            // (block 0 clears first thing: never expected) a data error, not a hang
        if (usable)
            for (int64_t j = threadIdx.x; j <= k; j += 64) p.out_tokens[o + b + j] = -1;
        if (threadIdx.x == 0) {
            p.out_n[b] = -1;
            if (p.out_emit_prob) p.out_emit_prob[b] = NAN;
            plan.done[b] = kDecided;
            plan.task[b].kind = kNone;
        }
        return;
    }
    accept_sequence<true>(p, plan, b, plan.lead, plan.done + b);
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
