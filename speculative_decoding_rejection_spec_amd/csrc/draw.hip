// draw.hip -- the staged draw: draw_sums (grid sequence x chunk, 256
// threads) and draw_pick (one 1024- or 512-thread workgroup per sequence).
// The kernel boundary publishes the chunk sums; the work itself is in
// draw_pass.h.
#include "draw_pass.h"

namespace sv {
namespace {

template <int DT>
__global__ __launch_bounds__(kThreads) void draw_sums_kernel(Problem p, Plan plan) {
    const int64_t w = blockIdx.x;
    const int32_t b = static_cast<int32_t>(w / plan.nchunk);
    const int32_t c = static_cast<int32_t>(w - static_cast<int64_t>(b) * plan.nchunk);
    __shared__ drawpass::TabEntry tbl[256];
    __shared__ DrawLds lds;
    load_exp2_table(tbl, kThreads);            // overlaps the task load
    const DrawTask task = load_task<false>(p, plan, b);
    if (task.kind == kNone) return;            // the whole workgroup leaves
    __syncthreads();
    draw_chunk<DT, false>(p, plan, task, b, c, tbl, lds);
}

// Early exit with the draws beside the rows (plan.queued): a sequence whose
// wait in the second round ran out (or every sequence, SV_QUEUE_FINAL) is
// redone here first -- its accept scan if its leading positions left it
// undecided, then every chunk -- with the chunk pass of a 256-thread
// workgroup (the other threads only take part in its barriers).
template <int DT, int kPickThreads>
__global__ __launch_bounds__(kPickThreads) void draw_pick_kernel(Problem p, Plan plan) {
    const int32_t b = blockIdx.x;
    __shared__ drawpass::TabEntry tbl[256];
    __shared__ union {
        PickLds<kPickThreads> pick;
        DrawLds draw;
    } lds;
    const bool redo = plan.queued && (plan.queue_mode == SV_QUEUE_FINAL || plan.aband[b] != 0);
    if (redo) {
        load_exp2_table(tbl, kPickThreads);
        if (plan.done[b] == kUndecided) {
            if (threadIdx.x < 64) accept_sequence<true>(p, plan, b);
            wait_stores();
        }
        __syncthreads();
        const DrawTask task = load_task<true>(p, plan, b);
        if (task.kind == kNone) return;
        for (int32_t c = 0; c < plan.nchunk; ++c)
            draw_chunk<DT, true, kPickThreads>(p, plan, task, b, c, tbl, lds.draw);
        wait_stores();
        __syncthreads();
        pick_sequence<DT, kPickThreads, true>(p, plan, task, b, tbl, lds.pick);
        return;
    }
    const DrawTask task = load_task<false>(p, plan, b);   // (issued before the table's loads)
    load_exp2_table(tbl, kPickThreads);
    if (task.kind == kNone) return;
    if (task.kind == kResidual && !(fabsf(task.m_d) <= 3.4e38f)) {
        // The gathered form reads the rejected position's draft row only
        // now: a non-finite maximum there makes the sequence a data error.
        const int64_t o = p.offsets ? static_cast<int64_t>(p.offsets[b]) : static_cast<int64_t>(b) * p.k_uniform;
        const int64_t k = p.offsets ? static_cast<int64_t>(p.offsets[b + 1]) - o : p.k_uniform;
        for (int64_t i = threadIdx.x; i <= k; i += kPickThreads) p.out_tokens[o + b + i] = -1;
        if (threadIdx.x == 0) {
            p.out_n[b] = -1;
            if (p.out_emit_prob) p.out_emit_prob[b] = NAN;
        }
        return;
    }
    __syncthreads();
    pick_sequence<DT, kPickThreads, false>(p, plan, task, b, tbl, lds.pick);
}

}  // namespace

hipError_t launch_draw_sums(const Problem& p, const Plan& plan, hipStream_t s) {
    const int64_t blocks = static_cast<int64_t>(p.B) * plan.nchunk;
    if (p.dtype == SV_BF16)
        draw_sums_kernel<SV_BF16><<<dim3(static_cast<uint32_t>(blocks)), dim3(kThreads), 0, s>>>(p, plan);
    else
        draw_sums_kernel<SV_F32><<<dim3(static_cast<uint32_t>(blocks)), dim3(kThreads), 0, s>>>(p, plan);
    return hipGetLastError();
}

// One workgroup per sequence: 1024 threads while the sequences fit one per
// CU, else 512 (two per CU, so the picks still run in one round).
hipError_t launch_draw_pick(const Problem& p, const Plan& plan, hipStream_t s) {
    const dim3 grid(static_cast<uint32_t>(p.B));
    const bool wide = p.B <= plan.cus;
    if (p.dtype == SV_BF16) {
        if (wide) draw_pick_kernel<SV_BF16, 1024><<<grid, dim3(1024), 0, s>>>(p, plan);
        else draw_pick_kernel<SV_BF16, 512><<<grid, dim3(512), 0, s>>>(p, plan);
    } else {
        if (wide) draw_pick_kernel<SV_F32, 1024><<<grid, dim3(1024), 0, s>>>(p, plan);
        else draw_pick_kernel<SV_F32, 512><<<grid, dim3(512), 0, s>>>(p, plan);
    }
    return hipGetLastError();
}

}  // namespace sv
