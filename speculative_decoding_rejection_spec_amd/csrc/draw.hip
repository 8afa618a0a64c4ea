// draw.hip -- the staged draw: draw_sums (grid sequence x chunk, 256
// threads) and draw_pick (one 256-thread workgroup per sequence),
// where the kernel boundary publishes the chunk sums; or, for one-pass calls
// whose draw fits one round of workgroups, draw_all, which also runs the
// accept scans and the picks.  The work itself is in accept_scan.h and
// draw_pass.h.
#include "draw_pass.h"

namespace sv {
namespace {

template <int DT>
__global__ __launch_bounds__(kThreads) void draw_sums_kernel(Problem p, Plan plan) {
    plan.epoch = call_epoch(plan);
    const int64_t w = blockIdx.x;
    const int32_t b = static_cast<int32_t>(w / plan.nchunk);
    const int32_t c = static_cast<int32_t>(w - static_cast<int64_t>(b) * plan.nchunk);
    __shared__ drawpass::TabEntry tbl[256];
    __shared__ DrawLds lds;
    load_exp2_table(tbl, kThreads);            // overlaps the task load
    const DrawTask task = load_task<false>(p, plan, b);
    // (the whole workgroup leaves; a task the accept scan did not write is
    // the pick's data error)
    if (task.kind == kNone || task.kind == kTaskUnset) return;
    __syncthreads();
    draw_chunk<DT, false>(p, plan, task, b, c, tbl, lds);
}

// Early exit with the draws beside the rows (plan.queued): a sequence whose
// wait in the second round ran out (or every sequence, SV_QUEUE_FINAL) is
// redone here first -- its accept scan if its leading positions left it
// undecided, then every chunk -- with the chunk pass of a 256-thread
// workgroup (the other threads only take part in its barriers).  A call
// whose second round could not find an item's work (never expected) makes
// every sequence a data error.
// (At 4 waves per SIMD four 256-thread workgroups share a CU: at most 128 VGPRs.)
template <int DT, int kPickThreads>
__global__ __launch_bounds__(kPickThreads, 4) void draw_pick_kernel(Problem p, Plan plan) {
    plan.epoch = call_epoch(plan);
    const int32_t b = blockIdx.x;
    __shared__ drawpass::TabEntry tbl[256];
    __shared__ union {
        PickLds<kPickThreads> pick;
        DrawLds draw;
    } lds;
    // The loads of the common path are issued together, before anything
    // depends on them: the redo flag, the task, chunk threadIdx.x's sums.
    const int32_t ab = plan.queued ? plan.aband[b] : 0;
    const uint32_t stall = plan.queued ? *plan.stall : 0u;
    const DrawTask task0 = load_task<false>(p, plan, b);
    const PickPrefetch pf = pick_prefetch<false>(plan, b);
    auto data_error = [&]() {
        const int64_t o = p.offsets ? static_cast<int64_t>(p.offsets[b]) : static_cast<int64_t>(b) * p.k_uniform;
        const int64_t o1 = p.offsets ? static_cast<int64_t>(p.offsets[b + 1]) : o + p.k_uniform;
        if (o >= 0 && o1 >= o && o1 - o <= kKMax && o1 <= p.total)
            for (int64_t i = threadIdx.x; i <= o1 - o; i += kPickThreads) p.out_tokens[o + b + i] = -1;
        if (threadIdx.x == 0) {
            p.out_n[b] = -1;
            if (p.out_emit_prob) p.out_emit_prob[b] = NAN;
        }
    };
    if (plan.queued && stall == plan.epoch) {
        data_error();
        return;
    }
    const bool redo = plan.queued && (plan.queue_mode == SV_QUEUE_FINAL || ab != 0);
    if (redo) {
        load_exp2_table(tbl, kPickThreads);
        if (plan.done[b] == kUndecided) {
            if (threadIdx.x < 64) accept_sequence<true>(p, plan, b, kKMax + 1, nullptr, nullptr, true, nullptr, false);
            wait_stores();
        }
        __syncthreads();
        const DrawTask task = load_task<true>(p, plan, b);
        if (task.kind == kTaskUnset) {         // (not expected: the scan above or the first round wrote it)
            data_error();
            return;
        }
        if (task.kind == kNone) return;
        for (int32_t c = 0; c < plan.nchunk; ++c)
            draw_chunk<DT, true, kPickThreads>(p, plan, task, b, c, tbl, lds.draw);
        wait_stores();
        __syncthreads();
        pick_sequence<DT, kPickThreads, true>(p, plan, task, b, tbl, lds.pick, pick_prefetch<true>(plan, b));
        return;
    }
    const DrawTask task = task0;
    load_exp2_table(tbl, kPickThreads);
    if (task.kind == kTaskUnset) {             // (not expected: every accept scan writes its task)
        data_error();
        return;
    }
    if (task.kind == kNone) return;
    if (task.kind == kResidual && !(fabsf(task.m_d) <= 3.4e38f)) {
        // The gathered form reads the rejected position's draft row only
        // now: a non-finite maximum there makes the sequence a data error.
        data_error();
        return;
    }
    __syncthreads();
    pick_sequence<DT, kPickThreads, false>(p, plan, task, b, tbl, lds.pick, pf);
}

// One pass, small calls: the accept scan, the chunk sums and the pick in
// one launch (grid sequence x chunk, 256 threads).  Every workgroup of
// sequence b runs b's accept scan to learn its draw task (workgroup 0 of
// the sequence writes the scan's outputs, the others write nothing); the
// workgroup that completes the sequence's count of summed chunks (the
// sums written through before the count) picks the token.
template <int DT>
__global__ __launch_bounds__(kThreads) void draw_all_kernel(Problem p, Plan plan) {
    plan.epoch = call_epoch(plan);
    const int64_t w = blockIdx.x;
    const int32_t b = static_cast<int32_t>(w / plan.nchunk);
    const int32_t c = static_cast<int32_t>(w - static_cast<int64_t>(b) * plan.nchunk);
    __shared__ drawpass::TabEntry tbl[256];
    __shared__ union {
        DrawLds draw;
        PickLds<kThreads> pick;
    } lds;
    __shared__ DrawTask s_task;
    __shared__ int32_t s_last;
    load_exp2_table(tbl, kThreads);
    if (threadIdx.x < 64) {
        DrawTask t;
        accept_sequence<false>(p, plan, b, kKMax + 1, nullptr, &t, c == 0);
        if (threadIdx.x == 0) s_task = t;
    }
    __syncthreads();
    const DrawTask task = s_task;
    if (task.kind == kNone) return;            // greedy or a data error: nothing to draw
    draw_chunk<DT, true>(p, plan, task, b, c, tbl, lds.draw);
    wait_stores();
    __syncthreads();
    if (threadIdx.x == 0)
        s_last = __hip_atomic_fetch_add(plan.picked + b, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u ==
                 static_cast<uint32_t>(plan.nchunk);
    __syncthreads();
    if (s_last) pick_sequence<DT, kThreads, true>(p, plan, task, b, tbl, lds.pick, pick_prefetch<true>(plan, b));
}

}  // namespace

hipError_t launch_draw_all(const Problem& p, const Plan& plan, hipStream_t s) {
    const int64_t blocks = static_cast<int64_t>(p.B) * plan.nchunk;
    if (p.dtype == SV_BF16)
        draw_all_kernel<SV_BF16><<<dim3(static_cast<uint32_t>(blocks)), dim3(kThreads), 0, s>>>(p, plan);
    else
        draw_all_kernel<SV_F32><<<dim3(static_cast<uint32_t>(blocks)), dim3(kThreads), 0, s>>>(p, plan);
    return hipGetLastError();
}

hipError_t launch_draw_sums(const Problem& p, const Plan& plan, hipStream_t s) {
    const int64_t blocks = static_cast<int64_t>(p.B) * plan.nchunk;
    if (p.dtype == SV_BF16)
        draw_sums_kernel<SV_BF16><<<dim3(static_cast<uint32_t>(blocks)), dim3(kThreads), 0, s>>>(p, plan);
    else
        draw_sums_kernel<SV_F32><<<dim3(static_cast<uint32_t>(blocks)), dim3(kThreads), 0, s>>>(p, plan);
    return hipGetLastError();
}

// One 256-thread workgroup per sequence.  The pick is a chain of round
// trips and workgroup-wide reductions; fewer waves per barrier outweigh the
// longer per-lane share of its final scan (8 tokens): 256 sequences of
// V = 152064 took 11.8 against 12.0 us with 512 threads and 13.3 against
// 11.5 with 1024 (one per CU); 512 ragged sequences of V = 128256 12.1
// against 12.9 us.
hipError_t launch_draw_pick(const Problem& p, const Plan& plan, hipStream_t s) {
    const dim3 grid(static_cast<uint32_t>(p.B));
    if (p.dtype == SV_BF16)
        draw_pick_kernel<SV_BF16, 256><<<grid, dim3(256), 0, s>>>(p, plan);
    else
        draw_pick_kernel<SV_F32, 256><<<grid, dim3(256), 0, s>>>(p, plan);
    return hipGetLastError();
}

}  // namespace sv
