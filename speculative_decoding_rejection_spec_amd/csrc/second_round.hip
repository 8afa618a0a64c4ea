// second_round.hip -- early exit outside the gathered form: the second round,
// which streams the remaining rows and makes the draws beside them.
//
// Second round (rest_draws_kernel).  The lead accept scan listed, for each
// undecided sequence (a block), its remaining row segments, followed lag_a
// blocks later by an accept item for it and lag_c blocks later by its
// nchunk draw items (list_rest in accept_scan.h); the draw chunks of the
// sequences the leading positions settled are interleaved evenly.
// Workgroup w takes item w:
//   * a row segment: streams it and writes its statistics (written through,
//     so workgroups on other XCDs see them); it waits for nothing.
//   * an accept item: polls until every statistic and captured logit of its
//     sequence's rows is written (the lead accept scan marked them unset),
//     then runs the sequence's accept scan, whose draw task is written with
//     its kind last.
//   * a draw item: polls until its sequence's task kind is set, then sums
//     its chunk.
// Items are dispatched in grid order, so by the time an item waits, what it
// waits for is running or done (the lags put about a resident grid of
// row segments in between, so it is usually done).  Each wait is bounded; a
// sequence whose wait runs out is marked and redone by the pick launch.
//
// Then the staged pick (draw_pick_kernel) redoes any marked sequence and
// picks every emitted token.
#include "draw_pass.h"
#include "row_pass.h"

namespace sv {
namespace {

constexpr uint32_t kPolls = 1u << 14;

// True once every row segment statistic (and captured logit) that the
// accept scan of sequence b reads past the leading positions is written.
// Run by one whole wave; lane i checks position i.
__device__ __forceinline__ bool rows_written(const Problem& p, const Plan& plan, int32_t b) {
    const int lane = threadIdx.x & 63;
    const int64_t o = p.offsets ? static_cast<int64_t>(p.offsets[b]) : static_cast<int64_t>(b) * p.k_uniform;
    const int64_t k = p.offsets ? static_cast<int64_t>(p.offsets[b + 1]) - o : p.k_uniform;
    const bool greedy = p.temperature[b] == 0.f;
    const int64_t ntarget = p.total + p.B;
    bool ok = true;
    if (lane >= plan.lead && lane <= k) {
        const int64_t trow = o + b + lane, drow = ntarget + o + lane;
        for (int32_t sg = 0; sg < plan.nseg; ++sg) {
            const SegStat* t = plan.seg + trow * plan.nseg + sg;
            if (greedy || lane < k)                // (a sampling sequence's bonus row is not listed)
                ok = ok && ld_co<true>(&t->head) != kUnset64 &&
                     __double_as_longlong(ld_co<true>(&t->s)) != static_cast<long long>(kUnset64);
            if (!greedy && lane < k) {
                const SegStat* d = plan.seg + drow * plan.nseg + sg;
                ok = ok && ld_co<true>(&d->head) != kUnset64 &&
                     __double_as_longlong(ld_co<true>(&d->s)) != static_cast<long long>(kUnset64);
            }
        }
        if (!greedy && lane < k)
            ok = ok && __float_as_uint(ld_co<true>(&plan.xlogit[trow])) != kUnset32 &&
                 __float_as_uint(ld_co<true>(&plan.xlogit[drow])) != kUnset32;
    }
    return !__any(!ok);
}

// The same for a sampling sequence whose rows have at most kPolledSegs
// segments, keeping what it loads: lane i < k loads position i's target and
// draft segment statistics and captured logits (also those of the leading
// positions, written by an earlier launch) into *pre, which the accept scan
// then uses without loading them again.
__device__ __forceinline__ bool rows_written_polled(const Problem& p, const Plan& plan, int32_t b, Polled* pre) {
    const int lane = threadIdx.x & 63;
    const int64_t o = p.offsets ? static_cast<int64_t>(p.offsets[b]) : static_cast<int64_t>(b) * p.k_uniform;
    const int64_t k = p.offsets ? static_cast<int64_t>(p.offsets[b + 1]) - o : p.k_uniform;
    const int64_t ntarget = p.total + p.B;
    bool ok = true;
    if (lane < k) {
        const int64_t trow = o + b + lane, drow = ntarget + o + lane;
#pragma unroll
        for (int sg = 0; sg < kPolledSegs; ++sg) {
            if (sg < plan.nseg) {
                const SegStat* t = plan.seg + trow * plan.nseg + sg;
                const SegStat* d = plan.seg + drow * plan.nseg + sg;
                pre->th[sg] = ld_co<true>(&t->head);
                pre->ts[sg] = ld_co<true>(&t->s);
                pre->dh[sg] = ld_co<true>(&d->head);
                pre->ds[sg] = ld_co<true>(&d->s);
                ok = ok && pre->th[sg] != kUnset64 && pre->dh[sg] != kUnset64 &&
                     __double_as_longlong(pre->ts[sg]) != static_cast<long long>(kUnset64) &&
                     __double_as_longlong(pre->ds[sg]) != static_cast<long long>(kUnset64);
            }
        }
        pre->xt = ld_co<true>(&plan.xlogit[trow]);
        pre->xd = ld_co<true>(&plan.xlogit[drow]);
        ok = ok && __float_as_uint(pre->xt) != kUnset32 && __float_as_uint(pre->xd) != kUnset32;
    }
    return !__any(!ok);
}

template <int DT>
__global__ __launch_bounds__(kThreads) void rest_draws_kernel(Problem p, Plan plan) {
    __shared__ union {
        RowLds row;
        struct {
            drawpass::TabEntry tbl[256];
            DrawLds draw;
        } d;
    } lds;
    __shared__ int32_t s_ready;
    const int tid = threadIdx.x;
    const int64_t w = blockIdx.x;
    const int64_t nchunk = plan.nchunk;
    const uint64_t ctr = *plan.blk_ctr;
    const int64_t nblk = static_cast<int64_t>(ctr >> 32), nr = static_cast<int64_t>(ctr & 0xffffffffu);
    const int64_t nvirt = nr + nblk * (1 + nchunk);
    const int64_t ne = static_cast<int64_t>(*plan.early_n) * nchunk;
    const int64_t all = nvirt + ne;
    if (w >= all) return;
    int32_t b, c;
    // Even interleave: item w is an early draw chunk iff the count of early
    // chunks among the first w + 1 items, floor((w + 1) ne / all), steps up at w.
    const int64_t d0 = (w * ne) / all, d1 = ((w + 1) * ne) / all;
    if (d1 > d0) {
        if (plan.queue_mode == SV_QUEUE_FINAL) return;
        b = plan.early[d0 / nchunk];
        c = static_cast<int32_t>(d0 % nchunk);
    } else {
        const int64_t v = w - d0;
        const int64_t la = plan.lag_a, lc = plan.lag_c;
        const int64_t vend = nr + max(static_cast<int64_t>(0), nblk - la) + nchunk * max(static_cast<int64_t>(0), nblk - lc);
        RestItem it;
        if (v < vend) {
            it = plan.sched[v];
        } else {                                       // the items of the last blocks
            int64_t t = v - vend;
            const int64_t na = min(nblk, la);
            if (t < na) {
                it = rest_item(static_cast<int32_t>(nblk - na + t), 0, kItemAccept, 0, -1);
            } else {
                t -= na;
                it = rest_item(static_cast<int32_t>(nblk - min(nblk, lc) + t / nchunk), 0, kItemChunk,
                               static_cast<int32_t>(t % nchunk), -1);
            }
        }
        const int32_t kind = item_kind(it);
        if (kind == kItemTarget || kind == kItemDraft) {
            row_segment<DT, true>(p, plan, it.b, kind == kItemTarget, it.row, item_seg(it), lds.row, it.x);
            return;
        }
        b = plan.blk_seq[it.b];
        if (plan.queue_mode == SV_QUEUE_FINAL) return;
        if (kind == kItemAccept) {
            if (tid >= 64) return;                     // one wave runs it
            bool ready = plan.queue_mode != SV_QUEUE_HANDOFF;
            // (a sampling sequence with short segment lists keeps what its
            // last poll loaded, saving the scan a round trip to memory)
            const bool keep = p.temperature[b] != 0.f && plan.nseg <= kPolledSegs;
            Polled pre;
            for (uint32_t polls = 0; ready; ++polls) {
                if (keep ? rows_written_polled(p, plan, b, &pre) : rows_written(p, plan, b)) break;
                if (polls == kPolls) ready = false;
                __builtin_amdgcn_s_sleep(8);
            }
            if (ready) {
                // (the lead scan found the sequence's offsets in order)
                if (keep) accept_sequence<true>(p, plan, b, kKMax + 1, nullptr, nullptr, true, &pre, false);
                else accept_sequence<true>(p, plan, b, kKMax + 1, nullptr, nullptr, true, nullptr, false);
            }
            else if (tid == 0) plan.aband[b] = 1;    // the pick launch redoes the sequence
            return;
        }
        // a draw chunk of an undecided sequence
        if (p.temperature[b] == 0.f) return;       // greedy: nothing to draw
        c = item_seg(it);
        if (tid == 0) {
            bool ready = false;
            if (plan.queue_mode != SV_QUEUE_HANDOFF)
                for (uint32_t polls = 0; polls < kPolls; ++polls) {
                    if (ld_co<true>(&plan.task[b].kind) != kTaskUnset) { ready = true; break; }
                    __builtin_amdgcn_s_sleep(8);
                }
            if (!ready) plan.aband[b] = 1;
            s_ready = ready;
        }
        __syncthreads();
        if (!s_ready) return;
    }
    load_exp2_table(lds.d.tbl, kThreads);
    const DrawTask task = load_task<true>(p, plan, b);
    if (task.kind == kNone) return;                // a data error found past the leading positions
    __syncthreads();
    draw_chunk<DT, false>(p, plan, task, b, c, lds.d.tbl, lds.d.draw);
}

}  // namespace

hipError_t rest_blocks_per_cu(int32_t dtype, int32_t* blocks) {
    int n = 0;
    const hipError_t e = dtype == SV_BF16
        ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, rest_draws_kernel<SV_BF16>, kThreads, 0)
        : hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, rest_draws_kernel<SV_F32>, kThreads, 0);
    *blocks = n;
    return e;
}

hipError_t launch_rest_draws(const Problem& p, const Plan& plan, hipStream_t s) {
    const int64_t blocks = (2 * p.total + p.B) * static_cast<int64_t>(plan.nseg) +
                           static_cast<int64_t>(p.B) * (1 + plan.nchunk);
    if (p.dtype == SV_BF16)
        rest_draws_kernel<SV_BF16><<<dim3(static_cast<uint32_t>(blocks)), dim3(kThreads), 0, s>>>(p, plan);
    else
        rest_draws_kernel<SV_F32><<<dim3(static_cast<uint32_t>(blocks)), dim3(kThreads), 0, s>>>(p, plan);
    return hipGetLastError();
}

}  // namespace sv
