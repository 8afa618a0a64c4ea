// second_round.hip -- early exit outside the gathered form: both rounds in
// one launch (rounds_kernel), then the staged pick (draw.hip).
//
// First round (lead_pass.h): the rows of the leading positions of every
// sequence and their accept scans.  Each scan lists in the second round's
// schedule what its sequence still needs (list_rest in accept_scan.h): an
// undecided sequence becomes a block of its remaining row segments, whose
// accept item comes lag_a blocks later and its nchunk draw items lag_c
// blocks later; a settled sampling sequence lists its nchunk draw chunks at
// once.  The second round's workgroups follow the first round's in the
// grid; workgroup nlead + v takes item v:
//   * a row segment: streams it and writes its statistics (written through,
//     so workgroups on other XCDs see them);
//   * an accept item: polls until every statistic and captured logit of its
//     sequence's rows is written (the lister marked them unset), then runs
//     the sequence's accept scan, which writes its draw task as an
//     epoch-tagged record (TaskRec);
//   * a draw item: polls until its sequence's task record is this call's (a
//     settled sequence's is written just before its chunks are listed), then
//     sums its chunk.
// Items are dispatched in grid order, so by the time an item waits, what it
// waits for is running or done (the lags put about a resident grid of row
// segments in between, so it is usually done).
//
// Then the staged pick (draw_pick_kernel) redoes any sequence a wait left
// to it and picks every emitted token.
#include "draw_pass.h"
#include "host_args.h"
#include "lead_pass.h"

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

// Thread 0 of a second-round workgroup: item v of the schedule.  Waits
// until its entry carries this call's epoch, or until every sequence is
// counted on lead_done: then the whole schedule is written, and an item
// past the written entries (the accept and draw items of the last blocks)
// follows from the final counts.  For an accept or kItemChunk item, also the
// undecided sequence of its block (*seq).  Returns false past the schedule's
// end, and when a wait runs out (the call is then marked stalled: never
// expected, see the kernel).
__device__ __forceinline__ bool find_item(const Problem& p, const Plan& plan, int64_t v, RestItem* out,
                                          int32_t* seq) {
    bool listed = false, final_counts = false;
    RestItem it{};
    const uint64_t all_done = (static_cast<uint64_t>(plan.epoch) << 32) | static_cast<uint32_t>(p.B);
    // first an ordinary load: an entry written long ago usually comes back current
    if (load_entry<false>(plan.sched + v, plan.epoch, &it)) {
        *out = it;
        listed = true;
    }
    for (uint32_t polls = 0; !listed; ++polls) {
        // (lead_done, one word every waiting workgroup reads, only on every
        // fourth poll)
        const bool count = (polls & 3) == 0;
        const bool got = load_entry<true>(plan.sched + v, plan.epoch, &it);
        const uint64_t d = count ? ld_co<true>(plan.lead_done) : 0;
        if (got) { listed = true; break; }
        if (d == all_done) { final_counts = true; break; }
        if (polls >= plan.item_polls) break;
        __builtin_amdgcn_s_sleep(8);
    }
    if (!listed && final_counts) {
        const uint64_t ctr = ld_co<true>(plan.blk_ctr);
        const int64_t nblk = static_cast<int64_t>(ctr >> 32), nr = static_cast<int64_t>(ctr & 0xffffffffu);
        const int64_t la = plan.lag_a, lc = plan.lag_c, nchunk = plan.nchunk;
        const int64_t vend = nr + max(static_cast<int64_t>(0), nblk - la) + nchunk * max(static_cast<int64_t>(0), nblk - lc);
        if (v >= nr + nblk * (1 + nchunk)) return false;             // past the schedule
        if (v < vend) {
            // (written before its lister counted its sequence)
            listed = load_entry<true>(plan.sched + v, plan.epoch, &it);
        } else {                                   // the items of the last blocks
            int64_t t = v - vend;
            const int64_t na = min(nblk, la);
            if (t < na) {
                it = rest_item(static_cast<int32_t>(nblk - na + t), 0, kItemAccept, 0, -1);
            } else {
                t -= na;
                it = rest_item(static_cast<int32_t>(nblk - min(nblk, lc) + t / nchunk), 0, kItemChunk,
                               static_cast<int32_t>(t % nchunk), -1);
            }
            listed = true;
        }
    }
    if (!listed) {
        st_co<true>(plan.stall, plan.epoch);
        return false;
    }
    *out = it;
    const int32_t kind = item_kind(it);
    if (kind == kItemAccept || kind == kItemChunk) {
        // the block's sequence: written by its lister, which has counted the
        // block and so is running (an ordinary load first, as for the entry)
        for (uint32_t polls = 0;; ++polls) {
            const uint64_t s = polls == 0 ? plan.blk_seq[it.b] : ld_co<true>(plan.blk_seq + it.b);
            if (static_cast<uint32_t>(s >> 32) == plan.epoch) {
                *seq = static_cast<int32_t>(static_cast<uint32_t>(s));
                break;
            }
            if (polls >= plan.item_polls) {
                st_co<true>(plan.stall, plan.epoch);
                return false;
            }
            if (polls > 0) __builtin_amdgcn_s_sleep(8);
        }
    } else if (kind == kItemChunkSeq) {
        *seq = it.b;
    }
    return true;
}

// Both rounds of early exit in one launch.  Workgroups [0, nlead) run the
// first round (lead_pass.h); workgroup nlead + v runs item v of the
// schedule the first round's accept scans list (list_rest).
//
// Every wait ends: workgroups are dispatched in order of their index (on
// each XCD, which receives every eighth one), a first-round workgroup never
// waits for a second-round one, so every first-round workgroup runs to its
// end, after which every entry is written.  The waits are bounded all the
// same: an item wait that runs out marks the call stalled, and the pick
// launch then reports every sequence as a data error; an accept or draw
// wait that runs out leaves its sequence to the pick launch, which redoes
// it.
template <int DT>
__global__ __launch_bounds__(kThreads) void rounds_kernel(Problem p, Plan plan, uint32_t nlead) {
    plan.epoch = begin_epoch(plan);                // (the call's first kernel)
    __shared__ union {
        RowLds row;
        struct {
            drawpass::TabEntry tbl[256];
            DrawLds draw;
        } d;
    } lds;
    __shared__ int32_t s_flag;
    __shared__ DrawTask s_task;
    __shared__ RestItem s_item;
    __shared__ int32_t s_seq;
    const int tid = threadIdx.x;
    if (blockIdx.x < nlead) {
        lead_workgroup<DT>(p, plan, blockIdx.x, lds.row, s_flag);
        return;
    }
    const int64_t v = static_cast<int64_t>(blockIdx.x) - nlead;
    if (tid == 0) {
        RestItem it;
        int32_t seq = 0;
        const bool found = find_item(p, plan, v, &it, &seq);
        s_flag = found;
        s_item = it;
        s_seq = seq;
    }
    __syncthreads();
    if (!s_flag) return;
    const RestItem it = s_item;
    const int32_t kind = item_kind(it);
    if (kind == kItemTarget || kind == kItemDraft) {
        row_segment<DT, true>(p, plan, it.b, kind == kItemTarget, it.row, item_seg(it), lds.row, it.x);
        return;
    }
    if (plan.queue_mode == SV_QUEUE_FINAL) return;
    const int32_t b = s_seq;
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
        else if (tid == 0) st_co<true>(plan.aband + b, 1);   // the pick launch redoes the sequence
        return;
    }
    // a draw chunk: thread 0 waits for the sequence's task (a settled
    // sequence's was written just before its chunks were listed, an
    // undecided one's comes from its accept item) while the others load the
    // exp2 table
    if (p.temperature[b] == 0.f) return;           // greedy: nothing to draw
    const int32_t c = item_seg(it);
    if (tid == 0) {
        DrawTask t{};
        t.kind = kTaskUnset;
        if (kind == kItemChunkSeq || plan.queue_mode != SV_QUEUE_HANDOFF) {
            t = load_task<true>(p, plan, b);
            for (uint32_t polls = 0; polls < kPolls && t.kind == kTaskUnset; ++polls) {
                __builtin_amdgcn_s_sleep(8);
                t = load_task<true, false>(p, plan, b);
            }
        }
        if (t.kind == kTaskUnset) st_co<true>(plan.aband + b, 1);   // the pick launch redoes the sequence
        s_task = t;
    }
    load_exp2_table(lds.d.tbl, kThreads);
    __syncthreads();
    const DrawTask task = s_task;
    // (kNone: a data error found past the leading positions)
    if (task.kind == kTaskUnset || task.kind == kNone) return;
    draw_chunk<DT, false>(p, plan, task, b, c, lds.d.tbl, lds.d.draw);
}

}  // namespace

hipError_t rounds_blocks_per_cu(int32_t dtype, int32_t* blocks) {
    int n = 0;
    const hipError_t e = dtype == SV_BF16
        ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, rounds_kernel<SV_BF16>, kThreads, 0)
        : hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, rounds_kernel<SV_F32>, kThreads, 0);
    *blocks = n;
    return e;
}

hipError_t launch_rounds(const Problem& p, const Plan& plan, hipStream_t s) {
    const int64_t nlead = host::rounds_lead_blocks(p.B, plan.lead, plan.nseg);
    const dim3 grid(static_cast<uint32_t>(
        nlead + host::rounds_rest_blocks(p.B, p.total, p.offsets != nullptr, p.k_uniform, plan.lead, plan.nseg,
                                         plan.nchunk)));
    if (p.dtype == SV_BF16)
        rounds_kernel<SV_BF16><<<grid, dim3(kThreads), 0, s>>>(p, plan, static_cast<uint32_t>(nlead));
    else
        rounds_kernel<SV_F32><<<grid, dim3(kThreads), 0, s>>>(p, plan, static_cast<uint32_t>(nlead));
    return hipGetLastError();
}

}  // namespace sv
