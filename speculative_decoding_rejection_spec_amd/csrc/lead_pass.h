// lead_pass.h -- early exit's first round: the rows of the leading
// positions of every sequence, and their accept scans.
//
// The pages verify one position at a time and stop at the first rejection,
// so rows after it are never needed (page "投机解码", section
// 投机解码的三步流程, step 3; page "大模型推理无损加速:投机采样...", section 三).
// The first round therefore reads positions < lead of every sequence; the
// accept scan over them settles a sequence (a rejection among them, or all
// of its rows read) or lists the rows it still needs for the second round.
//
// Workgroup w of the round maps to (sequence, position, target/draft,
// segment), the sequences in a scrambled order (Plan::lead_mul): the
// second round's schedule follows the order in which the scans finish, and
// sequences that settle early should not come in one run because the
// caller grouped them.  A workgroup whose row does not exist (position past k_b, a
// draft row the tests do not use, or a sequence whose offsets describe no
// usable range) streams nothing.  With one leading position and rows of at
// most kPolledSegs segments (the usual case), every workgroup writes its
// statistics as an epoch-tagged record (LeadRec) and leaves; the sequence's
// last workgroup (highest index) polls the records and runs the accept
// scan on them.  Otherwise every workgroup counts itself on its sequence's
// counter (cleared by workgroup 0 before it publishes lead_clr; a plain
// atomic add), its statistics written through first, and the one that
// completes the count (all lead x 2 x nseg workgroups of the sequence) runs
// the accept scan.  Either way the scans run beside the streaming of other
// sequences' rows.  Finally the scan counts the sequence on plan.lead_done, after
// everything the scan listed is visible: a second-round workgroup that sees
// every sequence counted knows the whole schedule is written.  (lead_done
// takes a plain atomic add: the sequences finish their scans at nearly the
// same time, and a compare-and-swap loop on one word would serialise them
// into a chain of round trips to memory.)
#pragma once

#include "accept_scan.h"
#include "row_pass.h"

namespace sv {

// Bound of the wait for workgroup 0's clearing of the list counters (it
// clears them first thing, so the wait is never expected to run out; if it
// does the sequence becomes a data error rather than a hang).
constexpr uint32_t kClearPolls = 1u << 22;
constexpr uint32_t kPaceSleeps = 4096;   // bound of the first round's pacing wait (Plan::lead_pace)

// The accept scan of sequence b from the first round's records (LeadRec:
// one leading position, rows of at most kPolledSegs segments), run by wave
// 0 of the sequence's last first-round workgroup: each lane polls one word
// of the sequence's records (an ordinary load first, then written-through
// loads) until all carry the call's epoch and the list counters are
// cleared, and lane 0 gets position 0's statistics and captured logits
// (Polled), so the scan loads no statistics itself.
__device__ __forceinline__ void lead_scan_polled(const Problem& p, const Plan& plan, int32_t b, bool usable,
                                                 int64_t o, int64_t k) {
    const int lane = threadIdx.x & 63;
    const int32_t nseg = plan.nseg;
    const int32_t nw = 2 * nseg * 5;                     // (at most 20 words)
    const uint64_t* words = plan.lead_rec[static_cast<int64_t>(b) * 2 * nseg].w;
    // the drafted token of position 0 names the segment that captured its logits
    const int32_t x = (usable && k >= 1) ? p.tokens[o] : -1;
    uint64_t wv = lane < nw ? words[lane] : 0;
    bool cur = lane >= nw || static_cast<uint32_t>(wv >> 32) == plan.epoch;
    uint32_t clr = ld_co<true>(plan.lead_clr);
    bool ready = false;
    for (uint32_t polls = 0; polls < kClearPolls; ++polls) {
        ready = __ballot(!cur) == 0 && __shfl(clr, 0, 64) == plan.epoch;
        if (ready) break;
        __builtin_amdgcn_s_sleep(2);
        if (!cur) {
            wv = ld_co<true>(words + lane);
            cur = static_cast<uint32_t>(wv >> 32) == plan.epoch;
        }
        if (clr != plan.epoch) clr = ld_co<true>(plan.lead_clr);
    }
    if (!ready) {
        // (not expected: every first-round workgroup writes its record)
        if (usable)
            for (int64_t j = lane; j <= k; j += 64) p.out_tokens[o + b + j] = -1;
        if (lane == 0) {
            p.out_n[b] = -1;
            if (p.out_emit_prob) p.out_emit_prob[b] = NAN;
            plan.done[b] = kDecided;
            store_no_task<true>(plan, b);
        }
        return;
    }
    auto word = [&](int rec, int j) {              // (every lane takes part)
        return static_cast<uint32_t>(__shfl(static_cast<int>(static_cast<uint32_t>(wv)), rec * 5 + j, 64));
    };
    Polled pre;
#pragma unroll
    for (int sg = 0; sg < kPolledSegs; ++sg) {
        const int st = sg < nseg ? sg : 0, sd = nseg + st;
        pre.th[sg] = (static_cast<uint64_t>(word(st, 1)) << 32) | word(st, 0);
        pre.ts[sg] = __hiloint2double(static_cast<int>(word(st, 3)), static_cast<int>(word(st, 2)));
        pre.dh[sg] = (static_cast<uint64_t>(word(sd, 1)) << 32) | word(sd, 0);
        pre.ds[sg] = __hiloint2double(static_cast<int>(word(sd, 3)), static_cast<int>(word(sd, 2)));
    }
    int32_t sx = (x >= 0 && x < p.V) ? static_cast<int32_t>(x / plan.seg_len) : 0;
    if (sx >= nseg) sx = nseg - 1;
    pre.xt = __uint_as_float(word(sx, 4));
    pre.xd = __uint_as_float(word(nseg + sx, 4));
    // (cleared before the sequence is listed: a second-round item marks it
    // only after a long wait of its own)
    if (lane == 0) st_co<true>(plan.aband + b, 0);
    accept_sequence<true>(p, plan, b, 1, plan.done + b, nullptr, true, &pre);
}

// s_last: an LDS word of the calling kernel.
template <int DT>
__device__ __forceinline__ void lead_workgroup(const Problem& p, const Plan& plan, int64_t w, RowLds& lds,
                                               int32_t& s_last) {
    const bool recs = plan.lead == 1 && plan.nseg <= kPolledSegs;   // (see below)
    if (w == 0) {
        // The accept scans below fill these lists and count themselves on
        // lead_done, and without records every workgroup counts itself on
        // its sequence's lead_ctr: cleared (written through) before the
        // epoch that lets them be used.  lead_done keeps the epoch in its
        // high half, so a reader tells this call's count from an earlier
        // call's.
        // (with records only thread 0 takes part: the other threads go on
        // to stream their segment at once)
        if (!recs) {
            for (int32_t j = threadIdx.x; j < p.B; j += kThreads) st_co<true>(plan.lead_ctr + j, uint64_t{0});
            wait_stores();
            __syncthreads();
        }
        if (threadIdx.x == 0) {
            st_co<true>(plan.blk_ctr, uint64_t{0});
            st_co<true>(plan.dlist_n, 0u);
            st_co<true>(plan.lead_done, static_cast<uint64_t>(plan.epoch) << 32);
            wait_stores();
            st_co<true>(plan.lead_clr, plan.epoch);
        }
    }
    int64_t q = w;
    const int64_t seg = q % plan.nseg;
    q /= plan.nseg;
    const bool is_target = (q & 1) == 0;
    q >>= 1;
    const int32_t i = static_cast<int32_t>(q % plan.lead);
    const int32_t b = static_cast<int32_t>((q / plan.lead) * plan.lead_mul % p.B);
    // One leading position, rows of at most kPolledSegs segments (recs): the
    // sequence's workgroups hand their statistics over as records (LeadRec)
    // and the last of them runs the scan, with no count of arrivals.
    // (cleared by one of the sequence's own workgroups, before it counts
    // itself: the sequence is listed, and a second-round item can mark it,
    // only after that)
    if (!recs && i == 0 && is_target && seg == 0 && threadIdx.x == 0) st_co<true>(plan.aband + b, 0);
    const int64_t o = first_slot(p, b);
    const int64_t o1 = p.offsets ? static_cast<int64_t>(p.offsets[b + 1]) : o + p.k_uniform;
    const int64_t k = o1 - o;
    const bool usable = o >= 0 && o1 >= o && k <= kKMax && o1 <= p.total;
    const bool exists = usable && (is_target ? i <= k : (i < k && !p.draft_probs));
    LeadRec* rec = recs ? plan.lead_rec + (static_cast<int64_t>(b) * 2 + (is_target ? 0 : 1)) * plan.nseg + seg
                        : nullptr;
    // (the second half waits: Plan::lead_pace; s_memrealtime counts at 100 MHz.
    // The wait also ends after kPaceSleeps sleeps of ~640 clocks, ~1 ms, whatever
    // the counter reads.)
    if (plan.lead_pace != 0 && w >= static_cast<int64_t>(p.B) * plan.lead * plan.nseg) {
        const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
        for (uint32_t n = 0; n < kPaceSleeps && __builtin_amdgcn_s_memrealtime() - t0 < plan.lead_pace; ++n)
            __builtin_amdgcn_s_sleep(10);
    }
    if (exists)
        row_segment<DT, true>(p, plan, b, is_target, is_target ? o + b + i : o + i, seg, lds, kXFromOffsets, rec);
    else if (rec && threadIdx.x == 0)
        store_lead_rec(rec, plan.epoch, 0, 0.0, 0.f);
    if (recs) {
        // The scan: the draft row's last segment, the sequence's highest
        // index, so it waits only for workgroups dispatched before it.
        if (is_target || seg != plan.nseg - 1 || threadIdx.x >= 64) return;
        lead_scan_polled(p, plan, b, usable, o, k);
        if (threadIdx.x == 0) {
            wait_stores();                         // (the wave's listing stores, every lane's)
            __hip_atomic_fetch_add(plan.lead_done, uint64_t{1}, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        return;
    }
    if (threadIdx.x == 0) {
        // One arrival (a plain atomic add: the lead x 2 x nseg workgroups of
        // a sequence would serialise a compare-and-swap loop into a chain of
        // round trips) on the counter workgroup 0 has cleared, after this
        // workgroup's statistics are visible.  (lead_clr is loaded while
        // those stores complete: the wait for them covers both round trips.)
        uint32_t clr = ld_co<true>(plan.lead_clr);
        wait_stores();
        for (uint32_t polls = 0; polls < kClearPolls && clr != plan.epoch; ++polls) {
            __builtin_amdgcn_s_sleep(2);
            clr = ld_co<true>(plan.lead_clr);
        }
        // (a clear never seen, not expected: no arrival, so the sequence is
        // never scanned; this workgroup makes it a data error and marks the
        // call stalled -- after the two-round launch the pick launch then
        // makes every sequence a data error, since the second round's waits
        // for the uncounted sequence run out)
        if (clr != plan.epoch)
            s_last = -1;
        else
            s_last = __hip_atomic_fetch_add(plan.lead_ctr + b, uint64_t{1}, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT) +
                             1 ==
                         static_cast<uint64_t>(plan.lead * 2 * plan.nseg);
    }
    __syncthreads();
    if (s_last == 0 || threadIdx.x >= 64) return;
    if (s_last < 0) {
        if (usable)
            for (int64_t j = threadIdx.x; j <= k; j += 64) p.out_tokens[o + b + j] = -1;
        if (threadIdx.x == 0) {
            p.out_n[b] = -1;
            if (p.out_emit_prob) p.out_emit_prob[b] = NAN;
            plan.done[b] = kDecided;
            store_no_task<true>(plan, b);
            st_co<true>(plan.stall, plan.epoch);
        }
        return;
    }
    accept_sequence<true>(p, plan, b, plan.lead, plan.done + b);
    if (threadIdx.x == 0) {
        wait_stores();                             // (the wave's listing stores, every lane's)
        __hip_atomic_fetch_add(plan.lead_done, uint64_t{1}, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

}  // namespace sv
