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
// usable range) streams nothing.  Every workgroup then counts itself on its
// sequence's counter, its statistics written through first; the one that
// completes the count (all lead x 2 x nseg workgroups of the sequence) runs
// the accept scan, so the scans run beside the streaming of other
// sequences' rows.  Finally it counts the sequence on plan.lead_done, after
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

// s_last, s_clr: LDS words of the calling kernel.
template <int DT>
__device__ __forceinline__ void lead_workgroup(const Problem& p, const Plan& plan, int64_t w, RowLds& lds,
                                               int32_t& s_last, uint32_t& s_clr) {
    if (w == 0 && threadIdx.x == 0) {
        // The accept scans below fill these lists and count themselves on
        // lead_done: cleared (written through) before the epoch that lets a
        // scan use them.  lead_done keeps the epoch in its high half, so a
        // reader tells this call's count from an earlier call's.
        st_co<true>(plan.blk_ctr, uint64_t{0});
        st_co<true>(plan.dlist_n, 0u);
        st_co<true>(plan.lead_done, static_cast<uint64_t>(plan.epoch) << 32);
        wait_stores();
        st_co<true>(plan.lead_clr, plan.epoch);
    }
    int64_t q = w;
    const int64_t seg = q % plan.nseg;
    q /= plan.nseg;
    const bool is_target = (q & 1) == 0;
    q >>= 1;
    const int32_t i = static_cast<int32_t>(q % plan.lead);
    const int32_t b = static_cast<int32_t>((q / plan.lead) * plan.lead_mul % p.B);
    // (cleared by one of the sequence's own workgroups, before it counts
    // itself: the sequence is listed, and a second-round item can mark it,
    // only after that)
    if (i == 0 && is_target && seg == 0 && threadIdx.x == 0) st_co<true>(plan.aband + b, 0);
    const int64_t o = first_slot(p, b);
    const int64_t o1 = p.offsets ? static_cast<int64_t>(p.offsets[b + 1]) : o + p.k_uniform;
    const int64_t k = o1 - o;
    const bool usable = o >= 0 && o1 >= o && k <= kKMax && o1 <= p.total;
    const bool exists = usable && (is_target ? i <= k : (i < k && !p.draft_probs));
    if (exists) row_segment<DT, true>(p, plan, b, is_target, is_target ? o + b + i : o + i, seg, lds);
    if (threadIdx.x == 0) {
        // (the counter and lead_clr are loaded while the statistics' stores
        // complete: the wait for those covers both round trips)
        const uint64_t old = ld_co<true>(plan.lead_ctr + b);
        s_clr = ld_co<true>(plan.lead_clr);
        wait_stores();
        s_last = arrive_from(plan.lead_ctr + b, plan.epoch, old) ==
                 static_cast<uint32_t>(plan.lead * 2 * plan.nseg);
    }
    __syncthreads();
    if (!s_last || threadIdx.x >= 64) return;
    bool cleared = s_clr == plan.epoch;
    for (uint32_t polls = 0; polls < kClearPolls && !cleared; ++polls) {
        cleared = ld_co<true>(plan.lead_clr) == plan.epoch;
        if (!cleared) __builtin_amdgcn_s_sleep(2);
    }
    if (cleared) {
        accept_sequence<true>(p, plan, b, plan.lead, plan.done + b);
    } else {
        if (usable)
            for (int64_t j = threadIdx.x; j <= k; j += 64) p.out_tokens[o + b + j] = -1;
        if (threadIdx.x == 0) {
            p.out_n[b] = -1;
            if (p.out_emit_prob) p.out_emit_prob[b] = NAN;
            plan.done[b] = kDecided;
            store_no_task<true>(plan, b);
        }
    }
    if (threadIdx.x == 0) {
        wait_stores();                             // (the wave's listing stores, every lane's)
        __hip_atomic_fetch_add(plan.lead_done, uint64_t{1}, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

}  // namespace sv
