// accept_scan.h -- the accept scan of one sequence, run by one wave64;
// shared by the accept kernels, the second round and the one-launch draw.
//
// Lane i (i <= k_b) owns position i of its sequence.  It merges the segment
// statistics of target row i (and draft row i) into the row maximum and the
// normaliser, gathers the logits of the drafted token x_i, and runs the
// accept test u_i < alpha_i = min(1, p_i(x_i) / q_i(x_i)) (page "投机解码",
// section 投机解码的三步流程 step 3; page "大模型推理无损加速:投机采样...",
// section 二.1).  All k tests run at once; a ballot of the rejections and a
// find-first-set give n, the first rejection (or k) -- the same n as a scan
// that stops at the first rejection.  Greedy sequences (T = 0) accept while
// x_i equals the target argmax and emit the argmax of row n (section 动手实践,
// greedy branch).
//
// The row pass keeps S_R = sum_v 2^(z_v c - R) with c = log2(e)/T rounded to
// fp32 and an integer reference R, and captures z_x, the logit of the
// drafted token of each row; p(x) = 2^(z_x c - R) / S_R exactly as the row
// pass summed it (a softmax at the temperature log2(e)/c, within
// 6e-8 relative of T); it is formed in fp64.  Worst-case relative error of
// S_R: under 3e-6 (fp32 partial sums of at most 42 terms: 2.5e-6; v_exp_f32
// and the rounded exponent argument, below 3 in magnitude: 3e-7; the merges
// are in fp64); alpha is therefore within 6e-6 of its exact value, inside
// the 1e-5 band where |u - alpha| counts as a tie.
//
// Sampling sequences leave the emitted token to the draw and record a
// DrawTask: a residual draw at row n if n < k, a bonus draw at row k
// otherwise.
#pragma once

#include "sv_internal.h"

namespace sv {

struct RowStat {
    float m;       // row maximum
    int32_t arg;   // greedy: lowest token id holding m
    float R;       // sampling: reference exponent
    double S;      // sampling: sum of 2^(z c - R)
};

// Merges the nseg segment statistics of one row in segment order: sampling
// rows by exact power-of-two rescaling to the largest reference exponent
// seen so far (the same sum as rescaling every term to the final one);
// greedy rows keep the lowest id among tied maxima.  Statistics are loaded
// four segments at a time so their round trips overlap.
// Merges the statistics (h = SegStat::head, v = SegStat::s) of the next
// segment of a row into r, segments in order.
__device__ __forceinline__ void merge_seg(RowStat& r, uint64_t h, double v, bool greedy) {
    const float m = head_m(h);
    if (greedy) {
        const int32_t a = static_cast<int32_t>(head_hi(h));
        if (m > r.m || (m == r.m && a < r.arg)) { r.m = m; r.arg = a; }
        return;
    }
    const float R = __uint_as_float(head_hi(h));
    r.m = fmaxf(r.m, m);
    if (R == -INFINITY) return;                                  // an empty segment
    if (R > r.R) {
        if (r.R != -INFINITY) r.S = ldexp(r.S, static_cast<int>(fmaxf(r.R - R, -2048.f)));
        r.R = R;
    }
    r.S += ldexp(v, static_cast<int>(fmaxf(R - r.R, -2048.f)));
}

template <bool kCo>
__device__ __forceinline__ RowStat merge_row(const SegStat* seg, int32_t nseg, bool greedy) {
    constexpr int kBatch = 4;
    RowStat r{-INFINITY, INT32_MAX, -INFINITY, 0.0};
    for (int32_t s0 = 0; s0 < nseg; s0 += kBatch) {
        uint64_t h[kBatch];
        double v[kBatch];
#pragma unroll
        for (int i = 0; i < kBatch; ++i) {
            const int32_t s = s0 + i < nseg ? s0 + i : nseg - 1;   // clamped; used only when in range
            h[i] = ld_co<kCo>(&seg[s].head);
            v[i] = greedy ? 0.0 : ld_co<kCo>(&seg[s].s);
        }
#pragma unroll
        for (int i = 0; i < kBatch; ++i) {
            if (s0 + i >= nseg) break;
            merge_seg(r, h[i], v[i], greedy);
        }
    }
    return r;
}

// The statistics a sampling sequence's accept scan reads, loaded by the wave
// that polled for them (rows of at most kPolledSegs segments): lane i holds
// position i's target and draft row segments and captured logits.
struct Polled {
    uint64_t th[kPolledSegs], dh[kPolledSegs];
    double ts[kPolledSegs], ds[kPolledSegs];
    float xt, xd;
};

// log2 of the normaliser sum_v 2^((z_v - m) c) of a merged sampling row.
__device__ __forceinline__ double log2_norm(const RowStat& r, float c) {
    return log2(r.S) + (static_cast<double>(r.R) - static_cast<double>(r.m) * c);
}

// Early exit: lists what sequence b needs from the second round.  An
// undecided sequence becomes block i of the schedule: its remaining rows
// (target rows limit..k, then draft rows limit..k-1 unless no_draft), nseg
// segments each, whose statistics and captured logits it marks unset; after
// block i come the accept item of block i - lag_a and the nchunk draw items
// of block i - lag_c (those of the last blocks follow the whole schedule,
// where the second round finds them by arithmetic), so an item is
// dispatched about lag blocks after the rows it needs.  The task of an
// undecided sampling sequence keeps an earlier call's epoch until its accept
// item writes it, so its draw items read it as unset (load_task) and wait.
// A sampling sequence its leading positions settled (settled) lists only its
// nchunk draw chunks (kItemChunkSeq), at the schedule's current end: its
// task was written just before, so they can run at once, beside the rows of
// the sequences listed around it (a chunk that finds its entry before the
// task's words waits for them like any draw item).
//
// One atomic add on blk_ctr (undecided blocks << 32 | row segments and
// settled chunks listed) places the listing; the marks an undecided
// sequence's accept item waits on are written through and visible before
// the entries, which carry the call's epoch (store_entry).
//
// The place in the schedule is taken first (list_reserve, lane 0's atomic
// add); a settled sequence takes it as soon as its scan decides, before its
// task is written, so that the listings keep the order in which the scans
// decide.
__device__ __forceinline__ uint64_t list_reserve(const Plan& plan, bool settled, int32_t cnt) {
    uint64_t pos = 0;
    if ((threadIdx.x & 63) == 0)
        pos = atomicAdd(reinterpret_cast<unsigned long long*>(plan.blk_ctr),
                        (settled ? 0ull : (1ull << 32)) | static_cast<uint64_t>(cnt));
    return pos;                                    // (lane 0's; list_rest broadcasts it)
}

__device__ __forceinline__ void list_rest(const Problem& p, const Plan& plan, int32_t b, int64_t o, int32_t k,
                                          int32_t limit, bool no_draft, bool greedy, bool skip_bonus_row,
                                          int32_t xtok, bool settled, uint64_t reserved = ~0ull) {
    const int lane = threadIdx.x & 63;
    const int64_t ntarget = p.total + p.B;
    const int32_t nseg = plan.nseg;
    const int64_t nchunk = plan.nchunk;
    const int32_t nt = settled ? 0 : k - limit + (skip_bonus_row ? 0 : 1);
    const int32_t nd = (settled || no_draft) ? 0 : k - limit;
    const int32_t cnt = settled ? static_cast<int32_t>(nchunk) : (nt + nd) * nseg;
    if (!settled) {
        // The marks first, visible before any entry that leads to them.  They
        // need no place in the schedule, so the reservation below goes out
        // with them and one store-completion wait covers both.
        for (int32_t e = lane; e < cnt; e += 64) {
            const int32_t j = e / nseg, sg = e - j * nseg;
            const bool tgt = j < nt;
            const int32_t ps = limit + (tgt ? j : j - nt);            // position in the sequence
            const int64_t row = tgt ? o + b + ps : o + ps;
            SegStat* st = plan.seg + (tgt ? row : ntarget + row) * nseg + sg;
            st_co<true>(&st->head, kUnset64);
            st_co<true>(&st->s, __longlong_as_double(static_cast<long long>(kUnset64)));
            if (sg == 0 && !greedy) st_co<true>(&plan.xlogit[tgt ? row : ntarget + row], __uint_as_float(kUnset32));
        }
    }
    uint64_t pos = reserved != ~0ull ? reserved : list_reserve(plan, settled, cnt);
    if (!settled) wait_stores();                   // (the marks, and the reply)
    pos = __shfl(pos, 0, 64);
    const int64_t i = static_cast<int64_t>(pos >> 32), base = static_cast<int64_t>(pos & 0xffffffffu);
    const int64_t at = base + max(static_cast<int64_t>(0), i - plan.lag_a) +
                       nchunk * max(static_cast<int64_t>(0), i - plan.lag_c);
    if (settled) {
        for (int32_t c = lane; c < cnt; c += 64)
            store_entry(plan.sched + at + c, rest_item(b, 0, kItemChunkSeq, c, -1), plan.epoch);
        return;
    }
    if (lane == 0) st_co<true>(plan.blk_seq + i, (static_cast<uint64_t>(plan.epoch) << 32) | static_cast<uint32_t>(b));
    for (int32_t e0 = 0; e0 < cnt; e0 += 64) {           // (uniform trip count: every lane shuffles)
        const int32_t e = e0 + lane;
        const int32_t j = e / nseg, sg = e - j * nseg;
        const bool tgt = j < nt;
        const int32_t ps = limit + (tgt ? j : j - nt);
        // the drafted token of position ps, from the lane that holds it
        const int32_t xs = __shfl(xtok, ps < 64 ? ps : 0, 64);
        if (e >= cnt) continue;
        const int64_t row = tgt ? o + b + ps : o + ps;
        const int32_t x = (!greedy && ps < k) ? xs : -1;
        store_entry(plan.sched + at + e, rest_item(b, static_cast<int32_t>(row), tgt ? kItemTarget : kItemDraft, sg, x),
                    plan.epoch);
    }
    int64_t q = at + cnt;
    if (i >= plan.lag_a) {
        if (lane == 0)
            store_entry(plan.sched + q, rest_item(static_cast<int32_t>(i - plan.lag_a), 0, kItemAccept, 0, -1),
                        plan.epoch);
        ++q;
    }
    if (i >= plan.lag_c)
        for (int32_t c = lane; c < nchunk; c += 64)
            store_entry(plan.sched + q + c, rest_item(static_cast<int32_t>(i - plan.lag_c), 0, kItemChunk, c, -1),
                        plan.epoch);
}

// Whether sequence b's offsets are in order with every other sequence's
// (reading R28): no earlier offset above o = offsets[b] and no later one
// (past b + 1) below o1 = offsets[b + 1].  Otherwise its range overlaps
// another sequence's, whose rows, uniforms and slots it would share.  Run
// by the whole wave (the offsets are read eight per lane at a time, so a
// batch of up to 511 sequences costs one round trip); the same in every
// lane.
__device__ __forceinline__ bool offsets_in_order(const Problem& p, int32_t b, int64_t o, int64_t o1) {
    if (!p.offsets) return true;
    constexpr int kU = 8;
    const int lane = threadIdx.x & 63;
    bool ok = true;
    for (int32_t j0 = 0; j0 <= p.B; j0 += 64 * kU) {
        int32_t v[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {             // (clamped: no load under a branch)
            const int32_t j = j0 + u * 64 + lane;
            v[u] = p.offsets[j <= p.B ? j : p.B];
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int32_t j = j0 + u * 64 + lane;
            if (j < b && v[u] > o) ok = false;
            if (j > b + 1 && j <= p.B && v[u] < o1) ok = false;
        }
    }
    return !__any(!ok);
}

// Accept scan of sequence b (0 <= b < B), run by every lane of one wave.
// kCo: the SegStats and captured logits come from other workgroups of the
// same launch, and the DrawTask goes to others.
//
// Early exit: only the rows of positions < limit have been read.  If their
// tests already decide the outcome (a rejection among them, or every
// position including the bonus row read) the scan writes everything and
// sets *done to kDecided, or to kDecidedEarlyDraw for a sampling sequence,
// whose draw chunks it then lists for the second round (list_rest);
// otherwise (the first rejection, if any, lies at or past limit) it writes
// nothing but *done = kUndecided, lists the rows still needed (list_rest)
// and runs again once they are read.  The scan stops at the first
// rejection, like the pages' loop over positions, so rows after it never
// influence the result.
// Diagnostics of rows that were not read are NaN.  Returns (the same in
// every lane) whether the scan settled the sequence with a draw still to
// make, i.e. wrote a DrawTask other than kNone.
//
// task_out (one pass only): also returns the DrawTask in every lane (kind
// kNone when there is nothing to draw).  emit = false: the scan writes
// nothing at all -- for workgroups that need the task of a sequence whose
// outputs another workgroup writes (the same scan over the same inputs
// gives the same task).  pre (sampling sequences outside the gathered form,
// rows of at most kPolledSegs segments, every position read): the rows'
// statistics already loaded, used instead of loading them again.
// check_order = false skips offsets_in_order for a sequence an earlier scan
// of the same call has already found in order (early exit's later scans).
template <bool kCo>
__device__ __forceinline__ bool accept_sequence(const Problem& p, const Plan& plan, int32_t b,
                                                int32_t limit = kKMax + 1, int32_t* done = nullptr,
                                                DrawTask* task_out = nullptr, bool emit = true,
                                                const Polled* pre = nullptr, bool check_order = true) {
    const int lane = threadIdx.x & 63;
    int64_t o, o1;
    if (p.offsets) { o = p.offsets[b]; o1 = p.offsets[b + 1]; }
    else { o = static_cast<int64_t>(b) * p.k_uniform; o1 = o + p.k_uniform; }
    const int64_t k64 = o1 - o;
    const float Tf = p.temperature[b];
    const int64_t ntarget = p.total + p.B;
    // (the order check, reading R28, comes after this lane's loads are
    // issued; its verdict joins ok before anything depends on it)
    bool ok = o >= 0 && k64 >= 0 && k64 <= kKMax && o1 <= p.total && temperature_ok(Tf);
    const int k = ok ? static_cast<int>(k64) : 0;
    const bool greedy = (Tf == 0.f);
    const bool gathered = p.draft_probs != nullptr;   // q_i(x_i) from the drafter
    const float c = greedy ? 0.f : row_scale(Tf);
    // Early exit beside the draws: the bonus row of a sampling sequence is
    // read by its draw alone, only when the bonus is drawn (kBonusSelf).
    const bool bonus_unread = plan.queued && !greedy && !gathered;
    const int64_t trow = o + b + lane;             // this lane's target row
    const int64_t drow = o + lane;                 // this lane's draft row

    // Every load this lane needs, issued together before any is used: the
    // indices are clamped into their arrays so that no load sits under a
    // branch (a value of a lane past k_b, or of a sequence found bad, is
    // never used).  Rows of at most kSegBatch segments have their segment
    // statistics loaded here too.
    const bool drafts = p.total > 0;               // (tokens and draft rows may be absent otherwise)
    const bool dstats = !greedy && !gathered && drafts;   // the draft rows' softmax enters the tests
    const int64_t trow_c = trow < 0 ? 0 : (trow >= ntarget ? ntarget - 1 : trow);
    const int64_t drow_c = drow < 0 ? 0 : (drow >= p.total ? p.total - 1 : drow);
    const int32_t x_ld = drafts ? p.tokens[drow_c] : -1;
    const float qg_ld = (gathered && drafts) ? p.draft_probs[drow_c] : NAN;
    const float u_ld = p.uniforms[trow_c];
    constexpr int kSegBatch = 4;
    const bool batched = !pre && plan.nseg <= kSegBatch;
    uint64_t th[kSegBatch] = {}, dh[kSegBatch] = {};
    double ts[kSegBatch] = {}, ds[kSegBatch] = {};
    float xt_ld = 0.f, xd_ld = 0.f;
    // (no draft rows in the call: the draft-side loads read the target row
    // again, so every address stays inside its array)
    const int64_t drow_all = drafts ? ntarget + drow_c : trow_c;   // index among all rows
    if (batched) {
        const SegStat* st = plan.seg + trow_c * plan.nseg;
        const SegStat* sd = plan.seg + drow_all * plan.nseg;
#pragma unroll
        for (int sg = 0; sg < kSegBatch; ++sg) {   // (segments past nseg reload the last one: unused)
            const int sgc = sg < plan.nseg ? sg : plan.nseg - 1;
            th[sg] = ld_co<kCo>(&st[sgc].head);
            ts[sg] = ld_co<kCo>(&st[sgc].s);
            dh[sg] = ld_co<kCo>(&sd[sgc].head);
            ds[sg] = ld_co<kCo>(&sd[sgc].s);
        }
    }
    if (!pre) {
        xt_ld = ld_co<kCo>(&plan.xlogit[trow_c]);
        xd_ld = ld_co<kCo>(&plan.xlogit[drow_all]);
    }

    int32_t x = -1;
    float qg = NAN;
    if (ok && lane < k) {
        x = x_ld;
        if (x < 0 || x >= p.V) ok = false;
        if (gathered && !greedy) {
            qg = qg_ld;
            if (!(qg > 0.f && qg <= 1.f)) ok = false;   // not a probability x could be drawn with
        }
    }
    RowStat rt{0.f, 0, 0.f, 1.0}, rd{0.f, 0, 0.f, 1.0};
    const bool read = lane < limit;                // this position's rows have been read
    const bool tread = read && !(bonus_unread && lane == k);   // ... and its target row
    bool row_bad = false;                          // a row of this position has a non-finite maximum
    if (ok && lane <= k && tread) {
        if (pre || batched) {
            rt = RowStat{-INFINITY, INT32_MAX, -INFINITY, 0.0};
#pragma unroll
            for (int sg = 0; sg < kSegBatch; ++sg) {
                if (sg >= plan.nseg || (pre && sg >= kPolledSegs)) break;
                merge_seg(rt, pre ? pre->th[sg] : th[sg], greedy ? 0.0 : (pre ? pre->ts[sg] : ts[sg]), greedy);
            }
        } else {
            rt = merge_row<kCo>(plan.seg + trow * plan.nseg, plan.nseg, greedy);
        }
        row_bad = !(fabsf(rt.m) <= 3.4e38f);
        if (!greedy && !gathered && lane < k) {
            if (pre || batched) {
                rd = RowStat{-INFINITY, INT32_MAX, -INFINITY, 0.0};
#pragma unroll
                for (int sg = 0; sg < kSegBatch; ++sg) {
                    if (sg >= plan.nseg || (pre && sg >= kPolledSegs)) break;
                    merge_seg(rd, pre ? pre->dh[sg] : dh[sg], pre ? pre->ds[sg] : ds[sg], false);
                }
            } else {
                rd = merge_row<kCo>(plan.seg + (ntarget + drow) * plan.nseg, plan.nseg, false);
            }
            row_bad = row_bad || !(fabsf(rd.m) <= 3.4e38f);
        }
    }
    if (check_order && !offsets_in_order(p, b, o, o1)) ok = false;
    ok = !__any(!ok);                              // one verdict for the whole sequence

    // Data error: the sequence's own token slots (when its offsets describe
    // a range inside the batch) are all -1.
    auto data_error = [&]() {
        if (task_out) task_out->kind = kNone;
        if (!emit) return;
        if (o >= 0 && o1 >= o && o1 <= p.total)
            for (int64_t i = lane; i <= k64; i += 64) p.out_tokens[o + b + i] = -1;
        if (lane == 0) {
            p.out_n[b] = -1;
            if (p.out_emit_prob) p.out_emit_prob[b] = NAN;
            store_no_task<kCo>(plan, b);
            if (done) *done = kDecided;
        }
    };
    if (!ok) {
        data_error();
        return false;
    }

    const float u_draw = __shfl(u_ld, k, 64);     // slot k_b: the draw uniform (k <= 63)
    bool reject = false;
    double px = NAN, qx = NAN;
    if (lane < k && read) {
        if (greedy) {
            reject = (x != rt.arg);
        } else {
            const double zt = pre ? pre->xt : xt_ld;   // captured by the row pass
            px = exp2(zt * c - rt.R) / rt.S;
            if (gathered) {
                qx = qg;
            } else {
                const double zd = pre ? pre->xd : xd_ld;
                qx = exp2(zd * c - rd.R) / rd.S;
            }
            const double alpha = fmin(1.0, px / qx);
            reject = !(static_cast<double>(u_ld) < alpha);
        }
    }
    // A row with a non-finite maximum ends the scan where it stands, like a
    // rejection, and makes the sequence a data error if the scan gets there
    // (rows past the first rejection are never looked at).
    const uint64_t bad = __ballot(row_bad);
    const uint64_t mask = __ballot(reject) | bad;
    if (!mask && (bonus_unread ? k > limit : k >= limit)) {   // undecided: rows past limit are needed
        if (done) {
            if (lane == 0) *done = kUndecided;
            list_rest(p, plan, b, o, k, limit, greedy || gathered, greedy, bonus_unread, x, false);
        }
        return false;
    }
    const int n = mask ? __ffsll(static_cast<unsigned long long>(mask)) - 1 : k;
    if ((bad >> n) & 1ull) {
        data_error();
        return false;
    }
    // Settled by its leading positions: a sampling sequence draws in the
    // second round, beside the remaining rows (not in the gathered form,
    // whose second round only streams rows); it is listed below, once its
    // task is written.
    const bool early_draw = done && !greedy && !gathered;
    if (done && lane == n) *done = early_draw ? kDecidedEarlyDraw : kDecided;
    const uint64_t reserved = early_draw ? list_reserve(plan, true, plan.nchunk) : ~0ull;

    const int32_t kind = greedy ? kNone : (n < k ? kResidual : (bonus_unread ? kBonusSelf : kBonus));
    if (task_out) {
        // (gathered form excluded: its residual needs the draft row read later)
        DrawTask& t = *task_out;
        t.kind = kind;
        t.out_slot = static_cast<int32_t>(o + b + n);
        t.trow = o + b + n;
        t.drow = o + n;
        t.m_t = __shfl(rt.m, n, 64);
        t.m_d = n < k ? __shfl(rd.m, n, 64) : 0.f;
        t.T = Tf;
        t.u = u_draw;
        const double th = (!greedy && n < k) ? log2_norm(rt, c) - log2_norm(rd, c) : 0.0;
        t.theta = __shfl(th, n, 64);
    }
    if (!emit) return !greedy;

    // Slot n of a sampling sequence is written by the draw alone: in the
    // one-launch forms the draw runs in another workgroup, possibly on another XCD,
    // and two plain stores to one slot from different L2s would land in the
    // order the caches happen to write back.
    if (lane <= k && (lane != n || greedy)) p.out_tokens[trow] = lane < n ? x : (lane == n ? rt.arg : -1);
    if (lane == n) {
        p.out_n[b] = n;
        if (greedy && p.out_emit_prob) p.out_emit_prob[b] = 1.f;   // the T -> 0 limit: a point mass
        // Gathered form: draft row n has not been read; list it, and leave
        // log2 S_p in theta until its statistics resolve the task.
        const bool pending = gathered && !greedy && n < k;
        if (pending) {
            const uint32_t base = atomicAdd(plan.dlist_n, static_cast<uint32_t>(plan.nseg));
            for (int32_t sg = 0; sg < plan.nseg; ++sg) {
                plan.dlist[base + sg] = rest_item(b, static_cast<int32_t>(drow), kItemDraft, sg, -1);
            }
        }
        store_task<kCo>(plan, b, greedy ? kNone : (n < k ? (pending ? kResidualPending : kResidual) : kind), trow,
                        drow, rt.m, n < k ? rd.m : 0.f, Tf, u_draw,
                        (!greedy && n < k) ? log2_norm(rt, c) - (pending ? 0.0 : log2_norm(rd, c)) : 0.0);
    }
    if (early_draw) list_rest(p, plan, b, o, k, limit, true, greedy, bonus_unread, x, true, reserved);
    if (p.out_p && lane < k) {
        p.out_p[drow] = static_cast<float>(px);
        p.out_q[drow] = static_cast<float>(qx);
    }
    if (p.out_row_max && lane <= k) {
        const bool dread = read && !greedy && !gathered;
        p.out_row_max[trow] = tread ? rt.m : NAN;
        p.out_row_sum[trow] = (greedy || !tread) ? NAN : static_cast<float>(exp2(log2_norm(rt, c)));
        if (lane < k) {
            p.out_row_max[ntarget + drow] = dread ? rd.m : NAN;
            p.out_row_sum[ntarget + drow] = dread ? static_cast<float>(exp2(log2_norm(rd, c))) : NAN;
        }
    }
    return !greedy;
}

// The DrawTask of sequence b as written by accept_sequence (store_task); a
// pending residual of the gathered form is completed from its draft row's
// SegStats (read after the accept scan): its maximum, and theta = log2 S_p -
// log2 S_q.  kind = kTaskUnset when the record is not (yet) this call's: a
// word still carries another call's epoch.  kCo: the task comes from another
// workgroup of the same launch; an ordinary load is tried first (a record
// this XCD has not cached since it was written comes back current) unless
// kPlainFirst is false, then one written-through load.
template <bool kCo>
__device__ __forceinline__ bool fetch_task(const TaskRec* t, uint32_t epoch, uint64_t* w) {
#pragma unroll
    for (int i = 0; i < 9; ++i) w[i] = ld_co<kCo>(&t->w[i]);
    bool cur = true;
#pragma unroll
    for (int i = 0; i < 9; ++i) cur = cur && static_cast<uint32_t>(w[i] >> 32) == epoch;
    return cur;
}
template <bool kCo, bool kPlainFirst = true>
__device__ __forceinline__ DrawTask load_task(const Problem& p, const Plan& plan, int32_t b) {
    const TaskRec* t = plan.task + b;
    uint64_t w[9];
    bool cur = false;
    if constexpr (kPlainFirst || !kCo) cur = fetch_task<false>(t, plan.epoch, w);
    if constexpr (kCo) {
        if (!cur) cur = fetch_task<true>(t, plan.epoch, w);
    }
    DrawTask r;
    auto lo = [&](int i) { return static_cast<uint32_t>(w[i]); };
    r.kind = cur ? static_cast<int32_t>(lo(0)) : static_cast<int32_t>(kTaskUnset);
    r.trow = lo(1);
    r.out_slot = static_cast<int32_t>(lo(1));
    r.drow = lo(2);
    r.m_t = __uint_as_float(lo(3));
    r.m_d = __uint_as_float(lo(4));
    r.T = __uint_as_float(lo(5));
    r.u = __uint_as_float(lo(6));
    r.theta = __hiloint2double(static_cast<int>(lo(8)), static_cast<int>(lo(7)));
    if (r.kind == kResidualPending) {
        const RowStat rd = merge_row<kCo>(plan.seg + (p.total + p.B + r.drow) * plan.nseg, plan.nseg, false);
        r.m_d = rd.m;
        r.theta -= log2_norm(rd, row_scale(r.T));
        r.kind = kResidual;
    }
    return r;
}

}  // namespace sv
