// sv_internal.h -- declarations shared by the HIP sources of libspecverify.
//
// Data flow of one call, staged form (every kernel is enqueued on the
// caller's stream; kernel boundaries publish each step's results).  One pass
// (Plan::lead == 0):
//   1. row pass    (row_stats.hip, row_pass.h): one workgroup per (logit row,
//                  segment) streams the segment once and writes a SegStat;
//   2. accept scan (accept.hip, accept_scan.h): one wave64 per sequence
//                  merges the segments of its rows, runs the k accept tests,
//                  finds the first rejection, writes the accepted tokens and
//                  a DrawTask;
//   3. draw_sums   (draw.hip, draw_pass.h): one workgroup per (sequence,
//                  chunk) of the one rejected or bonus row pair accumulates
//                  fp64 chunk sums;
//   4. draw_pick   (draw.hip, draw_pass.h): one workgroup per sequence
//                  locates the chunk that holds u * Z and the token inside it.
// Early exit (Plan::lead > 0): one launch (second_round.hip) runs two
// rounds.  Its first workgroups read the leading positions of every
// sequence (lead_pass.h), and the sequence's last workgroup (or, with more
// leading positions or segments, the one that completes its count of
// arrivals) runs its accept scan, which settles the sequence or lists
// its remaining rows; the later workgroups take the listed items in order:
// those rows, the undecided sequences' accept scans and every draw chunk.
// Then draw_pick picks.  The gathered form runs the first round as its own
// launch (row_lead), streams the listed rows (sched_rows), then runs steps
// 2-4 with the draft rows at rejections read in between (row_list).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/specverify.h"
#include "sv_layout.h"
#include "sv_tuning.h"

namespace sv {

// (constants, workspace records: sv_layout.h)

__device__ __forceinline__ uint64_t seg_head(float m, uint32_t hi) {
    return static_cast<uint64_t>(__float_as_uint(m)) | (static_cast<uint64_t>(hi) << 32);
}
__device__ __forceinline__ float head_m(uint64_t h) { return __uint_as_float(static_cast<uint32_t>(h)); }
__device__ __forceinline__ uint32_t head_hi(uint64_t h) { return static_cast<uint32_t>(h >> 32); }

__device__ __forceinline__ RestItem rest_item(int32_t b, int32_t row, int32_t kind, int32_t seg, int32_t x) {
    return RestItem{b, row, (kind << 28) | seg, x};
}
__device__ __forceinline__ int32_t item_kind(const RestItem& it) { return it.kseg >> 28; }
__device__ __forceinline__ int32_t item_seg(const RestItem& it) { return it.kseg & 0x0FFFFFFF; }

// The caller's arguments, passed by value to every kernel.
struct Problem {
    const void* target;
    const void* draft;
    const int32_t* tokens;
    const int32_t* offsets;   // nullptr => k_uniform
    const float* uniforms;
    const float* temperature;
    int32_t* out_tokens;
    int32_t* out_n;
    float* out_p;             // diagnostics, may be nullptr
    float* out_q;
    float* out_row_max;
    float* out_row_sum;
    const float* draft_probs; // gathered form: [total] q_i(x_i) from the drafter (nullptr otherwise)
    float* out_emit_prob;     // [B] probability of the emitted token under its draw, may be nullptr
    int64_t V;
    int64_t total;            // total drafted tokens = offsets[B]
    int32_t B;
    int32_t k_uniform;
    int32_t dtype;            // SV_F32 / SV_BF16
};

// Work decomposition and workspace pointers of one call.
struct Plan {
    int32_t nseg;        // segments per logit row in the row pass
    int64_t seg_len;     // elements per segment (multiple of 8)
    int32_t nchunk;      // chunks per row in the draw
    int64_t chunk_len;   // elements per chunk (multiple of 8)
    SegStat* seg;        // [(2 * total + B) * nseg]; target rows first
    TaskRec* task;       // [B]
    ChunkSums* csum;     // [B * nchunk * kWaves]: one per sub-chunk (wave) of each chunk
    int32_t* band_n;     // [B * nchunk * kWaves]: band tokens seen per sub-chunk (wave) of a chunk
    double* band_w;      // [B * nchunk * kWaves * kWaveCap * 2]: their (w_t, w_d)
    float* xlogit;       // [2 * total + B]: logit of the drafted token of each row
    int32_t lead;        // early exit: positions every sequence reads first (0: one pass over all rows)
    int64_t lead_mul;    // early exit: the first round's j-th sequence is (j * lead_mul) mod B
    int32_t* done;       // early exit: [B], kUndecided / kDecided / kDecidedEarlyDraw after the lead scan
    SchedEntry* sched;   // early exit: [(2 * total + B) * nseg + B * (1 + nchunk)], the second round's items
    uint64_t* blk_ctr;   // early exit: (undecided sequences listed) << 32 | (row segments listed)
    RestItem* dlist;     // gathered form: [B * nseg], segments of the draft rows at rejections
    uint32_t* dlist_n;   // gathered form: number of entries in dlist
    uint64_t* blk_seq;   // early exit: [B] epoch << 32 | the undecided sequence listed as block i
    int32_t lag_a, lag_c;// early exit: the accept item of block j follows block j + lag_a, its chunks
                         // follow block j + lag_c (huge: none inserted, the gathered form)
    int32_t* aband;      // [B] 1: sequence b is left to the pick launch
    uint32_t* picked;    // one pass, single draw launch: [B] chunks of sequence b summed so far
    int32_t queued;      // early exit with the draws beside the rows (not the gathered form)
    int32_t cus;         // compute units of the device
    int32_t queue_mode;  // SV_QUEUE_*: where the second round's draw chunks are summed
    uint32_t epoch;      // this call's number (never 0): tags the counters below; set on the
                         // device by each kernel (begin_epoch / call_epoch), not by the host
    uint32_t* epoch_ctr; // [2] at the workspace's start: the calls counter, this call's epoch
    uint64_t* lead_ctr;  // early exit without records: [B] leading segments of sequence b finished
                         // (cleared before lead_clr is published)
    uint32_t* lead_clr;  // early exit: the epoch of the call whose first round has cleared the list counters
    uint64_t* lead_done; // early exit: epoch << 32 | sequences whose leading accept scan has finished
                         // (set to epoch << 32 before lead_clr is published)
    LeadRec* lead_rec;   // early exit, lead 1, nseg <= kPolledSegs: [B][2][nseg] first-round records
    uint32_t lead_pace;  // early exit: 100 MHz ticks the first round's second half waits before streaming (0: none)
    uint32_t* stall;     // early exit: the epoch of a call whose second round could not find an item's work
    uint32_t item_polls; // early exit: bound of a second-round workgroup's wait for its item
};


// Plan::done values (early exit).  kDecidedEarlyDraw: settled with a draw
// that the second round makes.
enum : int32_t { kUndecided = 0, kDecided = 1, kDecidedEarlyDraw = 2 };

// Host-side launchers (one per kernel).
hipError_t launch_row_stats(const Problem& p, const Plan& plan, hipStream_t s);
hipError_t launch_row_list(const Problem& p, const Plan& plan, const RestItem* list, const uint32_t* count,
                           int64_t max_items, hipStream_t s);
hipError_t launch_sched_rows(const Problem& p, const Plan& plan, const uint32_t* count, int64_t max_items,
                             hipStream_t s);
hipError_t launch_rounds(const Problem& p, const Plan& plan, hipStream_t s);
hipError_t launch_row_lead(const Problem& p, const Plan& plan, hipStream_t s);
hipError_t launch_accept(const Problem& p, const Plan& plan, hipStream_t s);
hipError_t launch_draw_sums(const Problem& p, const Plan& plan, hipStream_t s);
hipError_t launch_draw_pick(const Problem& p, const Plan& plan, hipStream_t s);
hipError_t launch_draw_all(const Problem& p, const Plan& plan, hipStream_t s);
hipError_t launch_sample_sums(const Problem& p, const Plan& plan, hipStream_t s);
hipError_t launch_sample_pick(const Problem& p, const Plan& plan, hipStream_t s);
// Workgroups of the two-round launch one compute unit holds at once
// (occupancy query).
hipError_t rounds_blocks_per_cu(int32_t dtype, int32_t* blocks);

hipError_t launch_commit(const int32_t* out_tokens, const int32_t* out_n, const int32_t* offsets,
                         int32_t k_uniform, int32_t B, int32_t* seq_tokens, int32_t* seq_len,
                         int32_t max_len, int32_t* committed, int32_t* committed_offsets, hipStream_t s);
hipError_t launch_adapt_k(const int32_t* out_n, const int32_t* offsets, int32_t k_uniform, int32_t B,
                          int32_t min_k, int32_t max_k, double* history, int32_t* rounds, int32_t* k,
                          hipStream_t s);
hipError_t launch_ngram_draft(const int32_t* seq_tokens, const int32_t* seq_len, int32_t B, int32_t max_len,
                              int32_t ngram_max, int32_t ngram_min, int32_t k_max, int32_t* cont_start,
                              int32_t* draft_tokens, int32_t* draft_offsets, hipStream_t s);
hipError_t launch_stream_probe(const void* data, int64_t bytes, int64_t seg_bytes, uint32_t* out,
                               hipStream_t s);

// ---- device helpers shared by the kernels ---------------------------------

__device__ __forceinline__ float load_logit(const void* base, int32_t dtype, int64_t idx) {
    if (dtype == SV_BF16)
        return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(base)[idx]) << 16);
    return static_cast<const float*>(base)[idx];
}

// Data handed between workgroups of ONE launch (early exit's second round,
// the one-launch draw).  The L2 of each XCD is not coherent with the others
// for ordinary accesses, so such data is stored and loaded with agent-scope
// relaxed atomics (global_store / global_load with sc1: written through to,
// and read from, the point where all XCDs agree).  kCo = false gives
// ordinary accesses where a kernel boundary publishes the data.
template <bool kCo, class T>
__device__ __forceinline__ T ld_co(const T* ptr) {
    if constexpr (kCo) return __hip_atomic_load(ptr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else return *ptr;
}
template <bool kCo, class T>
__device__ __forceinline__ void st_co(T* ptr, T v) {
    if constexpr (kCo) __hip_atomic_store(ptr, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else *ptr = v;
}

// Waits until every global store this thread has issued has completed
// (s_waitcnt vmcnt(0): on gfx9-family GPUs vmcnt also counts stores, and a
// write-through store completes once it is visible at agent scope).  The
// signal fences keep the compiler from moving memory operations across it.
// Used before a counter increment that hands the stored data to another
// workgroup; cheaper than an agent-scope release fence, which would also
// write back the whole L2.
__device__ __forceinline__ void wait_stores() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0), expcnt and lgkmcnt unchanged
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// The call's epoch comes from device memory, so that a call replayed from a
// captured graph (the same kernel arguments every time) still gets a number
// of its own.  The call's first kernel takes the workspace's counter plus
// one (never 0) in every workgroup -- no kernel of the call writes the
// counter while the first one runs -- and workgroup 0 publishes it in
// epoch_ctr[1]; the call's later kernels read it back there, and their
// workgroup 0 advances the counter to it for the next call.  Kept at the
// workspace's start, the counter survives calls of other sizes.
__device__ __forceinline__ uint32_t begin_epoch(const Plan& plan) {
    uint32_t e = plan.epoch_ctr[0] + 1u;
    if (e == 0u) e = 1u;
    if (blockIdx.x == 0 && threadIdx.x == 0) plan.epoch_ctr[1] = e;
    return e;
}
__device__ __forceinline__ uint32_t call_epoch(const Plan& plan) {
    const uint32_t e = plan.epoch_ctr[1];
    if (blockIdx.x == 0 && threadIdx.x == 0) plan.epoch_ctr[0] = e;
    return e;
}

// Early exit's schedule entries (SchedEntry): written through, one word at a
// time, by a lister whose earlier stores (what the item needs) are already
// visible; read with the epoch checked on every word.
__device__ __forceinline__ void store_entry(SchedEntry* dst, const RestItem& it, uint32_t epoch) {
    const uint64_t e = static_cast<uint64_t>(epoch) << 32;
    st_co<true>(&dst->w[0], e | static_cast<uint32_t>(it.b));
    st_co<true>(&dst->w[1], e | static_cast<uint32_t>(it.row));
    st_co<true>(&dst->w[2], e | static_cast<uint32_t>(it.kseg));
    st_co<true>(&dst->w[3], e | static_cast<uint32_t>(it.x));
}
// True when every word of the entry carries `epoch`; *it gets the fields.
template <bool kCo>
__device__ __forceinline__ bool load_entry(const SchedEntry* src, uint32_t epoch, RestItem* it) {
    const uint64_t w0 = ld_co<kCo>(&src->w[0]), w1 = ld_co<kCo>(&src->w[1]);
    const uint64_t w2 = ld_co<kCo>(&src->w[2]), w3 = ld_co<kCo>(&src->w[3]);
    *it = RestItem{static_cast<int32_t>(static_cast<uint32_t>(w0)), static_cast<int32_t>(static_cast<uint32_t>(w1)),
                   static_cast<int32_t>(static_cast<uint32_t>(w2)), static_cast<int32_t>(static_cast<uint32_t>(w3))};
    return static_cast<uint32_t>(w0 >> 32) == epoch && static_cast<uint32_t>(w1 >> 32) == epoch &&
           static_cast<uint32_t>(w2 >> 32) == epoch && static_cast<uint32_t>(w3 >> 32) == epoch;
}

// Sequence b's DrawTask record (TaskRec): every word carries the call's
// epoch, so the stores need no order among themselves (kCo: written through,
// for workgroups of the same launch).
template <bool kCo>
__device__ __forceinline__ void store_task(const Plan& plan, int32_t b, int32_t kind, int64_t trow, int64_t drow,
                                           float m_t, float m_d, float T, float u, double theta) {
    TaskRec* r = plan.task + b;
    const uint64_t e = static_cast<uint64_t>(plan.epoch) << 32;
    st_co<kCo>(&r->w[1], e | static_cast<uint32_t>(trow));
    st_co<kCo>(&r->w[2], e | static_cast<uint32_t>(drow));
    st_co<kCo>(&r->w[3], e | __float_as_uint(m_t));
    st_co<kCo>(&r->w[4], e | __float_as_uint(m_d));
    st_co<kCo>(&r->w[5], e | __float_as_uint(T));
    st_co<kCo>(&r->w[6], e | __float_as_uint(u));
    st_co<kCo>(&r->w[7], e | static_cast<uint32_t>(__double2loint(theta)));
    st_co<kCo>(&r->w[8], e | static_cast<uint32_t>(__double2hiint(theta)));
    st_co<kCo>(&r->w[0], e | static_cast<uint32_t>(kind));
}
// A task that draws nothing (greedy, or a data error).
// A first-round workgroup's LeadRec (written through).
__device__ __forceinline__ void store_lead_rec(LeadRec* r, uint32_t epoch, uint64_t head, double s, float x) {
    const uint64_t e = static_cast<uint64_t>(epoch) << 32;
    st_co<true>(&r->w[0], e | static_cast<uint32_t>(head));
    st_co<true>(&r->w[1], e | static_cast<uint32_t>(head >> 32));
    st_co<true>(&r->w[2], e | static_cast<uint32_t>(__double2loint(s)));
    st_co<true>(&r->w[3], e | static_cast<uint32_t>(__double2hiint(s)));
    st_co<true>(&r->w[4], e | __float_as_uint(x));
}

template <bool kCo>
__device__ __forceinline__ void store_no_task(const Plan& plan, int32_t b) {
    store_task<kCo>(plan, b, kNone, 0, 0, 0.f, 0.f, 0.f, 0.f, 0.0);
}

// c = log2(e) / T as the row pass uses it (the accept scan must form the same
// float).  Capped at 2^60: beyond that every non-maximal term underflows.
__device__ __forceinline__ float row_scale(float T) {
    return static_cast<float>(fmin(1.4426950408889634 / static_cast<double>(T), 0x1p60));
}

// First drafted slot of sequence b (offsets, or k_uniform per sequence).
__device__ __forceinline__ int64_t first_slot(const Problem& p, int32_t b) {
    return p.offsets ? static_cast<int64_t>(p.offsets[b]) : static_cast<int64_t>(b) * p.k_uniform;
}

// Sequence owning target row r: the largest b with first_draft(b) + b <= r.
__device__ __forceinline__ int32_t seq_of_target_row(const Problem& p, int64_t r) {
    if (!p.offsets) return static_cast<int32_t>(r / (p.k_uniform + 1));
    int32_t lo = 0, hi = p.B - 1;
    while (lo < hi) {
        const int32_t mid = (lo + hi + 1) >> 1;
        if (static_cast<int64_t>(p.offsets[mid]) + mid <= r) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// Sequence owning draft row r: the largest b with first_draft(b) <= r.
__device__ __forceinline__ int32_t seq_of_draft_row(const Problem& p, int64_t r) {
    if (!p.offsets) return static_cast<int32_t>(r / p.k_uniform);
    int32_t lo = 0, hi = p.B - 1;
    while (lo < hi) {
        const int32_t mid = (lo + hi + 1) >> 1;
        if (static_cast<int64_t>(p.offsets[mid]) <= r) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// Temperature usable: T == 0 is greedy, T > 0 finite is sampling.
__device__ __forceinline__ bool temperature_ok(float T) { return T >= 0.f && T <= 3.4e38f; }

// Sum of a double over the workgroup; the result is valid in every thread.
__device__ __forceinline__ double block_sum(double x, double* lds /* [kWaves] */) {
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
    const int wave = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) lds[wave] = x;
    __syncthreads();
    double t = 0.0;
    for (int w = 0; w < kWaves; ++w) t += lds[w];
    return t;
}

}  // namespace sv
