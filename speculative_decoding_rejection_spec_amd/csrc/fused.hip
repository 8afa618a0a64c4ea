// fused.hip -- the whole verify step in one persistent launch.
//
// The staged form runs a kernel per step back to back; the draw (fp64, bound by
// vector ALU) then waits for the end of the row pass (bound by HBM), and
// each kernel boundary drains the GPU.  Here one grid of resident
// workgroups takes work items from a device-side queue in a fixed order:
//
//   super-step s = 0 .. B+L-1:  the row segments of sequence s (s < B),
//                               then the draw chunks of sequence s-L (s >= L)
//
// A row item streams one segment of one row (row_pass.h).  The workgroup
// that completes the last row item of a sequence runs that sequence's
// accept scan (accept_scan.h) and marks it ready.  A draw item waits until
// its sequence is ready (it almost never waits: its rows were queued L
// super-steps earlier), accumulates one chunk (draw_pass.h), and the
// workgroup that completes the last chunk of a sequence runs its pick.  So
// the fp64 draws of earlier sequences can run on the vector ALUs while later
// sequences' rows stream from HBM.
//
// Measured on MI355X (B=256, k=8, V=152064 bf16) this form is SLOWER than
// the staged one (0.32-0.49 ms per step against 0.27 ms), so it runs only
// when asked for (spec_verify_set_mode).  Two effects dominate: the draw and
// pick parts need about 120 VGPRs, which halves the resident workgroups
// (4 per CU against the row pass's 8) and with them the loads in flight;
// and every item costs a few microseconds of serial round trips (claim,
// store completion, counter) that a persistent workgroup cannot hide
// behind others.  Interleaving draws with rows made it slower still: a
// workgroup busy with fp64 arithmetic issues no loads.
//
// Every wait ends: items are claimed in increasing order, a draw item only
// waits for row items of its own sequence, which precede it in the queue,
// were claimed by running workgroups and never wait themselves.  The waits
// are nevertheless bounded; on expiry the launch is abandoned (every
// workgroup stops claiming work) rather than allowed to hang.
//
// Data handed between workgroups of the launch (segment statistics, the
// captured logits, draw tasks, chunk sums, band lists) is written with
// write-through stores and read with loads that bypass the per-XCD L2
// (ld_co / st_co); each writer waits for its stores to complete before the
// counter increment that hands them on (wait_stores).  Outputs are ordinary
// stores written back at the end of the launch, so every output element has
// exactly one writer in the launch (the emitted token of a sampling sequence
// is written by its pick alone, never also by its accept scan).
#include "draw_pass.h"
#include "row_pass.h"

namespace sv {
namespace {

constexpr uint32_t kSpinLimit = 1u << 16;   // waits of ~1-2 us each before abandoning
// At least 4 waves per SIMD: every part then fits 128 VGPRs.
constexpr int kFusedWavesPerEU = 4;

struct FusedLds {
    int32_t E[kFusedMaxB + 1];               // E[b]: drafted rows scheduled before sequence b
    drawpass::TabEntry tbl[256];
    union {
        RowLds row;
        DrawLds draw;
        PickLds<kThreads, kFusedMaxChunks * kWaves> pick;
    } u;
    int32_t scan[kWaves];
    uint32_t item;
    int32_t flag;
};

// Whether the offsets of sequence b describe a usable range of the batch.
__device__ __forceinline__ bool range_ok(const Problem& p, int32_t b) {
    if (!p.offsets) return true;
    const int64_t o = p.offsets[b], o1 = p.offsets[b + 1];
    return o >= 0 && o1 >= o && o1 - o <= kKMax && o1 <= p.total;
}

// Drafted positions scheduled for sequence b (2 k + 1 row items per
// segment): k_b when its range is usable, otherwise 0 (the sequence is then
// reported as a data error by its accept scan and reads nothing).
__device__ __forceinline__ int32_t sched_k(const Problem& p, int32_t b) {
    if (!p.offsets) return p.k_uniform;
    return range_ok(p, b) ? p.offsets[b + 1] - p.offsets[b] : 0;
}

// First item of super-step s (0 <= s <= B + lag).
__device__ __forceinline__ int64_t step_start(const int32_t* E, int32_t lag, int32_t B, int64_t nseg,
                                              int64_t nchunk, int32_t s) {
    const int32_t m = min(s, B);
    const int32_t d = min(max(s - lag, 0), B);
    return nseg * (2 * static_cast<int64_t>(E[m]) + m) + nchunk * d;
}

// The four kinds of work, each compiled as a function of its own so that
// every part gets its own register allocation within the kernel's budget:
// inlined into one loop body they need more than 200 VGPRs between them.
// (Inlining the row part alone, with a 16-deep load window to make up for
// the halved occupancy, measured slower.)
template <int DT>
__device__ __noinline__ void do_row(const Problem& p, const Plan& plan, int32_t b, bool is_target, int64_t r,
                                    int64_t seg, RowLds& lds) {
    row_segment<DT, true>(p, plan, b, is_target, r, seg, lds);
}
__device__ __noinline__ void do_accept(const Problem& p, const Plan& plan, int32_t b) {
    accept_sequence<true>(p, plan, b);
}
template <int DT>
__device__ __noinline__ void do_chunk(const Problem& p, const Plan& plan, const DrawTask& task, int32_t b,
                                      int32_t c, const drawpass::TabEntry* tbl, DrawLds& lds) {
    draw_chunk<DT, true>(p, plan, task, b, c, tbl, lds);
}
template <int DT>
__device__ __noinline__ void do_pick(const Problem& p, const Plan& plan, const DrawTask& task, int32_t b,
                                     const drawpass::TabEntry* tbl, PickLds<kThreads, kFusedMaxChunks * kWaves>& lds) {
    pick_sequence<DT, kThreads, true, kFusedMaxChunks * kWaves>(p, plan, task, b, tbl, lds, pick_prefetch<true>(plan, b));
}

template <int DT>
__global__ __launch_bounds__(kThreads, kFusedWavesPerEU) void fused_kernel(Problem p, Plan plan, Fused f) {
    __shared__ FusedLds L;
    const int tid = threadIdx.x;
    const int32_t B = p.B;
    const int64_t nseg = plan.nseg;
    uint32_t* const queue = plan.ctr + kCtrQueue;
    uint32_t* const rows_done = plan.ctr + kCtrHeader;
    uint32_t* const ready = rows_done + B;
    uint32_t* const chunks_done = ready + B;

    // Prologue: the exp2 table and the schedule prefix E (a workgroup-wide
    // exclusive scan of sched_k, kFusedMaxB / kThreads entries per thread).
    load_exp2_table(L.tbl, kThreads);
    {
        constexpr int kPer = kFusedMaxB / kThreads;
        int32_t v[kPer];
        int32_t sum = 0;
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int32_t b = tid * kPer + i;
            v[i] = b < B ? sched_k(p, b) : 0;
            sum += v[i];
        }
        int32_t inc = sum;
        for (int off = 1; off < 64; off <<= 1) {
            const int32_t y = __shfl_up(inc, off, 64);
            if ((tid & 63) >= off) inc += y;
        }
        if ((tid & 63) == 63) L.scan[tid >> 6] = inc;
        __syncthreads();
        int32_t run = inc - sum;
        for (int w = 0; w < (tid >> 6); ++w) run += L.scan[w];
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int32_t b = tid * kPer + i;
            if (b <= B) L.E[b] = run;
            run += v[i];
        }
        if (tid == kThreads - 1 && B == kFusedMaxB) L.E[B] = run;   // no thread owns b = kFusedMaxB
    }
    __syncthreads();

    const int32_t nsteps = B + f.lag;
    const int64_t nchunk = plan.nchunk;
    const int64_t nitems = step_start(L.E, f.lag, B, nseg, nchunk, nsteps);
    // Claims run one item ahead: the claim of the next item is issued when
    // the current one starts, so its round trip overlaps the current work.
    // (A workgroup then holds at most one item it has not started; claims
    // stay in increasing order, so the argument above still holds.)  An
    // abandoned launch hands out items past the end.
    uint32_t next = 0;
    if (tid == 0) next = __hip_atomic_fetch_add(queue, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (;;) {
        __syncthreads();                      // every thread is done with the previous item and its LDS
        if (tid == 0) {
            L.item = next;
            next = __hip_atomic_fetch_add(queue, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
        const int64_t w = L.item;
        if (w >= nitems) break;

        // Super-step of item w: the largest s with step_start(s) <= w.
        int32_t lo = 0, hi = nsteps - 1;
        while (lo < hi) {
            const int32_t mid = (lo + hi + 1) >> 1;
            if (step_start(L.E, f.lag, B, nseg, nchunk, mid) <= w) lo = mid; else hi = mid - 1;
        }
        const int32_t s = lo;
        const int64_t off = w - step_start(L.E, f.lag, B, nseg, nchunk, s);
        const int32_t ks = s < B ? L.E[s + 1] - L.E[s] : 0;
        const int64_t rows_s = s < B ? nseg * (2 * static_cast<int64_t>(ks) + 1) : 0;

        if (off < rows_s) {
            // ---- row item: segment off % nseg of row off / nseg of sequence s
            const int32_t b = s;
            const int64_t j = off / nseg, seg = off - j * nseg;
            const int64_t o = p.offsets ? static_cast<int64_t>(p.offsets[b]) : static_cast<int64_t>(b) * p.k_uniform;
            if (range_ok(p, b)) {
                if (j <= ks) do_row<DT>(p, plan, b, true, o + b + j, seg, L.u.row);
                else do_row<DT>(p, plan, b, false, o + (j - ks - 1), seg, L.u.row);
            }
            wait_stores();
            __syncthreads();
            if (tid == 0) {
                const uint32_t done = __hip_atomic_fetch_add(rows_done + b, 1u, __ATOMIC_RELAXED,
                                                             __HIP_MEMORY_SCOPE_AGENT);
                L.flag = (done + 1 == static_cast<uint32_t>(rows_s));
            }
            __syncthreads();
            if (L.flag && tid < 64) {
                do_accept(p, plan, b);
                wait_stores();
                if (tid == 0) __hip_atomic_store(ready + b, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        } else {
            // ---- draw item: chunk c of sequence b
            const int32_t b = s - f.lag;
            const int32_t c = static_cast<int32_t>(off - rows_s);
            const float T = p.temperature[b];
            if (!(T > 0.f && T <= 3.4e38f)) continue;      // greedy or unusable: no draw
            if (tid == 0) {
                uint32_t spins = 0;
                while (!__hip_atomic_load(ready + b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
                    if (++spins > kSpinLimit) break;
                    __builtin_amdgcn_s_sleep(2);
                }
                L.flag = spins <= kSpinLimit;
                if (!L.flag) __hip_atomic_fetch_or(queue, kQueueAbandoned, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            __syncthreads();
            if (!L.flag) continue;
            const DrawTask task = load_task<true>(p, plan, b);
            if (task.kind == kNone) continue;
            do_chunk<DT>(p, plan, task, b, c, L.tbl, L.u.draw);
            wait_stores();
            __syncthreads();
            if (tid == 0) {
                const uint32_t done = __hip_atomic_fetch_add(chunks_done + b, 1u, __ATOMIC_RELAXED,
                                                             __HIP_MEMORY_SCOPE_AGENT);
                L.flag = (done + 1 == static_cast<uint32_t>(nchunk));
            }
            __syncthreads();
            if (L.flag) do_pick<DT>(p, plan, task, b, L.tbl, L.u.pick);
        }
    }
}

// Zeroes the queue, the abort flag and the per-sequence counters.
__global__ __launch_bounds__(kThreads) void fused_reset_kernel(uint32_t* ctr, int64_t n) {
    for (int64_t i = blockIdx.x * static_cast<int64_t>(kThreads) + threadIdx.x; i < n;
         i += static_cast<int64_t>(gridDim.x) * kThreads)
        ctr[i] = 0u;
}

template <int DT>
int resident_blocks_per_cu() {
    static int cached = -1;                  // per dtype; the same on every gfx950 device
    if (cached < 0) {
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fused_kernel<DT>, kThreads, 0) != hipSuccess)
            return -1;
        cached = n;
    }
    return cached;
}

}  // namespace

int64_t fused_counter_words(int32_t B) { return kCtrHeader + 3 * static_cast<int64_t>(B); }

hipError_t launch_fused_reset(const Problem& p, const Plan& plan, hipStream_t s) {
    const int64_t n = fused_counter_words(p.B);
    int64_t blocks = (n + kThreads - 1) / kThreads;
    if (blocks > 1024) blocks = 1024;
    fused_reset_kernel<<<dim3(static_cast<uint32_t>(blocks)), dim3(kThreads), 0, s>>>(plan.ctr, n);
    return hipGetLastError();
}

hipError_t fused_grid(int32_t dtype, int32_t* blocks) {
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    const int per = dtype == SV_BF16 ? resident_blocks_per_cu<SV_BF16>() : resident_blocks_per_cu<SV_F32>();
    if (per <= 0) return hipErrorInvalidValue;
    *blocks = cus * per;
    return hipSuccess;
}

hipError_t launch_fused(const Problem& p, const Plan& plan, const Fused& f, hipStream_t s) {
    const int64_t blocks = f.blocks;
    if (blocks <= 0) return hipSuccess;
    if (p.dtype == SV_BF16)
        fused_kernel<SV_BF16><<<dim3(static_cast<uint32_t>(blocks)), dim3(kThreads), 0, s>>>(p, plan, f);
    else
        fused_kernel<SV_F32><<<dim3(static_cast<uint32_t>(blocks)), dim3(kThreads), 0, s>>>(p, plan, f);
    return hipGetLastError();
}

}  // namespace sv
