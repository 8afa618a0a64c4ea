// specverify.hip -- host side of the libspecverify C ABI: argument checks,
// work geometry, workspace, kernel launches and the benchmark timing probe.
// The operation and every argument are documented in include/specverify.h.
#include <stdlib.h>

#include <mutex>

#include "sv_internal.h"

namespace {
using namespace sv;

constexpr int64_t kDefaultSegElems = 65536;   // row-pass segment length before rounding
// Row-pass segments are whole load windows: 256 lanes x 16 B x the window
// depth (8 loads for bf16, 4 for fp32), so only a row's last segment can end
// inside a window.
int64_t row_unit(sv_dtype_t dtype) { return dtype == SV_BF16 ? 256 * 8 * 8 : 256 * 4 * 4; }
constexpr int64_t kDefaultChunkElems = 8192;  // draw chunk length before rounding
// Early exit is worth its two extra launches (~15 us) only when the rows
// it may skip take longer than that to stream: automatic mode (lead -1)
// uses one leading position when all rows together hold at least
// kAutoLeadBytes, and one full pass otherwise.
constexpr int32_t kAutoLead = -1;
constexpr int64_t kAutoLeadBytes = 512ll << 20;
constexpr int kMaxDevices = 64;
constexpr int kNumKernels = 13;
enum { kKRowStats, kKAccept, kKDrawSums, kKDrawPick, kKFusedReset, kKFused, kKRowLead, kKAcceptLead,
       kKRowDraft, kKRest, kKDrawAll, kKSampleSums, kKSamplePick };

const char* const kKernelNames[kNumKernels] = {"row_stats", "accept",      "draw_sums",   "draw_pick",
                                               "fused_reset", "fused",     "row_lead",    "accept_lead",
                                               "row_draft", "rest",        "draw_all",    "sample_sums",
                                               "sample_pick"};

std::mutex g_mutex;
int64_t g_seg_elems = 0;                     // 0: automatic (auto_lengths)
int64_t g_chunk_elems = 0;

// Automatic segment and chunk lengths: the defaults suit batches that fill
// the GPU many times over (256 sequences of k = 8, V = 152064: 8704 row
// workgroups, 4864 draw workgroups);
// a small call is cut finer so its row pass still has about kRowBlocks
// workgroups and its draw about kDrawBlocks (no finer than kMinSeg /
// kMinChunk logits).
constexpr int64_t kRowBlocks = 2048, kDrawBlocks = 1024;
constexpr int64_t kMinSeg = 8192, kMinChunk = 1024;
void auto_lengths(int32_t B, int64_t total, int64_t V, int64_t* seg, int64_t* chunk) {
    const int64_t rows = 2 * total + B;
    int64_t s = rows * V / kRowBlocks, c = static_cast<int64_t>(B) * V / kDrawBlocks;
    s = s < kMinSeg ? kMinSeg : (s > kDefaultSegElems ? kDefaultSegElems : s);
    c = c < kMinChunk ? kMinChunk : (c > kDefaultChunkElems ? kDefaultChunkElems : c);
    *seg = g_seg_elems ? g_seg_elems : s;
    *chunk = g_chunk_elems ? g_chunk_elems : c;
}
int32_t g_mode = SV_MODE_AUTO;
int32_t g_fused_lag = 0;                     // 0: chosen from the resident grid
int32_t g_lead = kAutoLead;                  // early exit: leading positions read first (0: off)
int32_t g_queue_mode = SV_QUEUE_OVERLAP;
int32_t g_lag_a = 0, g_lag_c = 0;            // 0: chosen from the resident grid
int32_t g_draw_mode = SV_DRAW_AUTO;
// One pass: the draw runs as one launch (draw_all) while its workgroups
// (sequences x chunks) fit one round on the CUs, counted at this many per
// CU; a larger draw takes three launches (accept, draw_sums, draw_pick),
// since the pick's count of summed chunks makes the workgroup that finishes
// a sequence last do its pick, and with several rounds in flight those
// land on whichever XCD already lags, which then lags further.
constexpr int kDrawAllWgsPerCu = 4;
constexpr int kRestWgsPerCu = 5;             // resident second-round workgroups per CU (its register count)

hipError_t device_cus(int* cus) {
    static int cached[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    if (!cached[dev]) {
        e = hipDeviceGetAttribute(&cached[dev], hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
    }
    *cus = cached[dev];
    return hipSuccess;
}

int32_t effective_lead(int64_t B, int64_t total, int64_t V, sv_dtype_t dtype) {
    if (g_mode == SV_MODE_FUSED) return 0;      // the fused form reads every row
    if (g_lead != kAutoLead) return g_lead;
    if (total == 0) return 0;                    // only bonus rows: nothing to skip
    const int64_t bytes = (2 * total + B) * V * (dtype == SV_BF16 ? 2 : 4);
    return bytes >= kAutoLeadBytes ? 1 : 0;
}
constexpr double kLagFactor = 1.5;           // resident grids of items between rows and draw

// Library-owned workspace, one grow-only buffer per device.
void* g_ws[kMaxDevices] = {};
size_t g_ws_bytes[kMaxDevices] = {};

// Timing probe state: a ring of event pairs for the last kTimedCalls calls.
constexpr int kTimedCalls = 256;
uint32_t g_timing = 0;                // bit i: time kernel i
int32_t g_timing_every = 1;           // record one call in this many
int64_t g_timing_seen = 0;            // calls made since the probe was enabled
int64_t g_timed_calls = 0;            // calls recorded since the probe was enabled
int g_timing_device = -1;
hipEvent_t g_ev[kTimedCalls][2 * kNumKernels] = {};
uint32_t g_ev_mask[kTimedCalls] = {};        // kernels recorded in each call

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

struct Geometry {
    int32_t nseg, nchunk;
    int64_t seg_len, chunk_len;
    size_t off_seg, off_task, off_csum, off_band_n, off_band_w, off_xlogit, off_ctr, off_done, off_sched,
        off_blk_ctr, off_blk_seq, off_dlist, off_dlist_n, off_nbuf, off_early, off_early_n, off_aband, off_picked, bytes;
};

// Splits a row of V logits into n <= max_pieces pieces of about `target`
// elements (at most max_len when that fits max_pieces; max_len a multiple of
// unit), each a multiple of `unit` elements long, none empty.
void split(int64_t V, int64_t target, int64_t max_pieces, int64_t unit, int64_t max_len, int32_t& n,
           int64_t& len) {
    int64_t pieces = (V + target / 2) / target;
    if (pieces < ceil_div(V, max_len)) pieces = ceil_div(V, max_len);
    if (pieces < 1) pieces = 1;
    if (pieces > max_pieces) pieces = max_pieces;
    len = ceil_div(ceil_div(V, pieces), unit) * unit;
    n = static_cast<int32_t>(ceil_div(V, len));
}

bool make_geometry(int32_t B, int64_t total, int64_t V, sv_dtype_t dtype, int64_t seg_elems,
                   int64_t chunk_elems, Geometry& g) {
    const int64_t unit = row_unit(dtype);
    split(V, seg_elems, 1 << 20, seg_elems >= unit ? unit : 8, max_seg_elems(dtype), g.nseg, g.seg_len);
    split(V, chunk_elems, kMaxChunks, 8, V, g.nchunk, g.chunk_len);
    const int64_t rows = 2 * total + B;
    // (the second round's grid holds every row segment and every draw chunk)
    if (rows * g.nseg + static_cast<int64_t>(B) * (1 + g.nchunk) > 0x7FFFFFFFll) return false;
    size_t off = 0;
    g.off_seg = off;
    off = align256(off + sizeof(SegStat) * static_cast<size_t>(rows) * g.nseg);
    g.off_task = off;
    off = align256(off + sizeof(DrawTask) * static_cast<size_t>(B));
    g.off_csum = off;
    off = align256(off + sizeof(ChunkSums) * kWaves * static_cast<size_t>(B) * g.nchunk);
    g.off_band_n = off;
    off = align256(off + sizeof(int32_t) * kWaves * static_cast<size_t>(B) * g.nchunk);
    g.off_band_w = off;
    off = align256(off + sizeof(double) * 2 * kWaves * kWaveCap * static_cast<size_t>(B) * g.nchunk);
    g.off_xlogit = off;
    off = align256(off + sizeof(float) * static_cast<size_t>(rows));
    g.off_ctr = off;
    off = align256(off + sizeof(uint32_t) * static_cast<size_t>(fused_counter_words(B)));
    g.off_done = off;
    off = align256(off + sizeof(int32_t) * static_cast<size_t>(B));
    g.off_sched = off;
    off = align256(off + sizeof(RestItem) * (static_cast<size_t>(rows) * g.nseg +
                                             static_cast<size_t>(B) * (1 + g.nchunk)));
    g.off_blk_ctr = off;
    off = align256(off + sizeof(uint64_t));
    g.off_blk_seq = off;
    off = align256(off + sizeof(int32_t) * static_cast<size_t>(B));
    g.off_dlist = off;
    off = align256(off + sizeof(RestItem) * static_cast<size_t>(B) * g.nseg);
    g.off_dlist_n = off;
    off = align256(off + sizeof(uint32_t));
    g.off_nbuf = off;                                   // accept counts of spec_draft_sample
    off = align256(off + sizeof(int32_t) * static_cast<size_t>(B));
    g.off_early = off;
    off = align256(off + sizeof(int32_t) * static_cast<size_t>(B));
    g.off_early_n = off;
    off = align256(off + sizeof(uint32_t));
    g.off_aband = off;
    off = align256(off + sizeof(int32_t) * static_cast<size_t>(B));
    g.off_picked = off;
    off = align256(off + sizeof(uint32_t) * static_cast<size_t>(B));
    g.bytes = off;
    return true;
}

bool aligned(const void* ptr, size_t a) { return (reinterpret_cast<uintptr_t>(ptr) % a) == 0; }

sv_status_t check_args(const void* target, const void* draft, const int32_t* tokens,
                       const int32_t* offsets, int32_t k_uniform, int64_t total, int32_t B,
                       int64_t V, sv_dtype_t dtype, const float* uniforms, const float* temperature,
                       const int32_t* out_tokens, const int32_t* out_n) {
    if (B < 0 || total < 0) return SV_ERR_SHAPE;
    if (dtype != SV_F32 && dtype != SV_BF16) return SV_ERR_DTYPE;
    if (!target || !uniforms || !temperature || !out_tokens || !out_n) return SV_ERR_NULL;
    if (total > 0 && (!draft || !tokens)) return SV_ERR_NULL;
    if (V < 1 || V > 0x7FFFFFFFll) return SV_ERR_SHAPE;
    if (!offsets) {
        if (k_uniform < 0 || k_uniform > SV_K_MAX || total != static_cast<int64_t>(B) * k_uniform)
            return SV_ERR_SHAPE;
    } else if (total > static_cast<int64_t>(B) * SV_K_MAX) {
        return SV_ERR_SHAPE;
    }
    const size_t elt = dtype == SV_BF16 ? 2 : 4;
    if (!aligned(target, elt) || !aligned(draft, elt) || !aligned(tokens, 4) ||
        !aligned(offsets, 4) || !aligned(uniforms, 4) || !aligned(temperature, 4) ||
        !aligned(out_tokens, 4) || !aligned(out_n, 4))
        return SV_ERR_ALIGN;
    return SV_OK;
}

// Returns a workspace of at least `bytes` on the current device.
sv_status_t owned_workspace(size_t bytes, void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SV_ERR_HIP;
    if (g_ws_bytes[dev] < bytes) {
        if (g_ws[dev]) {
            if (hipFree(g_ws[dev]) != hipSuccess) return SV_ERR_HIP;   // waits for the device
            g_ws[dev] = nullptr;
            g_ws_bytes[dev] = 0;
        }
        const size_t grow = bytes + bytes / 4;
        if (hipMalloc(&g_ws[dev], grow) != hipSuccess) { g_ws[dev] = nullptr; return SV_ERR_HIP; }
        g_ws_bytes[dev] = grow;
    }
    *out = g_ws[dev];
    return SV_OK;
}

// sample: the drafter's sampling step (spec_draft_sample), k = 0 for every
// row: two launches of its own (sample.hip) instead of the verify's.
sv_status_t run(const Problem& p, void* workspace, size_t workspace_bytes, hipStream_t stream,
                bool sample = false) {
    if (p.B == 0) return SV_OK;
    std::lock_guard<std::mutex> lock(g_mutex);
    Geometry g;
    int64_t seg_elems, chunk_elems;
    auto_lengths(p.B, p.total, p.V, &seg_elems, &chunk_elems);
    if (!make_geometry(p.B, p.total, p.V, static_cast<sv_dtype_t>(p.dtype), seg_elems, chunk_elems, g))
        return SV_ERR_SHAPE;
    if (workspace) {
        if (workspace_bytes < g.bytes) return SV_ERR_WORKSPACE;
        if (!aligned(workspace, 16)) return SV_ERR_ALIGN;
    } else {
        sv_status_t st = owned_workspace(g.bytes, &workspace);
        if (st != SV_OK) return st;
    }
    char* ws = static_cast<char*>(workspace);
    Plan plan;
    plan.nseg = g.nseg;
    plan.seg_len = g.seg_len;
    plan.nchunk = g.nchunk;
    plan.chunk_len = g.chunk_len;
    plan.seg = reinterpret_cast<SegStat*>(ws + g.off_seg);
    plan.task = reinterpret_cast<DrawTask*>(ws + g.off_task);
    plan.csum = reinterpret_cast<ChunkSums*>(ws + g.off_csum);
    plan.band_n = reinterpret_cast<int32_t*>(ws + g.off_band_n);
    plan.band_w = reinterpret_cast<double*>(ws + g.off_band_w);
    plan.xlogit = reinterpret_cast<float*>(ws + g.off_xlogit);
    plan.ctr = reinterpret_cast<uint32_t*>(ws + g.off_ctr);
    plan.done = reinterpret_cast<int32_t*>(ws + g.off_done);
    plan.sched = reinterpret_cast<RestItem*>(ws + g.off_sched);
    plan.blk_ctr = reinterpret_cast<uint64_t*>(ws + g.off_blk_ctr);
    plan.blk_seq = reinterpret_cast<int32_t*>(ws + g.off_blk_seq);
    plan.dlist = reinterpret_cast<RestItem*>(ws + g.off_dlist);
    plan.dlist_n = reinterpret_cast<uint32_t*>(ws + g.off_dlist_n);
    plan.early = reinterpret_cast<int32_t*>(ws + g.off_early);
    plan.early_n = reinterpret_cast<uint32_t*>(ws + g.off_early_n);
    plan.aband = reinterpret_cast<int32_t*>(ws + g.off_aband);
    plan.picked = reinterpret_cast<uint32_t*>(ws + g.off_picked);
    plan.queue_mode = g_queue_mode;
    Problem pr = p;
    if (!pr.out_n) pr.out_n = reinterpret_cast<int32_t*>(ws + g.off_nbuf);

    // The fused form needs the schedule prefix and the pick's chunk masses
    // in LDS, and an item count below 2^31.
    const int64_t max_items = (2 * p.total + p.B) * static_cast<int64_t>(g.nseg) +
                              static_cast<int64_t>(p.B) * g.nchunk;
    const bool fused_fits = p.B <= kFusedMaxB && g.nchunk <= kFusedMaxChunks && max_items < (1ll << 31);
    // The fused form measured slower than the staged one on MI355X (see
    // fused.hip), so it runs only when asked for.
    // The gathered form reads draft rows after the accept scans, which only
    // the staged form does.
    const bool fused = g_mode == SV_MODE_FUSED && !p.draft_probs && !sample;
    if (fused && !fused_fits) return SV_ERR_SHAPE;
    plan.lead = fused ? 0 : effective_lead(p.B, p.total, p.V, static_cast<sv_dtype_t>(p.dtype));
    if (device_cus(&plan.cus) != hipSuccess) return SV_ERR_HIP;
    plan.lag_a = plan.lag_c = 1 << 30;             // no accept or draw items in the schedule
    plan.queued = plan.lead > 0 && !p.draft_probs;
    if (plan.queued) {
        if (g_lag_a > 0) {
            plan.lag_a = g_lag_a;
            plan.lag_c = g_lag_c > g_lag_a ? g_lag_c : g_lag_a;
        } else {
            // An item waiting for what it needs holds its CU slot, so items
            // start well after their rows: the accept item about 1.4 resident
            // grids of row segments later, the draw items about 2.3 (measured
            // on MI355X; shorter lags wait more than they overlap).
            const double window = static_cast<double>(plan.cus) * kRestWgsPerCu;
            double per_block = (2.0 * static_cast<double>(p.total) / p.B - 2.0 * plan.lead + 1.0) * g.nseg;
            if (per_block < g.nseg) per_block = g.nseg;
            plan.lag_a = static_cast<int32_t>(1.4 * window / per_block) + 1;
            plan.lag_c = static_cast<int32_t>(2.3 * window / per_block) + 2;
        }
    }
    Fused f{};
    if (fused) {
        if (fused_grid(p.dtype, &f.blocks) != hipSuccess) return SV_ERR_HIP;
        if (g_fused_lag > 0) {
            f.lag = g_fused_lag;
        } else {
            const double per_step = g.nseg * (2.0 * p.total / p.B + 1.0) + g.nchunk;
            f.lag = static_cast<int32_t>(kLagFactor * f.blocks / per_step + 1.0);
        }
        if (f.lag > p.B) f.lag = p.B;
        if (f.lag < 1) f.lag = 1;
    }

    hipEvent_t* ev = nullptr;
    if (g_timing && (g_timing_seen++ % g_timing_every) == 0) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess) return SV_ERR_HIP;
        if (g_timing_device != dev) {
            for (auto& call : g_ev)
                for (auto& e : call) {
                    if (e) (void)hipEventDestroy(e);
                    e = nullptr;
                }
            for (auto& call : g_ev)
                for (auto& e : call)
                    if (hipEventCreate(&e) != hipSuccess) return SV_ERR_HIP;
            g_timing_device = dev;
            g_timed_calls = 0;
        }
        ev = g_ev[g_timed_calls % kTimedCalls];
    }
    uint32_t recorded = 0;
    auto launch = [&](int i, auto&& fn) -> bool {
        const bool timed = ev && ((g_timing >> i) & 1u);
        if (timed && hipEventRecord(ev[2 * i], stream) != hipSuccess) return false;
        if (fn() != hipSuccess) return false;
        if (timed && hipEventRecord(ev[2 * i + 1], stream) != hipSuccess) return false;
        if (timed) recorded |= 1u << i;
        return true;
    };
    bool ok;
    if (sample) {
        ok = launch(kKSampleSums, [&] { return launch_sample_sums(pr, plan, stream); }) &&
             launch(kKSamplePick, [&] { return launch_sample_pick(pr, plan, stream); });
    } else if (fused) {
        ok = launch(kKFusedReset, [&] { return launch_fused_reset(pr, plan, stream); }) &&
             launch(kKFused, [&] { return launch_fused(pr, plan, f, stream); });
    } else {
        // Row pass: one pass over every needed row, or (early exit) the
        // leading positions, their accept scan, then the listed remainder.
        // Early exit outside the gathered form ends in two launches: the
        // remaining rows with the draws beside them, and the picks (with the
        // redo of anything that round left over, usually nothing).
        const bool queued = plan.queued != 0;
        if (plan.lead > 0)
            ok = launch(kKRowLead, [&] { return launch_row_lead(pr, plan, stream); }) &&
                 launch(kKAcceptLead, [&] { return launch_accept_lead(pr, plan, stream); });
        else
            ok = launch(kKRowStats, [&] { return launch_row_stats(pr, plan, stream); });
        if (queued) {
            ok = ok && launch(kKRest, [&] { return launch_rest_draws(pr, plan, stream); }) &&
                 launch(kKDrawPick, [&] { return launch_draw_pick(pr, plan, stream); });
            if (ev) {
                g_ev_mask[g_timed_calls % kTimedCalls] = recorded;
                ++g_timed_calls;
            }
            return ok ? SV_OK : SV_ERR_HIP;
        }
        if (plan.lead > 0)   // gathered form: a settled sequence has no early draw
            ok = ok && launch(kKRowStats, [&] {
                return launch_row_list(pr, plan, plan.sched, reinterpret_cast<const uint32_t*>(plan.blk_ctr),
                                       (2 * p.total + p.B) * static_cast<int64_t>(g.nseg), stream);
            });
        // One pass, outside the gathered form: a draw that fits one round of
        // workgroups runs as one launch with the accept scans and the picks.
        const bool draw_all = !pr.draft_probs && plan.lead == 0 &&
                              (g_draw_mode == SV_DRAW_ONE ||
                               (g_draw_mode == SV_DRAW_AUTO &&
                                static_cast<int64_t>(p.B) * g.nchunk <= static_cast<int64_t>(kDrawAllWgsPerCu) * plan.cus));
        if (draw_all) {
            ok = ok && launch(kKDrawAll, [&] { return launch_draw_all(pr, plan, stream); });
            if (ev) {
                g_ev_mask[g_timed_calls % kTimedCalls] = recorded;
                ++g_timed_calls;
            }
            return ok ? SV_OK : SV_ERR_HIP;
        }
        ok = ok && launch(kKAccept, [&] { return launch_accept(pr, plan, stream); });
        // Gathered form: the draft rows at the rejections.
        if (ok && pr.draft_probs)
            ok = launch(kKRowDraft, [&] {
                return launch_row_list(pr, plan, plan.dlist, plan.dlist_n, static_cast<int64_t>(p.B) * g.nseg, stream);
            });
        ok = ok && launch(kKDrawSums, [&] { return launch_draw_sums(pr, plan, stream); }) &&
             launch(kKDrawPick, [&] { return launch_draw_pick(pr, plan, stream); });
    }
    if (ev) {
        g_ev_mask[g_timed_calls % kTimedCalls] = recorded;
        ++g_timed_calls;
    }
    return ok ? SV_OK : SV_ERR_HIP;
}

}  // namespace

extern "C" {

size_t spec_verify_workspace_size(int32_t B, int64_t total_draft, int64_t V, sv_dtype_t dtype) {
    if (B < 0 || total_draft < 0 || V < 1 || V > 0x7FFFFFFFll) return 0;
    if (dtype != SV_F32 && dtype != SV_BF16) return 0;
    std::lock_guard<std::mutex> lock(g_mutex);
    Geometry g;
    int64_t seg_elems, chunk_elems;
    auto_lengths(B, total_draft, V, &seg_elems, &chunk_elems);
    if (!make_geometry(B, total_draft, V, dtype, seg_elems, chunk_elems, g)) return 0;
    return g.bytes;
}

sv_status_t spec_verify_probs(const void* target_logits, const void* draft_logits,
                              const int32_t* draft_tokens, const int32_t* offsets,
                              int32_t k_uniform, int64_t total_draft, int32_t B, int64_t V,
                              sv_dtype_t dtype, const float* uniforms, const float* temperature,
                              int32_t* out_tokens, int32_t* out_n_accepted, float* out_p,
                              float* out_q, float* out_row_max, float* out_row_sumexp,
                              void* workspace, size_t workspace_bytes, hipStream_t stream) {
    sv_status_t st = check_args(target_logits, draft_logits, draft_tokens, offsets, k_uniform,
                                total_draft, B, V, dtype, uniforms, temperature, out_tokens,
                                out_n_accepted);
    if (st != SV_OK) return st;
    if ((out_p == nullptr) != (out_q == nullptr) ||
        (out_row_max == nullptr) != (out_row_sumexp == nullptr))
        return SV_ERR_NULL;
    if (!aligned(out_p, 4) || !aligned(out_q, 4) || !aligned(out_row_max, 4) ||
        !aligned(out_row_sumexp, 4))
        return SV_ERR_ALIGN;
    Problem p;
    p.target = target_logits;
    p.draft = draft_logits;
    p.tokens = draft_tokens;
    p.offsets = offsets;
    p.uniforms = uniforms;
    p.temperature = temperature;
    p.out_tokens = out_tokens;
    p.out_n = out_n_accepted;
    p.out_p = out_p;
    p.out_q = out_q;
    p.out_row_max = out_row_max;
    p.out_row_sum = out_row_sumexp;
    p.draft_probs = nullptr;
    p.out_emit_prob = nullptr;
    p.V = V;
    p.total = total_draft;
    p.B = B;
    p.k_uniform = offsets ? 0 : k_uniform;
    p.dtype = dtype;
    return run(p, workspace, workspace_bytes, stream);
}

sv_status_t spec_verify(const void* target_logits, const void* draft_logits,
                        const int32_t* draft_tokens, const int32_t* offsets, int32_t k_uniform,
                        int64_t total_draft, int32_t B, int64_t V, sv_dtype_t dtype,
                        const float* uniforms, const float* temperature, int32_t* out_tokens,
                        int32_t* out_n_accepted, void* workspace, size_t workspace_bytes,
                        hipStream_t stream) {
    return spec_verify_probs(target_logits, draft_logits, draft_tokens, offsets, k_uniform,
                             total_draft, B, V, dtype, uniforms, temperature, out_tokens,
                             out_n_accepted, nullptr, nullptr, nullptr, nullptr, workspace,
                             workspace_bytes, stream);
}

sv_status_t spec_verify_gathered(const void* target_logits, const void* draft_logits,
                                 const int32_t* draft_tokens, const float* draft_probs,
                                 const int32_t* offsets, int32_t k_uniform, int64_t total_draft,
                                 int32_t B, int64_t V, sv_dtype_t dtype, const float* uniforms,
                                 const float* temperature, int32_t* out_tokens,
                                 int32_t* out_n_accepted, float* out_emit_prob, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
    sv_status_t st = check_args(target_logits, draft_logits, draft_tokens, offsets, k_uniform,
                                total_draft, B, V, dtype, uniforms, temperature, out_tokens,
                                out_n_accepted);
    if (st != SV_OK) return st;
    if (total_draft > 0 && !draft_probs) return SV_ERR_NULL;
    if (!aligned(draft_probs, 4) || !aligned(out_emit_prob, 4)) return SV_ERR_ALIGN;
    Problem p{};
    p.target = target_logits;
    p.draft = draft_logits;
    p.tokens = draft_tokens;
    p.offsets = offsets;
    p.uniforms = uniforms;
    p.temperature = temperature;
    p.out_tokens = out_tokens;
    p.out_n = out_n_accepted;
    p.draft_probs = total_draft > 0 ? draft_probs : nullptr;
    p.out_emit_prob = out_emit_prob;
    p.V = V;
    p.total = total_draft;
    p.B = B;
    p.k_uniform = offsets ? 0 : k_uniform;
    p.dtype = dtype;
    return run(p, workspace, workspace_bytes, stream);
}

sv_status_t spec_draft_sample(const void* logits, int32_t rows, int64_t V, sv_dtype_t dtype,
                              const float* temperature, const float* uniforms, int32_t* out_tokens,
                              float* out_probs, void* workspace, size_t workspace_bytes,
                              hipStream_t stream) {
    // A verify of `rows` sequences with no drafted tokens: each row is the
    // bonus row of its sequence, so its token is drawn from softmax(z / T)
    // by the verify's inverse CDF (or is the argmax at T = 0).
    if (rows < 0) return SV_ERR_SHAPE;
    if (dtype != SV_F32 && dtype != SV_BF16) return SV_ERR_DTYPE;
    if (!logits || !temperature || !uniforms || !out_tokens) return SV_ERR_NULL;
    if (V < 1 || V > 0x7FFFFFFFll) return SV_ERR_SHAPE;
    const size_t elt = dtype == SV_BF16 ? 2 : 4;
    if (!aligned(logits, elt) || !aligned(temperature, 4) || !aligned(uniforms, 4) ||
        !aligned(out_tokens, 4) || !aligned(out_probs, 4))
        return SV_ERR_ALIGN;
    Problem p{};
    p.target = logits;
    p.uniforms = uniforms;
    p.temperature = temperature;
    p.out_tokens = out_tokens;
    p.out_n = nullptr;                           // the workspace holds the (zero) counts
    p.out_emit_prob = out_probs;
    p.V = V;
    p.total = 0;
    p.B = rows;
    p.k_uniform = 0;
    p.dtype = dtype;
    return run(p, workspace, workspace_bytes, stream, /*sample=*/true);
}

sv_status_t spec_commit(const int32_t* out_tokens, const int32_t* out_n_accepted, const int32_t* offsets,
                        int32_t k_uniform, int32_t B, int32_t* seq_tokens, int32_t* seq_len, int32_t max_len,
                        int32_t* committed, int32_t* committed_offsets, hipStream_t stream) {
    if (B < 0 || max_len < 0 || (!offsets && (k_uniform < 0 || k_uniform > SV_K_MAX))) return SV_ERR_SHAPE;
    if (!out_tokens || !out_n_accepted || !seq_tokens || !seq_len || !committed_offsets) return SV_ERR_NULL;
    if (!aligned(out_tokens, 4) || !aligned(out_n_accepted, 4) || !aligned(offsets, 4) ||
        !aligned(seq_tokens, 4) || !aligned(seq_len, 4) || !aligned(committed, 4) ||
        !aligned(committed_offsets, 4))
        return SV_ERR_ALIGN;
    return launch_commit(out_tokens, out_n_accepted, offsets, k_uniform, B, seq_tokens, seq_len, max_len,
                         committed, committed_offsets, stream) == hipSuccess ? SV_OK : SV_ERR_HIP;
}

sv_status_t spec_adapt_k(const int32_t* out_n_accepted, const int32_t* offsets, int32_t k_uniform, int32_t B,
                         int32_t min_k, int32_t max_k, double* history, int32_t* rounds, int32_t* k,
                         hipStream_t stream) {
    if (B < 0 || min_k < 1 || max_k < min_k || max_k > SV_K_MAX ||
        (!offsets && (k_uniform < 0 || k_uniform > SV_K_MAX)))
        return SV_ERR_SHAPE;
    if (B > 0 && (!out_n_accepted || !history || !rounds || !k)) return SV_ERR_NULL;
    if (!aligned(out_n_accepted, 4) || !aligned(offsets, 4) || !aligned(history, 8) || !aligned(rounds, 4) ||
        !aligned(k, 4))
        return SV_ERR_ALIGN;
    return launch_adapt_k(out_n_accepted, offsets, k_uniform, B, min_k, max_k, history, rounds, k, stream) ==
                   hipSuccess ? SV_OK : SV_ERR_HIP;
}

sv_status_t spec_stream_probe(const void* data, int64_t bytes, int64_t seg_bytes, uint32_t* out,
                              hipStream_t stream) {
    if (bytes < 0 || seg_bytes < 4096 || seg_bytes % 16 != 0 || seg_bytes > (1ll << 30)) return SV_ERR_SHAPE;
    if ((bytes + seg_bytes - 1) / seg_bytes > 0x7FFFFFFFll) return SV_ERR_SHAPE;
    if (bytes > 0 && (!data || !out)) return SV_ERR_NULL;
    if (!aligned(data, 16) || !aligned(out, 4)) return SV_ERR_ALIGN;
    return launch_stream_probe(data, bytes, seg_bytes, out, stream) == hipSuccess ? SV_OK : SV_ERR_HIP;
}

size_t spec_ngram_workspace_size(int32_t B) {
    return B < 0 ? 0 : align256(sizeof(int32_t) * (static_cast<size_t>(B) + 1));
}

sv_status_t spec_ngram_draft(const int32_t* seq_tokens, const int32_t* seq_len, int32_t B, int32_t max_len,
                             int32_t ngram_max, int32_t ngram_min, int32_t k_max, int32_t* draft_tokens,
                             int32_t* draft_offsets, void* workspace, size_t workspace_bytes,
                             hipStream_t stream) {
    if (B < 0 || max_len < 0 || ngram_min < 1 || ngram_max < ngram_min || k_max < 0 || k_max > SV_K_MAX)
        return SV_ERR_SHAPE;
    if (!draft_offsets || (B > 0 && (!seq_tokens || !seq_len || (k_max > 0 && !draft_tokens))))
        return SV_ERR_NULL;
    if (!aligned(seq_tokens, 4) || !aligned(seq_len, 4) || !aligned(draft_tokens, 4) ||
        !aligned(draft_offsets, 4))
        return SV_ERR_ALIGN;
    const size_t need = spec_ngram_workspace_size(B);
    if (workspace) {
        if (workspace_bytes < need) return SV_ERR_WORKSPACE;
        if (!aligned(workspace, 4)) return SV_ERR_ALIGN;
    } else {
        std::lock_guard<std::mutex> lock(g_mutex);
        const sv_status_t st = owned_workspace(need, &workspace);
        if (st != SV_OK) return st;
    }
    return launch_ngram_draft(seq_tokens, seq_len, B, max_len, ngram_max, ngram_min, k_max,
                              static_cast<int32_t*>(workspace), draft_tokens, draft_offsets, stream) ==
                   hipSuccess ? SV_OK : SV_ERR_HIP;
}

const char* spec_verify_status_string(sv_status_t status) {
    switch (status) {
        case SV_OK: return "ok";
        case SV_ERR_NULL: return "a required pointer is NULL";
        case SV_ERR_SHAPE: return "B, V, k or total_draft out of range or inconsistent";
        case SV_ERR_DTYPE: return "unsupported logit dtype";
        case SV_ERR_ALIGN: return "pointer not aligned to its element size";
        case SV_ERR_WORKSPACE: return "workspace smaller than spec_verify_workspace_size()";
        case SV_ERR_HIP: return "HIP call or kernel launch failed";
    }
    return "unknown status";
}

void spec_verify_release(void) {
    std::lock_guard<std::mutex> lock(g_mutex);
    int cur = 0;
    const bool have_cur = hipGetDevice(&cur) == hipSuccess;
    for (int d = 0; d < kMaxDevices; ++d) {
        if (!g_ws[d]) continue;
        if (hipSetDevice(d) == hipSuccess) (void)hipFree(g_ws[d]);
        g_ws[d] = nullptr;
        g_ws_bytes[d] = 0;
    }
    if (have_cur) (void)hipSetDevice(cur);
}

sv_status_t spec_verify_timing(int32_t kernels, int32_t every) {
    std::lock_guard<std::mutex> lock(g_mutex);
    if (every < 1) return SV_ERR_SHAPE;
    g_timing = static_cast<uint32_t>(kernels) & ((1u << kNumKernels) - 1u);
    g_timing_every = every;
    g_timing_seen = 0;
    g_timed_calls = 0;
    return SV_OK;
}

int32_t spec_verify_kernel_times(float* ms, int32_t max_kernels) {
    std::lock_guard<std::mutex> lock(g_mutex);
    if (g_timed_calls == 0 || !ms || !g_timing) return -1;
    const int64_t ncalls = g_timed_calls < kTimedCalls ? g_timed_calls : kTimedCalls;
    const int64_t last = (g_timed_calls - 1) % kTimedCalls;
    const uint32_t last_mask = g_ev_mask[last];
    if (last_mask == 0) return -1;
    const int last_kernel = 31 - __builtin_clz(last_mask);
    if (hipEventSynchronize(g_ev[last][2 * last_kernel + 1]) != hipSuccess) return -1;
    const int n = max_kernels < kNumKernels ? max_kernels : kNumKernels;
    for (int i = 0; i < n; ++i) {
        double sum = 0.0;
        int64_t cnt = 0;
        for (int64_t c = 0; c < ncalls; ++c) {
            if (!((g_ev_mask[c] >> i) & 1u)) continue;
            float t = 0.f;
            if (hipEventElapsedTime(&t, g_ev[c][2 * i], g_ev[c][2 * i + 1]) != hipSuccess) return -1;
            sum += t;
            ++cnt;
        }
        ms[i] = cnt ? static_cast<float>(sum / cnt) : __builtin_nanf("");
    }
    return kNumKernels;
}

const char* spec_verify_kernel_name(int32_t i) {
    return (i >= 0 && i < kNumKernels) ? kKernelNames[i] : nullptr;
}

sv_status_t spec_verify_set_mode(int32_t mode, int32_t fused_lag) {
    if (mode < SV_MODE_AUTO || mode > SV_MODE_FUSED || fused_lag < 0) return SV_ERR_SHAPE;
    std::lock_guard<std::mutex> lock(g_mutex);
    g_mode = mode;
    g_fused_lag = fused_lag;
    return SV_OK;
}

sv_status_t spec_verify_set_early_exit(int32_t lead_positions) {
    if (lead_positions < kAutoLead || lead_positions > SV_K_MAX + 1) return SV_ERR_SHAPE;
    std::lock_guard<std::mutex> lock(g_mutex);
    g_lead = lead_positions;
    return SV_OK;
}

sv_status_t spec_verify_set_queue(int32_t mode, int32_t lag_accept, int32_t lag_draw) {
    if (mode < SV_QUEUE_OVERLAP || mode > SV_QUEUE_HANDOFF || lag_accept < 0 || lag_draw < 0) return SV_ERR_SHAPE;
    std::lock_guard<std::mutex> lock(g_mutex);
    g_queue_mode = mode;
    g_lag_a = lag_accept;
    g_lag_c = lag_draw;
    return SV_OK;
}

sv_status_t spec_verify_set_draw(int32_t mode) {
    if (mode < SV_DRAW_AUTO || mode > SV_DRAW_THREE) return SV_ERR_SHAPE;
    std::lock_guard<std::mutex> lock(g_mutex);
    g_draw_mode = mode;
    return SV_OK;
}

sv_status_t spec_verify_set_geometry(int64_t seg_elems, int64_t chunk_elems) {
    if (seg_elems < 0 || chunk_elems < 0) return SV_ERR_SHAPE;
    std::lock_guard<std::mutex> lock(g_mutex);
    g_seg_elems = seg_elems;
    g_chunk_elems = chunk_elems;
    return SV_OK;
}

}  // extern "C"
