// specverify.hip -- host side of the libspecverify C ABI: argument checks,
// work geometry, workspace, kernel launches, and the per-call tuning hooks
// of sv_tuning.h.  The operation and every argument are documented in
// include/specverify.h.
#include <stdlib.h>

#include <mutex>

#include "host_args.h"
#include "sv_internal.h"
#include "sv_tuning.h"

// The scratch of spec_verify_noalloc: one copy on each GPU the library runs
// on, for the life of the process.  In host code `scratch` only names the
// symbol; its device address comes from hipGetSymbolAddress (scratch_address).
static __device__ __align__(256) unsigned char scratch[SV_NOALLOC_SCRATCH_BYTES];

namespace {
using namespace sv;
using namespace sv::host;

constexpr int kMaxDevices = 64;
enum { kKRowStats, kKAccept, kKDrawSums, kKDrawPick, kKRowLead, kKRowDraft, kKRounds, kKDrawAll, kKSampleSums,
       kKSamplePick, kNumKernels };
static_assert(kNumKernels == SV_NUM_KERNELS, "kernel count");

const char* const kKernelNames[kNumKernels] = {"row_stats", "accept",   "draw_sums", "draw_pick",
                                               "row_lead",  "row_draft", "rounds",    "draw_all",
                                               "sample_sums", "sample_pick"};

// One pass: the draw runs as one launch (draw_all) while its workgroups
// (sequences x chunks) fit one round on the CUs, counted at this many per
// CU; a larger draw takes three launches (accept, draw_sums, draw_pick),
// since the pick's count of summed chunks makes the workgroup that finishes
// a sequence last do its pick, and with several rounds in flight those
// land on whichever XCD already lags, which then lags further.
constexpr int kDrawAllWgsPerCu = 4;

// Per-device facts, queried once: compute units, and workgroups of the
// two-round launch a compute unit holds at once (its register count decides).
std::mutex g_mutex;                          // guards the caches and the owned workspace
struct DeviceInfo {
    int cus = 0;
    int rest_per_cu[2] = {0, 0};             // by dtype
};
DeviceInfo g_dev[kMaxDevices];

hipError_t device_info(int32_t dtype, int* cus, int* rest_per_cu) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mutex);
    DeviceInfo& d = g_dev[dev];
    if (!d.cus) {
        e = hipDeviceGetAttribute(&d.cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
    }
    const int di = dtype == SV_BF16 ? 1 : 0;
    if (!d.rest_per_cu[di]) {
        int32_t n = 0;
        e = rounds_blocks_per_cu(dtype, &n);
        if (e != hipSuccess) return e;
        d.rest_per_cu[di] = n > 0 ? n : 1;
    }
    *cus = d.cus;
    *rest_per_cu = d.rest_per_cu[di];
    return hipSuccess;
}

// Library-owned workspace, one grow-only buffer per device.
void* g_ws[kMaxDevices] = {};
size_t g_ws_bytes[kMaxDevices] = {};
// Device address of `scratch` on each device (looked up on first use).
void* g_scratch[kMaxDevices] = {};

// The address of this device's copy of `scratch`: hipGetSymbolAddress once
// per device, with that device current.  Allocates nothing.
sv_status_t scratch_address(void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SV_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_mutex);
    if (!g_scratch[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return SV_ERR_HIP;
        g_scratch[dev] = ptr;
    }
    *out = g_scratch[dev];
    return SV_OK;
}

// Returns a workspace of at least `bytes` on the current device.
sv_status_t owned_workspace(size_t bytes, void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SV_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_mutex);
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
                const Tuning& tu, bool sample = false) {
    if (tu.launched) *tu.launched = 0u;
    if (p.B == 0) return SV_OK;
    Geometry g;
    int64_t seg_elems, chunk_elems;
    auto_lengths(p.B, p.total, p.V, tu, &seg_elems, &chunk_elems);
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
    plan.task = reinterpret_cast<TaskRec*>(ws + g.off_task);
    plan.csum = reinterpret_cast<ChunkSums*>(ws + g.off_csum);
    plan.band_n = reinterpret_cast<int32_t*>(ws + g.off_band_n);
    plan.band_w = reinterpret_cast<double*>(ws + g.off_band_w);
    plan.xlogit = reinterpret_cast<float*>(ws + g.off_xlogit);
    plan.done = reinterpret_cast<int32_t*>(ws + g.off_done);
    plan.sched = reinterpret_cast<SchedEntry*>(ws + g.off_sched);
    plan.blk_ctr = reinterpret_cast<uint64_t*>(ws + g.off_blk_ctr);
    plan.blk_seq = reinterpret_cast<uint64_t*>(ws + g.off_blk_seq);
    plan.dlist = reinterpret_cast<RestItem*>(ws + g.off_dlist);
    plan.dlist_n = reinterpret_cast<uint32_t*>(ws + g.off_dlist_n);
    plan.aband = reinterpret_cast<int32_t*>(ws + g.off_aband);
    plan.picked = reinterpret_cast<uint32_t*>(ws + g.off_picked);
    plan.lead_ctr = reinterpret_cast<uint64_t*>(ws + g.off_lead_ctr);
    plan.lead_clr = reinterpret_cast<uint32_t*>(ws + g.off_lead_clr);
    plan.lead_done = reinterpret_cast<uint64_t*>(ws + g.off_lead_done);
    plan.lead_rec = reinterpret_cast<LeadRec*>(ws + g.off_lead_rec);
    plan.lead_pace = 0;
    plan.stall = reinterpret_cast<uint32_t*>(ws + g.off_stall);
    plan.item_polls = tu.item_polls;
    plan.epoch = 0;                                // (each kernel takes the call's epoch on the device)
    plan.epoch_ctr = reinterpret_cast<uint32_t*>(ws + g.off_epoch);
    plan.queue_mode = tu.queue_mode;
    Problem pr = p;
    if (!pr.out_n) pr.out_n = reinterpret_cast<int32_t*>(ws + g.off_nbuf);

    plan.lead = sample ? 0
                       : effective_lead(p.B, p.total, p.V, static_cast<sv_dtype_t>(p.dtype), tu,
                                        p.draft_probs != nullptr);
    plan.lead_mul = lead_multiplier(p.B);
    int rest_per_cu = 1;
    if (device_info(p.dtype, &plan.cus, &rest_per_cu) != hipSuccess) return SV_ERR_HIP;
    plan.lag_a = plan.lag_c = 1 << 30;             // no accept or draw items in the schedule
    plan.queued = plan.lead > 0 && !p.draft_probs;
    // (a call whose two-round grid would not fit 2^31 - 1 workgroups runs as one pass)
    if (plan.queued && rounds_lead_blocks(p.B, plan.lead, g.nseg) +
                           rounds_rest_blocks(p.B, p.total, p.offsets != nullptr, p.k_uniform, plan.lead, g.nseg,
                                              g.nchunk) > 0x7FFFFFFFll)
        plan.lead = plan.queued = 0;
    if (plan.queued) {
        if (tu.lag_a > 0) {
            plan.lag_a = tu.lag_a;
            plan.lag_c = tu.lag_c > tu.lag_a ? tu.lag_c : tu.lag_a;
        } else {
            // An item waiting for what it needs holds its CU slot, so items
            // start after their rows: the accept item about 0.8 resident grids
            // of an undecided block's row segments later, the draw items about
            // 1.3 (measured on MI355X, B=256 k=8 and B=512 ragged k: the
            // settled sequences' draw chunks listed between the blocks stretch
            // each block's share of the schedule; lags 1.4 / 2.3 took 2-4 us
            // longer, much shorter ones wait more than they overlap).
            const double window = static_cast<double>(plan.cus) * rest_per_cu;
            double per_block = (2.0 * static_cast<double>(p.total) / p.B - 2.0 * plan.lead + 1.0) * g.nseg;
            if (per_block < g.nseg) per_block = g.nseg;
            plan.lag_a = static_cast<int32_t>(0.8 * window / per_block) + 1;
            plan.lag_c = static_cast<int32_t>(1.3 * window / per_block) + 2;
        }
        // Pacing of the first round when all of it is resident at once (one
        // leading position, records): its second half of workgroups waits
        // about 90% of the time the first half takes to stream its rows at
        // the read ceiling (~7 TB/s), so that the first half's scans list
        // second-round work while the second half streams instead of all
        // scans finishing together (C4: 2-3 us shorter; a first round larger
        // than the resident grid staggers by itself, and pacing it was slower).
        const int64_t nlead = rounds_lead_blocks(p.B, plan.lead, g.nseg);
        if (plan.lead == 1 && g.nseg <= kPolledSegs &&
            static_cast<double>(nlead) <= static_cast<double>(plan.cus) * rest_per_cu) {
            const double half_bytes = static_cast<double>(p.B) * p.V * (p.dtype == SV_BF16 ? 2 : 4);
            plan.lead_pace = static_cast<uint32_t>(0.9 * half_bytes / 7.0e12 * 1e8);
        }
    }

    uint32_t recorded = 0;
    auto launch = [&](int i, auto&& fn) -> bool {
        hipEvent_t* ev = ((tu.timed >> i) & 1u) ? tu.events : nullptr;
        if (ev && hipEventRecord(ev[2 * i], stream) != hipSuccess) return false;
        if (fn() != hipSuccess) return false;
        if (ev && hipEventRecord(ev[2 * i + 1], stream) != hipSuccess) return false;
        recorded |= 1u << i;
        return true;
    };
    auto finish = [&](bool ok) {
        if (tu.launched) *tu.launched = recorded;
        return ok ? SV_OK : SV_ERR_HIP;
    };
    bool ok;
    if (sample) {
        ok = launch(kKSampleSums, [&] { return launch_sample_sums(pr, plan, stream); }) &&
             launch(kKSamplePick, [&] { return launch_sample_pick(pr, plan, stream); });
        return finish(ok);
    }
    // Early exit outside the gathered form: two launches, both rounds (the
    // leading positions with their accept scans, then the remaining rows
    // with the draws beside them), and the picks (with the redo of anything
    // the rounds left over, usually nothing).
    if (plan.queued) {
        ok = launch(kKRounds, [&] { return launch_rounds(pr, plan, stream); }) &&
             launch(kKDrawPick, [&] { return launch_draw_pick(pr, plan, stream); });
        return finish(ok);
    }
    // Row pass: one pass over every needed row, or (the gathered form's
    // early exit) the leading positions with their accept scans, then the
    // listed remainder.
    if (plan.lead > 0)
        ok = launch(kKRowLead, [&] { return launch_row_lead(pr, plan, stream); });
    else
        ok = launch(kKRowStats, [&] { return launch_row_stats(pr, plan, stream); });
    if (plan.lead > 0)   // gathered form: a settled sequence has no early draw
        ok = ok && launch(kKRowStats, [&] {
            return launch_sched_rows(pr, plan, reinterpret_cast<const uint32_t*>(plan.blk_ctr),
                                     (2 * p.total + p.B) * static_cast<int64_t>(g.nseg), stream);
        });
    // One pass, outside the gathered form: a draw that fits one round of
    // workgroups runs as one launch with the accept scans and the picks.
    const bool draw_all = !pr.draft_probs && plan.lead == 0 &&
                          (tu.draw_mode == SV_DRAW_ONE ||
                           (tu.draw_mode == SV_DRAW_AUTO &&
                            static_cast<int64_t>(p.B) * g.nchunk <= static_cast<int64_t>(kDrawAllWgsPerCu) * plan.cus));
    if (draw_all) {
        ok = ok && launch(kKDrawAll, [&] { return launch_draw_all(pr, plan, stream); });
        return finish(ok);
    }
    ok = ok && launch(kKAccept, [&] { return launch_accept(pr, plan, stream); });
    // Gathered form: the draft rows at the rejections.
    if (ok && pr.draft_probs)
        ok = launch(kKRowDraft, [&] {
            return launch_row_list(pr, plan, plan.dlist, plan.dlist_n, static_cast<int64_t>(p.B) * g.nseg, stream);
        });
    ok = ok && launch(kKDrawSums, [&] { return launch_draw_sums(pr, plan, stream); }) &&
         launch(kKDrawPick, [&] { return launch_draw_pick(pr, plan, stream); });
    return finish(ok);
}

sv_status_t verify_probs(const Tuning& tu, const void* target_logits, const void* draft_logits,
                         const int32_t* draft_tokens, const int32_t* offsets, int32_t k_uniform,
                         int64_t total_draft, int32_t B, int64_t V, sv_dtype_t dtype, const float* uniforms,
                         const float* temperature, int32_t* out_tokens, int32_t* out_n_accepted, float* out_p,
                         float* out_q, float* out_row_max, float* out_row_sumexp, void* workspace,
                         size_t workspace_bytes, hipStream_t stream) {
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
    Problem p{};
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
    return run(p, workspace, workspace_bytes, stream, tu);
}

sv_status_t verify_gathered(const Tuning& tu, const void* target_logits, const void* draft_logits,
                            const int32_t* draft_tokens, const float* draft_probs, const int32_t* offsets,
                            int32_t k_uniform, int64_t total_draft, int32_t B, int64_t V, sv_dtype_t dtype,
                            const float* uniforms, const float* temperature, int32_t* out_tokens,
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
    return run(p, workspace, workspace_bytes, stream, tu);
}

sv_status_t draft_sample(const Tuning& tu, const void* logits, int32_t rows, int64_t V, sv_dtype_t dtype,
                         const float* temperature, const float* uniforms, int32_t* out_tokens, float* out_probs,
                         void* workspace, size_t workspace_bytes, hipStream_t stream) {
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
    return run(p, workspace, workspace_bytes, stream, tu, /*sample=*/true);
}

}  // namespace

extern "C" {

size_t spec_verify_workspace_size(int32_t B, int64_t total_draft, int64_t V, sv_dtype_t dtype) {
    return workspace_bytes_for(B, total_draft, V, dtype, Tuning{});
}

sv_status_t spec_verify_probs(const void* target_logits, const void* draft_logits,
                              const int32_t* draft_tokens, const int32_t* offsets,
                              int32_t k_uniform, int64_t total_draft, int32_t B, int64_t V,
                              sv_dtype_t dtype, const float* uniforms, const float* temperature,
                              int32_t* out_tokens, int32_t* out_n_accepted, float* out_p,
                              float* out_q, float* out_row_max, float* out_row_sumexp,
                              void* workspace, size_t workspace_bytes, hipStream_t stream) {
    return verify_probs(Tuning{}, target_logits, draft_logits, draft_tokens, offsets, k_uniform, total_draft, B,
                        V, dtype, uniforms, temperature, out_tokens, out_n_accepted, out_p, out_q, out_row_max,
                        out_row_sumexp, workspace, workspace_bytes, stream);
}

sv_status_t spec_verify(const void* target_logits, const void* draft_logits,
                        const int32_t* draft_tokens, const int32_t* offsets, int32_t k_uniform,
                        int64_t total_draft, int32_t B, int64_t V, sv_dtype_t dtype,
                        const float* uniforms, const float* temperature, int32_t* out_tokens,
                        int32_t* out_n_accepted, void* workspace, size_t workspace_bytes,
                        hipStream_t stream) {
    return verify_probs(Tuning{}, target_logits, draft_logits, draft_tokens, offsets, k_uniform, total_draft, B,
                        V, dtype, uniforms, temperature, out_tokens, out_n_accepted, nullptr, nullptr, nullptr,
                        nullptr, workspace, workspace_bytes, stream);
}

sv_status_t spec_verify_noalloc(const void* target_logits, const void* draft_logits,
                                const int32_t* draft_tokens, const int32_t* offsets, int32_t k_uniform,
                                int64_t total_draft, int32_t B, int64_t V, sv_dtype_t dtype,
                                const float* uniforms, const float* temperature, int32_t* out_tokens,
                                int32_t* out_n_accepted, hipStream_t stream) {
    const sv_status_t st = check_args(target_logits, draft_logits, draft_tokens, offsets, k_uniform, total_draft,
                                      B, V, dtype, uniforms, temperature, out_tokens, out_n_accepted);
    if (st != SV_OK) return st;
    if (B == 0) return SV_OK;
    const size_t need = workspace_bytes_for(B, total_draft, V, dtype, Tuning{});
    if (need == 0) return SV_ERR_SHAPE;
    if (need > SV_NOALLOC_SCRATCH_BYTES) return SV_ERR_SCRATCH;
    void* ws = nullptr;
    const sv_status_t sa = scratch_address(&ws);
    if (sa != SV_OK) return sa;
    return verify_probs(Tuning{}, target_logits, draft_logits, draft_tokens, offsets, k_uniform, total_draft, B,
                        V, dtype, uniforms, temperature, out_tokens, out_n_accepted, nullptr, nullptr, nullptr,
                        nullptr, ws, SV_NOALLOC_SCRATCH_BYTES, stream);
}

sv_status_t spec_verify_gathered(const void* target_logits, const void* draft_logits,
                                 const int32_t* draft_tokens, const float* draft_probs,
                                 const int32_t* offsets, int32_t k_uniform, int64_t total_draft,
                                 int32_t B, int64_t V, sv_dtype_t dtype, const float* uniforms,
                                 const float* temperature, int32_t* out_tokens,
                                 int32_t* out_n_accepted, float* out_emit_prob, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
    return verify_gathered(Tuning{}, target_logits, draft_logits, draft_tokens, draft_probs, offsets, k_uniform,
                           total_draft, B, V, dtype, uniforms, temperature, out_tokens, out_n_accepted,
                           out_emit_prob, workspace, workspace_bytes, stream);
}

sv_status_t spec_draft_sample(const void* logits, int32_t rows, int64_t V, sv_dtype_t dtype,
                              const float* temperature, const float* uniforms, int32_t* out_tokens,
                              float* out_probs, void* workspace, size_t workspace_bytes,
                              hipStream_t stream) {
    return draft_sample(Tuning{}, logits, rows, V, dtype, temperature, uniforms, out_tokens, out_probs, workspace,
                        workspace_bytes, stream);
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
        case SV_ERR_SCRATCH: return "call needs more than spec_verify_noalloc's static scratch";
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


// ---- sv_tuning.h: test and benchmark hooks --------------------------------

void spec_tuning_defaults(sv_tuning_t* t) {
    if (!t) return;
    *t = sv_tuning_t{};
    t->lead = kAutoLead;
    t->queue_mode = SV_QUEUE_OVERLAP;
    t->draw_mode = SV_DRAW_AUTO;
}

size_t spec_verify_workspace_size_tuned(const sv_tuning_t* t, int32_t B, int64_t total_draft, int64_t V,
                                        sv_dtype_t dtype) {
    Tuning tu;
    if (!resolve(t, tu)) return 0;
    return workspace_bytes_for(B, total_draft, V, dtype, tu);
}

sv_status_t spec_verify_tuned(const sv_tuning_t* t, const void* target_logits, const void* draft_logits,
                              const int32_t* draft_tokens, const int32_t* offsets, int32_t k_uniform,
                              int64_t total_draft, int32_t B, int64_t V, sv_dtype_t dtype,
                              const float* uniforms, const float* temperature, int32_t* out_tokens,
                              int32_t* out_n_accepted, float* out_p, float* out_q, float* out_row_max,
                              float* out_row_sumexp, void* workspace, size_t workspace_bytes,
                              hipStream_t stream) {
    Tuning tu;
    if (!resolve(t, tu)) return SV_ERR_SHAPE;
    return verify_probs(tu, target_logits, draft_logits, draft_tokens, offsets, k_uniform, total_draft, B, V,
                        dtype, uniforms, temperature, out_tokens, out_n_accepted, out_p, out_q, out_row_max,
                        out_row_sumexp, workspace, workspace_bytes, stream);
}

sv_status_t spec_verify_gathered_tuned(const sv_tuning_t* t, const void* target_logits,
                                       const void* draft_logits, const int32_t* draft_tokens,
                                       const float* draft_probs, const int32_t* offsets, int32_t k_uniform,
                                       int64_t total_draft, int32_t B, int64_t V, sv_dtype_t dtype,
                                       const float* uniforms, const float* temperature, int32_t* out_tokens,
                                       int32_t* out_n_accepted, float* out_emit_prob, void* workspace,
                                       size_t workspace_bytes, hipStream_t stream) {
    Tuning tu;
    if (!resolve(t, tu)) return SV_ERR_SHAPE;
    return verify_gathered(tu, target_logits, draft_logits, draft_tokens, draft_probs, offsets, k_uniform,
                           total_draft, B, V, dtype, uniforms, temperature, out_tokens, out_n_accepted,
                           out_emit_prob, workspace, workspace_bytes, stream);
}

sv_status_t spec_draft_sample_tuned(const sv_tuning_t* t, const void* logits, int32_t rows, int64_t V,
                                    sv_dtype_t dtype, const float* temperature, const float* uniforms,
                                    int32_t* out_tokens, float* out_probs, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream) {
    Tuning tu;
    if (!resolve(t, tu)) return SV_ERR_SHAPE;
    return draft_sample(tu, logits, rows, V, dtype, temperature, uniforms, out_tokens, out_probs, workspace,
                        workspace_bytes, stream);
}

const char* spec_verify_kernel_name(int32_t i) {
    return (i >= 0 && i < kNumKernels) ? kKernelNames[i] : nullptr;
}

sv_status_t spec_timing_events_create(int32_t n, hipEvent_t* ev) {
    if (n < 0) return SV_ERR_SHAPE;
    if (n > 0 && !ev) return SV_ERR_NULL;
    for (int32_t i = 0; i < n; ++i) {
        if (hipEventCreate(&ev[i]) != hipSuccess) {
            for (int32_t j = 0; j < i; ++j) (void)hipEventDestroy(ev[j]);
            return SV_ERR_HIP;
        }
    }
    return SV_OK;
}

sv_status_t spec_timing_elapsed(hipEvent_t start, hipEvent_t stop, float* ms) {
    if (!start || !stop || !ms) return SV_ERR_NULL;
    if (hipEventSynchronize(stop) != hipSuccess) return SV_ERR_HIP;
    return hipEventElapsedTime(ms, start, stop) == hipSuccess ? SV_OK : SV_ERR_HIP;
}

sv_status_t spec_timing_events_destroy(int32_t n, hipEvent_t* ev) {
    if (n < 0) return SV_ERR_SHAPE;
    if (n > 0 && !ev) return SV_ERR_NULL;
    sv_status_t st = SV_OK;
    for (int32_t i = 0; i < n; ++i)
        if (ev[i] && hipEventDestroy(ev[i]) != hipSuccess) st = SV_ERR_HIP;
    return st;
}

sv_status_t spec_stream_probe(const void* data, int64_t bytes, int64_t seg_bytes, uint32_t* out,
                              hipStream_t stream) {
    if (bytes < 0 || seg_bytes < 4096 || seg_bytes % 16 != 0 || seg_bytes > (1ll << 30)) return SV_ERR_SHAPE;
    if ((bytes + seg_bytes - 1) / seg_bytes > 0x7FFFFFFFll) return SV_ERR_SHAPE;
    if (bytes > 0 && (!data || !out)) return SV_ERR_NULL;
    if (!aligned(data, 16) || !aligned(out, 4)) return SV_ERR_ALIGN;
    return launch_stream_probe(data, bytes, seg_bytes, out, stream) == hipSuccess ? SV_OK : SV_ERR_HIP;
}

}  // extern "C"
