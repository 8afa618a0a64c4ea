// host_args_check.cpp -- drives the host-side argument checks and work
// geometry (speculative_decoding_rejection_spec_amd/csrc/host_args.cpp)
// through valid, invalid and extreme arguments; tests/test_sanitizers.py
// builds it with address and undefined-behaviour sanitizers (any overflow,
// out-of-bounds access or misaligned read aborts the run).  Prints "ok" and
// exits 0 when every check holds.
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <random>
#include <vector>

#include "host_args.h"

using namespace sv;
using namespace sv::host;

static int failures = 0;
#define CHECK(cond)                                                              \
    do {                                                                         \
        if (!(cond)) {                                                           \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
            ++failures;                                                          \
        }                                                                        \
    } while (0)

static const void* fake(uintptr_t a) { return reinterpret_cast<const void*>(a); }

static sv_status_t call(const void* target, const void* draft, const void* tokens, const void* offsets, int32_t k,
                        int64_t total, int32_t B, int64_t V, int32_t dtype, const void* unif, const void* temp,
                        const void* out_tok, const void* out_n) {
    return check_args(target, draft, static_cast<const int32_t*>(tokens), static_cast<const int32_t*>(offsets), k,
                      total, B, V, static_cast<sv_dtype_t>(dtype), static_cast<const float*>(unif),
                      static_cast<const float*>(temp), static_cast<const int32_t*>(out_tok),
                      static_cast<const int32_t*>(out_n));
}

// The geometry of a call covers every logit once, in pieces of the promised
// sizes, and lays the workspace out in increasing, 256-byte-aligned blocks.
static void check_geometry(int32_t B, int64_t total, int64_t V, sv_dtype_t dt, const Tuning& tu) {
    int64_t seg = 0, chunk = 0;
    auto_lengths(B, total, V, tu, &seg, &chunk);
    Geometry g;
    if (!make_geometry(B, total, V, dt, seg, chunk, g)) {
        CHECK(workspace_bytes_for(B, total, V, dt, tu) == 0);
        return;
    }
    CHECK(g.nseg >= 1 && g.seg_len >= 1 && g.nseg * g.seg_len >= V && (g.nseg - 1) * g.seg_len < V);
    CHECK(g.nchunk >= 1 && g.nchunk <= kMaxChunks && g.nchunk * g.chunk_len >= V &&
          (g.nchunk - 1) * g.chunk_len < V);
    CHECK(g.chunk_len % 8 == 0);
    if (V > max_seg_elems(dt) && tu.seg_elems == 0) CHECK(g.seg_len <= max_seg_elems(dt));
    const size_t offs[] = {g.off_epoch,   g.off_seg,     g.off_task,     g.off_csum,     g.off_band_n,    g.off_band_w,
                           g.off_xlogit,  g.off_done,     g.off_sched,    g.off_blk_ctr,   g.off_blk_seq,
                           g.off_dlist,   g.off_dlist_n,  g.off_nbuf,     g.off_aband,     g.off_picked,
                           g.off_lead_ctr, g.off_lead_clr, g.off_lead_done, g.off_stall,    g.off_lead_rec,
                           g.bytes};
    for (size_t i = 0; i < sizeof(offs) / sizeof(offs[0]); ++i) {
        CHECK(offs[i] % 256 == 0);
        if (i > 0) CHECK(offs[i] >= offs[i - 1]);
    }
    // every record the kernels index fits before the next block; the epoch
    // counter (two words) first, at the same offset for every geometry
    CHECK(g.off_epoch == 0 && g.off_seg >= 2 * sizeof(uint32_t));
    const size_t rows = static_cast<size_t>(2 * total + B);
    CHECK(g.off_task - g.off_seg >= sizeof(SegStat) * rows * static_cast<size_t>(g.nseg));
    CHECK(g.off_task + sizeof(TaskRec) * static_cast<size_t>(B) <= g.off_csum);
    const size_t entries = rows * g.nseg + static_cast<size_t>(B) * (1 + g.nchunk);
    CHECK(g.off_sched + sizeof(SchedEntry) * entries <= g.off_blk_ctr);
    CHECK(g.off_blk_seq + sizeof(uint64_t) * static_cast<size_t>(B) <= g.off_dlist);
    CHECK(g.off_lead_rec + sizeof(LeadRec) * 2 * kPolledSegs * static_cast<size_t>(B) <= g.bytes);
    CHECK(g.bytes == workspace_bytes_for(B, total, V, dt, tu));
}

int main() {
    // ---- argument checks: the codes the C ABI documents --------------------
    const void *t = fake(0x10000), *d = fake(0x20000), *x = fake(0x30000), *u = fake(0x40000),
               *T = fake(0x50000), *ot = fake(0x60000), *on = fake(0x70000), *off = fake(0x90000);
    CHECK(call(t, d, x, nullptr, 4, 4, 1, 32000, SV_F32, u, T, ot, on) == SV_OK);
    CHECK(call(nullptr, d, x, nullptr, 4, 4, 1, 32000, SV_F32, u, T, ot, on) == SV_ERR_NULL);
    CHECK(call(t, d, x, nullptr, 4, 4, 1, 32000, SV_F32, nullptr, T, ot, on) == SV_ERR_NULL);
    CHECK(call(t, nullptr, x, nullptr, 4, 4, 1, 32000, SV_F32, u, T, ot, on) == SV_ERR_NULL);
    CHECK(call(t, nullptr, nullptr, nullptr, 0, 0, 1, 32000, SV_F32, u, T, ot, on) == SV_OK);
    CHECK(call(t, d, x, nullptr, 4, 4, 1, 32000, 2, u, T, ot, on) == SV_ERR_DTYPE);
    CHECK(call(t, d, x, nullptr, 4, 4, 1, 0, SV_F32, u, T, ot, on) == SV_ERR_SHAPE);
    CHECK(call(t, d, x, nullptr, 4, 4, 1, 1ll << 31, SV_F32, u, T, ot, on) == SV_ERR_SHAPE);
    CHECK(call(t, d, x, nullptr, 4, 4, -1, 32000, SV_F32, u, T, ot, on) == SV_ERR_SHAPE);
    CHECK(call(t, d, x, nullptr, 64, 64, 1, 32000, SV_F32, u, T, ot, on) == SV_ERR_SHAPE);
    CHECK(call(t, d, x, nullptr, -1, -1, 1, 32000, SV_F32, u, T, ot, on) == SV_ERR_SHAPE);
    CHECK(call(t, d, x, nullptr, 4, 5, 1, 32000, SV_F32, u, T, ot, on) == SV_ERR_SHAPE);
    CHECK(call(t, d, x, off, 0, 64 * 2, 2, 32000, SV_F32, u, T, ot, on) == SV_ERR_SHAPE);
    CHECK(call(t, d, x, off, 0, 0x7FFFFFFFll * 63, 0x7FFFFFFF, 32000, SV_F32, u, T, ot, on) == SV_OK);
    CHECK(call(fake(0x10002), d, x, nullptr, 4, 4, 1, 32000, SV_F32, u, T, ot, on) == SV_ERR_ALIGN);
    CHECK(call(fake(0x10001), d, x, nullptr, 4, 4, 1, 32000, SV_BF16, u, T, ot, on) == SV_ERR_ALIGN);
    CHECK(call(t, d, fake(0x30002), nullptr, 4, 4, 1, 32000, SV_F32, u, T, ot, on) == SV_ERR_ALIGN);
    CHECK(call(t, d, x, fake(0x90001), 0, 4, 1, 32000, SV_F32, u, T, ot, on) == SV_ERR_ALIGN);
    CHECK(call(t, d, x, nullptr, 0x7FFFFFFF / 63, (0x7FFFFFFF / 63) * 0x7FFFFFFFll, 0x7FFFFFFF, 1,
               SV_F32, u, T, ot, on) == SV_ERR_SHAPE);

    // ---- tuning fields -----------------------------------------------------
    Tuning tu;
    CHECK(resolve(nullptr, tu) && tu.lead == kAutoLead && tu.seg_elems == 0);
    sv_tuning_t raw{};
    raw.lead = kAutoLead;
    CHECK(resolve(&raw, tu));
    const int32_t bad_lead[] = {-2, SV_K_MAX + 2, -1000000};
    for (int32_t l : bad_lead) { raw.lead = l; CHECK(!resolve(&raw, tu)); }
    raw.lead = 0;
    raw.queue_mode = 3; CHECK(!resolve(&raw, tu)); raw.queue_mode = 0;
    raw.draw_mode = -1; CHECK(!resolve(&raw, tu)); raw.draw_mode = 0;
    raw.lag_accept = -1; CHECK(!resolve(&raw, tu)); raw.lag_accept = 0;
    raw.seg_elems = -5; CHECK(!resolve(&raw, tu)); raw.seg_elems = 0;
    CHECK(resolve(&raw, tu) && tu.lead == 0 && tu.item_polls == kItemPolls);
    raw.item_polls = 3;
    CHECK(resolve(&raw, tu) && tu.item_polls == 3);

    // ---- geometry and workspace layout -------------------------------------
    const Tuning dflt;
    const int64_t Vs[] = {1, 2, 7, 8, 1000, 4099, 32000, 40000, 128256, 152064, 1 << 20};
    const int32_t Bs[] = {1, 2, 64, 256, 512, 2049};
    for (int64_t V : Vs)
        for (int32_t B : Bs)
            for (int dt = 0; dt < 2; ++dt) {
                check_geometry(B, 0, V, static_cast<sv_dtype_t>(dt), dflt);
                check_geometry(B, static_cast<int64_t>(B) * 8, V, static_cast<sv_dtype_t>(dt), dflt);
                check_geometry(B, static_cast<int64_t>(B) * SV_K_MAX, V, static_cast<sv_dtype_t>(dt), dflt);
            }
    std::mt19937_64 rng(7);
    for (int i = 0; i < 2000; ++i) {
        const int32_t B = static_cast<int32_t>(rng() % 5000);
        const int64_t total = static_cast<int64_t>(B) * static_cast<int64_t>(rng() % (SV_K_MAX + 1));
        const int64_t V = 1 + static_cast<int64_t>(rng() % 300000);
        Tuning tt;
        if (i % 3 == 0) { tt.seg_elems = 1 + static_cast<int64_t>(rng() % 200000); }
        if (i % 5 == 0) { tt.chunk_elems = 1 + static_cast<int64_t>(rng() % 50000); }
        check_geometry(B, total, V, static_cast<sv_dtype_t>(i & 1), tt);
        CHECK(effective_lead(B, total, V, static_cast<sv_dtype_t>(i & 1), dflt) >= 0);
        CHECK(effective_lead(B, total, V, static_cast<sv_dtype_t>(i & 1), dflt, true) >= 0);
    }
    // the automatic form at the measured crossovers: one pass below 192 MiB
    // of rows (target and draft), early exit above; the gathered form counts
    // target rows against 320 MiB; calls without drafts take one pass; a
    // lead set in the tuning wins
    CHECK(effective_lead(64, 64 * 4, 128256, SV_BF16, dflt) == 0);          // C3: 148 MB
    CHECK(effective_lead(32, 32 * 8, 152064, SV_BF16, dflt) == 0);          // 165 MB
    CHECK(effective_lead(48, 48 * 8, 152064, SV_BF16, dflt) == 1);          // 248 MB
    CHECK(effective_lead(256, 256 * 8, 152064, SV_BF16, dflt) == 1);        // C4
    CHECK(effective_lead(96, 96 * 8, 152064, SV_BF16, dflt, true) == 0);    // gathered: 280 MB of target rows
    CHECK(effective_lead(128, 128 * 8, 152064, SV_BF16, dflt, true) == 1);  // gathered: 373 MB
    CHECK(effective_lead(4096, 0, 152064, SV_BF16, dflt) == 0);             // bonus rows only
    {
        Tuning t0;
        t0.lead = 0;
        CHECK(effective_lead(256, 256 * 8, 152064, SV_BF16, t0) == 0);
        t0.lead = 3;
        CHECK(effective_lead(1, 1, 100, SV_F32, t0) == 3);
    }
    // extremes: sizes whose workspace or grid cannot be formed give 0, without overflow
    CHECK(workspace_bytes_for(0x7FFFFFFF, 0x7FFFFFFFll * 63, 0x7FFFFFFF, SV_BF16, dflt) == 0);
    CHECK(workspace_bytes_for(-1, 0, 10, SV_F32, dflt) == 0);
    CHECK(workspace_bytes_for(1, -1, 10, SV_F32, dflt) == 0);
    CHECK(workspace_bytes_for(1, 0, 0, SV_F32, dflt) == 0);
    CHECK(workspace_bytes_for(1, 0, 10, static_cast<sv_dtype_t>(7), dflt) == 0);
    check_geometry(1, 0, 0x7FFFFFFF, SV_F32, dflt);
    check_geometry(4096, 4096ll * 8, 152064, SV_BF16, dflt);

    // the two-round grid holds every item the first round's scans can list:
    // an undecided greedy sequence lists target rows lead..k (when k >= lead),
    // an undecided sampling sequence target and draft rows lead..k-1 (its bonus
    // row is read by its draw alone; when k > lead), each nseg segments, plus
    // an accept item and nchunk draw items; a settled sampling sequence nchunk
    // draw items
    auto max_items = [](int64_t k, int64_t lead, int64_t nseg, int64_t nchunk) {
        int64_t m = nchunk;                                              // settled, sampling
        if (k >= lead) m = std::max(m, (k - lead + 1) * nseg + 1 + nchunk);        // undecided, greedy
        if (k > lead) m = std::max(m, 2 * (k - lead) * nseg + 1 + nchunk);         // undecided, sampling
        return m;
    };
    const int32_t nsegs[] = {1, 2, 3, 19}, nchunks[] = {1, 19, 256};
    for (int32_t k = 0; k <= SV_K_MAX; ++k)
        for (int32_t lead = 1; lead <= SV_K_MAX + 1; ++lead)
            for (int32_t ns : nsegs)
                for (int32_t nc : nchunks) {
                    const int32_t B = 3;
                    CHECK(rounds_rest_blocks(B, static_cast<int64_t>(B) * k, false, k, lead, ns, nc) >=
                          B * max_items(k, lead, ns, nc));
                    CHECK(rounds_lead_blocks(B, lead, ns) == static_cast<int64_t>(B) * lead * 2 * ns);
                }
    for (int i = 0; i < 500; ++i) {              // ragged k with offsets
        const int32_t B = 1 + static_cast<int32_t>(rng() % 300);
        const int32_t lead = 1 + static_cast<int32_t>(rng() % 4);
        const int32_t ns = nsegs[rng() % 4], nc = nchunks[rng() % 3];
        int64_t total = 0, need = 0;
        for (int32_t b = 0; b < B; ++b) {
            const int64_t k = static_cast<int64_t>(rng() % (SV_K_MAX + 1));
            total += k;
            need += max_items(k, lead, ns, nc);
        }
        CHECK(rounds_rest_blocks(B, total, true, 0, lead, ns, nc) >= need);
    }

    // the first round's order visits every sequence once
    for (int32_t B = 1; B <= 3000; B += (B < 600 ? 1 : 97)) {
        const int64_t m = lead_multiplier(B);
        CHECK(m >= 1);
        std::vector<char> seen(static_cast<size_t>(B), 0);
        for (int64_t j = 0; j < B; ++j) seen[static_cast<size_t>(j * m % B)] = 1;
        for (int32_t b = 0; b < B; ++b) CHECK(seen[static_cast<size_t>(b)]);
    }
    CHECK(lead_multiplier(0x7FFFFFFF) >= 1);

    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("ok\n");
    return 0;
}
