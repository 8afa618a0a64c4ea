// host_args.cpp -- host-side argument checks and work geometry (declared,
// with what each computes, in host_args.h).
#include "host_args.h"

namespace sv {
namespace host {

bool resolve(const sv_tuning_t* t, Tuning& r) {
    r = Tuning{};
    if (!t) return true;
    if (t->seg_elems < 0 || t->chunk_elems < 0 || t->lead < kAutoLead || t->lead > SV_K_MAX + 1 ||
        t->queue_mode < SV_QUEUE_OVERLAP || t->queue_mode > SV_QUEUE_HANDOFF || t->lag_accept < 0 ||
        t->lag_draw < 0 || t->draw_mode < SV_DRAW_AUTO || t->draw_mode > SV_DRAW_THREE)
        return false;
    r.seg_elems = t->seg_elems;
    r.chunk_elems = t->chunk_elems;
    r.lead = t->lead;
    r.queue_mode = t->queue_mode;
    r.lag_a = t->lag_accept;
    r.lag_c = t->lag_draw;
    r.draw_mode = t->draw_mode;
    r.item_polls = t->item_polls ? t->item_polls : kItemPolls;
    r.timed = t->timed;
    r.events = t->events;
    r.launched = t->launched;
    return true;
}

void auto_lengths(int32_t B, int64_t total, int64_t V, const Tuning& tu, int64_t* seg, int64_t* chunk) {
    const int64_t rows = 2 * total + B;
    // (a product that would pass the default length saturates there: for the
    // largest arguments rows * V does not fit 64 bits)
    int64_t s = rows > kDefaultSegElems * kRowBlocks / V ? kDefaultSegElems : rows * V / kRowBlocks;
    int64_t c = B > kDefaultChunkElems * kDrawBlocks / V ? kDefaultChunkElems : static_cast<int64_t>(B) * V / kDrawBlocks;
    s = s < kMinSeg ? kMinSeg : (s > kDefaultSegElems ? kDefaultSegElems : s);
    c = c < kMinChunk ? kMinChunk : (c > kDefaultChunkElems ? kDefaultChunkElems : c);
    *seg = tu.seg_elems ? tu.seg_elems : s;
    *chunk = tu.chunk_elems ? tu.chunk_elems : c;
}

int64_t lead_multiplier(int32_t B) {
    if (B <= 2) return 1;
    int64_t m = static_cast<int64_t>(0.6180339887498949 * B);
    if (m < 1) m = 1;
    auto gcd = [](int64_t a, int64_t b) {
        while (b) {
            const int64_t t = a % b;
            a = b;
            b = t;
        }
        return a;
    };
    while (gcd(m, B) != 1) ++m;                  // (ends: B - 1 is coprime with B)
    return m;
}

int64_t rounds_lead_blocks(int32_t B, int32_t lead, int32_t nseg) {
    return static_cast<int64_t>(B) * lead * 2 * nseg;
}

int64_t rounds_rest_blocks(int32_t B, int64_t total, bool has_offsets, int32_t k_uniform, int32_t lead, int32_t nseg,
                           int32_t nchunk) {
    int64_t per = 2 * (static_cast<int64_t>(k_uniform) - lead) + 1;
    if (per < 0) per = 0;
    const int64_t rows = has_offsets ? 2 * total + B : static_cast<int64_t>(B) * per;
    return rows * nseg + static_cast<int64_t>(B) * (1 + nchunk);
}

int32_t effective_lead(int64_t B, int64_t total, int64_t V, sv_dtype_t dtype, const Tuning& tu, bool gathered) {
    if (tu.lead != kAutoLead) return tu.lead;
    if (total == 0) return 0;                    // only bonus rows: nothing to skip
    // (in double: no product of the sizes can overflow)
    const double rows = static_cast<double>(gathered ? total + B : 2 * total + B);
    const double bytes = rows * static_cast<double>(V) * (dtype == SV_BF16 ? 2.0 : 4.0);
    return bytes >= static_cast<double>(gathered ? kAutoLeadBytesGathered : kAutoLeadBytes) ? 1 : 0;
}

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
    if (rows > 0x7FFFFFFFll / g.nseg) return false;   // (checked first: rows * nseg may not fit 64 bits)
    if (rows * g.nseg + static_cast<int64_t>(B) * (1 + g.nchunk) > 0x7FFFFFFFll) return false;
    // (the epoch counter first, at the same place for every geometry)
    g.off_epoch = 0;
    size_t off = align256(2 * sizeof(uint32_t));
    g.off_seg = off;
    off = align256(off + sizeof(SegStat) * static_cast<size_t>(rows) * g.nseg);
    g.off_task = off;
    off = align256(off + sizeof(TaskRec) * static_cast<size_t>(B));
    g.off_csum = off;
    off = align256(off + sizeof(ChunkSums) * kWaves * static_cast<size_t>(B) * g.nchunk);
    g.off_band_n = off;
    off = align256(off + sizeof(int32_t) * kWaves * static_cast<size_t>(B) * g.nchunk);
    g.off_band_w = off;
    off = align256(off + sizeof(double) * 2 * kWaves * kWaveCap * static_cast<size_t>(B) * g.nchunk);
    g.off_xlogit = off;
    off = align256(off + sizeof(float) * static_cast<size_t>(rows));
    g.off_done = off;
    off = align256(off + sizeof(int32_t) * static_cast<size_t>(B));
    const size_t entries = static_cast<size_t>(rows) * g.nseg + static_cast<size_t>(B) * (1 + g.nchunk);
    g.off_sched = off;
    off = align256(off + sizeof(SchedEntry) * entries);
    g.off_blk_ctr = off;
    off = align256(off + sizeof(uint64_t));
    g.off_blk_seq = off;
    off = align256(off + sizeof(uint64_t) * static_cast<size_t>(B));
    g.off_dlist = off;
    off = align256(off + sizeof(RestItem) * static_cast<size_t>(B) * g.nseg);
    g.off_dlist_n = off;
    off = align256(off + sizeof(uint32_t));
    g.off_nbuf = off;                                   // accept counts of spec_draft_sample
    off = align256(off + sizeof(int32_t) * static_cast<size_t>(B));
    g.off_aband = off;
    off = align256(off + sizeof(int32_t) * static_cast<size_t>(B));
    g.off_picked = off;
    off = align256(off + sizeof(uint32_t) * static_cast<size_t>(B));
    g.off_lead_ctr = off;
    off = align256(off + sizeof(uint64_t) * static_cast<size_t>(B));
    g.off_lead_clr = off;
    off = align256(off + sizeof(uint32_t));
    g.off_lead_done = off;
    off = align256(off + sizeof(uint64_t));
    g.off_stall = off;
    off = align256(off + sizeof(uint32_t));
    g.off_lead_rec = off;
    off = align256(off + sizeof(LeadRec) * 2 * kPolledSegs * static_cast<size_t>(B));
    g.bytes = off;
    return true;
}


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

size_t workspace_bytes_for(int32_t B, int64_t total, int64_t V, sv_dtype_t dtype, const Tuning& tu) {
    if (B < 0 || total < 0 || V < 1 || V > 0x7FFFFFFFll) return 0;
    if (dtype != SV_F32 && dtype != SV_BF16) return 0;
    Geometry g;
    int64_t seg_elems, chunk_elems;
    auto_lengths(B, total, V, tu, &seg_elems, &chunk_elems);
    if (!make_geometry(B, total, V, dtype, seg_elems, chunk_elems, g)) return 0;
    return g.bytes;
}

}  // namespace host
}  // namespace sv
