// host_args.h -- the host-side checks and work geometry of a call: argument
// validation, per-call tuning, segment and chunk lengths, and the layout of
// the workspace.  Plain C++ (no device code), so that it also builds with a
// host compiler under address and undefined-behaviour sanitizers.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/specverify.h"
#include "sv_layout.h"
#include "sv_tuning.h"

namespace sv {
namespace host {

constexpr int64_t kDefaultSegElems = 65536;   // row-pass segment length before rounding
// Row-pass segments are whole load windows: 256 lanes x 16 B x the window
// depth (8 loads for bf16, 4 for fp32), so only a row's last segment can end
// inside a window.
inline int64_t row_unit(sv_dtype_t dtype) { return dtype == SV_BF16 ? 256 * 8 * 8 : 256 * 4 * 4; }
constexpr int64_t kDefaultChunkElems = 8192;  // draw chunk length before rounding
// Early exit pays for its first round's scans and its pick launch only when
// the rows it may skip take longer than those to stream: automatic mode
// (lead -1) uses one leading position when the rows a full pass reads hold
// at least kAutoLeadBytes (target and draft rows) or, in the gathered form
// (target rows only, with its own launches), kAutoLeadBytesGathered, and
// one full pass otherwise.  Both are the sizes where the two forms took
// equally long on an MI355X (bf16, V = 128256 and 152064, one full pass
// against one leading position over a range of batch sizes).
constexpr int32_t kAutoLead = -1;
constexpr int64_t kAutoLeadBytes = 192ll << 20;
constexpr int64_t kAutoLeadBytesGathered = 320ll << 20;

// Early exit: bound of a second-round workgroup's wait for its item (one
// poll takes a memory round trip and a short sleep, about a microsecond).
constexpr uint32_t kItemPolls = 1u << 22;

// One call's tuning (sv_tuning.h), resolved: every field in range.
struct Tuning {
    int64_t seg_elems = 0, chunk_elems = 0;   // 0: automatic (auto_lengths)
    int32_t lead = kAutoLead;
    int32_t queue_mode = SV_QUEUE_OVERLAP;
    int32_t lag_a = 0, lag_c = 0;             // 0: chosen from the resident grid
    int32_t draw_mode = SV_DRAW_AUTO;
    uint32_t item_polls = kItemPolls;
    uint32_t timed = 0;                       // kernels whose events are recorded
    hipEvent_t* events = nullptr;
    uint32_t* launched = nullptr;
};

// Reads a caller's tuning (NULL: the defaults); false if a field is out of range.
bool resolve(const sv_tuning_t* t, Tuning& r);

// Automatic segment and chunk lengths: the defaults suit batches that fill
// the GPU many times over (256 sequences of k = 8, V = 152064: 8704 row
// workgroups, 4864 draw workgroups);
// a small call is cut finer so its row pass still has about kRowBlocks
// workgroups and its draw about kDrawBlocks (no finer than kMinSeg /
// kMinChunk logits).
constexpr int64_t kRowBlocks = 2048, kDrawBlocks = 1024;
constexpr int64_t kMinSeg = 8192, kMinChunk = 1024;
void auto_lengths(int32_t B, int64_t total, int64_t V, const Tuning& tu, int64_t* seg, int64_t* chunk);

// Leading positions read first (early exit): the tuning's, or 1 when the
// rows a full pass reads hold at least kAutoLeadBytes (kAutoLeadBytesGathered
// in the gathered form), 0 for calls without drafts.
int32_t effective_lead(int64_t B, int64_t total, int64_t V, sv_dtype_t dtype, const Tuning& tu,
                       bool gathered = false);

// The first round visits sequence (j * m) mod B as its j-th: m is coprime
// with B (so every sequence is visited once) and near 0.618 B, which spreads
// neighbouring sequences apart, so that the order in which the first round
// finishes, and lists, does not follow how the caller ordered the batch.
int64_t lead_multiplier(int32_t B);

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

struct Geometry {
    int32_t nseg, nchunk;
    int64_t seg_len, chunk_len;
    size_t off_seg, off_task, off_csum, off_band_n, off_band_w, off_xlogit, off_done, off_sched,
        off_blk_ctr, off_blk_seq, off_dlist, off_dlist_n, off_nbuf, off_aband, off_picked,
        off_lead_ctr, off_lead_clr, off_lead_done, off_stall, off_lead_rec, off_epoch, bytes;
};

// Splits a row of V logits into n <= max_pieces pieces of about `target`
// elements, each a multiple of `unit` long (see host_args.cpp).
void split(int64_t V, int64_t target, int64_t max_pieces, int64_t unit, int64_t max_len, int32_t& n,
           int64_t& len);

// The segment and chunk geometry and the workspace layout of a call; false
// when the second round's grid would not fit 2^31 - 1 workgroups (a call
// whose two-round launch, the first round's workgroups included, would not
// fit runs as one pass).
bool make_geometry(int32_t B, int64_t total, int64_t V, sv_dtype_t dtype, int64_t seg_elems,
                   int64_t chunk_elems, Geometry& g);

// Workgroups of early exit's two-round launch: the first round's (every
// sequence's leading rows, lead x 2 x nseg each), then enough for every item
// the first round's scans can list.  An undecided sequence lists its
// remaining row segments, an accept item and nchunk draw items; a settled
// sampling sequence nchunk draw items.  With a uniform k an undecided
// sequence has at most 2 (k - lead) + 1 remaining rows (none when lead > k);
// with offsets, every row of the call bounds them.
int64_t rounds_lead_blocks(int32_t B, int32_t lead, int32_t nseg);
int64_t rounds_rest_blocks(int32_t B, int64_t total, bool has_offsets, int32_t k_uniform, int32_t lead, int32_t nseg,
                           int32_t nchunk);

inline bool aligned(const void* ptr, size_t a) { return (reinterpret_cast<uintptr_t>(ptr) % a) == 0; }

// The argument checks of spec_verify and its variants (before anything is enqueued).
sv_status_t check_args(const void* target, const void* draft, const int32_t* tokens,
                       const int32_t* offsets, int32_t k_uniform, int64_t total, int32_t B,
                       int64_t V, sv_dtype_t dtype, const float* uniforms, const float* temperature,
                       const int32_t* out_tokens, const int32_t* out_n);

// Workspace bytes of a call (0 on bad sizes).
size_t workspace_bytes_for(int32_t B, int64_t total, int64_t V, sv_dtype_t dtype, const Tuning& tu);

}  // namespace host
}  // namespace sv
