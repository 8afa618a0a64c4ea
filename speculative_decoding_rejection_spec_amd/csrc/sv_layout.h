// sv_layout.h -- sizes and records of the workspace, shared by the kernels
// and the host code that lays the workspace out (plain C++: the host-side
// argument checks in host_args.cpp compile with any C++17 compiler).
#pragma once

#include <stdint.h>

#include "../../include/specverify.h"

namespace sv {

constexpr int kThreads = 256;          // workgroup size of every kernel (4 x wave64)
constexpr int kWaves = kThreads / 64;
constexpr int kKMax = SV_K_MAX;
constexpr int kWaveCap = 8;            // band tokens listed per wave of a draw chunk
constexpr int kMaxChunks = 256;        // draw chunks per row (the pick keeps a mass per sub-chunk in LDS)
// Row pass: the longest segment, so that each lane's fp32 partial sums
// take at most 40 vectors (16 bytes: 8 bf16 or 4 fp32 logits) each.
constexpr int64_t max_seg_elems(int32_t dtype) {
    return 40 * kThreads * (dtype == SV_BF16 ? 8 : 4);
}

// Statistics of one segment of one logit row, as two 64-bit words, each
// written and read whole.  `head` packs the largest logit m of the segment
// (exact; low 32 bits, fp32) with, for sampling rows, the integer-valued
// reference exponent R >= max(z) * c - 2, c = log2(e)/T (row_scale below;
// fp32 bits), and for greedy rows the lowest token id holding m.  `s` is, for
// sampling rows, the sum over the segment of 2^(z*c - R) (0 for greedy
// rows), so every rescale is an exact power of two.  kUnset64 in a word
// marks it not yet written; a captured logit not yet written is kUnset32.
struct SegStat {
    uint64_t head;
    double s;
};
constexpr uint64_t kUnset64 = ~0ull;
constexpr uint32_t kUnset32 = ~0u;

// kResidualPending: a residual draw of the gathered form, whose draft row n
// is read after the accept scan (its maximum and normaliser come from that
// row's SegStats; DrawTask::theta holds log2 S_p until then).
// kTaskUnset: what a read of a task the call has not (yet) written returns
// (its record still carries an earlier call's epoch).
// kBonusSelf: a bonus draw whose row the row pass did not read (early exit
// beside the draws): the draw takes the weights relative to references of
// its own, and the pick checks the row's maximum (a non-finite one makes the
// sequence a data error).
enum : int32_t { kTaskUnset = -1, kNone = 0, kResidual = 1, kBonus = 2, kResidualPending = 3, kBonusSelf = 4 };

// The draw one sequence still needs after the accept scan (as a kernel
// holds it; TaskRec is its form in the workspace).
struct DrawTask {
    int32_t kind;      // kNone (greedy, error), kResidual (n < k), kBonus or kBonusSelf (n = k)
    int32_t out_slot;  // index into out_tokens of the emitted token
    int64_t trow;      // target row at position n
    int64_t drow;      // draft row at position n (kResidual only)
    float m_t, m_d;    // exact maxima of those rows
    float T, u;        // temperature and the draw uniform
    double theta;      // log2(S_p / S_q) from the row pass: p_v > q_v iff d_v > theta
};

// Rows of at most this many segments have their statistics handed to an
// accept scan by the wave that polled for them (accept_scan.h's Polled;
// LeadRec below).
constexpr int kPolledSegs = 2;

// What one first-round workgroup of early exit (one leading position per
// sequence, rows of at most kPolledSegs segments) hands to its sequence's
// accept scan: its segment's head (two words: low, high half) and sum (two
// words), and the logit of the drafted token if its segment holds it (one
// word, else 0), each word with the call's epoch in its high half.  Every
// first-round workgroup writes its record, also one whose row is not read
// (then the words carry the epoch and nothing else), so the scan waits for
// a fixed set of records.  Indexed [sequence][target, draft][segment].
struct LeadRec {
    uint64_t w[5];
};

// A DrawTask in the workspace: nine 64-bit words, each with the number
// (epoch) of the call that wrote it in its high half and one 32-bit field in
// its low half: kind, trow, drow, m_t, m_d, T, u, and theta's low and high
// words (out_slot is trow).  A reader takes the task once every word carries
// its call's epoch, so the writer's stores may land in any order and a task
// of an earlier call reads as not yet written.  One record per 128-byte line.
struct alignas(128) TaskRec {
    uint64_t w[9];
};

// Partial sums of the draw over one sub-chunk (fp64).
struct ChunkSums {
    double sp;   // sum of w_t = exp((z_t - m_t)/T) over the chunk
    double sq;   // sum of w_d over the chunk (residual)
    double a;    // sum of w_t over tokens robustly classified p > q
    double b;    // sum of w_d over the same tokens
};

// One work item of the second early-exit round: a row segment (kind
// kItemDraft / kItemTarget), the accept scan of an undecided sequence
// (kItemAccept), or one draw chunk of such a sequence (kItemChunk).  The
// gathered form's row lists use the row-segment kinds.
// kItemChunkSeq: a draw chunk of a sampling sequence its leading positions
// settled (b is the sequence itself; its task is written before the item is
// listed).
enum : int32_t { kItemDraft = 0, kItemTarget = 1, kItemAccept = 2, kItemChunk = 3, kItemChunkSeq = 4 };
struct RestItem {
    int32_t b;      // row segments and kItemChunkSeq: the sequence; accept and kItemChunk items: its block
    int32_t row;    // row segments: row index in its array
    int32_t kseg;   // kind << 28 | segment (row segments) or chunk (draw items)
    int32_t x;      // row segments: the drafted token whose logit the row's segments capture, or -1
};

// An entry of early exit's schedule: the four fields of a RestItem, each in
// a 64-bit word whose high half is the number (epoch) of the call that wrote
// it.  A reader takes the entry once all four words carry its call's epoch.
struct alignas(32) SchedEntry {
    uint64_t w[4];
};

}  // namespace sv
