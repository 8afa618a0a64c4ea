// bookkeeping.hip -- what follows a verify round on the device: committing
// the round's tokens to each sequence, the adaptive draft length, and
// n-gram (prompt-lookup) drafting for the next round.
//
// * commit (page "【大模型】- 推测解码", sections 基础推测解码器 / 批量推测解码;
//   page "投机解码", section 动手实践): sequence b appends its n_b accepted
//   drafts and its emitted token, cut to the room left in its row.  One
//   workgroup scans the committed counts into offsets; then one wave per
//   sequence copies its tokens into its row and into the packed list.
// * adaptive k (page "【大模型】- 推测解码", section 自适应推测解码; page
//   "大模型推理无损加速:投机采样...", section 四): each sequence records its rate
//   n/k; once 10 rates are held the mean of the last 10 (summed oldest first
//   in fp64, the order the rule states) above 0.8 raises k, below 0.5 lowers
//   it, within [min_k, max_k].  One thread per sequence; the last 10 rates
//   live in a ring.
// * n-gram drafting (page "投机解码", section Lookahead 与 n-gram 投机; page
//   "大模型推理无损加速:投机采样...", section 四): the drafts are the tokens
//   that follow the most recent earlier occurrence of the sequence's last n
//   tokens, n from ngram_max down to ngram_min.  One workgroup per sequence
//   tests every candidate start in parallel (lane-strided) and keeps the
//   largest matching one; a scan and a copy then pack the drafts in the
//   layout spec_verify takes (prefix offsets).
#include "sv_internal.h"

namespace sv {
namespace {

constexpr int kScanThreads = 1024;

// Exclusive scan of counts[0..B) into offsets[0..B] by one workgroup, in
// chunks of kScanThreads with a running carry.  count(b) supplies the counts.
template <class Count>
__device__ __forceinline__ void scan_into(int32_t B, int32_t* offsets, Count count) {
    __shared__ int32_t wsum[kScanThreads / 64];
    __shared__ int32_t carry;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (tid == 0) carry = 0;
    __syncthreads();
    for (int32_t base = 0; base < B; base += kScanThreads) {
        const int32_t b = base + tid;
        const int32_t c = b < B ? count(b) : 0;
        int32_t inc = c;
        for (int off = 1; off < 64; off <<= 1) {
            const int32_t y = __shfl_up(inc, off, 64);
            if (lane >= off) inc += y;
        }
        if (lane == 63) wsum[wave] = inc;
        __syncthreads();
        int32_t before = carry;
        for (int w2 = 0; w2 < wave; ++w2) before += wsum[w2];
        if (b < B) offsets[b] = before + inc - c;
        __syncthreads();
        if (tid == kScanThreads - 1) carry = before + inc;
        __syncthreads();
    }
    if (tid == 0) offsets[B] = carry;
}

// ---- commit ------------------------------------------------------------------

struct CommitArgs {
    const int32_t* out_tokens;
    const int32_t* out_n;
    const int32_t* offsets;   // nullptr => k_uniform
    int32_t k_uniform;
    int32_t B;
    int32_t* seq_tokens;      // [B, max_len]
    int32_t* seq_len;         // [B]
    int32_t max_len;
    int32_t* committed;       // packed, may be nullptr
    int32_t* committed_offsets;   // [B+1]
};

__device__ __forceinline__ int32_t commit_count(const CommitArgs& a, int32_t b) {
    const int32_t n = a.out_n[b];
    const int32_t len = a.seq_len[b];
    const int32_t room = len < a.max_len ? a.max_len - (len > 0 ? len : 0) : 0;
    const int32_t c = n >= 0 ? n + 1 : 0;
    return c < room ? c : room;
}

__global__ __launch_bounds__(kScanThreads) void commit_scan_kernel(CommitArgs a) {
    scan_into(a.B, a.committed_offsets, [&](int32_t b) { return commit_count(a, b); });
}

__global__ __launch_bounds__(kThreads) void commit_copy_kernel(CommitArgs a) {
    const int32_t b = blockIdx.x * kWaves + (threadIdx.x >> 6);
    if (b >= a.B) return;
    const int lane = threadIdx.x & 63;
    const int32_t p0 = a.committed_offsets[b], c = a.committed_offsets[b + 1] - p0;
    const int64_t slot = a.offsets ? static_cast<int64_t>(a.offsets[b]) + b
                                   : static_cast<int64_t>(b) * (a.k_uniform + 1);
    const int32_t len = a.seq_len[b] > 0 ? a.seq_len[b] : 0;
    int32_t* row = a.seq_tokens + static_cast<int64_t>(b) * a.max_len;
    for (int32_t i = lane; i < c; i += 64) {
        const int32_t t = a.out_tokens[slot + i];
        row[len + i] = t;
        if (a.committed) a.committed[p0 + i] = t;
    }
    if (lane == 0) a.seq_len[b] = len + c;
}

// ---- adaptive k ------------------------------------------------------------

__global__ __launch_bounds__(kThreads) void adapt_k_kernel(const int32_t* out_n, const int32_t* offsets,
                                                           int32_t k_uniform, int32_t B, int32_t min_k,
                                                           int32_t max_k, double* history, int32_t* rounds,
                                                           int32_t* k) {
    const int32_t b = blockIdx.x * kThreads + threadIdx.x;
    if (b >= B) return;
    const int32_t n = out_n[b];
    const int32_t ku = offsets ? offsets[b + 1] - offsets[b] : k_uniform;
    if (n < 0 || ku < 1) return;                       // data error / nothing drafted: unchanged
    double* h = history + static_cast<int64_t>(b) * 10;
    const int32_t r = rounds[b];                       // rates recorded so far
    h[r % 10] = n > 0 ? static_cast<double>(n) / static_cast<double>(ku) : 0.0;
    int32_t r1 = r + 1;
    if (r1 >= 1000000000) r1 -= 500000000;             // stays >= 10, same ring position
    rounds[b] = r1;
    if (r1 < 10) return;
    double sum = 0.0;                                  // oldest first: the ring from r1 % 10
    for (int i = 0; i < 10; ++i) sum += h[(r1 + i) % 10];
    const double avg = sum / 10.0;
    int32_t kb = k[b];
    if (avg > 0.8) kb = kb + 1 < max_k ? kb + 1 : max_k;
    else if (avg < 0.5) kb = kb - 1 > min_k ? kb - 1 : min_k;
    k[b] = kb;
}

// ---- n-gram drafting -------------------------------------------------------

// Per sequence: the start of the continuation and its length, in
// draft_offsets[b + 1] (the scan turns the counts into offsets in place).
__global__ __launch_bounds__(kThreads) void ngram_find_kernel(const int32_t* seq_tokens, const int32_t* seq_len,
                                                              int32_t max_len, int32_t ngram_max,
                                                              int32_t ngram_min, int32_t k_max,
                                                              int32_t* cont_start, int32_t* draft_offsets) {
    const int32_t b = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    __shared__ int32_t best[kWaves];
    const int32_t* t = seq_tokens + static_cast<int64_t>(b) * max_len;
    int32_t L = seq_len[b];
    L = L < 0 ? 0 : (L > max_len ? max_len : L);
    int32_t start = -1;
    for (int32_t n = ngram_max; n >= ngram_min; --n) {
        if (L < n + 1) continue;                        // uniform over the workgroup
        int32_t mine = -1;
        for (int32_t j = tid; j <= L - n - 1; j += kThreads) {
            bool eq = true;
            for (int32_t i = 0; i < n && eq; ++i) eq = t[j + i] == t[L - n + i];
            if (eq) mine = j;                           // j grows: keep the largest
        }
        for (int off = 32; off > 0; off >>= 1) mine = max(mine, __shfl_xor(mine, off, 64));
        __syncthreads();
        if (lane == 0) best[wave] = mine;
        __syncthreads();
        int32_t j = best[0];
        for (int w2 = 1; w2 < kWaves; ++w2) j = max(j, best[w2]);
        if (j >= 0) { start = j + n; break; }
    }
    if (tid == 0) {
        int32_t c = start >= 0 ? L - start : 0;
        c = c < k_max ? c : k_max;
        cont_start[b] = start;
        draft_offsets[b + 1] = c;
    }
}

__global__ __launch_bounds__(kScanThreads) void ngram_scan_kernel(int32_t B, int32_t* draft_offsets) {
    // The counts sit in draft_offsets[1..B]; every thread reads its count
    // (scan_into reads a chunk before writing it) -- but the write of
    // offsets[b] could overwrite count b-1's slot before it is read in the
    // next chunk, so the counts are read from a shifted view: count(b) =
    // draft_offsets[b + 1], written slots are offsets[b] <= b, and chunk
    // boundaries are synchronised by scan_into.
    scan_into(B, draft_offsets, [&](int32_t b) { return draft_offsets[b + 1]; });
}

__global__ __launch_bounds__(kThreads) void ngram_copy_kernel(const int32_t* seq_tokens, int32_t B,
                                                              int32_t max_len, const int32_t* cont_start,
                                                              const int32_t* draft_offsets,
                                                              int32_t* draft_tokens) {
    const int32_t b = blockIdx.x * kWaves + (threadIdx.x >> 6);
    if (b >= B) return;
    const int lane = threadIdx.x & 63;
    const int32_t p0 = draft_offsets[b], c = draft_offsets[b + 1] - p0;
    const int32_t* t = seq_tokens + static_cast<int64_t>(b) * max_len + cont_start[b];
    for (int32_t i = lane; i < c; i += 64) draft_tokens[p0 + i] = t[i];
}

}  // namespace

hipError_t launch_commit(const int32_t* out_tokens, const int32_t* out_n, const int32_t* offsets,
                         int32_t k_uniform, int32_t B, int32_t* seq_tokens, int32_t* seq_len,
                         int32_t max_len, int32_t* committed, int32_t* committed_offsets, hipStream_t s) {
    const CommitArgs a{out_tokens, out_n, offsets, k_uniform, B, seq_tokens, seq_len, max_len, committed,
                       committed_offsets};
    commit_scan_kernel<<<dim3(1), dim3(kScanThreads), 0, s>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || B == 0) return e;
    commit_copy_kernel<<<dim3(static_cast<uint32_t>((B + kWaves - 1) / kWaves)), dim3(kThreads), 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_adapt_k(const int32_t* out_n, const int32_t* offsets, int32_t k_uniform, int32_t B,
                          int32_t min_k, int32_t max_k, double* history, int32_t* rounds, int32_t* k,
                          hipStream_t s) {
    if (B == 0) return hipSuccess;
    adapt_k_kernel<<<dim3(static_cast<uint32_t>((B + kThreads - 1) / kThreads)), dim3(kThreads), 0, s>>>(
        out_n, offsets, k_uniform, B, min_k, max_k, history, rounds, k);
    return hipGetLastError();
}

hipError_t launch_ngram_draft(const int32_t* seq_tokens, const int32_t* seq_len, int32_t B, int32_t max_len,
                              int32_t ngram_max, int32_t ngram_min, int32_t k_max, int32_t* cont_start,
                              int32_t* draft_tokens, int32_t* draft_offsets, hipStream_t s) {
    if (B > 0) {
        ngram_find_kernel<<<dim3(static_cast<uint32_t>(B)), dim3(kThreads), 0, s>>>(
            seq_tokens, seq_len, max_len, ngram_max, ngram_min, k_max, cont_start, draft_offsets);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    ngram_scan_kernel<<<dim3(1), dim3(kScanThreads), 0, s>>>(B, draft_offsets);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || B == 0) return e;
    ngram_copy_kernel<<<dim3(static_cast<uint32_t>((B + kWaves - 1) / kWaves)), dim3(kThreads), 0, s>>>(
        seq_tokens, B, max_len, cont_start, draft_offsets, draft_tokens);
    return hipGetLastError();
}

}  // namespace sv
