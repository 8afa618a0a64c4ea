/*
 * specverify.h -- C ABI of libspecverify, the speculative-sampling verify
 * step on AMD Instinct MI355X (gfx950).
 *
 * The operation (pages cited by title and section):
 *   * "投机解码" (docs.ifdog.com), section 投机解码的三步流程, step 3: each
 *     drafted token x_i is accepted with probability min(1, p(x_i)/q(x_i));
 *     at the first rejection a replacement is drawn from the normalised
 *     max(0, p - q) and later drafts are dropped; if all k are accepted a
 *     bonus token is drawn from the target distribution at position k+1.
 *     Its section 动手实践 tempers the distributions with softmax(logits/T)
 *     and, at T = 0, accepts while the draft equals the target argmax.
 *   * "大模型推理无损加速:投机采样(Speculative Decoding)数学原理与工业级落地实践"
 *     (bbs.huaweicloud.com), section 二 (alpha(x), residual p'(x)) and
 *     section 三 (one verify step over gamma drafts with the bonus draw).
 *   * "【大模型】- 推测解码" (sxl-space.tk), section 批量推测解码: a batch of
 *     sequences verified independently.
 * Readings where the pages leave a step open: every target and draft row is
 * divided by T; strict u < alpha; no epsilon guards; the residual uses the
 * full q row; the bonus is always drawn; the uniform of slot k_b drives the
 * draw; the draw is an inverse CDF over ascending token ids that picks
 * t* = min{t : sum_{v<=t} r_v > u * sum_v r_v}; greedy ties go to the lowest
 * token id.
 *
 * Conventions shared by every call below:
 *   * All array arguments are DEVICE pointers (memory of the GPU that is
 *     current on the calling thread), owned by the caller.  The library keeps
 *     no pointer after the call returns.
 *   * Calls only enqueue work on `stream` (0 = the null stream) and never
 *     synchronise the host; results are valid once the stream has completed.
 *   * Sequence b (0 <= b < B) has k_b drafted tokens, 0 <= k_b <= SV_K_MAX.
 *     With `offsets` (int32 [B+1], offsets[0] = 0, non-decreasing,
 *     offsets[B] = total_draft) k_b = offsets[b+1] - offsets[b]; with
 *     offsets == NULL every k_b = k_uniform and total_draft = B * k_uniform.
 *   * Row layout (row-major, V logits per row, dtype fp32 or bf16):
 *       target_logits [total_draft + B, V]: position i = 0..k_b of sequence b
 *         is row offsets[b] + b + i (row i scores drafted token i; row k_b is
 *         the bonus row);
 *       draft_logits  [total_draft, V]: position i = 0..k_b-1 of b is row
 *         offsets[b] + i.  Draft rows of greedy (T = 0) sequences are never
 *         read.
 *   * draft_tokens int32 [total_draft] (slot offsets[b] + i);
 *     uniforms fp32 [total_draft + B] in [0, 1) (slot offsets[b] + b + i:
 *     the accept uniform of position i for i < k_b, the draw uniform for
 *     i = k_b); temperature fp32 [B] (0 = greedy, > 0 = sampling).
 *   * Outputs: out_tokens int32 [total_draft + B] (slot offsets[b] + b + i):
 *     the n_b accepted drafts, then the emitted token, then -1;
 *     out_n_accepted int32 [B]: n_b in 0..k_b, or -1 for a per-sequence data
 *     error (k_b out of range; offsets out of order: offsets[b+1] below
 *     offsets[b], an earlier offset above offsets[b] or a later one below
 *     offsets[b+1], so that the range overlaps another sequence's -- two
 *     overlapping ranges are both errors; T < 0 or not finite; a drafted
 *     token outside [0, V); or a logit row with a non-finite maximum that
 *     the scan reaches: target and draft rows up to and including the
 *     first rejection -- rows past it are never looked at, whichever form
 *     reads them); that sequence's token slots, when its range lies inside
 *     the batch, are all -1.  Every other sequence is verified as usual.
 *     NaN logits are otherwise outside the contract.
 *   * Argument errors are detected on the host before anything is enqueued
 *     and return a negative sv_status_t with no output written.
 *   * Pointers must be aligned to their element size; 16-byte aligned logit
 *     rows (V * element size % 16 == 0 and 16-byte aligned bases) stream
 *     fastest.
 *   * workspace == NULL selects a library-owned, grow-only device buffer per
 *     GPU (allocated with hipMalloc on first use or growth); calls that use it
 *     must not overlap in time on one GPU.  Callers that run concurrent
 *     streams pass their own workspace of spec_verify_workspace_size() bytes
 *     per stream.
 *   * A call with a caller workspace, or through spec_verify_noalloc, may be
 *     captured in a HIP graph and replayed: each replay is a call of its own
 *     (its kernels number it from a counter at the workspace's start), and
 *     replays, like calls, must not overlap in time on one workspace.  The
 *     library-owned buffer is allocated on a call's first use of a size,
 *     which capture does not allow.
 */
#ifndef SPECVERIFY_H
#define SPECVERIFY_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SV_K_MAX 63 /* k_b + 1 positions fit one 64-lane wavefront */

typedef enum { SV_F32 = 0, SV_BF16 = 1 } sv_dtype_t;

typedef enum {
    SV_OK = 0,
    SV_ERR_NULL = -1,      /* a required pointer is NULL */
    SV_ERR_SHAPE = -2,     /* B, V, k_uniform or total_draft out of range or inconsistent */
    SV_ERR_DTYPE = -3,     /* dtype is not SV_F32 / SV_BF16 */
    SV_ERR_ALIGN = -4,     /* a pointer is not aligned to its element size */
    SV_ERR_WORKSPACE = -5, /* workspace_bytes smaller than spec_verify_workspace_size() */
    SV_ERR_HIP = -6,       /* a HIP call or kernel launch failed */
    SV_ERR_SCRATCH = -7    /* the call needs more than spec_verify_noalloc's static scratch */
} sv_status_t;

/* Bytes of device workspace one call needs for these sizes (0 on bad sizes). */
size_t spec_verify_workspace_size(int32_t B, int64_t total_draft, int64_t V, sv_dtype_t dtype);

/* The verify step for B sequences (layout above).  Pass 1 streams every needed
 * logit row once (row maximum, sum of exp((z - max)/T), or the argmax for
 * greedy rows); one wavefront per sequence then runs the accept tests and
 * finds the first rejection; a last fp64 pass over the one rejected or bonus
 * row pair draws the emitted token by inverse CDF.  Calls whose logit rows
 * hold at least 192 MiB read the rows in position order and stop at each
 * sequence's first rejection (early exit, two launches); smaller calls read
 * every needed row in one pass (two to four launches).  The outputs do not
 * depend on the form. */
sv_status_t spec_verify(const void *target_logits, const void *draft_logits,
                        const int32_t *draft_tokens, const int32_t *offsets,
                        int32_t k_uniform, int64_t total_draft, int32_t B, int64_t V,
                        sv_dtype_t dtype, const float *uniforms, const float *temperature,
                        int32_t *out_tokens, int32_t *out_n_accepted, void *workspace,
                        size_t workspace_bytes, hipStream_t stream);

/* spec_verify for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * The same operation, arguments and outputs as spec_verify, without the
 * workspace: the library uses a static device array of
 * SV_NOALLOC_SCRATCH_BYTES on each GPU (held until the process ends; its
 * address is looked up once per GPU, on the first call there) and calls no
 * allocating routine.  A call whose workspace (spec_verify_workspace_size)
 * exceeds the array returns SV_ERR_SCRATCH before anything is enqueued
 * (256 sequences of k = 8 at V = 152064 need 3.7 MiB, 512 of k <= 10 at
 * V = 128256 6.1 MiB).  Every call on one GPU shares that GPU's array and
 * finds it holding the previous call's contents (each call re-initialises
 * what it reads): calls that overlap in time on one GPU, on different
 * streams, race and give wrong results. */
#define SV_NOALLOC_SCRATCH_BYTES (16u << 20)
sv_status_t spec_verify_noalloc(const void *target_logits, const void *draft_logits,
                                const int32_t *draft_tokens, const int32_t *offsets,
                                int32_t k_uniform, int64_t total_draft, int32_t B, int64_t V,
                                sv_dtype_t dtype, const float *uniforms, const float *temperature,
                                int32_t *out_tokens, int32_t *out_n_accepted, hipStream_t stream);

/* spec_verify plus diagnostics (each may be NULL):
 *   out_p, out_q fp32 [total_draft]: p_i(x_i), q_i(x_i) of the tempered
 *     softmax at every drafted position of sampling sequences (NaN for greedy
 *     sequences);
 *   out_row_max, out_row_sumexp fp32 [2 * total_draft + B]: per logit row
 *     (target rows first, then draft rows) the maximum logit and
 *     sum_v exp((z_v - max)/T); sumexp is NaN for greedy rows and both are NaN
 *     for rows that are never read (with early exit: rows past a sequence's
 *     first rejection, and the bonus row of a sampling sequence, which its
 *     draw alone reads). */
sv_status_t spec_verify_probs(const void *target_logits, const void *draft_logits,
                              const int32_t *draft_tokens, const int32_t *offsets,
                              int32_t k_uniform, int64_t total_draft, int32_t B, int64_t V,
                              sv_dtype_t dtype, const float *uniforms,
                              const float *temperature, int32_t *out_tokens,
                              int32_t *out_n_accepted, float *out_p, float *out_q,
                              float *out_row_max, float *out_row_sumexp, void *workspace,
                              size_t workspace_bytes, hipStream_t stream);

/* The verify step with the drafter's gathered probabilities (page
 * "大模型推理无损加速:投机采样..." section 三: the draft stage keeps
 * q_prob.gather(next_token), the accept test divides by it, and the full
 * draft distribution is rebuilt only at the rejected position; page
 * "【大模型】- 推测解码" section 基础推测解码器: target_verify(input_ids,
 * draft_tokens, draft_probs)).
 *   draft_probs fp32 [total_draft] (slot offsets[b] + i): q_i(x_i) as the
 *     drafter computed it when it sampled x_i; for sampling sequences it
 *     must lie in (0, 1], otherwise the sequence is a data error (-1).
 *     Ignored for greedy sequences.
 *   out_emit_prob fp32 [B] (may be NULL): the probability of the emitted
 *     token under the distribution it was drawn from (the residual
 *     max(0, p_n - q_n)/Z, or p_k for a bonus; 1 for greedy sequences; NaN
 *     for data errors).
 * Every other argument and output is as for spec_verify.  Only target rows
 * and, for each sequence that rejects at position n < k_b, draft row n are
 * read; early exit applies to the target rows (automatically when they
 * hold at least 320 MiB). */
sv_status_t spec_verify_gathered(const void *target_logits, const void *draft_logits,
                                 const int32_t *draft_tokens, const float *draft_probs,
                                 const int32_t *offsets, int32_t k_uniform, int64_t total_draft,
                                 int32_t B, int64_t V, sv_dtype_t dtype, const float *uniforms,
                                 const float *temperature, int32_t *out_tokens,
                                 int32_t *out_n_accepted, float *out_emit_prob, void *workspace,
                                 size_t workspace_bytes, hipStream_t stream);

/* The drafter's sampling step (page "投机解码", section 动手实践: the draft
 * model's next token is drawn from softmax(logits / T), or is the argmax at
 * T = 0; page "大模型推理无损加速:投机采样..." section 三: the drawn token's
 * probability is gathered for the verify).
 *   logits [rows, V] (fp32 or bf16, one draft-model row per sequence);
 *   temperature fp32 [rows] (0 = greedy); uniforms fp32 [rows] in [0, 1).
 *   out_tokens int32 [rows]: x = min{t : sum_{v<=t} q_v > u} (the same fp64
 *     inverse CDF over ascending ids as the verify's draws), the lowest-id
 *     argmax at T = 0, -1 for an unusable temperature or a row whose maximum
 *     is not finite;
 *   out_probs fp32 [rows] (may be NULL): q(x) (1 at T = 0, NaN on error) --
 *     the draft_probs of spec_verify_gathered.
 * Two launches ("sample_sums", "sample_pick"), one read of each row.
 * Workspace as for spec_verify with B = rows and total_draft = 0. */
sv_status_t spec_draft_sample(const void *logits, int32_t rows, int64_t V, sv_dtype_t dtype,
                              const float *temperature, const float *uniforms,
                              int32_t *out_tokens, float *out_probs, void *workspace,
                              size_t workspace_bytes, hipStream_t stream);

/* ---- after the verify: bookkeeping and n-gram drafting -------------------
 * (page "【大模型】- 推测解码", sections 基础推测解码器, 批量推测解码 and
 * 自适应推测解码; page "投机解码", sections 动手实践 and Lookahead 与 n-gram 投机;
 * page "大模型推理无损加速:投机采样...", section 四).  Same conventions as above:
 * device pointers, enqueue-only on `stream`, argument errors returned before
 * anything is enqueued. */

/* Commits one verify round: sequence b appends its n_b accepted drafts and
 * its emitted token (out_tokens slots offsets[b]+b .. offsets[b]+b+n_b, as
 * spec_verify wrote them; offsets == NULL means k_uniform drafts each) to row
 * b of seq_tokens [B, max_len] after its seq_len[b] tokens (0 <= seq_len[b]
 * <= max_len), cut to the room left; a data-error sequence (n_b < 0) appends
 * nothing.  seq_len is updated.  committed_offsets int32 [B+1] receives the
 * prefix sums of the appended counts and committed (int32, room for every
 * appended token: total_draft + B suffices; may be NULL) the appended tokens
 * in sequence order. */
sv_status_t spec_commit(const int32_t *out_tokens, const int32_t *out_n_accepted,
                        const int32_t *offsets, int32_t k_uniform, int32_t B,
                        int32_t *seq_tokens, int32_t *seq_len, int32_t max_len,
                        int32_t *committed, int32_t *committed_offsets, hipStream_t stream);

/* Adaptive draft length, one round (the adapt_k rule of section 自适应推测解码):
 * sequence b records its acceptance rate n_b / k_b (0 when n_b = 0; k_b from
 * offsets or k_uniform); once it holds 10 rates, the mean of the last 10
 * (summed oldest first in fp64) above 0.8 raises k[b] by one, below 0.5 lowers
 * it by one, within [min_k, max_k] (1 <= min_k <= max_k <= SV_K_MAX).  State:
 * history fp64 [B, 10] (a ring of the last rates) and rounds int32 [B] (rates
 * recorded), both zero before the first round; k int32 [B] is read and
 * updated (the pages start at (min_k + max_k) / 2).  Sequences with n_b < 0
 * or k_b = 0 are left unchanged. */
sv_status_t spec_adapt_k(const int32_t *out_n_accepted, const int32_t *offsets, int32_t k_uniform,
                         int32_t B, int32_t min_k, int32_t max_k, double *history,
                         int32_t *rounds, int32_t *k, hipStream_t stream);

/* n-gram (prompt-lookup) drafting, no draft model: for each sequence (row b
 * of seq_tokens [B, max_len], its first seq_len[b] tokens), the drafts are
 * the up to k_max (<= SV_K_MAX) tokens that follow the most recent earlier
 * occurrence of its last n tokens, trying n = ngram_max down to ngram_min
 * (>= 1) and taking the first n that matches; an occurrence must be followed
 * by at least one token, and the continuation stops at the end of the
 * sequence; no match gives no drafts.  Output in spec_verify's layout:
 * draft_offsets int32 [B+1] (prefix sums of the counts) and draft_tokens
 * int32 [B * k_max] (packed).  workspace: spec_ngram_workspace_size(B) bytes,
 * or NULL for the library-owned buffer (shared with spec_verify's). */
size_t spec_ngram_workspace_size(int32_t B);
sv_status_t spec_ngram_draft(const int32_t *seq_tokens, const int32_t *seq_len, int32_t B,
                             int32_t max_len, int32_t ngram_max, int32_t ngram_min, int32_t k_max,
                             int32_t *draft_tokens, int32_t *draft_offsets, void *workspace,
                             size_t workspace_bytes, hipStream_t stream);

/* Human-readable name of a status code (static storage). */
const char *spec_verify_status_string(sv_status_t status);

/* Frees the library-owned workspace of every GPU.  Not safe while a call
 * that uses it is still running. */
void spec_verify_release(void);

#ifdef __cplusplus
}
#endif

#endif /* SPECVERIFY_H */
