/*
 * oracle.c -- plain, slow, fp64 CPU oracle of the speculative-sampling verify
 * step.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the GPU library, and the GPU library never
 * calls it.
 *
 * Pages this follows (cited by title and section):
 *   [ifdog] "投机解码", docs.ifdog.com -- sections 投机解码的三步流程 (three-step
 *           flow), 无损保证：数学推导 (lossless proof, its equations for the
 *           accept path, the normaliser Z identity, the reject path and the
 *           output marginal), 动手实践 (worked transformers demo: temperature,
 *           greedy branch, bonus token).
 *   [hw]    "大模型推理无损加速:投机采样(Speculative Decoding)数学原理与工业级落地
 *           实践", bbs.huaweicloud.com -- section 二 (1. acceptance probability
 *           alpha(x) = min(1, p/q); 2. residual distribution p'(x); 3. marginal
 *           equivalence) and section 三 (one verify step incl. the bonus).
 *   [sxl]   "【大模型】- 推测解码", sxl-space.tk -- 基础推测解码器 (target_verify)
 *           and 批量推测解码 (per-row verify over a batch).
 *
 * What is computed, per sequence b (k = k_b drafted tokens x_0..x_{k-1}):
 *   T = 0 (greedy; [ifdog] 动手实践 greedy branch): a_i = argmax over the raw
 *     logits of target row i, lowest index on ties.  Accept while x_i == a_i;
 *     at the first mismatch i emit a_i; if all k match, emit a_k.
 *   T > 0: p_i = softmax(z_t[i] / T), q_i = softmax(z_d[i] / T) in fp64
 *     (every row tempered, see the readings below).  Position i is accepted
 *     iff u_i < alpha_i = min(1, p_i(x_i) / q_i(x_i))  ([ifdog] three-step
 *     flow step 3; [hw] 二.1).  The first rejection at i = n stops the scan.
 *     If n < k the emitted token is drawn from r = max(0, p_n - q_n) / Z
 *     ([ifdog] residual equation; [hw] 二.2); if n = k it is drawn from p_k
 *     (bonus, [ifdog] three-step flow last bullet; [hw] 三 step 4).  A draw
 *     with uniform u* = u_k picks t* = min{t : C_t > u* . Z}, C_t = the
 *     running sum of r over token ids 0..t, Z = C_{V-1}.
 *
 * Readings where the pages leave a step open (every one is also listed in
 * the design notes):
 *   R1 temperature divides every target and draft row (the lossless proof
 *      needs the same p in the test and the bonus draw);
 *   R2 strict u < alpha;
 *   R3 no epsilon guards (q(x) > 0 holds for finite logits);
 *   R4 the residual uses the full q_n row;
 *   R5 the bonus token is always drawn;
 *   R6 uniform slot k_b drives the draw, slots 0..k_b-1 the accept tests;
 *   R7 the pages' multinomial draw is an inverse CDF in ascending token id
 *      with a strict '>' (zero-mass tokens are never picked);
 *   R8 greedy ties go to the lowest token id;
 *   R11 if a rejection leaves Z < 1e-9 the draw falls back to p_n (flag D);
 *   R26 a logit row the scan reaches (positions up to the first rejection)
 *      whose maximum is not finite makes the sequence a data error (flag E);
 *   R28 the rows, uniforms and output slots of sequence b are its own only
 *      when its offsets are in order with every other sequence's:
 *      offsets[b] <= offsets[b+1], no earlier offset above offsets[b] and no
 *      later one below offsets[b+1].  Otherwise its range overlaps another
 *      sequence's (or runs backwards) and it is a data error (flag E); two
 *      overlapping ranges are thus both errors, and every other sequence is
 *      verified as usual.
 *
 * Two more entry points follow the same pages: oracle_verify_gathered (the
 * accept tests divide by the drafter's gathered q_i(x_i) instead of the draft
 * row's softmax; the full draft row enters only the residual) and
 * oracle_draft_sample (the drafter's own step: x ~ softmax(z / T) by the same
 * inverse CDF, or the argmax at T = 0, with q(x) reported).  The round's
 * bookkeeping follows: oracle_commit (append the committed tokens),
 * oracle_adapt_k (adaptive draft length) and oracle_ngram_draft
 * (prompt-lookup drafting without a draft model).
 *
 * Ambiguity flags (rows where float rounding order may legitimately decide
 * differently): A = some evaluated accept test has |u - alpha| < 1e-5;
 * B = u*.Z lies within 1e-12 (absolute) of a CDF boundary C_t; D = degenerate
 * residual (see R11); E = per-row data error (bad k, T, token).
 *
 * Sums are Neumaier-compensated running sums, in ascending token id.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_FLAG_A 1
#define ORC_FLAG_B 2
#define ORC_FLAG_D 4
#define ORC_FLAG_E 8

#define ORC_ACCEPT_BAND 1e-5
#define ORC_CDF_BAND 1e-12
#define ORC_DEGENERATE_Z 1e-9
#define ORC_K_MAX 63

/* ---- small helpers ------------------------------------------------------ */

/* Stored logit -> double.  dtype 0: fp32; dtype 1: bf16 (upper half of an
 * fp32 bit pattern), decoded exactly. */
static double orc_decode(const void *rows, int dtype, int64_t idx) {
    if (dtype == 0) return (double)((const float *)rows)[idx];
    uint32_t bits = ((uint32_t)((const uint16_t *)rows)[idx]) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* Neumaier compensated sum. */
typedef struct { double s, c; } orc_sum;

static void orc_sum_add(orc_sum *a, double x) {
    double t = a->s + x;
    if (fabs(a->s) >= fabs(x)) a->c += (a->s - t) + x;
    else a->c += (x - t) + a->s;
    a->s = t;
}

static double orc_sum_value(const orc_sum *a) { return a->s + a->c; }

/* ---- row-level definitions --------------------------------------------- */

/* Largest logit and the lowest token id holding it. */
static double orc_row_argmax(const void *rows, int dtype, int64_t row, int64_t V,
                             int64_t *arg) {
    const int64_t base = row * V;
    double best = orc_decode(rows, dtype, base);
    int64_t at = 0;
    for (int64_t v = 1; v < V; ++v) {
        double z = orc_decode(rows, dtype, base + v);
        if (z > best) { best = z; at = v; }
    }
    if (arg) *arg = at;
    return best;
}

/* A sequence whose scan reaches a logit row with a non-finite maximum:
 * every token slot -1, n = -1, flag E (reading R26). */
static void orc_row_error(int32_t *out, int k, int32_t *out_n, int32_t *out_flag) {
    for (int i = 0; i <= k; ++i) out[i] = -1;
    *out_n = -1;
    if (out_flag) *out_flag = ORC_FLAG_E;
}

/* Temperature softmax of one row: p_v = exp((z_v - m)/T) / S with
 * m = max z and S = sum_v exp((z_v - m)/T).  Writes p (length V) and
 * returns m and S.  [ifdog] 动手实践 applies softmax(logits / T). */
static void orc_softmax_row(const void *rows, int dtype, int64_t row, int64_t V, double T,
                            double *p, double *m_out, double *S_out) {
    const int64_t base = row * V;
    double m = orc_row_argmax(rows, dtype, row, V, NULL);
    orc_sum S = {0.0, 0.0};
    for (int64_t v = 0; v < V; ++v) {
        double w = exp((orc_decode(rows, dtype, base + v) - m) / T);
        p[v] = w;
        orc_sum_add(&S, w);
    }
    double s = orc_sum_value(&S);
    for (int64_t v = 0; v < V; ++v) p[v] /= s;
    *m_out = m;
    *S_out = s;
}

/* ---- the verify step on probability rows ------------------------------- */

/* Mass of token v in the draw: max(0, p_v - q_v) (residual) or p_v (q NULL). */
static double orc_mass(const double *pr, const double *qr, int64_t v) {
    return qr ? fmax(0.0, pr[v] - qr[v]) : pr[v];
}

/* Inverse-CDF draw over token ids in ascending order: Z = sum of all masses,
 * t* = min{t : C_t > u Z} with C_t the running sum up to t (strict '>', so a
 * zero-mass token is never picked).  If qr != NULL and Z < 1e-9 the draw
 * falls back to pr alone (*degenerate = 1): a rejection happens with
 * probability Z ([ifdog] Z identity), so this only arises from rounding.
 * Writes Z and the distance from u Z to the nearest C_t. */
static int64_t orc_draw(const double *pr, const double *qr, int64_t V, float u,
                        double *Z_out, double *gap_out, int *degenerate) {
    orc_sum Zs = {0.0, 0.0};
    for (int64_t v = 0; v < V; ++v) orc_sum_add(&Zs, orc_mass(pr, qr, v));
    double Z = orc_sum_value(&Zs);
    *degenerate = 0;
    if (qr && Z < ORC_DEGENERATE_Z) {
        *degenerate = 1;
        qr = NULL;
        Zs.s = Zs.c = 0.0;
        for (int64_t v = 0; v < V; ++v) orc_sum_add(&Zs, pr[v]);
        Z = orc_sum_value(&Zs);
    }
    const double target = (double)u * Z;
    orc_sum C = {0.0, 0.0};
    double gap = INFINITY;
    int64_t pick = -1, last_pos = -1;
    for (int64_t v = 0; v < V; ++v) {
        double r = orc_mass(pr, qr, v);
        if (r > 0.0) last_pos = v;
        orc_sum_add(&C, r);
        double c = orc_sum_value(&C), d = fabs(target - c);
        if (d < gap) gap = d;
        if (pick < 0 && c > target) pick = v;
    }
    /* u < 1 makes u Z < Z = C_{V-1}, so a pick always exists; keep a valid
     * token for the record anyway. */
    if (pick < 0) pick = last_pos >= 0 ? last_pos : 0;
    *Z_out = Z;
    *gap_out = gap;
    return pick;
}


typedef struct {
    int32_t n, token, flags;
    double Z, gap;
} orc_result;

/* One sequence, sampling path.  P[i] (i = 0..k) are target distributions,
 * Q[i] (i = 0..k-1) draft distributions, x the drafted tokens, u the k+1
 * uniforms (u[k] drives the draw). */
static orc_result orc_verify_probs_seq(const double *const *P, const double *const *Q,
                                       int64_t V, int k, const int32_t *x, const float *u,
                                       const float *qg, double *alpha_out, double *px_out,
                                       double *qx_out) {
    orc_result res = {k, -1, 0, 0.0, 0.0};

    /* Accept tests in order; stop at the first rejection ([ifdog] three-step
     * flow step 3; [hw] 二.1 alpha(x) = min(1, p(x)/q(x))).  qg != NULL: the
     * drafter's own q_i(x_i), gathered when it sampled x_i ([hw] 三 drafting
     * step, [sxl] 基础推测解码器 draft_probs), replaces Q[i][x_i]; the full q
     * row is then used only for the residual at the rejection. */
    for (int i = 0; i < k; ++i) {
        double px = P[i][x[i]], qx = qg ? (double)qg[i] : Q[i][x[i]];
        double ratio = px / qx;
        double alpha = ratio < 1.0 ? ratio : 1.0;
        if (alpha_out) alpha_out[i] = alpha;
        if (px_out) px_out[i] = px;
        if (qx_out) qx_out[i] = qx;
        if (fabs((double)u[i] - alpha) < ORC_ACCEPT_BAND) res.flags |= ORC_FLAG_A;
        if (!((double)u[i] < alpha)) { res.n = i; break; }
    }
    const int n = res.n;

    /* Draw: residual max(0, p_n - q_n) after a rejection ([ifdog] reject-path
     * equation; [hw] 二.2), else the bonus distribution p_k. */
    const double *pr = P[n];
    const double *qr = (n < k) ? Q[n] : NULL;
    int degenerate = 0;
    int64_t pick = orc_draw(pr, qr, V, u[k], &res.Z, &res.gap, &degenerate);
    if (degenerate) res.flags |= ORC_FLAG_D;
    if (res.gap < ORC_CDF_BAND) res.flags |= ORC_FLAG_B;
    res.token = (int32_t)pick;
    return res;
}

static void orc_write_tokens(int32_t *out, int k, const int32_t *x, int n, int32_t emitted) {
    for (int i = 0; i <= k; ++i) out[i] = -1;
    if (n < 0) return;
    for (int i = 0; i < n; ++i) out[i] = x[i];
    out[n] = emitted;
}

/* ---- exported entry points --------------------------------------------- */

/* Probability-domain entry (tests feed p and q directly, bypassing softmax).
 * Uniform k for all B sequences.  shared_rows != 0: every sequence uses the
 * same P [k+1, V] and Q [k, V]; otherwise P is [B*(k+1), V] and Q [B*k, V].
 * tokens [B*k], uniforms [B*(k+1)], out_tokens [B*(k+1)], out_n/out_flags
 * [B], out_Z/out_gap [B] (may be NULL).  Returns 0, or -1 on bad sizes. */
int oracle_verify_probs(const double *Pall, const double *Qall, int64_t V, int32_t B,
                        int32_t k, int32_t shared_rows, const int32_t *tokens,
                        const float *uniforms, int32_t *out_tokens, int32_t *out_n,
                        int32_t *out_flags, double *out_Z, double *out_gap) {
    if (V < 1 || B < 0 || k < 0 || k > ORC_K_MAX) return -1;
    const double *P[ORC_K_MAX + 1];
    const double *Q[ORC_K_MAX + 1];
    for (int32_t b = 0; b < B; ++b) {
        const int64_t pb = shared_rows ? 0 : (int64_t)b * (k + 1);
        const int64_t qb = shared_rows ? 0 : (int64_t)b * k;
        for (int i = 0; i <= k; ++i) P[i] = Pall + (pb + i) * V;
        for (int i = 0; i < k; ++i) Q[i] = Qall + (qb + i) * V;
        const int32_t *x = tokens + (int64_t)b * k;
        int bad = 0;
        for (int i = 0; i < k; ++i) bad |= (x[i] < 0 || x[i] >= V);
        orc_result r = {-1, -1, ORC_FLAG_E, 0.0, 0.0};
        if (!bad)
            r = orc_verify_probs_seq(P, Q, V, k, x, uniforms + (int64_t)b * (k + 1), NULL, NULL,
                                     NULL, NULL);
        orc_write_tokens(out_tokens + (int64_t)b * (k + 1), k, x, r.n, r.token);
        out_n[b] = r.n;
        if (out_flags) out_flags[b] = r.flags;
        if (out_Z) out_Z[b] = r.Z;
        if (out_gap) out_gap[b] = r.gap;
    }
    return 0;
}

/* Logit-domain entry with the same layout as the GPU library:
 *   target [total+B, V] (sequence b position i at row offsets[b]+b+i),
 *   draft  [total, V]   (row offsets[b]+i), dtype 0 = fp32, 1 = bf16 bits,
 *   tokens [total], uniforms [total+B] (slot offsets[b]+b+i),
 *   temperature [B] (0 = greedy).
 * Processes sequences b_begin..b_end-1 (so callers may split the batch over
 * threads).  Outputs: out_tokens [total+B], out_n [B] (-1 = data error),
 * out_flags [B]; optional (NULL to skip): out_alpha/out_px/out_qx [total]
 * (position diagnostics), out_Z/out_gap [B], out_row_max/out_row_sum
 * [2*total+B] (target rows first, then draft rows; NaN where unused).
 * Returns 0, -1 on bad arguments, -2 on allocation failure. */
static int orc_verify_range(const void *target, const void *draft, int32_t dtype, int64_t V,
                            int32_t B, const int32_t *offsets, const int32_t *tokens,
                            const float *draft_probs, const float *uniforms,
                            const float *temperature, int32_t b_begin, int32_t b_end,
                            int32_t *out_tokens, int32_t *out_n, int32_t *out_flags,
                            double *out_alpha, double *out_px, double *out_qx, double *out_Z,
                            double *out_gap, double *out_row_max, double *out_row_sum) {
    if (V < 1 || B < 0 || (dtype != 0 && dtype != 1) || b_begin < 0 || b_end > B ||
        b_begin > b_end)
        return -1;
    const int64_t total = offsets[B];
    double *buf = (double *)malloc(sizeof(double) * (size_t)V * (2 * ORC_K_MAX + 1));
    if (!buf) return -2;

    for (int32_t b = b_begin; b < b_end; ++b) {
        const int64_t o = offsets[b];
        const int k = (int)(offsets[b + 1] - offsets[b]);
        const double T = (double)temperature[b];
        const int64_t trow = o + b;     /* first target row of b */
        const int64_t drow = o;         /* first draft row of b  */
        int32_t *out = out_tokens + trow;
        int bad = (k < 0 || k > ORC_K_MAX || !(T >= 0.0) || isinf(T) || o < 0 ||
                   offsets[b + 1] > total);
        /* Reading R28: the range must be ordered against every other one. */
        for (int32_t j = 0; !bad && j < b; ++j) bad |= offsets[j] > o;
        for (int32_t j = b + 2; !bad && j <= B; ++j) bad |= offsets[j] < offsets[b + 1];
        const int32_t *x = tokens + drow;
        for (int i = 0; !bad && i < k; ++i) bad |= (x[i] < 0 || x[i] >= V);
        /* A gathered q(x) must be a probability the drafter could have drawn
         * x with: finite and > 0 (sampling sequences only). */
        const float *qg = draft_probs ? draft_probs + drow : NULL;
        for (int i = 0; !bad && qg && T > 0.0 && i < k; ++i)
            bad |= !(qg[i] > 0.0f && qg[i] <= 1.0f);
        if (bad) {
            /* The sequence's own slots, when its range lies inside the batch. */
            if (o >= 0 && k >= 0 && offsets[b + 1] <= total)
                for (int i = 0; i <= k; ++i) out[i] = -1;
            out_n[b] = -1;
            if (out_flags) out_flags[b] = ORC_FLAG_E;
            continue;
        }
        if (out_row_max)
            for (int i = 0; i <= k; ++i) {
                out_row_max[trow + i] = NAN;
                out_row_sum[trow + i] = NAN;
                if (i < k) {
                    out_row_max[total + B + drow + i] = NAN;
                    out_row_sum[total + B + drow + i] = NAN;
                }
            }

        if (T == 0.0) {
            /* Greedy: accept while the draft equals the target argmax. */
            int n = k, row_bad = 0;
            int64_t a = 0;
            for (int i = 0; i <= k; ++i) {
                double m = orc_row_argmax(target, dtype, trow + i, V, &a);
                if (out_row_max) out_row_max[trow + i] = m;
                if (!isfinite(m)) { row_bad = 1; break; }      /* reading R26 */
                if (i == k || x[i] != a) { n = i; break; }
            }
            if (row_bad) {
                orc_row_error(out, k, out_n + b, out_flags ? out_flags + b : NULL);
                continue;
            }
            orc_write_tokens(out, k, x, n, (int32_t)a);
            out_n[b] = n;
            if (out_flags) out_flags[b] = 0;
            if (out_Z) out_Z[b] = NAN;
            if (out_gap) out_gap[b] = NAN;
            continue;
        }

        /* Sampling: tempered softmax of every needed row, then the test. */
        const double *P[ORC_K_MAX + 1];
        const double *Q[ORC_K_MAX + 1];
        double mt[ORC_K_MAX + 1], md[ORC_K_MAX + 1];
        for (int i = 0; i <= k; ++i) {
            double *p = buf + (size_t)i * V, S;
            orc_softmax_row(target, dtype, trow + i, V, T, p, &mt[i], &S);
            P[i] = p;
            if (out_row_max) { out_row_max[trow + i] = mt[i]; out_row_sum[trow + i] = S; }
        }
        for (int i = 0; i < k; ++i) {
            double *q = buf + (size_t)(k + 1 + i) * V, S;
            orc_softmax_row(draft, dtype, drow + i, V, T, q, &md[i], &S);
            Q[i] = q;
            if (out_row_max) {
                out_row_max[total + B + drow + i] = md[i];
                out_row_sum[total + B + drow + i] = S;
            }
        }
        orc_result r = orc_verify_probs_seq(
            P, Q, V, k, x, uniforms + trow, qg, out_alpha ? out_alpha + drow : NULL,
            out_px ? out_px + drow : NULL, out_qx ? out_qx + drow : NULL);
        /* Reading R26: a row the scan reaches whose maximum is not finite
         * makes the sequence a data error -- target rows 0..n and draft rows
         * 0..n (the gathered form reads only draft row n, for the residual);
         * rows after the first rejection are never read. */
        int row_bad = 0;
        for (int i = 0; i <= r.n && !row_bad; ++i)
            row_bad = !isfinite(mt[i]) || (i < k && (!qg || i == r.n) && !isfinite(md[i]));
        if (row_bad) {
            orc_row_error(out, k, out_n + b, out_flags ? out_flags + b : NULL);
            if (out_Z) out_Z[b] = NAN;
            if (out_gap) out_gap[b] = NAN;
            continue;
        }
        orc_write_tokens(out, k, x, r.n, r.token);
        out_n[b] = r.n;
        if (out_flags) out_flags[b] = r.flags;
        if (out_Z) out_Z[b] = r.Z;
        if (out_gap) out_gap[b] = r.gap;
    }
    free(buf);
    return 0;
}

int oracle_verify(const void *target, const void *draft, int32_t dtype, int64_t V,
                  int32_t B, const int32_t *offsets, const int32_t *tokens,
                  const float *uniforms, const float *temperature, int32_t b_begin,
                  int32_t b_end, int32_t *out_tokens, int32_t *out_n, int32_t *out_flags,
                  double *out_alpha, double *out_px, double *out_qx, double *out_Z,
                  double *out_gap, double *out_row_max, double *out_row_sum) {
    return orc_verify_range(target, draft, dtype, V, B, offsets, tokens, NULL, uniforms,
                            temperature, b_begin, b_end, out_tokens, out_n, out_flags, out_alpha,
                            out_px, out_qx, out_Z, out_gap, out_row_max, out_row_sum);
}

/* The same verify step with the drafter's gathered probabilities:
 * draft_probs [total] holds q_i(x_i) as the drafter computed it when it
 * sampled x_i ([hw] 三 drafting step: q_prob.gather; [sxl] 基础推测解码器:
 * draft_generate returns the gathered probabilities and target_verify divides
 * by them).  The accept test uses it in place of the draft row's softmax;
 * the full draft row is needed only at the rejected position, for the
 * residual ([hw] 三 recomputes q there).  A sampling sequence whose gathered
 * value is not in (0, 1] is a data error (out_n = -1). */
int oracle_verify_gathered(const void *target, const void *draft, int32_t dtype, int64_t V,
                           int32_t B, const int32_t *offsets, const int32_t *tokens,
                           const float *draft_probs, const float *uniforms,
                           const float *temperature, int32_t b_begin, int32_t b_end,
                           int32_t *out_tokens, int32_t *out_n, int32_t *out_flags,
                           double *out_alpha, double *out_px, double *out_qx, double *out_Z,
                           double *out_gap) {
    if (!draft_probs) return -1;
    return orc_verify_range(target, draft, dtype, V, B, offsets, tokens, draft_probs, uniforms,
                            temperature, b_begin, b_end, out_tokens, out_n, out_flags, out_alpha,
                            out_px, out_qx, out_Z, out_gap, NULL, NULL);
}

/* Draft sampler: the drafter's step that produces each drafted token.  Row
 * r holds the draft model's logits; T = temperature[r].
 *   T = 0: x = argmax over the raw logits, lowest id on ties ([ifdog] 动手实践,
 *          greedy drafting); its probability is reported as 1 (the T -> 0
 *          limit of softmax(z / T) is a point mass on that id).
 *   T > 0: q = softmax(z / T) ([ifdog] 动手实践; [hw] 三 and [sxl] use T = 1),
 *          and x is drawn from q by the same inverse CDF as the verify draws
 *          (reading R7: x = min{t : C_t > u Z} with u = uniforms[r]); its
 *          probability q(x) is what the drafter gathers for the verify.
 *   T < 0 or not finite: data error, x = -1, probability NaN, flag E.
 * Rows r_begin..r_end-1.  Outputs: out_tokens/out_probs/out_flags [rows];
 * out_gap [rows] (may be NULL): distance from u Z to the nearest C_t (flag B
 * below 1e-12).  Returns 0, -1 on bad arguments, -2 on allocation failure. */
int oracle_draft_sample(const void *logits, int32_t dtype, int64_t V, int32_t rows,
                        const float *temperature, const float *uniforms, int32_t r_begin,
                        int32_t r_end, int32_t *out_tokens, double *out_probs,
                        int32_t *out_flags, double *out_gap) {
    if (V < 1 || rows < 0 || (dtype != 0 && dtype != 1) || r_begin < 0 || r_end > rows ||
        r_begin > r_end)
        return -1;
    double *q = (double *)malloc(sizeof(double) * (size_t)V);
    if (!q) return -2;
    for (int32_t r = r_begin; r < r_end; ++r) {
        const double T = (double)temperature[r];
        if (!(T >= 0.0) || isinf(T)) {
            out_tokens[r] = -1;
            out_probs[r] = NAN;
            out_flags[r] = ORC_FLAG_E;
            if (out_gap) out_gap[r] = NAN;
            continue;
        }
        if (T == 0.0) {
            int64_t a = 0;
            orc_row_argmax(logits, dtype, r, V, &a);
            out_tokens[r] = (int32_t)a;
            out_probs[r] = 1.0;
            out_flags[r] = 0;
            if (out_gap) out_gap[r] = NAN;
            continue;
        }
        double m, S, Z, gap;
        int degenerate;
        orc_softmax_row(logits, dtype, r, V, T, q, &m, &S);
        int64_t t = orc_draw(q, NULL, V, uniforms[r], &Z, &gap, &degenerate);
        out_tokens[r] = (int32_t)t;
        out_probs[r] = q[t];
        out_flags[r] = gap < ORC_CDF_BAND ? ORC_FLAG_B : 0;
        if (out_gap) out_gap[r] = gap;
    }
    free(q);
    return 0;
}

/* ---- post-verify bookkeeping and the n-gram drafter --------------------- */

/* Commit one verify round to each sequence ([sxl] 基础推测解码器 generate, step
 * 3 更新生成序列, and 批量推测解码 update_generated: the verified tokens are
 * appended to the generated sequence; [ifdog] 动手实践 and [hw] 三 append the
 * accepted drafts AND the replacement or bonus token -- [sxl]'s own loop
 * drops the replacement when some drafts were accepted, which reads as a
 * bug).  Sequence b (n = out_n[b]) commits out_tokens[o_b+b .. o_b+b+n],
 * n + 1 tokens, cut to the room left in its row of seq_tokens [B, max_len];
 * a data-error sequence (n < 0) commits nothing.  Updates seq_len; writes
 * committed_offsets [B+1] (prefix sums of the committed counts) and the
 * committed tokens packed in that order into committed [total+B]. */
int oracle_commit(const int32_t *out_tokens, const int32_t *out_n, const int32_t *offsets,
                  int32_t B, int32_t *seq_tokens, int32_t *seq_len, int32_t max_len,
                  int32_t *committed, int32_t *committed_offsets) {
    if (B < 0 || max_len < 0) return -1;
    committed_offsets[0] = 0;
    for (int32_t b = 0; b < B; ++b) {
        const int64_t slot = (int64_t)offsets[b] + b;
        int32_t c = out_n[b] >= 0 ? out_n[b] + 1 : 0;
        const int32_t room = seq_len[b] < max_len ? max_len - seq_len[b] : 0;
        if (c > room) c = room;
        for (int32_t i = 0; i < c; ++i) {
            seq_tokens[(int64_t)b * max_len + seq_len[b] + i] = out_tokens[slot + i];
            committed[committed_offsets[b] + i] = out_tokens[slot + i];
        }
        seq_len[b] += c;
        committed_offsets[b + 1] = committed_offsets[b] + c;
    }
    return 0;
}

/* Adaptive draft length, one round ([sxl] 自适应推测解码 adapt_k; [hw] 四
 * adaptive gamma): sequence b appends its acceptance rate n/k (n accepted of
 * the k it drafted; 0 when none were accepted, as [sxl] records 0 when
 * target_verify returns no accepted tokens) to a history of at most 100;
 * once it holds at least 10 rates, the mean of the last 10 (summed in order,
 * oldest first, in fp64) above 0.8 raises k by one (at most max_k), below
 * 0.5 lowers it by one (at least min_k).  k_used [B] is the k of this round;
 * k [B] is updated in place.  history [B, 100] and hist_count [B] are the
 * oracle's own state (initially zero).  Sequences with n < 0 (data errors) or
 * k_used < 1 are left unchanged. */
int oracle_adapt_k(const int32_t *out_n, const int32_t *k_used, int32_t B, int32_t min_k,
                   int32_t max_k, double *history, int32_t *hist_count, int32_t *k) {
    if (B < 0 || min_k < 1 || max_k < min_k) return -1;
    for (int32_t b = 0; b < B; ++b) {
        if (out_n[b] < 0 || k_used[b] < 1) continue;
        double *h = history + (int64_t)b * 100;
        const double rate = out_n[b] > 0 ? (double)out_n[b] / (double)k_used[b] : 0.0;
        if (hist_count[b] == 100) {            /* drop the oldest */
            memmove(h, h + 1, sizeof(double) * 99);
            hist_count[b] = 99;
        }
        h[hist_count[b]++] = rate;
        if (hist_count[b] >= 10) {
            double sum = 0.0;
            for (int32_t i = hist_count[b] - 10; i < hist_count[b]; ++i) sum += h[i];
            const double avg = sum / 10.0;
            if (avg > 0.8) k[b] = k[b] + 1 < max_k ? k[b] + 1 : max_k;
            else if (avg < 0.5) k[b] = k[b] - 1 > min_k ? k[b] - 1 : min_k;
        }
    }
    return 0;
}

/* n-gram (prompt-lookup) drafting ([ifdog] Lookahead 与 n-gram 投机; [hw] 四,
 * Prompt Lookup Decoding): no draft model -- the drafts are copied from the
 * sequence itself, after an earlier occurrence of its last n tokens.
 * Readings: n runs from ngram_max down to ngram_min and the first n with a
 * match wins; the match is the most recent one, i.e. the largest start j
 * with tokens[j .. j+n-1] equal to the last n tokens and j + n < L (at least
 * one token follows it, so the suffix itself never matches); the drafts are
 * the up to k_max tokens that follow the match, cut at the end of the
 * sequence; no match gives no drafts.  seq_tokens [B, max_len] with L =
 * seq_len[b].  Writes draft_offsets [B+1] (prefix sums of the counts) and the
 * drafts packed in that order into draft_tokens [B * k_max]. */
int oracle_ngram_draft(const int32_t *seq_tokens, const int32_t *seq_len, int32_t B,
                       int32_t max_len, int32_t ngram_max, int32_t ngram_min, int32_t k_max,
                       int32_t *draft_tokens, int32_t *draft_offsets) {
    if (B < 0 || ngram_min < 1 || ngram_max < ngram_min || k_max < 0) return -1;
    draft_offsets[0] = 0;
    for (int32_t b = 0; b < B; ++b) {
        const int32_t *t = seq_tokens + (int64_t)b * max_len;
        const int32_t L = seq_len[b] < max_len ? seq_len[b] : max_len;
        int32_t start = -1, n_used = 0;
        for (int32_t n = ngram_max; n >= ngram_min && start < 0; --n) {
            if (L < n + 1) continue;
            for (int32_t j = L - n - 1; j >= 0; --j) {
                int32_t eq = 1;
                for (int32_t i = 0; i < n && eq; ++i) eq = (t[j + i] == t[L - n + i]);
                if (eq) { start = j; n_used = n; break; }
            }
        }
        int32_t c = 0;
        if (start >= 0) {
            c = L - (start + n_used);
            if (c > k_max) c = k_max;
            for (int32_t i = 0; i < c; ++i) draft_tokens[draft_offsets[b] + i] = t[start + n_used + i];
        }
        draft_offsets[b + 1] = draft_offsets[b] + c;
    }
    return 0;
}

/* Softmax of stored rows (exposed so tests can pin it against a library
 * softmax).  Writes p [nrows, V], m [nrows], S [nrows]. */
int oracle_softmax_rows(const void *rows, int32_t dtype, int64_t nrows, int64_t V, double T,
                        double *p, double *m, double *S) {
    if (V < 1 || nrows < 0 || !(T > 0.0) || (dtype != 0 && dtype != 1)) return -1;
    for (int64_t r = 0; r < nrows; ++r) orc_softmax_row(rows, dtype, r, V, T, p + r * V, &m[r], &S[r]);
    return 0;
}

/* Draw only: given one non-negative mass row r [V] and a uniform, return
 * t* = min{t : C_t > u Z}; writes Z and the boundary gap. */
int64_t oracle_inverse_cdf(const double *r, int64_t V, float u, double *Z_out, double *gap_out) {
    double Z, gap;
    int degenerate;
    int64_t pick = orc_draw(r, NULL, V, u, &Z, &gap, &degenerate);
    if (Z_out) *Z_out = Z;
    if (gap_out) *gap_out = gap;
    return pick;
}
