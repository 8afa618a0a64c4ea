/*
 * sv_tuning.h -- test and benchmark hooks of libspecverify.
 *
 * Not part of the product interface (include/specverify.h).  The library
 * exports these symbols so that the test suite can force each launch form
 * and geometry and the benchmark can time single kernels.  Every hook is a
 * per-call option or a stateless helper: nothing here changes what another
 * caller's call does, and spec_verify_workspace_size() never depends on it.
 *
 * The operation, the layout and the error behaviour of every entry below are
 * those of the entry in include/specverify.h whose name it extends; the only
 * difference is the sv_tuning_t argument (NULL = the defaults, identical to
 * the plain entry).  Outputs never depend on the tuning: only the launch
 * sequence does, and with it the workspace size and the NaN diagnostics of
 * rows a form does not read.
 */
#ifndef SV_TUNING_H
#define SV_TUNING_H

#include "../../include/specverify.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Kernels a call may launch; bit i of sv_tuning_t::launched and events
 * 2i, 2i+1 belong to spec_verify_kernel_name(i). */
#define SV_NUM_KERNELS 10

/* Early exit's second round (queue_mode): SV_QUEUE_OVERLAP (the default)
 * sums the draw chunks beside the remaining rows, each accept scan lag_accept
 * sequences (blocks of rows) after its own rows and its chunks lag_draw
 * blocks after them, every wait bounded; SV_QUEUE_FINAL leaves every accept
 * scan and chunk of that round to the pick launch; SV_QUEUE_HANDOFF makes
 * the undecided sequences take the path of a wait that runs out (they are
 * redone by the pick launch). */
enum { SV_QUEUE_OVERLAP = 0, SV_QUEUE_FINAL = 1, SV_QUEUE_HANDOFF = 2 };

/* The draw of a one-pass call outside the gathered form (draw_mode):
 * SV_DRAW_ONE one launch ("draw_all": accept scan, chunk sums and pick);
 * SV_DRAW_THREE three ("accept", "draw_sums", "draw_pick"); SV_DRAW_AUTO
 * one launch while the draw's workgroups fit one round on the CUs. */
enum { SV_DRAW_AUTO = 0, SV_DRAW_ONE = 1, SV_DRAW_THREE = 2 };

typedef struct {
    int64_t seg_elems;    /* approx logits per row-pass segment; 0 = automatic (65536 for batches
                             that fill the GPU, shorter for small calls) */
    int64_t chunk_elems;  /* approx logits per draw chunk; 0 = automatic (8192, shorter for small calls) */
    int32_t lead;         /* early exit: leading positions read first; -1 = automatic (1 when the
                             rows a full pass reads hold >= 192 MiB, 320 MiB in the gathered form,
                             else 0), 0 = one pass, up to SV_K_MAX + 1 */
    int32_t queue_mode;   /* SV_QUEUE_* */
    int32_t lag_accept;   /* 0 = chosen from the resident grid */
    int32_t lag_draw;     /* 0 = chosen from the resident grid */
    int32_t draw_mode;    /* SV_DRAW_* */
    uint32_t item_polls;  /* early exit: bound of a second-round workgroup's wait for its schedule
                             entry (0 = automatic: several seconds); a wait that runs out makes every
                             sequence of the call a data error (out_n_accepted -1) */
    uint32_t timed;       /* with events: bit i set = record events around kernel i */
    hipEvent_t *events;   /* NULL, or 2 * SV_NUM_KERNELS events created by the caller: events[2i] is
                             recorded on the call's stream right before kernel i, events[2i+1] right
                             after it, for the timed kernels the call launches */
    uint32_t *launched;   /* NULL, or (host memory) receives the bitmask of the kernels launched */
} sv_tuning_t;

/* The defaults: every field automatic, no events. */
void spec_tuning_defaults(sv_tuning_t *t);

/* Workspace bytes a call with this tuning needs (0 on bad sizes or tuning). */
size_t spec_verify_workspace_size_tuned(const sv_tuning_t *t, int32_t B, int64_t total_draft, int64_t V,
                                        sv_dtype_t dtype);

/* spec_verify_probs, spec_verify_gathered and spec_draft_sample with a
 * tuning; SV_ERR_SHAPE for a field out of range. */
sv_status_t spec_verify_tuned(const sv_tuning_t *t, const void *target_logits, const void *draft_logits,
                              const int32_t *draft_tokens, const int32_t *offsets, int32_t k_uniform,
                              int64_t total_draft, int32_t B, int64_t V, sv_dtype_t dtype,
                              const float *uniforms, const float *temperature, int32_t *out_tokens,
                              int32_t *out_n_accepted, float *out_p, float *out_q, float *out_row_max,
                              float *out_row_sumexp, void *workspace, size_t workspace_bytes,
                              hipStream_t stream);
sv_status_t spec_verify_gathered_tuned(const sv_tuning_t *t, const void *target_logits,
                                       const void *draft_logits, const int32_t *draft_tokens,
                                       const float *draft_probs, const int32_t *offsets, int32_t k_uniform,
                                       int64_t total_draft, int32_t B, int64_t V, sv_dtype_t dtype,
                                       const float *uniforms, const float *temperature, int32_t *out_tokens,
                                       int32_t *out_n_accepted, float *out_emit_prob, void *workspace,
                                       size_t workspace_bytes, hipStream_t stream);
sv_status_t spec_draft_sample_tuned(const sv_tuning_t *t, const void *logits, int32_t rows, int64_t V,
                                    sv_dtype_t dtype, const float *temperature, const float *uniforms,
                                    int32_t *out_tokens, float *out_probs, void *workspace,
                                    size_t workspace_bytes, hipStream_t stream);

/* Name of kernel i (static storage), NULL outside 0 .. SV_NUM_KERNELS-1. */
const char *spec_verify_kernel_name(int32_t i);

/* Event helpers for the timing fields: create n timing events into ev[],
 * the milliseconds between two completed events, and destroy n events. */
sv_status_t spec_timing_events_create(int32_t n, hipEvent_t *ev);
sv_status_t spec_timing_elapsed(hipEvent_t start, hipEvent_t stop, float *ms);
sv_status_t spec_timing_events_destroy(int32_t n, hipEvent_t *ev);

/* Benchmark reference: a bare read-reduce over `bytes` of device memory at
 * `data` (16-byte aligned), one 256-thread workgroup per `seg_bytes` (a
 * multiple of 16, 4096 .. 2^30) reading it the way the row pass reads a
 * segment (16-byte raw buffer loads, 8 in flight per lane, non-temporal) and
 * writing the XOR of its whole 16-byte words to out[i] (uint32,
 * ceil(bytes / seg_bytes) entries, caller-owned).  Its bandwidth is the
 * practical ceiling of the row pass.  Enqueue-only on `stream`. */
sv_status_t spec_stream_probe(const void *data, int64_t bytes, int64_t seg_bytes, uint32_t *out,
                              hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SV_TUNING_H */
