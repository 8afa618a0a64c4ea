#!/usr/bin/env python3
"""Throughput of the speculative-sampling verify step on one MI355X.

Workload (default): B=256 sequences, k=8 drafted tokens each, V=152064, bf16
logits, T=1; half the sequences have near-identical drafts (target + N(0,
0.1^2): mostly all-accept plus a bonus draw), half have independent N(0, 2^2)
draft logits (mostly an early rejection plus a residual draw).  Inputs are
seeded synthetic logits generated on the host and copied to HBM before the
timed region; `--copies` copies are rotated between steps so no step finds
its rows in the 256 MB last-level cache.

One step = one spec_verify call (row pass, accept scan, fp64 draw) over the
whole batch.  Output: one JSON line with sequences/s, the achieved HBM
bandwidth on algorithmic bytes, the roofline of the dominant kernel and the
fp64 CPU oracle timed on this host as a baseline.  The dominant kernel is
early exit's two-round launch (every row the step reads and every draw row)
for C4 and C5, the one-pass row pass for smaller calls.

Algorithmic bytes per step: the logit rows the step reads, once each, plus
one extra read of each draw row (2 rows for a residual draw, 1 for a bonus
draw, 0 for greedy), V * element size per row; the small per-sequence arrays
are ignored.  Rows read: with early exit (--lead 1; the default for C4) the
leading positions of every sequence and the remaining positions of the
sequences they leave undecided; in one full pass (--lead 0), every target
row and the draft rows of sampling sequences.  Both
figures, and the minimum (the rows up to each sequence's first rejection),
are in the output line.

Settling: the GPU's clock control runs a step of this kind slower for the
first few tens of milliseconds after an idle spell (measured on C4, windows
of 25 steps after one idle second: 200, 199, 186, 178, 174 us per step, then
170-172 us for as long as the load lasts; the bare read probe loses only its
first window).  Before the warmup steps the bench therefore runs untimed
steps for --settle-ms milliseconds (default 60, 0 to skip), and reports
their per-window step times in the line's "settle" object, so the timed
steps measure the sustained rate a serving loop sees.
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
EVENT_EVERY = 8
METRIC = "sequences verified/s and achieved HBM GB/s (% of peak), B=256 k=8 V=152064 bf16"
# Counter summaries per roofline kernel, and the sources each kernel is built from.
COUNTERS = {"row_stats": os.path.join(ROOT, "profiles", "row_stats_c4_counters.txt"),
            "rounds": os.path.join(ROOT, "profiles", "rounds_c4_counters.txt")}
KERNEL_SOURCES = {"row_stats": ["row_stats.hip", "row_pass.h", "sv_internal.h"],
                  "rounds": ["second_round.hip", "lead_pass.h", "row_pass.h", "accept_scan.h", "draw_pass.h",
                             "sv_internal.h", "sv_layout.h"]}


def code_text(src: str) -> str:
    """C++ source without its comments and with runs of whitespace folded
    (the sources hold no comment markers inside string literals), so that a
    comment-only edit keeps the hash of a kernel's sources."""
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    return " ".join(src.split())


def source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "speculative_decoding_rejection_spec_amd", "csrc", f)) as fh:
            h.update(code_text(fh.read()).encode())
    return h.hexdigest()[:16]


def committed_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary, or None when missing or taken on different kernel sources."""
    path = COUNTERS.get(kernel)
    if not path or not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_sha256") != source_hash(kernel):
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--settle-ms", type=float, default=60.0,
                    help="untimed steps for this long before the warmup (GPU clock settling; 0 = none)")
    ap.add_argument("--workload", default="c4", help="c1 c2 c2g c3 c4 c4s c5 (c4s: C4 with shuffled halves)")
    ap.add_argument("--batch", type=int, default=0,
                    help="sequences in the batch (0 = the workload's own; other sizes keep its recipe)")
    ap.add_argument("--copies", type=int, default=4, help="input copies rotated between steps")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-kernel-events", action="store_true",
                    help="time without the per-kernel HIP events (no roofline)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration runs)")
    ap.add_argument("--seg", type=int, default=0, help="row-pass segment elements (0 = default)")
    ap.add_argument("--chunk", type=int, default=0, help="draw chunk elements (0 = default)")
    ap.add_argument("--entry", choices=["verify", "gathered", "draft", "ngram", "commit", "stream"],
                    default="verify",
                    help="verify: spec_verify; gathered: spec_verify_gathered with the drafts' q(x) "
                         "(the accept tests need no draft rows); draft: spec_draft_sample over one "
                         "draft-model row per sequence; ngram: spec_ngram_draft over B=512 token streams "
                         "of 4096; commit: spec_commit + spec_adapt_k of the workload's verify outputs; "
                         "stream: the bare read-reduce reference over the workload's logit bytes")
    ap.add_argument("--queue", type=int, default=0,
                    help="early exit: draws beside the rows (0) or all in the final launch (1)")
    ap.add_argument("--queue-lag", type=int, nargs=2, default=[0, 0], metavar=("ACCEPT", "DRAW"),
                    help="early exit: lags of the accept and draw items in sequences (0 0 = automatic)")
    ap.add_argument("--lead", type=int, default=-1,
                    help="early exit: leading positions read by every sequence (0 = one full pass, "
                         "-1 = the library's choice by batch size)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}): "
              "the verify step runs sequence-parallel on one device and this build has no "
              "multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import speculative_decoding_rejection_spec_amd as sv
    import workloads as wl

    if not os.path.exists(sv.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    sv.set_geometry(args.seg, args.chunk)
    sv.set_early_exit(args.lead)
    sv.set_queue(args.queue, *args.queue_lag)

    if args.entry == "ngram":
        return bench_ngram(args, sv, torch, np)
    if args.entry == "stream":
        return bench_stream(args, sv, torch, np)

    t_gen = time.perf_counter()
    # c4s: C4 with the near-identical and independent drafts on a random half
    # of the sequences each instead of the first and second half
    bsz = args.batch if args.batch > 0 else None
    w = (wl.make_workload("c4", B=bsz, shuffle_halves=True) if args.workload == "c4s"
         else wl.make_workload(args.workload, B=bsz))
    t_gen = time.perf_counter() - t_gen
    if args.entry == "commit":
        return bench_commit(args, sv, torch, np, w)

    def logits(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    copies = []
    for _ in range(max(1, args.copies)):
        copies.append(dict(target=logits(w.target), draft=logits(w.draft),
                           tokens=torch.from_numpy(w.tokens).to(dev),
                           offsets=torch.from_numpy(w.offsets).to(dev),
                           uniforms=torch.from_numpy(w.uniforms).to(dev),
                           temperature=torch.from_numpy(w.temperature).to(dev)))
    out_tok = torch.empty(w.total + w.B, dtype=torch.int32, device=dev)
    out_n = torch.empty(w.B, dtype=torch.int32, device=dev)
    ws = torch.empty(sv.spec_verify_workspace_size(w.B, w.total, w.V, sv.SV_BF16 if w.dtype == "bf16"
                                                   else sv.SV_F32), dtype=torch.uint8, device=dev)

    if args.entry == "gathered":
        # the drafter's gathered q_i(x_i), formed on the device from the draft
        # rows (input preparation, outside the timed region)
        for d in copies:
            tq = d["temperature"].repeat_interleave((d["offsets"][1:] - d["offsets"][:-1]).long())
            probs = torch.softmax(d["draft"].float() / tq.clamp_min(1e-30)[:, None], dim=-1)
            d["qg"] = probs.gather(1, d["tokens"].long()[:, None]).squeeze(1).contiguous()
            del probs
        emit = torch.empty(w.B, dtype=torch.float32, device=dev)
    if args.entry == "draft":
        # one draft-model row per sequence (its first draft row), its T, and
        # the sequence's first uniform
        for d in copies:
            first = d["offsets"][:-1].long()
            d["drow"] = d["draft"][first].contiguous()
            d["du"] = d["uniforms"][first + torch.arange(w.B, device=dev)].contiguous()
        dtok = torch.empty(w.B, dtype=torch.int32, device=dev)
        dprob = torch.empty(w.B, dtype=torch.float32, device=dev)
        ws = torch.empty(sv.spec_verify_workspace_size(w.B, 0, w.V, sv.SV_BF16 if w.dtype == "bf16"
                                                       else sv.SV_F32), dtype=torch.uint8, device=dev)

    def step(i):
        d = copies[i % len(copies)]
        if args.entry == "gathered":
            sv.spec_verify_gathered(d["target"], d["draft"], d["tokens"], d["qg"], d["offsets"],
                                    d["uniforms"], d["temperature"], out_tokens=out_tok,
                                    out_n_accepted=out_n, out_emit_prob=emit, workspace=ws)
        elif args.entry == "draft":
            sv.spec_draft_sample(d["drow"], d["temperature"], d["du"], out_tokens=dtok, out_probs=dprob,
                                 workspace=ws)
        else:
            sv.spec_verify(d["target"], d["draft"], d["tokens"], d["offsets"], d["uniforms"],
                           d["temperature"], out_tokens=out_tok, out_n_accepted=out_n, workspace=ws)

    if args.calibrate_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    settled = settle(torch, step, args.settle_ms)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # Which kernels a call launches (kernel_times() lists only those).
    sv.timing(True)
    step(0)
    torch.cuda.synchronize()
    launched = sv.kernel_times()
    queued = "rounds" in launched
    early = queued or "row_lead" in launched
    sv.timing(False)
    # The roofline kernel: the row pass (one launch, or the two launches of
    # early exit in the gathered form), or -- early exit -- the two-round
    # launch, which streams every row the step reads and every draw row.
    if "sample_sums" in launched:                # the draft sampler: one read of each row
        roof = ["sample_sums"]
    elif queued:
        roof = ["rounds"]
    else:
        roof = ["row_lead", "row_stats"] if early else ["row_stats"]
    if "row_draft" in launched:
        roof.append("row_draft")
    roof_kernel = "+".join(roof)

    # Timed region: HIP events around the roofline kernel(s) only, on one
    # step in EVENT_EVERY so their cost stays out of the step time.
    sv.timing(roof if not args.no_kernel_events else False, every=EVENT_EVERY)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    k1_live = None
    if not args.no_kernel_events:
        kt = sv.kernel_times()
        k1_live = sum(kt[k] for k in roof)
    sv.timing(False)
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    # Host cost of enqueueing one step (binding, C host code, launches),
    # timed without waiting for the GPU: below ms_per_step the GPU is the
    # bound, not the host.
    torch.cuda.synchronize()
    te = time.perf_counter()
    for i in range(8):
        step(i)
    host_ms = (time.perf_counter() - te) * 1e3 / 8
    torch.cuda.synchronize()
    # Per-step distribution: a further pass with an event pair around each step.
    step_ms = []
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(64)]
    for i, (e0, e1) in enumerate(evs):
        e0.record()
        step(i)
        e1.record()
    torch.cuda.synchronize()
    step_ms = sorted(e0.elapsed_time(e1) for e0, e1 in evs)
    # Per-kernel breakdown: a further untimed pass with events around every kernel.
    kern = {}
    if not args.no_kernel_events:
        sv.timing(True)
        for i in range(min(args.steps, 32)):
            step(i)
        torch.cuda.synchronize()
        kern = sv.kernel_times()
        sv.timing(False)

    # Algorithmic bytes from the realised accept counts.
    elt = w.elem_bytes
    sampling = w.temperature > 0
    if args.entry == "draft":
        # one row per sequence read once, plus its bonus-style draw row
        k = np.zeros(w.B, np.int64)
        n = np.zeros(w.B, np.int64)
    else:
        k = w.k.astype(np.int64)
        n = out_n.cpu().numpy().astype(np.int64)
    gathered = args.entry == "gathered"
    dsamp = sampling & (not gathered)          # sequences whose accept tests read draft rows
    full_rows = int(np.sum(k + 1) + np.sum(k[dsamp]))                     # every needed row, one pass
    min_rows = int(np.sum(n + 1) + np.sum(np.minimum(n + 1, k)[dsamp]))  # up to the first rejection
    if early:
        L = args.lead if args.lead > 0 else 1
        lead_rows = np.minimum(k, L - 1) + 1 + np.where(dsamp, np.minimum(k, L), 0)
        # (a sampling sequence's bonus row is read by its draw alone: the
        # sequence is settled once its k drafted positions are)
        decided = (n < L) | (k < L) | (dsamp & (k <= L))
        rest_rows = np.where(decided, 0, (k - L + 1) - dsamp + np.where(dsamp, k - L, 0))
        read_rows = int(np.sum(lead_rows + rest_rows))
    else:
        read_rows = full_rows
    if gathered:                                 # the draft row at each rejection
        extra = int(np.sum(sampling & (n < k)))
        read_rows += extra
        min_rows += extra
        full_rows += extra
    # (the draft sampler reads each row once: its sums pass re-reads a
    # sub-chunk from cache, its pick one sub-chunk)
    draw_rows = 0 if args.entry == "draft" else int(np.sum(np.where(sampling, np.where(n < k, 2, 1), 0)))
    row_bytes = w.V * elt
    k1_bytes = read_rows * row_bytes
    total_bytes = (read_rows + draw_rows) * row_bytes
    seq_per_s = w.B / (ms_per_step / 1e3)
    hbm_gbs = total_bytes / (ms_per_step / 1e3) / 1e9

    roofline = None
    # The committed counter summaries were taken on the C4 verify in the
    # default geometry: their traffic applies to no other workload or shape.
    counters_apply = (args.workload == "c4" and args.batch in (0, 256) and args.entry == "verify" and
                      args.seg == 0 and args.chunk == 0 and
                      args.lead in (-1, 0, 1) and args.queue == 0 and list(args.queue_lag) == [0, 0])
    if k1_live is not None:
        # The row pass reads every needed row once; the two-round launch also
        # reads the draw rows (unless they are all left to the pick launch).
        kbytes = (read_rows + (draw_rows if args.queue == 0 else 0)) * row_bytes if queued else k1_bytes
        achieved = kbytes / (k1_live / 1e3) / 1e9
        roofline = {"bound": "hbm", "kernel": roof_kernel, "achieved": round(achieved, 1),
                    "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                    "traffic": committed_traffic(roof_kernel) if counters_apply else None,
                    "algorithmic_bytes": kbytes,
                    "mean_ms": round(k1_live, 5)}

    cpu = None
    check = None
    if not args.no_cpu_baseline:
        import oracle
        threads = min(16, os.cpu_count() or 1)
        if args.entry == "draft":
            first = w.offsets[:-1].astype(np.int64)
            rows_in = np.ascontiguousarray(w.draft[first])
            du = copies[0]["du"].cpu().numpy()
            tc = time.perf_counter()
            ref = oracle.draft_sample(rows_in, w.temperature, du, threads=threads)
            tc = time.perf_counter() - tc
            agree = int(np.sum(ref["tokens"] == dtok.cpu().numpy()))
            what = "tokens"
        else:
            qg = copies[0]["qg"].cpu().numpy() if gathered else None
            tc = time.perf_counter()
            ref = oracle.verify(w, threads=threads, draft_probs=qg)
            tc = time.perf_counter() - tc
            # every token slot and accept count, sequence by sequence
            gtok = out_tok.cpu().numpy()
            same = np.array([ref["n"][b] == n[b] and np.array_equal(
                ref["tokens"][w.target_row(b, 0):w.target_row(b, int(w.k[b])) + 1],
                gtok[w.target_row(b, 0):w.target_row(b, int(w.k[b])) + 1]) for b in range(w.B)])
            flagged = (ref["flags"] & (oracle.FLAG_A | oracle.FLAG_B | oracle.FLAG_D)) != 0
            agree = int(same.sum())
            what = "accept counts and token slots"
            check = {"sequences": w.B, "identical": agree, "flagged": int(flagged.sum()),
                     "flag_rate": round(float(flagged.mean()), 6),
                     "differing_unflagged": int(np.sum(~same & ~flagged)),
                     "data_errors": int(np.sum(ref["n"] < 0))}
        cpu = {"value": round(w.B / tc, 2), "unit": "rows/s" if args.entry == "draft" else "sequences/s",
               "cores": threads, "kind": "oracle", "sample": f"the whole batch ({w.B} sequences) once, "
               f"fp64 C oracle split over {threads} threads; {what} agree with the "
               f"GPU on {agree}/{w.B} sequences", "cpu_model": cpu_model()}
        if args.entry != "draft":
            n1 = min(w.B, 32)
            t1 = time.perf_counter()
            oracle.verify(w, threads=1, seqs=(0, n1), draft_probs=qg)
            t1 = time.perf_counter() - t1
            cpu["single_thread"] = {"value": round(n1 / t1, 2), "sample": f"sequences 0..{n1 - 1}, one thread"}

    kdesc = f"k={int(w.k.max())}" if int(w.k.min()) == int(w.k.max()) else f"k={int(w.k.min())}..{int(w.k.max())}"
    base = f"sequences verified/s and achieved HBM GB/s (% of peak), B={w.B} {kdesc} V={w.V} {w.dtype}"
    metric = {"verify": base,
              "gathered": base + " (verify with the drafts' gathered q(x))",
              "draft": "draft rows sampled/s (spec_draft_sample), one row per sequence"}[args.entry]
    res = {
        "metric": metric, "value": round(seq_per_s, 1),
        "unit": "rows/s" if args.entry == "draft" else "sequences/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"verify {args.workload}: B={w.B} k={int(w.k.max()) if w.B else 0} "
                   f"V={w.V} {w.dtype} logits", "B": w.B, "V": w.V, "k_max": int(w.k.max()),
                   "total_draft": w.total, "logit_dtype": w.dtype,
                   "temperatures": sorted(set(float(t) for t in w.temperature)),
                   "input_copies": len(copies), "entry": args.entry,
                   "early_exit_lead": (args.lead if args.lead > 0 else 1) if early else 0},
        "hbm_gbs": round(hbm_gbs, 1), "hbm_frac": round(hbm_gbs / PEAK_HBM_GBS, 4),
        "algorithmic_bytes": total_bytes, "mean_accepted": round(float(n.mean()), 4),
        "host_ms_per_step": round(host_ms, 5),
        "rows_read": read_rows, "rows_full_pass": full_rows, "rows_minimum": min_rows,
        "rows_past_first_rejection": read_rows - min_rows, "draw_rows": draw_rows,
        "step_roofline": {"bound": "hbm", "achieved": round(hbm_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                          "frac": round(hbm_gbs / PEAK_HBM_GBS, 4), "bytes": total_bytes},
        "oracle_check": check, "settle": settled,
        "kernels_ms": {k: round(v, 5) for k, v in kern.items()},   # separate pass, all kernels evented
        "roofline": roofline, "cpu_baseline": cpu, "gen_s": round(t_gen, 2),
        "step_ms_events": {"median": round(step_ms[len(step_ms) // 2], 5), "p10": round(step_ms[6], 5),
                           "p90": round(step_ms[57], 5), "steps": len(step_ms)},
    }
    print(json.dumps(res), flush=True)


def settle(torch, fn, ms_target, windows=8):
    """Untimed calls of fn for about ms_target milliseconds of GPU time, in
    `windows` back-to-back windows timed with HIP events (no host wait
    between them, so the GPU never idles); returns what the line reports."""
    if ms_target <= 0:
        return None
    for i in range(2):                  # (first-call set-up out of the estimate)
        fn(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(4):
        fn(i)
    torch.cuda.synchronize()
    est = (time.perf_counter() - t0) * 1e3 / 4
    per = max(1, min(2000, int(ms_target / windows / max(est, 1e-3))))
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(windows + 1)]
    evs[0].record()
    for j in range(windows):
        for i in range(per):
            fn(4 + j * per + i)
        evs[j + 1].record()
    torch.cuda.synchronize()
    win = [round(evs[j].elapsed_time(evs[j + 1]) / per, 5) for j in range(windows)]
    return {"ms": ms_target, "steps": 6 + windows * per, "window_steps": per, "window_ms_per_step": win}


def _timed(torch, fn, steps, warmup):
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        fn(i)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _line(args, metric, value, unit, ms, config, extra, dtype="int32"):
    res = {"metric": metric, "value": round(value, 1), "unit": unit, "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": dtype, "data": "synthetic", "config": config, **extra}
    print(json.dumps(res), flush=True)


def bench_stream(args, sv, torch, np):
    """The bare read-reduce reference: the C4 logit arrays' bytes (1.32 GB)
    streamed by spec_stream_probe in the row pass's segment size, copies
    rotated like the verify bench."""
    dev = torch.device("cuda:0")
    nbytes = (2304 + 2048) * 152064 * 2
    bufs = [torch.randint(0, 1 << 15, (nbytes // 2,), dtype=torch.int16, device=dev)
            for _ in range(max(2, args.copies))]
    out = torch.empty((nbytes + 163839) // 163840, dtype=torch.int32, device=dev)
    settled = settle(torch, lambda i: sv.stream_probe(bufs[i % len(bufs)], out=out), args.settle_ms)
    for i in range(args.warmup):
        sv.stream_probe(bufs[i % len(bufs)], out=out)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        sv.stream_probe(bufs[i % len(bufs)], out=out)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    for i in range(args.steps):
        sv.stream_probe(bufs[i % len(bufs)], out=out)
    ev[1].record()
    torch.cuda.synchronize()
    ms_ev = ev[0].elapsed_time(ev[1]) / args.steps
    gbs = nbytes / (ms / 1e3) / 1e9
    _line(args, "bare read-reduce GB/s (spec_stream_probe over 1.32 GB, 163840-byte segments)", gbs,
          "GB/s", ms, {"workload": "stream 1.32 GB (the C4 logit arrays' bytes)", "bytes": nbytes},
          {"hbm_frac": round(gbs / PEAK_HBM_GBS, 4), "ms_per_call_events": round(ms_ev, 5), "settle": settled},
          dtype="u32")


def bench_ngram(args, sv, torch, np):
    """n-gram drafting over B=512 synthetic token streams of up to 4096 tokens
    (a 200-token alphabet with copied motifs, so suffixes recur)."""
    dev = torch.device("cuda:0")
    g = np.random.default_rng(2024)
    B, max_len, kmax = 512, 4096, 8
    seq = g.integers(0, 200, size=(B, max_len)).astype(np.int32)
    for b in range(B):
        for _ in range(16):
            m = int(g.integers(4, 32))
            src, dst = g.integers(0, max_len - m, size=2)
            seq[b, dst:dst + m] = seq[b, src:src + m]
    L = g.integers(max_len // 2, max_len + 1, size=B).astype(np.int32)
    dseq, dL = torch.from_numpy(seq).to(dev), torch.from_numpy(L).to(dev)
    tok = torch.empty(B * kmax, dtype=torch.int32, device=dev)
    off = torch.empty(B + 1, dtype=torch.int32, device=dev)
    ws = torch.empty(sv.lib().spec_ngram_workspace_size(B), dtype=torch.uint8, device=dev)
    ms = _timed(torch, lambda i: sv.spec_ngram_draft(dseq, dL, ngram_max=3, ngram_min=1, k_max=kmax,
                                                     draft_tokens=tok, draft_offsets=off, workspace=ws),
                args.steps, args.warmup)
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        tc = time.perf_counter()
        ref_t, ref_o = oracle.ngram_draft(seq, L, 3, 1, kmax)
        tc = time.perf_counter() - tc
        same = bool(np.array_equal(ref_o, off.cpu().numpy()))
        cpu = {"value": round(B / tc, 2), "unit": "sequences/s", "cores": 1, "kind": "oracle",
               "sample": f"the whole batch once, C oracle on one thread; offsets agree with the GPU: {same}"}
    drafted = int(off[-1].item())
    _line(args, "sequences n-gram-drafted/s (spec_ngram_draft, n = 3..1, k_max = 8)", B / (ms / 1e3),
          "sequences/s", ms, {"workload": f"ngram: B={B} token streams, lengths {max_len // 2}..{max_len}",
                              "B": B, "max_len": max_len, "k_max": kmax},
          {"drafts_per_sequence": round(drafted / B, 3), "token_bytes": int(L.sum()) * 4,
           "token_gbs": round(int(L.sum()) * 4 / (ms / 1e3) / 1e9, 1), "cpu_baseline": cpu})


def bench_commit(args, sv, torch, np, w):
    """spec_commit + spec_adapt_k on the outputs of one verify of the workload
    (each step appends one round to rows of 4096 tokens)."""
    dev = torch.device("cuda:0")
    def logits(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)
    off = torch.from_numpy(w.offsets).to(dev)
    tok, n = sv.spec_verify(logits(w.target), logits(w.draft), torch.from_numpy(w.tokens).to(dev), off,
                            torch.from_numpy(w.uniforms).to(dev), torch.from_numpy(w.temperature).to(dev))
    max_len = 4096
    steps = min(args.steps, 250)
    seq = torch.zeros((w.B, max_len), dtype=torch.int32, device=dev)
    L = torch.full((w.B,), 512, dtype=torch.int32, device=dev)
    com = torch.empty(w.total + w.B, dtype=torch.int32, device=dev)
    coff = torch.empty(w.B + 1, dtype=torch.int32, device=dev)
    hist = torch.zeros((w.B, 10), dtype=torch.float64, device=dev)
    rounds = torch.zeros(w.B, dtype=torch.int32, device=dev)
    k = torch.full((w.B,), 5, dtype=torch.int32, device=dev)

    def step(i):
        sv.spec_commit(tok, n, off, seq, L, committed=com, committed_offsets=coff)
        sv.spec_adapt_k(n, off, hist, rounds, k, min_k=1, max_k=10)
    args.steps = steps
    ms = _timed(torch, step, steps, min(args.warmup, 10))
    _line(args, "verify rounds committed/s (spec_commit + spec_adapt_k)", 1e3 / ms, "rounds/s", ms,
          {"workload": f"commit {args.workload}: B={w.B}", "B": w.B, "max_len": max_len},
          {"sequences_per_s": round(w.B / (ms / 1e3), 1)})


if __name__ == "__main__":
    main()
