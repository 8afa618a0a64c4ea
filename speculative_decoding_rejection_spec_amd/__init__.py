"""libspecverify: the speculative-sampling verify step on AMD MI355X (gfx950).

Thin Python binding over the C ABI in include/specverify.h.  The functions
below take torch tensors that already live on one GPU, check that they have
the layout the C call documents, and pass their pointers and the current HIP
stream to the library.  All arithmetic of the verify step runs in the HIP
kernels; torch is used for device memory and streams only.

set_geometry / set_early_exit / set_queue / set_draw and timing() are test
and benchmark options of this binding (csrc/sv_tuning.h): they are kept in
the calling Python process and passed to the library with each call, which
holds no such state itself.
"""
from __future__ import annotations

import ctypes

from ._lib import (LIB_PATH, SV_NOALLOC_SCRATCH_BYTES, SV_BF16, SV_DRAW_AUTO, SV_DRAW_ONE, SV_DRAW_THREE, SV_F32, SV_K_MAX, SV_NUM_KERNELS,
                   SV_QUEUE_FINAL, SV_QUEUE_HANDOFF, SV_QUEUE_OVERLAP, SpecVerifyError, Tuning, check, lib)

__all__ = [
    "spec_verify", "spec_verify_noalloc", "spec_verify_probs", "spec_verify_gathered", "spec_draft_sample",
    "spec_commit", "spec_adapt_k", "spec_ngram_draft",
    "spec_verify_workspace_size", "spec_verify_release",
    "stream_probe", "timing", "kernel_times", "set_geometry", "set_early_exit", "set_queue", "set_draw",
    "reset_options", "SpecVerifyError", "SV_F32", "SV_BF16", "SV_K_MAX", "SV_QUEUE_OVERLAP",
    "SV_QUEUE_FINAL", "SV_QUEUE_HANDOFF", "SV_DRAW_AUTO", "SV_DRAW_ONE", "SV_DRAW_THREE", "LIB_PATH", "lib",
]

# ---- per-call options (csrc/sv_tuning.h), held by this binding ------------
_DEFAULTS = dict(seg_elems=0, chunk_elems=0, lead=-1, queue_mode=SV_QUEUE_OVERLAP, lag_accept=0, lag_draw=0,
                 draw_mode=SV_DRAW_AUTO, item_polls=0)
_OPTS = dict(_DEFAULTS)
_TIMING = {"mask": 0, "every": 1, "seen": 0, "records": [], "free": []}
_MAX_RECORDS = 256
_POOL = 64          # event sets created when timing is turned on (none inside a timed loop)


def _options_set() -> bool:
    return _OPTS != _DEFAULTS


def _tuning(record: bool):
    """The sv_tuning_t for the next call (None: defaults, no timing), and the
    timing record it fills, if any."""
    rec = None
    if record and _TIMING["mask"]:
        if _TIMING["seen"] % _TIMING["every"] == 0:
            rec = _timing_record()
        _TIMING["seen"] += 1
    if rec is None and not _options_set():
        return None, None
    t = Tuning(**_OPTS)
    if rec is not None:
        t.timed = _TIMING["mask"]
        t.events = ctypes.cast(rec["events"], ctypes.c_void_p)
        t.launched = ctypes.cast(ctypes.pointer(rec["launched"]), ctypes.c_void_p)
    return t, rec


def _new_event_set():
    ev = (ctypes.c_void_p * (2 * SV_NUM_KERNELS))()
    check(lib().spec_timing_events_create(2 * SV_NUM_KERNELS, ev), "spec_timing_events_create")
    return ev


def _timing_record():
    recs = _TIMING["records"]
    if _TIMING["free"]:
        ev = _TIMING["free"].pop()
    elif len(recs) >= _MAX_RECORDS or len(recs) >= _POOL:
        ev = recs.pop(0)["events"]          # the oldest record's events are re-recorded
    else:
        ev = _new_event_set()
    rec = {"events": ev, "launched": ctypes.c_uint32(0), "mask": _TIMING["mask"]}
    recs.append(rec)
    return rec


def reset_options() -> None:
    """Every per-call option back to the library's defaults (timing off)."""
    _OPTS.update(_DEFAULTS)
    timing(False)


def _dtype_code(dtype) -> int:
    import torch
    if dtype == torch.float32:
        return SV_F32
    if dtype == torch.bfloat16:
        return SV_BF16
    raise TypeError(f"logits must be float32 or bfloat16, got {dtype}")


def _ptr(t):
    return None if t is None or t.numel() == 0 else ctypes.c_void_p(t.data_ptr())


def _need(t, name, dtype, device):
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _prepare(target_logits, draft_logits, draft_tokens, offsets, uniforms, temperature,
             k_uniform, out_tokens, out_n_accepted):
    import torch
    dev = target_logits.device
    if dev.type != "cuda":
        raise ValueError("target_logits must be on a GPU")
    if not target_logits.is_contiguous() or target_logits.dim() != 2:
        raise ValueError("target_logits must be a contiguous [rows, V] tensor")
    V = int(target_logits.shape[1])
    _need(draft_tokens, "draft_tokens", torch.int32, dev)
    _need(uniforms, "uniforms", torch.float32, dev)
    _need(temperature, "temperature", torch.float32, dev)
    if draft_logits.numel():
        _need(draft_logits, "draft_logits", target_logits.dtype, dev)
    if offsets is not None:
        _need(offsets, "offsets", torch.int32, dev)
    B = int(temperature.numel())
    total = int(draft_tokens.numel())
    # Shapes the kernels index by (checked here so no kernel reads past a tensor).
    if target_logits.shape[0] != total + B:
        raise ValueError(f"target_logits has {target_logits.shape[0]} rows, expected {total + B}")
    if total and tuple(draft_logits.shape) != (total, V):
        raise ValueError(f"draft_logits must be [{total}, {V}], got {tuple(draft_logits.shape)}")
    if uniforms.numel() != total + B:
        raise ValueError(f"uniforms must have {total + B} entries")
    if offsets is not None and offsets.numel() != B + 1:
        raise ValueError(f"offsets must have {B + 1} entries")
    if offsets is None and total != B * int(k_uniform):
        raise ValueError("without offsets, draft_tokens must hold B * k_uniform tokens")
    if out_tokens is None:
        out_tokens = torch.empty(total + B, dtype=torch.int32, device=dev)
    if out_n_accepted is None:
        out_n_accepted = torch.empty(B, dtype=torch.int32, device=dev)
    _need(out_tokens, "out_tokens", torch.int32, dev)
    _need(out_n_accepted, "out_n_accepted", torch.int32, dev)
    if out_tokens.numel() != total + B or out_n_accepted.numel() != B:
        raise ValueError("out_tokens / out_n_accepted have the wrong size")
    return dev, V, B, total, out_tokens, out_n_accepted


def _stream(dev, stream):
    import torch
    s = torch.cuda.current_stream(dev) if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def spec_verify(target_logits, draft_logits, draft_tokens, offsets, uniforms, temperature, *,
                k_uniform: int = 0, out_tokens=None, out_n_accepted=None, workspace=None,
                stream=None):
    """Runs spec_verify on the current (or given) stream; returns
    (out_tokens [total+B] int32, out_n_accepted [B] int32).  ``offsets`` is an
    int32 [B+1] tensor or None (then every sequence has ``k_uniform`` drafts).
    Results are ready once the stream completes."""
    dev, V, B, total, out_tokens, out_n_accepted = _prepare(
        target_logits, draft_logits, draft_tokens, offsets, uniforms, temperature, k_uniform,
        out_tokens, out_n_accepted)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = (_ptr(target_logits), _ptr(draft_logits), _ptr(draft_tokens), _ptr(offsets),
            int(k_uniform), total, B, V, _dtype_code(target_logits.dtype), _ptr(uniforms),
            _ptr(temperature), _ptr(out_tokens), _ptr(out_n_accepted))
    t, _ = _tuning(record=True)
    if t is None:
        st = lib().spec_verify(*args, _ptr(workspace), ws_bytes, _stream(dev, stream))
    else:
        st = lib().spec_verify_tuned(ctypes.byref(t), *args, None, None, None, None, _ptr(workspace), ws_bytes,
                                     _stream(dev, stream))
    check(st, "spec_verify")
    return out_tokens, out_n_accepted


def spec_verify_noalloc(target_logits, draft_logits, draft_tokens, offsets, uniforms, temperature, *,
                        k_uniform: int = 0, out_tokens=None, out_n_accepted=None, stream=None):
    """spec_verify without a workspace or any allocation inside the library
    (its static per-GPU scratch); pass out_tokens and out_n_accepted to keep
    the call itself allocation-free.  Returns (out_tokens, out_n_accepted)."""
    dev, V, B, total, out_tokens, out_n_accepted = _prepare(
        target_logits, draft_logits, draft_tokens, offsets, uniforms, temperature, k_uniform,
        out_tokens, out_n_accepted)
    st = lib().spec_verify_noalloc(
        _ptr(target_logits), _ptr(draft_logits), _ptr(draft_tokens), _ptr(offsets), int(k_uniform), total, B, V,
        _dtype_code(target_logits.dtype), _ptr(uniforms), _ptr(temperature), _ptr(out_tokens),
        _ptr(out_n_accepted), _stream(dev, stream))
    check(st, "spec_verify_noalloc")
    return out_tokens, out_n_accepted


def spec_verify_probs(target_logits, draft_logits, draft_tokens, offsets, uniforms, temperature,
                      *, k_uniform: int = 0, workspace=None, stream=None) -> dict:
    """spec_verify plus its fp32 diagnostics: p/q [total] (p_i(x_i), q_i(x_i)),
    row_max/row_sumexp [2*total+B] (target rows first)."""
    import torch
    dev, V, B, total, out_tokens, out_n = _prepare(
        target_logits, draft_logits, draft_tokens, offsets, uniforms, temperature, k_uniform,
        None, None)
    out_p = torch.full((total,), float("nan"), device=dev)
    out_q = torch.full((total,), float("nan"), device=dev)
    row_max = torch.full((2 * total + B,), float("nan"), device=dev)
    row_sum = torch.full((2 * total + B,), float("nan"), device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = (_ptr(target_logits), _ptr(draft_logits), _ptr(draft_tokens), _ptr(offsets),
            int(k_uniform), total, B, V, _dtype_code(target_logits.dtype), _ptr(uniforms),
            _ptr(temperature), _ptr(out_tokens), _ptr(out_n), _ptr(out_p) if total else None,
            _ptr(out_q) if total else None, _ptr(row_max), _ptr(row_sum), _ptr(workspace),
            ws_bytes, _stream(dev, stream))
    t, _ = _tuning(record=True)
    st = lib().spec_verify_probs(*args) if t is None else lib().spec_verify_tuned(ctypes.byref(t), *args)
    check(st, "spec_verify_probs")
    return dict(tokens=out_tokens, n=out_n, p=out_p, q=out_q, row_max=row_max, row_sumexp=row_sum)


def spec_verify_gathered(target_logits, draft_logits, draft_tokens, draft_probs, offsets, uniforms,
                         temperature, *, k_uniform: int = 0, out_tokens=None, out_n_accepted=None,
                         out_emit_prob=None, workspace=None, stream=None):
    """spec_verify with the drafter's gathered q_i(x_i) (``draft_probs``,
    float32 [total]); returns (out_tokens, out_n_accepted, out_emit_prob [B]
    float32: the emitted token's probability under its draw)."""
    import torch
    dev, V, B, total, out_tokens, out_n_accepted = _prepare(
        target_logits, draft_logits, draft_tokens, offsets, uniforms, temperature, k_uniform,
        out_tokens, out_n_accepted)
    _need(draft_probs, "draft_probs", torch.float32, dev)
    if draft_probs.numel() != total:
        raise ValueError(f"draft_probs must have {total} entries")
    if out_emit_prob is None:
        out_emit_prob = torch.empty(B, dtype=torch.float32, device=dev)
    _need(out_emit_prob, "out_emit_prob", torch.float32, dev)
    if out_emit_prob.numel() != B:
        raise ValueError(f"out_emit_prob must have {B} entries")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = (_ptr(target_logits), _ptr(draft_logits), _ptr(draft_tokens), _ptr(draft_probs),
            _ptr(offsets), int(k_uniform), total, B, V, _dtype_code(target_logits.dtype),
            _ptr(uniforms), _ptr(temperature), _ptr(out_tokens), _ptr(out_n_accepted),
            _ptr(out_emit_prob), _ptr(workspace), ws_bytes, _stream(dev, stream))
    t, _ = _tuning(record=True)
    st = lib().spec_verify_gathered(*args) if t is None else lib().spec_verify_gathered_tuned(ctypes.byref(t),
                                                                                              *args)
    check(st, "spec_verify_gathered")
    return out_tokens, out_n_accepted, out_emit_prob


def spec_draft_sample(logits, temperature, uniforms, *, out_tokens=None, out_probs=None,
                      workspace=None, stream=None):
    """The drafter's sampling step over ``logits`` [rows, V] (float32 or
    bfloat16): returns (tokens [rows] int32, probs [rows] float32 = q(x))."""
    import torch
    dev = logits.device
    if dev.type != "cuda" or logits.dim() != 2 or not logits.is_contiguous():
        raise ValueError("logits must be a contiguous [rows, V] GPU tensor")
    rows, V = int(logits.shape[0]), int(logits.shape[1])
    _need(temperature, "temperature", torch.float32, dev)
    _need(uniforms, "uniforms", torch.float32, dev)
    if temperature.numel() != rows or uniforms.numel() != rows:
        raise ValueError(f"temperature and uniforms must have {rows} entries")
    if out_tokens is None:
        out_tokens = torch.empty(rows, dtype=torch.int32, device=dev)
    if out_probs is None:
        out_probs = torch.empty(rows, dtype=torch.float32, device=dev)
    _need(out_tokens, "out_tokens", torch.int32, dev)
    _need(out_probs, "out_probs", torch.float32, dev)
    if out_tokens.numel() != rows or out_probs.numel() != rows:
        raise ValueError("out_tokens / out_probs have the wrong size")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = (_ptr(logits), rows, V, _dtype_code(logits.dtype), _ptr(temperature), _ptr(uniforms),
            _ptr(out_tokens), _ptr(out_probs), _ptr(workspace), ws_bytes, _stream(dev, stream))
    t, _ = _tuning(record=True)
    st = lib().spec_draft_sample(*args) if t is None else lib().spec_draft_sample_tuned(ctypes.byref(t), *args)
    check(st, "spec_draft_sample")
    return out_tokens, out_probs


def spec_commit(out_tokens, out_n_accepted, offsets, seq_tokens, seq_len, *, k_uniform: int = 0,
                committed=None, committed_offsets=None, stream=None):
    """Appends each sequence's accepted drafts and emitted token to its row
    of ``seq_tokens`` [B, max_len] (int32; ``seq_len`` [B] updated in place);
    returns (committed tokens packed, committed_offsets [B+1])."""
    import torch
    dev = seq_tokens.device
    B, max_len = int(seq_tokens.shape[0]), int(seq_tokens.shape[1])
    for t, nm in ((out_tokens, "out_tokens"), (out_n_accepted, "out_n_accepted"), (seq_tokens, "seq_tokens"),
                  (seq_len, "seq_len")):
        _need(t, nm, torch.int32, dev)
    if offsets is not None:
        _need(offsets, "offsets", torch.int32, dev)
        if offsets.numel() != B + 1:
            raise ValueError(f"offsets must have {B + 1} entries")
    total = out_tokens.numel() - B
    if out_n_accepted.numel() != B or seq_len.numel() != B or total < 0:
        raise ValueError("out_n_accepted / seq_len / out_tokens sizes do not match B")
    if offsets is None and total != B * int(k_uniform):
        raise ValueError("without offsets, out_tokens must hold B * (k_uniform + 1) entries")
    if committed is None:
        committed = torch.empty(max(1, total + B), dtype=torch.int32, device=dev)
    if committed_offsets is None:
        committed_offsets = torch.empty(B + 1, dtype=torch.int32, device=dev)
    _need(committed, "committed", torch.int32, dev)
    _need(committed_offsets, "committed_offsets", torch.int32, dev)
    if committed.numel() < total + B or committed_offsets.numel() != B + 1:
        raise ValueError("committed needs total + B entries and committed_offsets B + 1")
    check(lib().spec_commit(_ptr(out_tokens), _ptr(out_n_accepted), _ptr(offsets), int(k_uniform), B,
                            _ptr(seq_tokens), _ptr(seq_len), max_len, _ptr(committed),
                            _ptr(committed_offsets), _stream(dev, stream)), "spec_commit")
    return committed, committed_offsets


def spec_adapt_k(out_n_accepted, offsets, history, rounds, k, *, k_uniform: int = 0, min_k: int = 1,
                 max_k: int = 10, stream=None):
    """One round of the adaptive draft length; ``history`` float64 [B, 10],
    ``rounds`` int32 [B] (zero at the start) and ``k`` int32 [B] are updated
    in place."""
    import torch
    dev = k.device
    B = int(k.numel())
    _need(out_n_accepted, "out_n_accepted", torch.int32, dev)
    _need(history, "history", torch.float64, dev)
    _need(rounds, "rounds", torch.int32, dev)
    _need(k, "k", torch.int32, dev)
    if offsets is not None:
        _need(offsets, "offsets", torch.int32, dev)
        if offsets.numel() != B + 1:
            raise ValueError(f"offsets must have {B + 1} entries")
    if out_n_accepted.numel() != B or rounds.numel() != B or tuple(history.shape) != (B, 10):
        raise ValueError("out_n_accepted [B], rounds [B] and history [B, 10] expected")
    check(lib().spec_adapt_k(_ptr(out_n_accepted), _ptr(offsets), int(k_uniform), B, int(min_k), int(max_k),
                             _ptr(history), _ptr(rounds), _ptr(k), _stream(dev, stream)), "spec_adapt_k")
    return k


def spec_ngram_draft(seq_tokens, seq_len, *, ngram_max: int = 3, ngram_min: int = 1, k_max: int = 8,
                     draft_tokens=None, draft_offsets=None, workspace=None, stream=None):
    """n-gram drafts of each sequence: returns (draft_tokens packed
    [B * k_max], draft_offsets [B+1])."""
    import torch
    dev = seq_tokens.device
    B, max_len = int(seq_tokens.shape[0]), int(seq_tokens.shape[1])
    _need(seq_tokens, "seq_tokens", torch.int32, dev)
    _need(seq_len, "seq_len", torch.int32, dev)
    if seq_len.numel() != B:
        raise ValueError(f"seq_len must have {B} entries")
    if draft_tokens is None:
        draft_tokens = torch.empty(max(1, B * k_max), dtype=torch.int32, device=dev)
    if draft_offsets is None:
        draft_offsets = torch.empty(B + 1, dtype=torch.int32, device=dev)
    _need(draft_tokens, "draft_tokens", torch.int32, dev)
    _need(draft_offsets, "draft_offsets", torch.int32, dev)
    if draft_tokens.numel() < B * k_max or draft_offsets.numel() != B + 1:
        raise ValueError("draft_tokens needs B * k_max entries and draft_offsets B + 1")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    check(lib().spec_ngram_draft(_ptr(seq_tokens), _ptr(seq_len), B, max_len, int(ngram_max), int(ngram_min),
                                 int(k_max), _ptr(draft_tokens), _ptr(draft_offsets), _ptr(workspace), ws_bytes,
                                 _stream(dev, stream)), "spec_ngram_draft")
    return draft_tokens, draft_offsets


def spec_verify_workspace_size(B: int, total_draft: int, V: int, dtype) -> int:
    """Workspace bytes of a call of these sizes under the options currently
    set in this binding (the library's default size when none is set)."""
    code = dtype if isinstance(dtype, int) else _dtype_code(dtype)
    if not _options_set():
        return int(lib().spec_verify_workspace_size(B, total_draft, V, code))
    t = Tuning(**_OPTS)
    return int(lib().spec_verify_workspace_size_tuned(ctypes.byref(t), B, total_draft, V, code))


def spec_verify_release() -> None:
    lib().spec_verify_release()


def _set(**kw) -> None:
    new = dict(_OPTS, **kw)
    t = Tuning(**new)
    # the library validates the fields: a tuned size query of 0 for a tiny
    # valid problem means a field is out of range
    if lib().spec_verify_workspace_size_tuned(ctypes.byref(t), 1, 0, 8, SV_F32) == 0:
        raise SpecVerifyError(-2, f"options {kw}")
    _OPTS.update(kw)


def set_geometry(seg_elems: int = 0, chunk_elems: int = 0) -> None:
    """Approximate logits per row-pass segment and per draw chunk (0 =
    automatic) for this process's later calls."""
    _set(seg_elems=int(seg_elems), chunk_elems=int(chunk_elems))


def set_early_exit(lead_positions: int = -1) -> None:
    """Leading positions every sequence reads before the rest (0 = off,
    -1 = automatic by batch size)."""
    _set(lead=int(lead_positions))


def set_queue(mode: int = SV_QUEUE_OVERLAP, lag_accept: int = 0, lag_draw: int = 0, item_polls: int = 0) -> None:
    """Where early exit's second-round accept scans and draw chunks run, and
    their lags in sequences (0 = automatic); outputs do not change.
    item_polls: bound of a second-round workgroup's wait for its schedule
    entry (0 = automatic); a wait that runs out makes every sequence of the
    call a data error (a test hook for that path)."""
    _set(queue_mode=int(mode), lag_accept=int(lag_accept), lag_draw=int(lag_draw), item_polls=int(item_polls))


def set_draw(mode: int = SV_DRAW_AUTO) -> None:
    """One-pass draw as one launch (SV_DRAW_ONE), three (SV_DRAW_THREE) or
    chosen by size (SV_DRAW_AUTO); outputs do not change."""
    _set(draw_mode=int(mode))


def stream_probe(data, seg_bytes: int = 163840, out=None, stream=None):
    """Bare read-reduce over a contiguous device tensor (benchmark reference
    for the row pass's bandwidth); returns the per-workgroup XOR words."""
    import torch
    if data.device.type != "cuda" or not data.is_contiguous():
        raise ValueError("data must be a contiguous GPU tensor")
    nbytes = data.numel() * data.element_size()
    n = (nbytes + seg_bytes - 1) // seg_bytes
    if out is None:
        out = torch.empty(max(1, n), dtype=torch.int32, device=data.device)
    elif out.numel() < n or out.dtype != torch.int32 or out.device != data.device:
        raise ValueError(f"out must be int32 on {data.device} with at least {n} entries")
    check(lib().spec_stream_probe(_ptr(data), nbytes, seg_bytes, _ptr(out), _stream(data.device, stream)),
          "spec_stream_probe")
    return out


def kernel_names() -> list:
    return [lib().spec_verify_kernel_name(i).decode() for i in range(SV_NUM_KERNELS)]


def timing(enable=True, every: int = 1) -> None:
    """Records HIP events around every kernel (True), the named kernels (an
    iterable of names from kernel_names()), or none (False) of one verify
    call in `every`; kernel_times() reports them over the last 64 recorded
    calls.  Turning it on creates the events; turning it on or off clears
    what was recorded."""
    names = kernel_names()
    if enable is True:
        mask = (1 << SV_NUM_KERNELS) - 1
    elif not enable:
        mask = 0
    else:
        want = list(enable)
        unknown = [n for n in want if n not in names]
        if unknown:
            raise ValueError(f"unknown kernels {unknown}")
        mask = sum(1 << names.index(n) for n in set(want))
    if int(every) < 1:
        raise ValueError("every must be >= 1")
    _TIMING["free"].extend(r["events"] for r in _TIMING["records"])
    _TIMING.update(mask=mask, every=int(every), seen=0, records=[])
    while mask and len(_TIMING["free"]) < _POOL:
        _TIMING["free"].append(_new_event_set())


def kernel_times() -> dict:
    """Mean milliseconds per call of every timed kernel over the recorded
    calls that launched it (waits for their events); kernels a call did not
    launch are absent."""
    recs = _TIMING["records"]
    if not recs:
        raise RuntimeError("no timed call to report")
    names = kernel_names()
    sums, counts = {}, {}
    ms = ctypes.c_float(0.0)
    for rec in recs:
        done = rec["launched"].value & rec["mask"]
        for i in range(SV_NUM_KERNELS):
            if (done >> i) & 1:
                check(lib().spec_timing_elapsed(rec["events"][2 * i], rec["events"][2 * i + 1], ctypes.byref(ms)),
                      "spec_timing_elapsed")
                sums[names[i]] = sums.get(names[i], 0.0) + ms.value
                counts[names[i]] = counts.get(names[i], 0) + 1
    return {k: sums[k] / counts[k] for k in sums}
