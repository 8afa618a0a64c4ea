"""C-ABI checks that need no GPU: the library loads, exports every function
include/specverify.h (the product interface) and csrc/sv_tuning.h (test and
benchmark hooks) declare, and rejects bad arguments on the host before
anything is enqueued (every call here fails validation, so no kernel and no
HIP runtime call is ever made)."""
import ctypes
import os
import re

import pytest

from speculative_decoding_rejection_spec_amd import _lib as svlib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "specverify.h")
TUNING_HEADER = os.path.join(ROOT, "speculative_decoding_rejection_spec_amd", "csrc", "sv_tuning.h")

OK, NULL, SHAPE, DTYPE, ALIGN, WORKSPACE = 0, -1, -2, -3, -4, -5


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(svlib.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return svlib.lib()


def declared_functions(path=HEADER):
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(spec_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 9
    for n in names:
        assert hasattr(lib, n), f"{n} declared in specverify.h but not exported"
    assert sorted(svlib.SIGNATURES) == names, "binding signatures out of sync with the header"
    hooks = declared_functions(TUNING_HEADER)
    assert len(hooks) >= 9 and not set(hooks) & set(names)
    for n in hooks:
        assert hasattr(lib, n), f"{n} declared in sv_tuning.h but not exported"
    assert sorted(svlib.TUNING_SIGNATURES) == hooks, "hook signatures out of sync with sv_tuning.h"


def test_public_header_holds_no_tuning_hooks():
    """The product header declares the operation's calls only: no process-wide
    knobs, timing probes or benchmark references."""
    text = open(HEADER).read()
    for word in ("set_geometry", "set_mode", "set_early_exit", "set_queue", "set_draw", "timing",
                 "kernel_times", "stream_probe", "fused"):
        assert word not in text, word


def test_status_strings(lib):
    for code in (OK, NULL, SHAPE, DTYPE, ALIGN, WORKSPACE, -6, -7):
        s = lib.spec_verify_status_string(code).decode()
        assert s and s != "unknown status"
    assert lib.spec_verify_status_string(-99).decode() == "unknown status"
    assert lib.spec_verify_kernel_name(0).decode() == "row_stats"
    assert lib.spec_verify_kernel_name(3).decode() == "draw_pick"
    assert lib.spec_verify_kernel_name(svlib.SV_NUM_KERNELS - 1).decode() == "sample_pick"
    assert lib.spec_verify_kernel_name(svlib.SV_NUM_KERNELS) is None
    assert lib.spec_verify_kernel_name(-1) is None


def test_workspace_size(lib):
    ws = lib.spec_verify_workspace_size
    c4 = ws(256, 2048, 152064, 1)
    # at least the per-segment statistics (two segments of 16 bytes per row)
    assert c4 >= (2 * 2048 + 256) * 2 * 16
    assert ws(512, 2816, 128256, 1) > ws(64, 256, 128256, 1)
    assert c4 < ws(512, 4096, 152064, 1)
    assert ws(256, 2048, 152064, 0) >= c4            # fp32 rows: shorter segments, more of them
    assert ws(-1, 0, 10, 0) == 0
    assert ws(1, 0, 0, 0) == 0
    assert ws(1, 0, 10, 7) == 0
    assert ws(1, -1, 10, 0) == 0


def _fake(addr):
    return ctypes.c_void_p(addr)


def _call(lib, **kw):
    a = dict(target=_fake(0x10000), draft=_fake(0x20000), tokens=_fake(0x30000), offsets=None,
             k=4, total=4, B=1, V=32000, dtype=0, unif=_fake(0x40000), temp=_fake(0x50000),
             out_tok=_fake(0x60000), out_n=_fake(0x70000), ws=_fake(0x80000), ws_bytes=16,
             stream=None)
    a.update(kw)
    return lib.spec_verify(a["target"], a["draft"], a["tokens"], a["offsets"], a["k"], a["total"],
                           a["B"], a["V"], a["dtype"], a["unif"], a["temp"], a["out_tok"],
                           a["out_n"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(target=None), NULL),
    (dict(unif=None), NULL),
    (dict(temp=None), NULL),
    (dict(out_tok=None), NULL),
    (dict(out_n=None), NULL),
    (dict(draft=None), NULL),
    (dict(tokens=None), NULL),
    (dict(dtype=2), DTYPE),
    (dict(V=0), SHAPE),
    (dict(V=1 << 31), SHAPE),
    (dict(B=-1), SHAPE),
    (dict(k=64, total=64), SHAPE),
    (dict(k=-1, total=-1), SHAPE),
    (dict(k=4, total=5), SHAPE),
    (dict(offsets=_fake(0x90000), total=64 * 2, B=2), SHAPE),
    (dict(target=_fake(0x10002)), ALIGN),
    (dict(dtype=1, target=_fake(0x10001)), ALIGN),
    (dict(tokens=_fake(0x30002)), ALIGN),
    (dict(offsets=_fake(0x90001)), ALIGN),
    (dict(ws_bytes=16), WORKSPACE),
])
def test_argument_errors(lib, kw, code):
    assert _call(lib, **kw) == code


def test_noalloc_rejects_calls_beyond_its_scratch(lib):
    """The size check comes before any HIP call: 4096 sequences of k = 8 at
    V = 152064 need 55 MiB of workspace, more than the 16 MiB scratch."""
    f = _fake
    need = lib.spec_verify_workspace_size(4096, 4096 * 8, 152064, 1)
    assert need > svlib.SV_NOALLOC_SCRATCH_BYTES
    assert lib.spec_verify_workspace_size(256, 2048, 152064, 1) <= svlib.SV_NOALLOC_SCRATCH_BYTES
    assert lib.spec_verify_workspace_size(512, 5120, 128256, 1) <= svlib.SV_NOALLOC_SCRATCH_BYTES
    st = lib.spec_verify_noalloc(f(0x10000), f(0x20000), f(0x30000), None, 8, 4096 * 8, 4096, 152064, 1,
                                 f(0x40000), f(0x50000), f(0x60000), f(0x70000), None)
    assert st == -7
    assert "scratch" in lib.spec_verify_status_string(-7).decode()
    # argument errors as for spec_verify, and an empty batch does nothing
    assert lib.spec_verify_noalloc(None, f(0x20000), f(0x30000), None, 4, 4, 1, 32000, 0, f(0x40000),
                                   f(0x50000), f(0x60000), f(0x70000), None) == NULL
    assert lib.spec_verify_noalloc(f(0x10000), None, None, None, 0, 0, 0, 32000, 0, f(0x40000), f(0x50000),
                                   f(0x60000), f(0x70000), None) == OK


def test_empty_batch_is_a_no_op(lib):
    # B = 0: nothing to verify, nothing enqueued
    assert _call(lib, B=0, k=0, total=0) == OK


def test_probs_requires_pairs(lib):
    f = _fake
    st = lib.spec_verify_probs(f(0x10000), f(0x20000), f(0x30000), None, 4, 4, 1, 32000, 0,
                               f(0x40000), f(0x50000), f(0x60000), f(0x70000), f(0xA0000), None,
                               None, None, f(0x80000), 16, None)
    assert st == NULL


def _tuning(**kw):
    t = svlib.Tuning()
    svlib.lib().spec_tuning_defaults(ctypes.byref(t))
    for k, v in kw.items():
        setattr(t, k, v)
    return t


def test_tuned_workspace_size_has_no_global_effect(lib):
    base = lib.spec_verify_workspace_size(64, 256, 128256, 1)
    dflt = _tuning()
    assert dflt.lead == -1 and dflt.seg_elems == 0 and not dflt.events
    assert lib.spec_verify_workspace_size_tuned(ctypes.byref(dflt), 64, 256, 128256, 1) == base
    assert lib.spec_verify_workspace_size_tuned(None, 64, 256, 128256, 1) == base
    fine = _tuning(seg_elems=1024, chunk_elems=512)
    assert lib.spec_verify_workspace_size_tuned(ctypes.byref(fine), 64, 256, 128256, 1) > base
    # a tuned query leaves every other caller's size alone
    assert lib.spec_verify_workspace_size(64, 256, 128256, 1) == base


@pytest.mark.parametrize("field,value", [("seg_elems", -1), ("chunk_elems", -1), ("lead", -2), ("lead", 65),
                                         ("queue_mode", 3), ("queue_mode", -1), ("lag_accept", -1),
                                         ("lag_draw", -1), ("draw_mode", 3), ("draw_mode", -1)])
def test_tuning_fields_are_validated(lib, field, value):
    t = _tuning(**{field: value})
    assert lib.spec_verify_workspace_size_tuned(ctypes.byref(t), 64, 256, 128256, 1) == 0
    f = _fake
    st = lib.spec_verify_tuned(ctypes.byref(t), f(0x10000), f(0x20000), f(0x30000), None, 4, 4, 1, 32000, 0,
                               f(0x40000), f(0x50000), f(0x60000), f(0x70000), None, None, None, None,
                               f(0x80000), 1 << 30, None)
    assert st == SHAPE
    st = lib.spec_draft_sample_tuned(ctypes.byref(t), f(0x10000), 4, 32000, 0, f(0x50000), f(0x40000),
                                     f(0x60000), None, f(0x80000), 1 << 30, None)
    assert st == SHAPE


def test_tuned_entries_validate_like_the_plain_ones(lib):
    f = _fake
    t = _tuning(lead=0)
    # k = 64 exceeds SV_K_MAX; a NULL target; a misaligned bf16 base
    assert lib.spec_verify_tuned(ctypes.byref(t), f(0x10000), f(0x20000), f(0x30000), None, 64, 64, 1, 32000, 0,
                                 f(0x40000), f(0x50000), f(0x60000), f(0x70000), None, None, None, None,
                                 f(0x80000), 16, None) == SHAPE
    assert lib.spec_verify_tuned(None, None, f(0x20000), f(0x30000), None, 4, 4, 1, 32000, 0, f(0x40000),
                                 f(0x50000), f(0x60000), f(0x70000), None, None, None, None, f(0x80000), 16,
                                 None) == NULL
    assert lib.spec_verify_gathered_tuned(ctypes.byref(t), f(0x10001), f(0x20000), f(0x30000), f(0x90000), None,
                                          4, 4, 1, 32000, 1, f(0x40000), f(0x50000), f(0x60000), f(0x70000),
                                          None, f(0x80000), 16, None) == ALIGN


def test_timing_helpers_argument_errors(lib):
    assert lib.spec_timing_events_create(-1, None) == SHAPE
    assert lib.spec_timing_events_create(2, None) == NULL
    assert lib.spec_timing_events_create(0, None) == OK
    ms = ctypes.c_float()
    assert lib.spec_timing_elapsed(None, None, ctypes.byref(ms)) == NULL
    assert lib.spec_timing_events_destroy(-1, None) == SHAPE
    assert lib.spec_timing_events_destroy(3, None) == NULL


def test_binding_options_stay_in_the_process(lib):
    """The binding's option setters validate through the library and keep
    the options on the Python side; reset_options restores the defaults."""
    import speculative_decoding_rejection_spec_amd as sv
    base = sv.spec_verify_workspace_size(64, 256, 128256, sv.SV_BF16)
    try:
        sv.set_geometry(1024, 512)
        assert sv.spec_verify_workspace_size(64, 256, 128256, sv.SV_BF16) > base
        assert lib.spec_verify_workspace_size(64, 256, 128256, 1) == base
        with pytest.raises(sv.SpecVerifyError):
            sv.set_early_exit(-7)
        with pytest.raises(sv.SpecVerifyError):
            sv.set_queue(9)
    finally:
        sv.reset_options()
    assert sv.spec_verify_workspace_size(64, 256, 128256, sv.SV_BF16) == base


def test_stream_probe_argument_errors(lib):
    p = ctypes.c_void_p(0x100000)
    assert lib.spec_stream_probe(p, 1 << 20, 1024, p, None) == SHAPE        # segment too short
    assert lib.spec_stream_probe(p, 1 << 20, 4100, p, None) == SHAPE        # not a multiple of 16
    assert lib.spec_stream_probe(p, -1, 4096, p, None) == SHAPE
    assert lib.spec_stream_probe(None, 1 << 20, 4096, p, None) == NULL
    assert lib.spec_stream_probe(ctypes.c_void_p(0x100008), 1 << 20, 4096, p, None) == ALIGN


def test_bookkeeping_argument_errors(lib):
    """Host-side validation of the bookkeeping and n-gram entry points (every
    call fails before any HIP call)."""
    p = ctypes.c_void_p(16)                     # never dereferenced: validation fails first
    assert lib.spec_commit(p, p, None, 0, -1, p, p, 8, p, p, None) == SHAPE
    assert lib.spec_commit(p, p, None, 64, 1, p, p, 8, p, p, None) == SHAPE
    assert lib.spec_commit(None, p, None, 1, 1, p, p, 8, p, p, None) == NULL
    assert lib.spec_commit(p, p, None, 1, 1, p, p, 8, p, None, None) == NULL
    assert lib.spec_commit(ctypes.c_void_p(18), p, None, 1, 1, p, p, 8, p, p, None) == ALIGN
    assert lib.spec_adapt_k(p, None, 4, 1, 0, 10, p, p, p, None) == SHAPE
    assert lib.spec_adapt_k(p, None, 4, 1, 5, 4, p, p, p, None) == SHAPE
    assert lib.spec_adapt_k(p, None, 4, 1, 1, 64, p, p, p, None) == SHAPE
    assert lib.spec_adapt_k(None, None, 4, 1, 1, 10, p, p, p, None) == NULL
    assert lib.spec_adapt_k(p, None, 4, 1, 1, 10, ctypes.c_void_p(20), p, p, None) == ALIGN
    assert lib.spec_ngram_draft(p, p, 2, 16, 3, 0, 4, p, p, None, 0, None) == SHAPE
    assert lib.spec_ngram_draft(p, p, 2, 16, 2, 3, 4, p, p, None, 0, None) == SHAPE
    assert lib.spec_ngram_draft(p, p, 2, 16, 3, 1, 64, p, p, None, 0, None) == SHAPE
    assert lib.spec_ngram_draft(p, p, 2, 16, 3, 1, 4, p, None, None, 0, None) == NULL
    assert lib.spec_ngram_draft(p, p, 2, 16, 3, 1, 4, p, p, p, 1, None) == WORKSPACE
    assert lib.spec_ngram_workspace_size(-1) == 0
    assert lib.spec_ngram_workspace_size(1000) >= 4 * 1001
