"""GPU parity at the edges of the boundary: the degenerate residual, the
longest drafts a wave holds, per-sequence data errors beside clean
sequences, temperatures far from 1, and uniforms of 0 on masked rows.

Every case is compared with the fp64 oracle on the same inputs, through the
C ABI, in each launch form (early exit, one pass with the draw in one launch
or in three).  The bar is that of tests/test_gpu_parity.py; where a case is
built so that the oracle flags it, the test says what it requires instead.
"""
import numpy as np
import pytest

import oracle
import workloads as wl
from test_gpu_parity import compare, run_gpu, set_form

pytestmark = pytest.mark.gpu

FORMS = ["early", "full", "full3"]
FORM = {"name": None}


@pytest.fixture(scope="module", params=FORMS)
def sv(cuda, request):
    import os

    import speculative_decoding_rejection_spec_amd as sv
    if not os.path.exists(sv.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    set_form(sv, request.param)
    FORM["name"] = request.param
    print(f"[form {request.param}]", flush=True)
    yield sv
    sv.reset_options()


def _leads():
    return (1, 2, 64) if FORM["name"] == "early" else (None,)


def _run_leads(sv, w, cuda, ref, label):
    """Runs w in the current form (early exit: at several leads) and returns
    the outputs of the last run, each compared with the oracle."""
    out = None
    try:
        for lead in _leads():
            if lead is not None:
                sv.set_early_exit(lead)
            out = run_gpu(sv, w, cuda)
            compare(w, out, ref, f"{label} lead {lead}")
    finally:
        if FORM["name"] == "early":
            sv.set_early_exit(1)
    return out


# --------------------------------------------------------------------------
# the degenerate residual (reading R11)
# --------------------------------------------------------------------------
def degenerate_workload(dtype, V=4096, B=12):
    """Sequences rejected at a position whose target and draft rows are the
    same except at the drafted token x, where the draft logit is 2^-13
    higher; x's logit sits ~10 below the rest, so p(x) ~ 1e-8 and the
    residual mass Z = q(x) - p(x) ~ 1e-12, far below the 1e-9 threshold.
    alpha = 1 - 1.2e-4 and the accept uniform 1 - 2^-14 rejects it by 6e-5
    (outside the accept band).  Half the sequences reject at position 0,
    half at position 1 after an identical-row position 0; T is 1 or 0.5.
    All values are exact in bf16, so both dtypes see the same logits."""
    g = np.random.default_rng(1011)
    T_rows, D_rows, X, U, Ts, K = [], [], [], [], [], []
    for b in range(B):
        k = 1 + (b % 2)
        n = k - 1                                            # the rejected position
        t = wl.bf16_to_f32(wl.bf16_round(10.0 + g.standard_normal((k + 1, V)).astype(np.float32)))
        d = t[:k].copy()
        x = g.integers(0, V, size=k)
        t[n, x[n]] = 0.0
        d[n, x[n]] = 2.0 ** -13
        u = g.random(k + 1, dtype=np.float32)
        u[:n] = 0.25                                         # identical rows before n: alpha = 1, accepted
        u[n] = np.float32(1.0 - 2.0 ** -14)
        T_rows.append(t); D_rows.append(d); X.append(x); U.append(u)
        Ts.append(1.0 if b % 4 < 2 else 0.5); K.append(k)
    return wl.assemble(np.concatenate(T_rows), np.concatenate(D_rows), np.concatenate(X),
                       np.concatenate(U), np.array(Ts, np.float32), K, dtype=dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_degenerate_residual_falls_back_to_the_target_row(sv, cuda, dtype):
    """Every sequence is flagged D by the oracle, which then draws from
    p_n; the GPU must emit the same token bit for bit (only a flag-B gap
    would excuse a difference, and none of these draws has one)."""
    w = degenerate_workload(dtype)
    ref = oracle.verify(w, diag=True)
    assert np.all(ref["flags"] == oracle.FLAG_D), ref["flags"]
    assert np.all(ref["gap"] > 1e-9)
    assert np.all(ref["n"] == w.k - 1)
    for lead in _leads():
        if lead is not None:
            sv.set_early_exit(lead)
        try:
            gpu = run_gpu(sv, w, cuda)
        finally:
            if FORM["name"] == "early":
                sv.set_early_exit(1)
        np.testing.assert_array_equal(gpu["n"], ref["n"], err_msg=f"lead {lead}")
        np.testing.assert_array_equal(gpu["tokens"], ref["tokens"], err_msg=f"lead {lead}")


# --------------------------------------------------------------------------
# k_b = 63: every lane of the wave
# --------------------------------------------------------------------------
def k63_workload(dtype, V=2048):
    """k_b = 63 (SV_K_MAX, the bonus row on lane 63): (a) q == p, every draft
    accepted and the bonus drawn from row 63; (b) q == p up to position 61,
    a rejection at 62; (c) greedy, every draft the target argmax; (d) greedy
    with a mismatch at 62; (e) independent draft rows (an early rejection);
    (f) k = 0 beside them."""
    g = np.random.default_rng(63)
    K = [63, 63, 63, 63, 63, 0]
    Ts = [1.0, 0.8, 0.0, 0.0, 1.0, 1.0]
    T_rows, D_rows, X, U = [], [], [], []
    for case, k in enumerate(K):
        t = (g.standard_normal((k + 1, V)) * 2).astype(np.float32)
        if dtype == "bf16":
            t = wl.bf16_to_f32(wl.bf16_round(t))
        d = t[:k].copy()
        u = g.random(k + 1, dtype=np.float32)
        if case in (0, 1, 5):
            x = g.integers(0, V, size=k)
        if case == 1:
            d[62] = (g.standard_normal(V) * 2).astype(np.float32)
            d[62, x[62]] = t[62, x[62]] + 6.0              # q(x) >> p(x)
            u[62] = 0.99
        if case in (2, 3):
            x = np.argmax(t[:k], axis=1)
            if case == 3:
                x[62] = (x[62] + 1) % V
        if case == 4:
            d = (g.standard_normal((k, V)) * 2).astype(np.float32)
            x = np.argmax(d, axis=1)
        T_rows.append(t); D_rows.append(d); X.append(x); U.append(u)
    return wl.assemble(np.concatenate(T_rows), np.concatenate(D_rows), np.concatenate(X),
                       np.concatenate(U), np.array(Ts, np.float32), K, dtype=dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_k_max_63(sv, cuda, dtype):
    w = k63_workload(dtype)
    ref = oracle.verify(w)
    assert list(ref["n"][:4]) == [63, 62, 63, 62], ref["n"]
    gpu = _run_leads(sv, w, cuda, ref, f"k=63 {dtype}")
    assert list(gpu["n"][:4]) == [63, 62, 63, 62]
    # the bonus of (a) is drawn from row 63; (c) emits the argmax of row 63
    vals = wl.logits_as_f32(w.target)
    assert gpu["tokens"][w.target_row(2, 63)] == int(np.argmax(vals[w.target_row(2, 63)]))


# --------------------------------------------------------------------------
# per-sequence data errors beside clean sequences
# --------------------------------------------------------------------------
def bad_offsets_workload(dtype, V=3000):
    """offsets = [0, 4, 8, 6, 12, 15, 85, 90, 154, 160]: sequence 2 runs
    backwards (k = -2) and sequences 1 ([4, 8)) and 3 ([6, 12)) overlap
    (reading R28: all three are data errors); sequence 5 has k = 70 and
    sequence 7 k = 64, above SV_K_MAX; sequences 0, 4, 6 and 8 are clean,
    greedy and sampling, beside them."""
    offsets = np.array([0, 4, 8, 6, 12, 15, 85, 90, 154, 160], np.int32)
    B = len(offsets) - 1
    total = int(offsets[-1])
    g = np.random.default_rng(4242)
    target = (g.standard_normal((total + B, V)) * 2).astype(np.float32)
    draft = (target[:total] + g.standard_normal((total, V)).astype(np.float32) * 0.5).astype(np.float32)
    tokens = np.argmax(draft, axis=1).astype(np.int32)
    temps = np.array([0.0, 1.0, 1.0, 0.8, 1.0, 0.7, 0.6, 1.0, 0.9], np.float32)
    uniforms = g.random(total + B, dtype=np.float32)
    store = (lambda a: wl.bf16_round(a)) if dtype == "bf16" else (lambda a: a)
    return wl.Workload(name="bad offsets", V=V, B=B, dtype=dtype, k=np.diff(offsets).astype(np.int32),
                       offsets=offsets, target=store(target), draft=store(draft), tokens=tokens,
                       uniforms=uniforms, temperature=temps, sigma=np.zeros(B))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_data_errors_k_over_max_and_out_of_order_offsets(sv, cuda, dtype):
    w = bad_offsets_workload(dtype)
    ref = oracle.verify(w)
    assert list(ref["n"][[1, 2, 3, 5, 7]]) == [-1] * 5
    assert np.all(ref["n"][[0, 4, 6, 8]] >= 0)
    for lead in _leads():
        if lead is not None:
            sv.set_early_exit(lead)
        try:
            gpu = run_gpu(sv, w, cuda)
        finally:
            if FORM["name"] == "early":
                sv.set_early_exit(1)
        np.testing.assert_array_equal(gpu["n"], ref["n"], err_msg=f"lead {lead}")
        # every slot: the clean sequences' outputs, -1 in the ranges of the
        # error sequences that lie inside the batch
        np.testing.assert_array_equal(gpu["tokens"], ref["tokens"], err_msg=f"lead {lead}")


# --------------------------------------------------------------------------
# temperatures far from 1
# --------------------------------------------------------------------------
def temperature_workload(T, B=24, V=128256):
    """C3-shaped sequences (Zipf targets, draft noise sigma ~ U[0.2, 2]) at
    temperature T, drafts sampled from the draft rows at that T, plus four
    sequences of wide-range rows (N(0, 8^2) logits: at T = 0.05 the tail
    weights exp((z - m)/T) fall far below 2^-1023)."""
    w = wl.make_workload("c3", trial=5, B=B, V=V)
    g = np.random.default_rng(int(T * 1000) + 7)
    k = w.k.copy()
    target = wl.logits_as_f32(w.target).copy()
    draft = wl.logits_as_f32(w.draft).copy()
    for b in range(B - 4, B):
        for i in range(int(k[b]) + 1):
            target[w.target_row(b, i)] = (g.standard_normal(V) * 8).astype(np.float32)
        for i in range(int(k[b])):
            draft[w.draft_row(b, i)] = target[w.target_row(b, i)] + \
                (g.standard_normal(V) * 0.5).astype(np.float32)
    target = wl.bf16_to_f32(wl.bf16_round(target))
    draft = wl.bf16_to_f32(wl.bf16_round(draft))
    tokens = np.empty(w.total, np.int32)
    for r in range(w.total):                       # Gumbel-max draw from softmax(draft / T)
        tokens[r] = int(np.argmax(draft[r].astype(np.float64) / T - np.log(g.standard_exponential(V))))
    return wl.assemble(target, draft, tokens, w.uniforms, np.full(B, T, np.float32), k, dtype="bf16")


@pytest.mark.parametrize("T", [0.05, 0.2, 4.0])
def test_temperature_sweep(sv, cuda, T):
    w = temperature_workload(T)
    ref = oracle.verify(w, threads=16)
    _run_leads(sv, w, cuda, ref, f"T={T}")


# --------------------------------------------------------------------------
# a draw uniform of 0 on masked rows
# --------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_zero_draw_uniform_never_emits_a_masked_token(sv, cuda, dtype):
    """With u = 0 the inverse CDF picks the first token with positive mass.
    Masked (-inf) logits have none, so the token emitted after a masked
    prefix (or inside a masked block) is the first unmasked one with mass --
    the oracle's choice (it flags these rows B: u Z = 0 = C_t on the masked
    prefix) -- and never a masked token."""
    from test_gpu_parity import masked_workload
    w = masked_workload(dtype)
    for b in range(w.B):
        w.uniforms[w.uniform_slot(b, int(w.k[b]))] = 0.0
    ref = oracle.verify(w)
    gpu = run_gpu(sv, w, cuda)
    np.testing.assert_array_equal(gpu["n"], ref["n"])
    np.testing.assert_array_equal(gpu["tokens"], ref["tokens"])
    vals = wl.logits_as_f32(w.target)
    for b in range(w.B):
        n = int(gpu["n"][b])
        t = int(gpu["tokens"][w.target_row(b, n)])
        assert np.isfinite(vals[w.target_row(b, n), t]), (b, n, t)


# --------------------------------------------------------------------------
# a second-round wait that runs out
# --------------------------------------------------------------------------
def test_item_wait_that_runs_out_reports_data_errors(sv, cuda):
    """Early exit: a second-round workgroup whose wait for its schedule
    entry runs out (forced from the host with a bound of one poll, so that
    workgroups starting beside the first round give up) makes every sequence
    of the call a data error, never a hang or a wrong token; the next call,
    with the automatic bound, is exact again."""
    if FORM["name"] != "early":
        pytest.skip("early exit only")
    w = wl.make_workload("c3", trial=9, B=16, V=128256)
    ref = oracle.verify(w, threads=16)
    stalled = 0
    try:
        sv.set_queue(item_polls=1)
        for i in range(3):
            gpu = run_gpu(sv, w, cuda)
            if np.all(gpu["n"] == -1):
                assert np.all(gpu["tokens"] == -1)
                stalled += 1
            else:                                  # (every workgroup found its entry in time)
                compare(w, gpu, ref, f"item_polls 1, call {i}")
    finally:
        sv.set_queue()
    assert stalled >= 1
    compare(w, run_gpu(sv, w, cuda), ref, "after a stalled call")


# --------------------------------------------------------------------------
# the first round's two hand-overs to the accept scan
# --------------------------------------------------------------------------
@pytest.mark.parametrize("seg", [0, 32768, 12288])
def test_first_round_records_and_counts(sv, cuda, seg):
    """Early exit after one leading position hands each first-round
    workgroup's statistics to its sequence's scan as epoch-tagged records
    when a row has at most two segments (V = 50000 bf16: one segment by
    default, two at 32768 logits per segment), and through a count of
    arrivals otherwise (five segments at 12288).  Both against the oracle,
    over several calls (the records of one call must never pass for the
    next call's)."""
    if FORM["name"] != "early":
        pytest.skip("early exit only")
    w = wl.make_workload("c3", trial=11, B=24, V=50000)
    ref = oracle.verify(w, threads=16)
    try:
        sv.set_geometry(seg_elems=seg)
        sv.set_early_exit(1)
        for i in range(3):
            compare(w, run_gpu(sv, w, cuda), ref, f"seg {seg}, call {i}")
    finally:
        sv.set_geometry()


@pytest.mark.parametrize("lead", [2, 5, 64])
def test_counted_first_round_at_full_size(sv, cuda, lead):
    """The count of arrivals at the full C3 size (B = 64, k = 4, V = 128256
    bf16, two segments a row): every first-round workgroup of a sequence,
    lead x 2 x 2 of them (256 at lead 64, past k + 1 = 5 positions the
    workgroups have no row to read), counts itself on the sequence's
    counter, which the round clears; the one that completes the count runs
    the scan.  Two calls per lead against the oracle (a count left by one
    call must never complete the next call's)."""
    if FORM["name"] != "early":
        pytest.skip("early exit only")
    print(f"[c3 full size, lead {lead}]", flush=True)
    w = wl.make_workload("c3", trial=12)
    ref = oracle.verify(w, threads=16)
    try:
        sv.set_early_exit(lead)
        for i in range(2):
            compare(w, run_gpu(sv, w, cuda), ref, f"lead {lead}, call {i}")
    finally:
        sv.set_early_exit(1)
