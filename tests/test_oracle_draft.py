"""Pins of the oracle's drafter-side entry points against what the pages and
the mathematics fix (CPU only):

* draft sampler (the drafting step of the page "投机解码", section 动手实践,
  and of "大模型推理无损加速:投机采样..." section 三): the drawn token is
  numpy.searchsorted over a scipy softmax, its reported probability is that
  softmax's value, greedy rows give the lowest-index argmax with probability
  1, and 200K seeded draws follow softmax(z / T) (chi-square);
* verify with the drafter's gathered q(x) (the same section 三 and the page
  "【大模型】- 推测解码", section 基础推测解码器): equal to the plain verify when the
  gathered values are the draft rows' own probabilities, lossless by
  chi-square when the drafts are drawn from q, blind to every draft row but
  the rejected one, and a data error for a gathered value outside (0, 1].
"""
import math

import numpy as np
import pytest
import scipy.special
import scipy.stats

import oracle
import workloads as wl


def _rng(seed):
    return np.random.default_rng(seed)


# --------------------------------------------------------------------------
# draft sampler
# --------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_draft_sample_matches_scipy_searchsorted(dtype):
    g = _rng(11)
    rows, V = 64, 3000
    z = (g.standard_normal((rows, V)) * 2.5).astype(np.float32)
    stored = wl.bf16_round(z) if dtype == "bf16" else z
    vals = wl.logits_as_f32(stored).astype(np.float64)
    T = g.choice([0.5, 1.0, 1.7], size=rows).astype(np.float32)
    u = g.random(rows, dtype=np.float32)
    out = oracle.draft_sample(stored, T, u)
    for r in range(rows):
        q = scipy.special.softmax(vals[r] / float(T[r]))
        c = np.cumsum(q)
        t = int(np.searchsorted(c, float(u[r]) * c[-1], side="right"))
        if out["gap"][r] > 1e-9:          # away from a boundary both orders agree
            assert out["tokens"][r] == t, r
        assert abs(out["probs"][r] - q[out["tokens"][r]]) <= 1e-14 * q[out["tokens"][r]], r
        assert out["flags"][r] == 0


def test_draft_sample_greedy_and_errors():
    z = np.zeros((4, 50), np.float32)
    z[:, [40, 7, 23]] = 3.0                 # ties: the lowest id wins
    z[1, 7] = 2.5                           # row 1: 23 < 40 and 7 is lower now
    T = np.array([0.0, 0.0, -1.0, np.nan], np.float32)
    out = oracle.draft_sample(z, T, np.full(4, 0.5, np.float32))
    assert out["tokens"][0] == 7 and out["probs"][0] == 1.0
    assert out["tokens"][1] == 23 and out["probs"][1] == 1.0
    assert list(out["tokens"][2:]) == [-1, -1]
    assert np.all(out["flags"][2:] == oracle.FLAG_E) and np.all(np.isnan(out["probs"][2:]))


def test_draft_sample_hand_case():
    # softmax of log([1, 0, 2, 1]) = [1/4, 0, 1/2, 1/4]: u = 1/4 lands on the
    # boundary C_0 = 1/4, strict '>' skips the zero-mass token 1 and picks 2
    z = np.log(np.array([[1.0, 1e-300, 2.0, 1.0]])).astype(np.float32)
    z[0, 1] = -1e4                          # exp underflows to exactly 0
    out = oracle.draft_sample(z, [1.0], np.array([0.25], np.float32))
    assert out["tokens"][0] == 2
    out = oracle.draft_sample(z, [1.0], np.array([0.0], np.float32))
    assert out["tokens"][0] == 0


@pytest.mark.parametrize("T", [0.7, 1.0])
def test_draft_sample_chi_square(T):
    g = _rng(31)
    V, N = 16, 200_000
    z = (g.standard_normal(V) * 1.5).astype(np.float32)
    rows = np.ascontiguousarray(np.broadcast_to(z, (N, V)))
    out = oracle.draft_sample(rows, np.full(N, T, np.float32), g.random(N, dtype=np.float32),
                              threads=8)
    q = scipy.special.softmax(z.astype(np.float64) / T)
    hist = np.bincount(out["tokens"], minlength=V)
    assert scipy.stats.chisquare(hist, q * N).pvalue > 1e-3


# --------------------------------------------------------------------------
# verify with gathered draft probabilities
# --------------------------------------------------------------------------
def gathered_q(w):
    """q_i(x_i) of every drafted position from the stored draft rows (fp64
    scipy softmax, rounded to fp32 as a drafter would hand it over); 1.0 for
    greedy sequences, whose accept test never reads it."""
    d = wl.logits_as_f32(w.draft).astype(np.float64)
    qg = np.ones(w.total, np.float32)
    for b in range(w.B):
        T = float(w.temperature[b])
        if T <= 0:
            continue
        for i in range(int(w.k[b])):
            j = int(w.offsets[b]) + i
            qg[j] = np.float32(scipy.special.softmax(d[j] / T)[w.tokens[j]])
    return qg


@pytest.mark.parametrize("name,B", [("c1", 8), ("c3", 6), ("c5", 16)])
def test_gathered_equals_plain_verify(name, B):
    w = wl.make_workload(name, trial=2, B=B)
    ref = oracle.verify(w, diag=True)
    got = oracle.verify(w, diag=True, draft_probs=gathered_q(w))
    amb = ((ref["flags"] | got["flags"]) & (oracle.FLAG_A | oracle.FLAG_B)) != 0
    for b in range(w.B):
        if amb[b]:
            continue
        sl = slice(w.target_row(b, 0), w.target_row(b, int(w.k[b])) + 1)
        assert got["n"][b] == ref["n"][b], (name, b)
        assert np.array_equal(got["tokens"][sl], ref["tokens"][sl]), (name, b)
    ok = ~np.isnan(ref["qx"])
    assert np.all(np.abs(got["qx"][ok] - ref["qx"][ok]) <= 1e-7 * ref["qx"][ok] + 1e-30)


def test_gathered_lossless_chi_square():
    """k = 1, V = 16: drafts drawn from q with their gathered q(x) -> the first
    emitted token follows p; acceptance rate = sum min(p, q)."""
    g = _rng(41)
    V, N, T = 16, 200_000, 1.0
    zt = (g.standard_normal((2, V)) * 1.5).astype(np.float32)
    zd = (g.standard_normal(V) * 1.5).astype(np.float32)
    p0 = scipy.special.softmax(zt[0].astype(np.float64))
    q = scipy.special.softmax(zd.astype(np.float64))
    x = g.choice(V, size=N, p=q)
    target = np.ascontiguousarray(np.tile(zt, (N, 1)))
    draft = np.ascontiguousarray(np.broadcast_to(zd, (N, V)))
    w = wl.assemble(target, draft, x, g.random(2 * N, dtype=np.float32), np.full(N, T), [1] * N)
    out = oracle.verify(w, threads=8, draft_probs=q[x].astype(np.float32))
    first = np.bincount(out["tokens"][0::2], minlength=V)
    assert scipy.stats.chisquare(first, p0 * N).pvalue > 1e-3
    acc = np.mean(out["n"] == 1)
    expect = np.minimum(p0, q).sum()
    assert abs(acc - expect) < 5 * math.sqrt(expect * (1 - expect) / N)


def test_gathered_reads_only_the_rejected_draft_row():
    """Rewriting every draft row except the one at each sequence's first
    rejection changes nothing: the accept tests use the gathered values.
    (The rewritten rows put almost all mass on the drafted token, so a
    verify that read q(x) from them would reject far more often.)"""
    w = wl.make_workload("c5", trial=3, B=24, V=4000)
    qg = gathered_q(w)
    ref = oracle.verify(w, draft_probs=qg)
    assert (ref["n"][w.temperature > 0] > 0).sum() >= 4     # rows before n exist
    draft = wl.logits_as_f32(w.draft).copy()
    for b in range(w.B):
        for i in range(int(w.k[b])):
            if i != ref["n"][b]:
                j = int(w.offsets[b]) + i
                draft[j] = -10.0
                draft[j, w.tokens[j]] = 20.0
    stored = wl.bf16_round(draft) if w.draft.dtype == np.uint16 else draft
    w2 = wl.Workload(**{**w.__dict__, "draft": stored})
    got = oracle.verify(w2, draft_probs=qg)
    assert np.array_equal(got["n"], ref["n"]) and np.array_equal(got["tokens"], ref["tokens"])


def test_gathered_bad_values_are_data_errors():
    w = wl.make_workload("c3", trial=4, B=6, V=2000)
    qg = gathered_q(w)
    for bad in (0.0, -0.5, np.nan, np.inf, 1.5):
        q2 = qg.copy()
        q2[w.offsets[2] + 1] = bad
        out = oracle.verify(w, draft_probs=q2)
        assert out["n"][2] == -1 and out["flags"][2] == oracle.FLAG_E, bad
        ref = oracle.verify(w, draft_probs=qg)
        assert np.array_equal(np.delete(out["n"], 2), np.delete(ref["n"], 2))
