"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Nothing here compares the oracle with itself.  Each test checks one property
that a plausible mistake in ``oracle/oracle.c`` (a dropped term, a wrong sign,
'<=' for '<', a transposed p/q, a wrong uniform slot, an untempered row) would
break:

* softmax vs scipy.special.softmax (library routine), tempered;
* the normaliser identity of the lossless proof on the page "投机解码"
  (section 无损保证：数学推导): sum max(0,p-q) = sum max(0,q-p) = 1 - sum min(p,q);
* exact losslessness by enumeration over a dyadic grid of uniforms (the
  output marginal equation of the same section, and of the page
  "大模型推理无损加速:投机采样..." section 二.3) -- pins strict '<' in the
  accept test and strict '>' in the inverse CDF;
* statistical losslessness (chi-square, V=16, 10^6 trials) for several q;
* the accept-path equation P(accept, x=t) = min(p(t), q(t));
* inverse CDF == numpy.searchsorted(cumsum, u*Z, side='right');
* greedy path == argmax decoding, lowest index on ties;
* special cases: q == p, one-hot p, V = 2 closed form, k = 0;
* an independent numpy/scipy composition at real vocabulary sizes.
"""
from fractions import Fraction
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
# softmax
# --------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T", [0.6, 1.0, 2.5])
def test_softmax_matches_scipy(dtype, T):
    g = _rng(1)
    z = (g.standard_normal((4, 5000)) * 3).astype(np.float32)
    rows = wl.bf16_round(z) if dtype == "bf16" else z
    vals = wl.logits_as_f32(rows).astype(np.float64)
    p, m, S = oracle.softmax_rows(rows, T)
    ref = scipy.special.softmax(vals / T, axis=1)
    np.testing.assert_allclose(p, ref, rtol=1e-12, atol=1e-300)
    np.testing.assert_array_equal(m, vals.max(axis=1))
    for r in range(len(rows)):
        S_ref = math.fsum(np.exp((vals[r] - vals[r].max()) / T))
        assert abs(S[r] - S_ref) <= 1e-13 * S_ref
    assert np.all(np.abs(p.sum(axis=1) - 1) < 1e-13)


def test_softmax_temperature_not_dropped():
    # T must divide the logits: softmax(z/2) differs from softmax(z)
    z = np.array([[0.0, 1.0, 2.0, 3.0]], np.float32)
    p2, _, _ = oracle.softmax_rows(z, 2.0)
    p1, _, _ = oracle.softmax_rows(z, 1.0)
    assert abs(p2[0, 3] - math.exp(1.5) / sum(math.exp(x / 2) for x in range(4))) < 1e-15
    assert abs(p1[0, 3] - p2[0, 3]) > 0.1


# --------------------------------------------------------------------------
# Z identity (normaliser of the residual distribution)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("V", [16, 32000, 128256, 152064])
def test_residual_mass_identity(V):
    g = _rng(V)
    for trial in range(3):
        p = scipy.special.softmax(g.standard_normal(V) * 2)
        q = scipy.special.softmax(np.log(p) + g.standard_normal(V) * (0.1 + trial))
        # force a rejection at position 0: a token with p/q < 1, u just below 1
        x = int(np.argmin(p / q))
        assert p[x] / q[x] < 0.999
        P = np.stack([p, p])
        out = oracle.verify_probs(P, q[None], np.array([[x]]),
                                  np.array([[1 - 2 ** -24, 0.5]], np.float32), 1, True)
        assert out["n"][0] == 0
        Z = out["Z"][0]
        assert abs(Z - math.fsum(np.maximum(0, q - p))) < 1e-12
        assert abs(Z - (1 - math.fsum(np.minimum(p, q)))) < 1e-12


# --------------------------------------------------------------------------
# exact losslessness on a dyadic grid
# --------------------------------------------------------------------------
def _dyadic_case(seed):
    """q = powers of two, p = multiples of 1/64 with Z a power of two, so every
    quantity the oracle forms is exact in fp64."""
    q = np.array([Fraction(1, 2), Fraction(1, 4), Fraction(1, 8), Fraction(1, 16), Fraction(1, 16)])
    g = _rng(seed)
    while True:
        cuts = np.sort(g.integers(0, 65, size=4))
        c = np.diff(np.concatenate([[0], cuts, [64]]))
        p = np.array([Fraction(int(v), 64) for v in c])
        Z = sum(max(Fraction(0), a - b) for a, b in zip(p, q))
        if Z > 0 and (Z * 64).denominator == 1 and ((Z * 64).numerator & ((Z * 64).numerator - 1)) == 0:
            return p, q


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_lossless_exact_enumeration(seed):
    p, q = _dyadic_case(seed)
    p1 = np.array([Fraction(1, 8)] * 4 + [Fraction(1, 2)])      # bonus row
    V, G = len(p), 256
    grid = (np.arange(G) / G).astype(np.float32)                 # exact in fp32
    xs, u0, u1 = np.meshgrid(np.arange(V), grid, grid, indexing="ij")
    P = np.array([[float(a) for a in p], [float(a) for a in p1]])
    Q = np.array([[float(a) for a in q]])
    out = oracle.verify_probs(P, Q, xs.reshape(-1, 1),
                              np.stack([u0.ravel(), u1.ravel()], 1), 1, True)
    first = out["tokens"][:, 0].reshape(V, G * G)
    nacc = out["n"].reshape(V, G * G)
    second = out["tokens"][:, 1].reshape(V, G * G)
    # marginal of the first emitted token
    for t in range(V):
        prob = sum(q[x] * Fraction(int(np.sum(first[x] == t)), G * G) for x in range(V))
        assert prob == p[t], (t, prob, p[t])
    # accept-path equation: P(accept, x = t) = min(p(t), q(t))
    for t in range(V):
        acc = q[t] * Fraction(int(np.sum(nacc[t] == 1)), G * G)
        assert acc == min(p[t], q[t])
    # bonus token after an accept is distributed as the next target row
    for t in range(V):
        num = sum(q[x] * Fraction(int(np.sum((nacc[x] == 1) & (second[x] == t))), G * G)
                  for x in range(V))
        den = sum(q[x] * Fraction(int(np.sum(nacc[x] == 1)), G * G) for x in range(V))
        assert num / den == p1[t]
    assert not np.any(out["flags"] & oracle.FLAG_D)


# --------------------------------------------------------------------------
# statistical losslessness, V = 16, 10^6 trials
# --------------------------------------------------------------------------
def _q_cases(p, g):
    V = len(p)
    yield "identical", p.copy()
    d = g.dirichlet(np.full(V, 1.0))
    yield "random", d
    # q concentrated where p is small
    w = 1.0 / p ** 2
    yield "anti", w / w.sum()
    # near-disjoint support (tiny q on half the tokens)
    w = np.where(np.arange(V) < V // 2, 1.0, 1e-4)
    yield "disjointish", w / w.sum()


@pytest.mark.parametrize("case_idx", [0, 1, 2, 3])
def test_lossless_chi_square(case_idx):
    g = _rng(100 + case_idx)
    V, N = 16, 1_000_000
    p0 = g.dirichlet(np.full(V, 3.0))
    p0 = (p0 + 0.01) / (p0 + 0.01).sum()
    p1 = g.dirichlet(np.full(V, 3.0))
    p1 = (p1 + 0.01) / (p1 + 0.01).sum()
    name, q = list(_q_cases(p0, g))[case_idx]
    x = g.choice(V, size=N, p=q)
    u = g.random((N, 2), dtype=np.float32)
    out = oracle.verify_probs(np.stack([p0, p1]), q[None], x[:, None], u, 1, True)
    first = np.bincount(out["tokens"][:, 0], minlength=V)
    assert scipy.stats.chisquare(first, p0 * N).pvalue > 1e-3, name
    # acceptance rate = sum min(p, q) = 1 - Z
    acc = np.mean(out["n"] == 1)
    expect = np.minimum(p0, q).sum()
    assert abs(acc - expect) < 5 * math.sqrt(expect * (1 - expect) / N) + 1e-12, name
    # bonus token conditional on acceptance ~ p1
    sel = out["n"] == 1
    if sel.sum() > 1000:
        bonus = np.bincount(out["tokens"][sel, 1], minlength=V)
        assert scipy.stats.chisquare(bonus, p1 * sel.sum()).pvalue > 1e-3, name


def test_lossless_chain_k3():
    """With k = 3 the j-th emitted token, given the first j-1 were accepted
    drafts, is distributed as target row j-1 (chained positions)."""
    g = _rng(7)
    V, N, k = 16, 400_000, 3
    P = np.stack([(lambda d: (d + 0.02) / (d + 0.02).sum())(g.dirichlet(np.full(V, 2.0)))
                  for _ in range(k + 1)])
    Q = np.stack([g.dirichlet(np.full(V, 2.0)) for _ in range(k)])
    x = np.stack([g.choice(V, size=N, p=Q[i]) for i in range(k)], 1)
    u = g.random((N, k + 1), dtype=np.float32)
    out = oracle.verify_probs(P, Q, x, u, k, True)
    for j in range(k + 1):
        sel = out["n"] >= j
        tok = np.bincount(out["tokens"][sel, j], minlength=V)
        assert scipy.stats.chisquare(tok, P[j] * sel.sum()).pvalue > 1e-3, j


# --------------------------------------------------------------------------
# inverse CDF convention
# --------------------------------------------------------------------------
def test_inverse_cdf_hand_case():
    r = np.array([0.0, 0.25, 0.0, 0.5, 0.25])
    assert oracle.inverse_cdf(r, 0.25)[0] == 3      # C = .25 is not > .25: skip to t=3
    assert oracle.inverse_cdf(r, 0.0)[0] == 1       # zero-mass token 0 never picked
    assert oracle.inverse_cdf(r, 0.75)[0] == 4
    assert oracle.inverse_cdf(r, 0.7499999)[0] == 3
    assert oracle.inverse_cdf(r, 1 - 2 ** -24)[0] == 4
    t, Z, gap = oracle.inverse_cdf(r, 0.25)
    assert Z == 1.0 and gap == 0.0


def test_inverse_cdf_matches_searchsorted():
    g = _rng(3)
    for _ in range(200):
        V = int(g.integers(1, 3000))
        r = g.random(V) * (g.random(V) < 0.7)
        if r.sum() == 0:
            r[V // 2] = 1.0
        u = np.float32(g.random())
        t, Z, gap = oracle.inverse_cdf(r, u)
        C = np.cumsum(r)
        if gap < 1e-10:
            continue
        assert t == int(np.searchsorted(C, float(u) * C[-1], side="right"))
        assert r[t] > 0


# --------------------------------------------------------------------------
# greedy
# --------------------------------------------------------------------------
def test_greedy_equals_argmax_with_ties():
    V, k = 50, 3
    g = _rng(11)
    T_rows = g.standard_normal((k + 1, V)).astype(np.float32)
    T_rows[0, [7, 3, 20]] = 9.0          # tie: lowest index 3 wins
    T_rows[1, [5, 6]] = 9.0
    T_rows[2, 40] = 9.0
    T_rows[3, [0, 49]] = 9.0
    D_rows = g.standard_normal((k, V)).astype(np.float32)
    w = wl.assemble(T_rows, D_rows, [3, 5, 11], [0.9] * 4, [0.0], [k])
    out = oracle.verify(w)
    assert out["n"][0] == 2 and list(out["tokens"]) == [3, 5, 40, -1]
    w = wl.assemble(T_rows, D_rows, [3, 5, 40], [0.9] * 4, [0.0], [k])
    out = oracle.verify(w)
    assert out["n"][0] == 3 and list(out["tokens"]) == [3, 5, 40, 0]
    w = wl.assemble(T_rows, D_rows, [7, 5, 40], [0.9] * 4, [0.0], [k])
    out = oracle.verify(w)             # 7 ties the max but is not the lowest index
    assert out["n"][0] == 0 and list(out["tokens"]) == [3, -1, -1, -1]


def test_greedy_matches_numpy_argmax_bf16():
    w = wl.make_workload("c2g", V=4096)
    out = oracle.verify(w)
    vals = wl.logits_as_f32(w.target)
    a = [int(np.argmax(vals[i])) for i in range(w.k[0] + 1)]
    n = next((i for i in range(w.k[0]) if w.tokens[i] != a[i]), int(w.k[0]))
    assert out["n"][0] == n
    assert out["tokens"][n] == a[n]


# --------------------------------------------------------------------------
# special cases
# --------------------------------------------------------------------------
def test_identical_draft_accepts_everything():
    g = _rng(5)
    V, k, N = 300, 4, 400
    for trial in range(N):
        z = (g.standard_normal((k + 1, V)) * 2).astype(np.float32)
        x = g.integers(0, V, size=k)
        w = wl.assemble(z, z[:k], x, g.random(k + 1, dtype=np.float32), [1.0], [k])
        out = oracle.verify(w)
        assert out["n"][0] == k
        p = scipy.special.softmax(z[k].astype(np.float64))
        u = float(w.uniforms[k])
        assert out["tokens"][k] == np.searchsorted(np.cumsum(p), u * p.sum(), side="right")


def test_one_hot_target_always_emits_hot_token():
    g = _rng(6)
    V, k = 64, 3
    hot = 17
    for trial in range(200):
        zt = g.standard_normal((k + 1, V)).astype(np.float32)
        zt[:, hot] += 1000.0
        zd = (g.standard_normal((k, V)) * 3).astype(np.float32)
        x = g.integers(0, V, size=k)
        w = wl.assemble(zt, zd, x, g.random(k + 1, dtype=np.float32), [1.0], [k])
        out = oracle.verify(w)
        n = out["n"][0]
        assert all(out["tokens"][:n] == hot)
        assert out["tokens"][n] == hot


def test_v2_closed_form():
    # p = (a, 1-a), q = (b, 1-b): alpha(x=0) = min(1, a/b); residual is a point
    # mass on the token where p > q.
    for a, b in [(0.25, 0.75), (0.75, 0.25), (0.5, 0.5)]:
        P = np.array([[a, 1 - a], [0.5, 0.5]])
        Q = np.array([[b, 1 - b]])
        us = np.array([[u, 0.3] for u in np.linspace(0, 1, 1000, endpoint=False)], np.float32)
        out = oracle.verify_probs(P, Q, np.zeros((len(us), 1), np.int32), us, 1, True)
        alpha = min(1.0, a / b)
        np.testing.assert_array_equal(out["n"] == 1, us[:, 0] < alpha)
        rej = out["n"] == 0
        if rej.any():
            assert np.all(out["tokens"][rej, 0] == (0 if a > b else 1))


def test_k_zero_emits_bonus_or_argmax():
    g = _rng(9)
    z = (g.standard_normal((1, 100)) * 2).astype(np.float32)
    w = wl.assemble(z, np.zeros((0, 100), np.float32), [], [0.5], [1.0], [0])
    out = oracle.verify(w)
    p = scipy.special.softmax(z[0].astype(np.float64))
    assert out["n"][0] == 0
    assert out["tokens"][0] == np.searchsorted(np.cumsum(p), 0.5 * p.sum(), side="right")
    w = wl.assemble(z, np.zeros((0, 100), np.float32), [], [0.5], [0.0], [0])
    assert oracle.verify(w)["tokens"][0] == int(np.argmax(z[0]))


def test_data_errors_flag_rows():
    z = np.zeros((3, 8), np.float32)
    w = wl.assemble(z[:2], z[:1], [8], [0.1, 0.2], [1.0], [1])          # token out of range
    assert oracle.verify(w)["n"][0] == -1
    w = wl.assemble(z[:2], z[:1], [1], [0.1, 0.2], [-1.0], [1])         # negative T
    out = oracle.verify(w)
    assert out["n"][0] == -1 and out["flags"][0] & oracle.FLAG_E


def test_offsets_out_of_order_are_data_errors():
    """Reading R28: offsets [0, 4, 8, 6, 12, 15] run backwards at sequence 2
    (k = -2), and sequences 1 ([4, 8)) and 3 ([6, 12)) overlap, so all three
    are data errors with every slot of theirs -1; sequences 0 and 4, whose
    ranges are in order with every other, give exactly what they give when
    verified in a batch of their own."""
    g = _rng(28)
    V = 300
    offsets = np.array([0, 4, 8, 6, 12, 15], np.int32)
    B, total = len(offsets) - 1, 15
    t = (g.standard_normal((total + B, V)) * 2).astype(np.float32)
    d = (t[:total] + g.standard_normal((total, V)).astype(np.float32)).astype(np.float32)
    w = wl.Workload(name="order", V=V, B=B, dtype="f32", k=np.diff(offsets).astype(np.int32),
                    offsets=offsets, target=t, draft=d, tokens=g.integers(0, V, size=total).astype(np.int32),
                    uniforms=g.random(total + B, dtype=np.float32),
                    temperature=np.array([1.0, 1.0, 0.7, 0.0, 0.8], np.float32), sigma=np.zeros(B))
    out = oracle.verify(w)
    assert list(out["n"][[1, 2, 3]]) == [-1, -1, -1]
    assert all(out["flags"][[1, 2, 3]] == oracle.FLAG_E)
    assert np.all(out["tokens"][w.target_row(1, 0):w.target_row(1, 4) + 1] == -1)
    assert np.all(out["tokens"][w.target_row(3, 0):w.target_row(3, 6) + 1] == -1)
    alone = w.subset([0, 4])
    ref = oracle.verify(alone)
    assert out["n"][0] == ref["n"][0] >= 0 and out["n"][4] == ref["n"][1] >= 0
    np.testing.assert_array_equal(out["tokens"][0:5], ref["tokens"][0:5])
    np.testing.assert_array_equal(out["tokens"][16:20], ref["tokens"][5:9])


# --------------------------------------------------------------------------
# cross-check with an independent numpy / scipy composition at real V
# --------------------------------------------------------------------------
def _numpy_verify(w, b):
    kb = int(w.k[b])
    T = float(w.temperature[b])
    zt = [wl.logits_as_f32(w.target[w.target_row(b, i)]).astype(np.float64) for i in range(kb + 1)]
    zd = [wl.logits_as_f32(w.draft[w.draft_row(b, i)]).astype(np.float64) for i in range(kb)]
    x = w.tokens[w.offsets[b]:w.offsets[b + 1]]
    u = w.uniforms[w.uniform_slot(b, 0):w.uniform_slot(b, kb) + 1].astype(np.float64)
    if T == 0:
        a = [int(np.argmax(r)) for r in zt]
        n = next((i for i in range(kb) if x[i] != a[i]), kb)
        return n, a[n]
    p = [scipy.special.softmax(r / T) for r in zt]
    q = [scipy.special.softmax(r / T) for r in zd]
    n = kb
    for i in range(kb):
        if not u[i] < min(1.0, p[i][x[i]] / q[i][x[i]]):
            n = i
            break
    r = np.maximum(0, p[n] - q[n]) if n < kb else p[n]
    C = np.cumsum(r)
    return n, int(np.searchsorted(C, u[kb] * C[-1], side="right"))


@pytest.mark.parametrize("name,B", [("c1", 1), ("c2", 1), ("c2g", 1), ("c3", 6), ("c4", 6), ("c5", 12)])
def test_oracle_vs_numpy_composition(name, B):
    for trial in range(3 if B == 1 else 1):
        w = wl.make_workload(name, trial=trial, B=B)
        out = oracle.verify(w, diag=True, threads=4)
        for b in range(w.B):
            if out["flags"][b] & (oracle.FLAG_A | oracle.FLAG_D):
                continue
            if np.isfinite(out["gap"][b]) and out["gap"][b] < 1e-10:
                continue
            n, tok = _numpy_verify(w, b)
            assert out["n"][b] == n, (name, trial, b)
            assert out["tokens"][w.target_row(b, n)] == tok, (name, trial, b)
            kb = int(w.k[b])
            np.testing.assert_array_equal(
                out["tokens"][w.target_row(b, 0):w.target_row(b, n)],
                w.tokens[w.offsets[b]:w.offsets[b] + n])
            assert np.all(out["tokens"][w.target_row(b, n + 1):w.target_row(b, kb) + 1] == -1)


def test_alpha_has_no_epsilon_guard():
    # tiny q(x): alpha = p/q = 0.5 exactly; an additive guard on q would move it
    P = np.array([[5e-8, 1 - 5e-8], [0.5, 0.5]])
    Q = np.array([[1e-7, 1 - 1e-7]])
    us = np.array([[0.4999, 0.5], [0.5001, 0.5]], np.float32)
    out = oracle.verify_probs(P, Q, np.zeros((2, 1), np.int32), us, 1, True)
    assert list(out["n"]) == [1, 0]
