"""Pins of reading R26 in the oracle (CPU only): a logit row whose maximum is
not finite makes its sequence a data error (n = -1, every slot -1, flag E)
exactly when the verify reaches that row -- target and draft rows at
positions up to and including the first rejection (the gathered form reads a
draft row only at the rejection) -- and changes nothing when it lies past the
first rejection, where the pages' loop never looks.

The cases are built so the scan's stopping point is known without the oracle:
u = 0 accepts every position (alpha > 0 for finite rows), and a draft row
that puts its mass on a token the target row gives almost none rejects at
u = 0.5 (alpha ~ 1e-9).
"""
import numpy as np

import oracle
import workloads as wl

V, K = 64, 4


def base_rows(seed):
    g = np.random.default_rng(seed)
    t = g.standard_normal((K + 1, V)).astype(np.float32)
    d = g.standard_normal((K, V)).astype(np.float32)
    x = g.integers(0, V, size=K)
    return t, d, x


def run(t, d, x, u, T=1.0, qg=None):
    w = wl.assemble(t, d, x, u, [T], [K])
    return oracle.verify(w, draft_probs=qg)


def accept_all():
    return np.zeros(K + 1, np.float32)


def reject_at(t, d, x, i):
    """Uniforms and rows such that position i rejects (and earlier ones accept)."""
    d[i] = -30.0
    d[i, x[i]] = 30.0            # q(x_i) ~ 1
    t[i, x[i]] = -30.0           # p(x_i) ~ 1e-13
    u = np.zeros(K + 1, np.float32)
    u[i] = 0.5
    return u


def is_error(r):
    return r["n"][0] == -1 and np.all(r["tokens"] == -1) and r["flags"][0] & oracle.FLAG_E


def test_clean_rows_are_not_errors():
    t, d, x = base_rows(1)
    r = run(t, d, x, accept_all())
    assert r["n"][0] == K and not r["flags"][0] & oracle.FLAG_E
    t, d, x = base_rows(2)
    u = reject_at(t, d, x, 1)
    r = run(t, d, x, u)
    assert r["n"][0] == 1 and not r["flags"][0] & oracle.FLAG_E


def test_nonfinite_rows_the_scan_reaches():
    for pos in range(K + 1):
        for what in ("+inf", "all -inf"):
            t, d, x = base_rows(3)
            if what == "+inf":
                t[pos, (x[min(pos, K - 1)] + 7) % V] = np.inf
            else:
                t[pos] = -np.inf
            assert is_error(run(t, d, x, accept_all())), (pos, what)
    for pos in range(K):
        t, d, x = base_rows(4)
        d[pos, 5] = np.inf
        assert is_error(run(t, d, x, accept_all())), pos


def test_nonfinite_at_the_rejection():
    t, d, x = base_rows(5)
    u = reject_at(t, d, x, 2)
    t2 = t.copy()
    t2[2, (x[2] + 1) % V] = np.inf
    assert is_error(run(t2, d, x, u))
    d2 = d.copy()
    d2[2, (x[2] + 1) % V] = np.inf
    assert is_error(run(t, d2, x, u))


def test_nonfinite_past_the_rejection_changes_nothing():
    t, d, x = base_rows(6)
    u = reject_at(t, d, x, 1)
    clean = run(t, d, x, u)
    assert clean["n"][0] == 1
    for pos in (2, 3, 4):
        t2 = t.copy()
        t2[pos, 9] = np.inf
        r = run(t2, d, x, u)
        assert r["n"][0] == 1 and np.array_equal(r["tokens"], clean["tokens"]), pos
        assert not r["flags"][0] & oracle.FLAG_E
        if pos < K:
            d2 = d.copy()
            d2[pos] = np.nan
            r = run(t, d2, x, u)
            assert np.array_equal(r["tokens"], clean["tokens"]) and r["n"][0] == 1, pos


def test_greedy_reaches_rows_up_to_the_first_mismatch():
    g = np.random.default_rng(7)
    t = g.standard_normal((K + 1, V)).astype(np.float32)
    d = np.zeros((K, V), np.float32)
    x = np.argmax(t[:K], axis=1)
    x[3] = (x[3] + 1) % V                        # first mismatch at position 3
    clean = run(t, d, x, accept_all(), T=0.0)
    assert clean["n"][0] == 3
    t2 = t.copy()
    t2[1, x[1]] = np.inf                         # still the argmax at 1: accepted, but non-finite
    assert is_error(run(t2, d, x, accept_all(), T=0.0))
    t3 = t.copy()
    t3[4, 0] = np.inf                            # past the mismatch
    r = run(t3, d, x, accept_all(), T=0.0)
    assert r["n"][0] == 3 and np.array_equal(r["tokens"], clean["tokens"])


def test_gathered_form_reads_the_draft_row_only_at_the_rejection():
    t, d, x = base_rows(8)
    u = reject_at(t, d, x, 2)
    qg = np.full(K, 0.5, np.float32)
    qg[2] = 1.0                                  # the drafter was sure of x_2
    clean = run(t, d, x, u, qg=qg)
    assert clean["n"][0] == 2
    for pos in (0, 1, 3):                        # draft rows the gathered form never reads
        d2 = d.copy()
        d2[pos, 3] = np.inf
        r = run(t, d2, x, u, qg=qg)
        assert np.array_equal(r["tokens"], clean["tokens"]) and r["n"][0] == 2, pos
    d2 = d.copy()
    d2[2, 3] = np.inf                            # the residual's draft row
    assert is_error(run(t, d2, x, u, qg=qg))
