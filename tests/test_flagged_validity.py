"""CPU pins of the validity check that tests/test_gpu_parity.py applies to
sequences the oracle flags as ambiguous: it must accept the oracle's own
outcome and the outcome just across the flagged boundary, and reject
tokens with no mass, tokens far from u Z, and accept counts the bands
cannot explain."""
import numpy as np

import oracle
import workloads as wl
from test_gpu_parity import flagged_valid


def _masked_zero_uniform():
    """One sampling sequence (k = 2, identical rows: both drafts accepted)
    whose bonus row is masked on tokens 0..99, drawn with u = 0: the oracle
    flags it B (u Z = 0 = C_t on the masked prefix) and emits token 100."""
    g = np.random.default_rng(5)
    V = 500
    t = (g.standard_normal((3, V)) * 2).astype(np.float32)
    t[2, :100] = -np.inf
    w = wl.assemble(t, t[:2], [7, 9], [0.5, 0.5, 0.0], [1.0], [2])
    ref = oracle.verify(w)
    assert ref["flags"][0] == oracle.FLAG_B and ref["n"][0] == 2
    return w, ref


def test_accepts_the_oracle_outcome():
    w, ref = _masked_zero_uniform()
    assert list(ref["tokens"]) == [7, 9, 100]
    assert flagged_valid(w, 0, 2, ref["tokens"])


def test_rejects_a_masked_token():
    w, _ = _masked_zero_uniform()
    assert not flagged_valid(w, 0, 2, np.array([7, 9, 99]))
    assert not flagged_valid(w, 0, 2, np.array([7, 9, 0]))


def test_rejects_a_token_far_from_the_target():
    w, _ = _masked_zero_uniform()
    assert not flagged_valid(w, 0, 2, np.array([7, 9, 300]))


def test_rejects_counts_the_bands_cannot_explain():
    w, ref = _masked_zero_uniform()
    # alpha = 1 at both positions (identical rows), u = 0.5: a rejection at
    # 0 or 1 is impossible, and the accepted prefix must be the drafts
    assert not flagged_valid(w, 0, 0, np.array([100, -1, -1]))
    assert not flagged_valid(w, 0, 1, np.array([7, 100, -1]))
    assert not flagged_valid(w, 0, 2, np.array([7, 8, 100]))
    assert not flagged_valid(w, 0, 2, np.array([7, 9, 100])[::-1])


def test_accepts_the_token_across_a_flagged_boundary():
    """A bonus draw whose u Z lands exactly on C_t (the bonus row holds four
    equal logits: p = 1/4 each, u = 1/2): the oracle's strict '>' gives
    token 2, a draw rounding the other way gives token 1 -- both valid;
    token 0 or 3 is not."""
    z = np.zeros((1, 4), np.float32)
    w = wl.assemble(z, np.zeros((0, 4), np.float32), [], [0.5], [1.0], [0])
    ref = oracle.verify(w)
    assert ref["flags"][0] == oracle.FLAG_B and ref["tokens"][0] == 2
    assert flagged_valid(w, 0, 0, np.array([2]))
    assert flagged_valid(w, 0, 0, np.array([1]))
    assert not flagged_valid(w, 0, 0, np.array([0]))
    assert not flagged_valid(w, 0, 0, np.array([3]))
