"""Pins of the oracle's ambiguity flags and of its degenerate-residual
fallback (reading R11), against constructed cases whose answer is fixed by
hand or by numpy.searchsorted.

* Flag D and the fallback.  A rejection happens with probability Z (page
  "投机解码", section 无损保证：数学推导, the normaliser identity), so a
  rejection that leaves Z < 1e-9 can only come from rounding; the oracle then
  draws from p_n instead of the residual (page "大模型推理无损加速:投机采样...",
  section 二.2 defines p'(x) only for Z > 0).  The cases below build a rejected
  position whose p_n and q_n differ by a relative 1e-4 at the drafted token
  alone, so Z = 1e-4 q_n(x), and choose the draw uniform so that a draw from
  p_n, a draw from q_n and a residual draw give three different tokens.
* Flag A: |u - alpha| < 1e-5 on an accept test the scan evaluates (tests past
  the first rejection are never evaluated, so they never flag).
* Flag B: u Z within 1e-12 of a CDF boundary C_t.

Every case runs through oracle.verify_probs (the probability-domain entry:
no softmax), and tests/test_oracle_mutants.py plants the plausible mistakes
(fallback from q_n, no fallback, thresholds moved by orders of magnitude,
flags never set) that these pins must catch.
"""
import math

import numpy as np

import oracle

V = 1000
EPS = 1e-4                      # relative gap p_n(x) = q_n(x) (1 - EPS): alpha = 1 - EPS
U_REJECT = np.float32(0.99996)  # above alpha = 0.9999 by 6e-5: a rejection, outside the accept band


def _rows(q0, seed=0, V=V):
    """p_n, q_n over V tokens: token 0 is the drafted one with q_n(0) = q0,
    p_n(0) = q0 (1 - EPS); the other tokens share the rest in the same
    proportions s_v in both rows (so p_n(v) > q_n(v) for every v > 0)."""
    g = np.random.default_rng(seed)
    s = g.random(V)
    s[0] = 0.0
    s /= s.sum()
    p0 = q0 * (1.0 - EPS)
    p = s * (1.0 - p0)
    q = s * (1.0 - q0)
    p[0], q[0] = p0, q0
    return p, q


def _verify(p, q, u_draw, u_accept=U_REJECT):
    bonus = np.full(len(p), 1.0 / len(p))
    out = oracle.verify_probs(np.stack([p, bonus]), q[None], np.array([[0]]),
                              np.array([[u_accept, u_draw]], np.float32), 1, True)
    return int(out["n"][0]), int(out["tokens"][0, 0]), int(out["flags"][0]), float(out["Z"][0]), \
        float(out["gap"][0])


def _residual_mass(p, q):
    return math.fsum(np.maximum(0.0, p - q))


def _searchsorted(mass, u):
    C = np.cumsum(mass)
    return int(np.searchsorted(C, float(u) * C[-1], side="right"))


def test_degenerate_residual_draws_from_the_target_row():
    """Z = 1e-4 q_n(x) < 1e-9: flag D, and the token is the inverse-CDF draw
    from p_n -- not from q_n, not from the (rounding-level) residual."""
    u = np.float32(4 * 2 ** -20)                 # target u * sum(p_n) = u
    p, q = _rows(float(u) + 2e-10)               # C_p(0) = u - 1.8e-10 < target < C_q(0) = u + 2e-10
    n, tok, flags, Z, gap = _verify(p, q, u)
    assert n == 0
    assert flags == oracle.FLAG_D
    assert _residual_mass(p, q) < 1e-9
    assert abs(Z - math.fsum(p)) < 1e-15                # the reported Z is that of the fallback, p_n
    assert tok == _searchsorted(p, u) == 1       # from p_n: token 0's mass ends just below the target
    assert _searchsorted(q, u) == 0              # a draw from q_n would give token 0
    assert _searchsorted(np.maximum(0.0, p - q), u) >= 1
    assert gap > 1e-10                           # not a flag-B row


def test_degenerate_residual_can_emit_the_rejected_token():
    """With the target below p_n(x) the fallback emits the rejected token x
    itself, which the residual (zero mass at x) never could."""
    u = np.float32(2 * 2 ** -20)
    p, q = _rows(4 * 2 ** -20 + 2e-10)
    n, tok, flags, Z, gap = _verify(p, q, u)
    assert n == 0 and flags == oracle.FLAG_D and _residual_mass(p, q) < 1e-9
    assert tok == _searchsorted(p, u) == 0
    assert _searchsorted(np.maximum(0.0, p - q), u) >= 1


def test_small_but_usable_residual_is_drawn_normally():
    """Z = 1e-7 (above the 1e-9 threshold): no flag, the residual draw."""
    p, q = _rows(1e-3, seed=1)
    for u in (np.float32(0.5), np.float32(0.123), np.float32(0.9)):
        n, tok, flags, Z, gap = _verify(p, q, u)
        assert n == 0 and flags == 0
        assert abs(Z - 1e-7) < 1e-12
        assert tok == _searchsorted(np.maximum(0.0, p - q), u)
        assert tok >= 1


def test_degenerate_threshold_bracket():
    """Z = 2e-9 is drawn from the residual, Z = 5e-10 falls back.  (Eight
    tokens, so each residual mass, ~Z/7, lies far above the 1e-12 CDF band:
    at V = 1000 a residual of 2e-9 spreads ~2e-12 per token and nearly every
    draw lands within the band of some boundary, a flag-B row.)"""
    u = np.float32(0.37)
    p, q = _rows(2e-5, seed=2, V=8)              # Z = 2e-9
    _, tok, flags, _, _ = _verify(p, q, u)
    assert flags == 0 and tok == _searchsorted(np.maximum(0.0, p - q), u)
    p, q = _rows(5e-6, seed=2, V=8)              # Z = 5e-10
    _, tok, flags, _, _ = _verify(p, q, u)
    assert flags == oracle.FLAG_D and tok == _searchsorted(p, u)


# --------------------------------------------------------------------------
# flag A: the accept band
# --------------------------------------------------------------------------
P4 = np.array([[1 / 8, 3 / 8, 1 / 4, 1 / 4], [1 / 4, 1 / 4, 1 / 4, 1 / 4]])
Q4 = np.array([[1 / 4, 1 / 4, 1 / 4, 1 / 4]])    # alpha(x = 0) = 0.5 exactly


def _alpha_half(u0):
    out = oracle.verify_probs(P4, Q4, np.array([[0]]), np.array([[u0, 0.3]], np.float32), 1, True)
    return int(out["n"][0]), int(out["flags"][0])


def test_flag_a_inside_the_band():
    assert _alpha_half(0.5 + 2 ** -20) == (0, oracle.FLAG_A)    # rejected, 9.5e-7 from alpha
    assert _alpha_half(0.5 - 2 ** -20) == (1, oracle.FLAG_A)    # accepted, 9.5e-7 from alpha
    assert _alpha_half(0.5 + 2 ** -17) == (0, oracle.FLAG_A)    # 7.6e-6 from alpha


def test_flag_a_outside_the_band():
    assert _alpha_half(0.5 + 2 ** -16) == (0, 0)                # 1.5e-5 from alpha
    assert _alpha_half(0.5 - 2 ** -16) == (1, 0)
    assert _alpha_half(0.75) == (0, 0)


def test_flag_a_only_on_evaluated_tests():
    """Position 1 has alpha = 1 and u = 1 - 2^-24 (inside the band): it flags
    only when the scan reaches it."""
    P = np.array([[1 / 8, 3 / 8, 1 / 4, 1 / 4], [1 / 4] * 4, [1 / 4] * 4])
    Q = np.array([[1 / 4] * 4, [1 / 4] * 4])
    x = np.array([[0, 2]])
    u_hi = 1 - 2 ** -24
    out = oracle.verify_probs(P, Q, x, np.array([[0.9, u_hi, 0.3]], np.float32), 2, True)
    assert out["n"][0] == 0 and out["flags"][0] == 0           # rejected at 0: position 1 unseen
    out = oracle.verify_probs(P, Q, x, np.array([[0.1, u_hi, 0.3]], np.float32), 2, True)
    assert out["n"][0] == 2 and out["flags"][0] == oracle.FLAG_A


# --------------------------------------------------------------------------
# flag B: the CDF band
# --------------------------------------------------------------------------
def _bonus(pk, u):
    """k = 0: a bonus draw from pk with uniform u."""
    out = oracle.verify_probs(np.asarray(pk, float)[None], np.zeros((1, len(pk))),
                              np.zeros((1, 0), np.int32), np.array([[u]], np.float32), 0, True)
    return int(out["tokens"][0, 0]), int(out["flags"][0]), float(out["gap"][0])


def test_flag_b_on_an_exact_boundary():
    tok, flags, gap = _bonus([0, 1 / 4, 0, 1 / 2, 1 / 4], 0.25)
    assert (tok, flags, gap) == (3, oracle.FLAG_B, 0.0)         # C_1 = u Z exactly: strict '>' moves on
    tok, flags, _ = _bonus([0, 1 / 4, 0, 1 / 2, 1 / 4], 0.3)
    assert (tok, flags) == (3, 0)


def test_flag_b_band_width():
    """u Z 5e-14 from a boundary flags; 5e-12 from it does not."""
    for delta, flagged in ((5e-14, True), (5e-12, False)):
        pk = [0.25 + delta, 0.5 - delta, 0.25]
        tok, flags, gap = _bonus(pk, 0.25)
        assert tok == 0                                         # C_0 = 0.25 + delta > 0.25 Z
        assert abs(gap - delta) < 1e-15
        assert (flags == oracle.FLAG_B) == flagged, (delta, flags)
