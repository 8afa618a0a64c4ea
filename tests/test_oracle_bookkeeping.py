"""Pins of the oracle's post-verify bookkeeping and n-gram drafter (CPU only).

* commit (page "【大模型】- 推测解码", sections 基础推测解码器 / 批量推测解码;
  page "投机解码", section 动手实践): every sequence gains its accepted drafts
  and its emitted token, in order, up to its capacity; data errors gain
  nothing; the packed list is the concatenation in sequence order (checked
  against numpy slicing).
* adaptive k (page "【大模型】- 推测解码", section 自适应推测解码): k trajectories
  derived by hand from the page's rule -- start at (min_k + max_k) // 2,
  decide once 10 rates are held, mean of the last 10 strictly above 0.8 or
  below 0.5, clamp to [min_k, max_k] -- including the exact boundaries 0.8
  and 0.5 and a k that changes between rounds.
* n-gram drafter (page "投机解码", section Lookahead 与 n-gram 投机; page
  "大模型推理无损加速:投机采样...", section 四): hand cases (most recent match,
  fall back to shorter n-grams, continuation cut at the sequence end, no
  match) and a brute-force search with numpy sliding windows.
"""
import numpy as np
import pytest

import oracle


# --------------------------------------------------------------------------
# commit
# --------------------------------------------------------------------------
def test_commit_hand_case():
    # B = 3, k = [2, 0, 3]: slots at offsets[b] + b
    offsets = np.array([0, 2, 2, 5], np.int32)
    out_tokens = np.array([11, 12, 13, 21, 31, 32, 33, 34], np.int32)
    #                      seq0: n=1 -> 11, 12 (emitted) ; seq1: n=0 -> 21 ; seq2: n=-1 (error)
    out_n = np.array([1, 0, -1], np.int32)
    seq = np.zeros((3, 6), np.int32)
    seq[0, :2] = [1, 2]
    seq[1, :5] = [5, 5, 5, 5, 5]
    seq[2, :1] = [9]
    L = np.array([2, 5, 1], np.int32)
    s2, L2, com, coff = oracle.commit(out_tokens, out_n, offsets, seq, L)
    assert list(L2) == [4, 6, 1]
    assert list(s2[0, :4]) == [1, 2, 11, 12] and list(s2[1]) == [5, 5, 5, 5, 5, 21]
    assert list(com) == [11, 12, 21] and list(coff) == [0, 2, 3, 3]
    # capacity: seq 1 is full now; committing again adds nothing
    _, L3, com3, coff3 = oracle.commit(out_tokens, out_n, offsets, s2, L2)
    assert list(L3) == [6, 6, 1] and list(coff3) == [0, 2, 2, 2]


def test_commit_matches_numpy_slices():
    g = np.random.default_rng(3)
    B, max_len = 40, 64
    k = g.integers(0, 8, size=B).astype(np.int32)
    offsets = np.concatenate([[0], np.cumsum(k)]).astype(np.int32)
    out_tokens = g.integers(0, 1000, size=int(offsets[-1]) + B).astype(np.int32)
    out_n = np.array([g.integers(-1, kb + 1) for kb in k], np.int32)
    L = g.integers(0, max_len + 1, size=B).astype(np.int32)
    seq = g.integers(0, 1000, size=(B, max_len)).astype(np.int32)
    s2, L2, com, coff = oracle.commit(out_tokens, out_n, offsets, seq, L)
    parts = []
    for b in range(B):
        want = out_tokens[offsets[b] + b: offsets[b] + b + out_n[b] + 1] if out_n[b] >= 0 else []
        want = np.asarray(want, np.int32)[:max_len - L[b]]
        parts.append(want)
        np.testing.assert_array_equal(s2[b, :L[b]], seq[b, :L[b]])          # old tokens kept
        np.testing.assert_array_equal(s2[b, L[b]:L2[b]], want)
        np.testing.assert_array_equal(s2[b, L2[b]:], seq[b, L2[b]:])         # nothing past the end
    np.testing.assert_array_equal(com, np.concatenate(parts) if parts else [])
    np.testing.assert_array_equal(np.diff(coff), [len(p) for p in parts])


# --------------------------------------------------------------------------
# adaptive k
# --------------------------------------------------------------------------
def run_adapt(ns, ks, B=1, min_k=1, max_k=10):
    a = oracle.AdaptK(B, min_k, max_k)
    out = []
    for n, k in zip(ns, ks):
        out.append(int(a.update(np.full(B, n, np.int32), np.full(B, k, np.int32))[0]))
    return out


def test_adapt_k_starts_in_the_middle_and_waits_for_ten_rounds():
    assert oracle.AdaptK(1, 1, 10).k[0] == 5
    assert oracle.AdaptK(1, 2, 9).k[0] == 5
    # all drafts accepted: rate 1 > 0.8 from the 10th round on, one step per round, capped at 10
    assert run_adapt([5] * 16, [5] * 16) == [5] * 9 + [6, 7, 8, 9, 10, 10, 10]


def test_adapt_k_boundaries_are_strict():
    # rate exactly 0.8 (4 of 5) never raises k; exactly 0.5 (1 of 2) never lowers it
    assert run_adapt([4] * 20, [5] * 20) == [5] * 20
    assert run_adapt([1] * 20, [2] * 20) == [5] * 20
    # nothing accepted: rate 0 < 0.5 lowers k from the 10th round, floor 1
    assert run_adapt([0] * 16, [5] * 16) == [5] * 9 + [4, 3, 2, 1, 1, 1, 1]


def test_adapt_k_window_is_the_last_ten():
    # 10 rounds at rate 1, then rate 0: the mean of the last 10 is
    # (10 - j) / 10 after j zero rounds: > 0.8 for j = 0, 1; in [0.5, 0.8] for
    # j = 2..5; < 0.5 from j = 6 on.
    ns = [5] * 10 + [0] * 9
    got = run_adapt(ns, [5] * 19)
    assert got == [5] * 9 + [6] + [7] + [7, 7, 7, 7] + [6, 5, 4, 3]


def test_adapt_k_rate_uses_the_rounds_own_k():
    # n = 3 accepted of k = 3 drafted is rate 1; of k = 4 it is 0.75
    assert run_adapt([3] * 10, [3] * 10)[-1] == 6
    assert run_adapt([3] * 10, [4] * 10)[-1] == 5


def test_adapt_k_history_cap_and_errors():
    a = oracle.AdaptK(2, 1, 10)
    for r in range(150):
        a.update(np.array([5, -1], np.int32), np.array([5, 5], np.int32))
    assert a.k[0] == 10 and a.count[0] == 100
    assert a.k[1] == 5 and a.count[1] == 0          # data errors leave the state alone


# --------------------------------------------------------------------------
# n-gram drafter
# --------------------------------------------------------------------------
def draft_of(seq, n_max=3, n_min=1, k_max=4):
    s = np.zeros((1, 32), np.int32)
    s[0, :len(seq)] = seq
    toks, off = oracle.ngram_draft(s, [len(seq)], n_max, n_min, k_max)
    return list(toks[off[0]:off[1]])


def test_ngram_hand_cases():
    assert draft_of([1, 2, 3, 4, 1, 2, 3]) == [4, 1, 2, 3]          # trigram match at the start
    assert draft_of([7, 1, 5, 7, 1, 6, 7, 1], n_max=2) == [6, 7, 1]  # most recent of two matches
    assert draft_of([1, 2, 3, 9, 8, 2, 3], k_max=3) == [9, 8, 2]     # no trigram: the bigram [2, 3]
    assert draft_of([4, 5, 6, 4], n_max=3) == [5, 6, 4]              # unigram 4, cut at the end
    assert draft_of([1, 2, 3]) == []                                 # nothing repeats
    assert draft_of([5, 5]) == [5]                                   # the match may overlap the suffix
    assert draft_of([3]) == [] and draft_of([]) == []
    assert draft_of([1, 2, 1, 2], n_max=2, n_min=2, k_max=0) == []


def _brute(seq, n_max, n_min, k_max):
    from numpy.lib.stride_tricks import sliding_window_view
    seq = np.asarray(seq)
    L = len(seq)
    for n in range(n_max, n_min - 1, -1):
        if L < n + 1:
            continue
        win = sliding_window_view(seq[:L - 1], n)          # windows that end before the last token
        hits = np.nonzero((win == seq[L - n:]).all(axis=1))[0]
        if hits.size:
            j = int(hits.max())
            return list(seq[j + n: j + n + k_max])
    return []


def test_ngram_matches_brute_force():
    g = np.random.default_rng(17)
    B, max_len = 200, 96
    seq = g.integers(0, 6, size=(B, max_len)).astype(np.int32)       # small alphabet: many repeats
    L = g.integers(0, max_len + 1, size=B).astype(np.int32)
    for n_max, n_min, k_max in ((3, 1, 5), (4, 2, 8), (1, 1, 3)):
        toks, off = oracle.ngram_draft(seq, L, n_max, n_min, k_max)
        for b in range(B):
            assert list(toks[off[b]:off[b + 1]]) == _brute(seq[b, :L[b]], n_max, n_min, k_max), b
