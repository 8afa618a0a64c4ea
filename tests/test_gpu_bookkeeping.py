"""GPU parity of the post-verify bookkeeping and the n-gram drafter against
the oracle: spec_commit, spec_adapt_k and spec_ngram_draft, all integer work
(adapt_k decides on fp64 means formed in the same order on both sides), so
the bar is bit-exact.  A last test runs a whole greedy round on the device:
n-gram drafts, the verify, and the commit."""
import numpy as np
import pytest

import oracle
import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sv(cuda):
    import os

    import speculative_decoding_rejection_spec_amd as sv
    if not os.path.exists(sv.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return sv


def T(a, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def random_round(g, B, max_len, kmax=8):
    k = g.integers(0, kmax + 1, size=B).astype(np.int32)
    offsets = np.concatenate([[0], np.cumsum(k)]).astype(np.int32)
    out_tokens = g.integers(0, 50000, size=int(offsets[-1]) + B).astype(np.int32)
    out_n = np.array([g.integers(-1, kb + 1) for kb in k], np.int32)
    seq = g.integers(0, 50000, size=(B, max_len)).astype(np.int32)
    L = g.integers(0, max_len + 1, size=B).astype(np.int32)
    L[:3] = [max_len, max_len - 1, 0][:B]                 # full, almost full, empty
    return k, offsets, out_tokens, out_n, seq, L


@pytest.mark.parametrize("B,max_len", [(1, 16), (300, 64), (3000, 40)])
def test_commit_parity(sv, cuda, B, max_len):
    import torch
    g = np.random.default_rng(B)
    k, offsets, out_tokens, out_n, seq, L = random_round(g, B, max_len)
    want = oracle.commit(out_tokens, out_n, offsets, seq, L)
    dseq, dL = T(seq, cuda), T(L, cuda)
    com, coff = sv.spec_commit(T(out_tokens, cuda), T(out_n, cuda), T(offsets, cuda), dseq, dL)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(dseq.cpu().numpy(), want[0])
    np.testing.assert_array_equal(dL.cpu().numpy(), want[1])
    np.testing.assert_array_equal(coff.cpu().numpy(), want[3])
    np.testing.assert_array_equal(com.cpu().numpy()[:want[3][-1]], want[2])


def test_commit_uniform_k_and_verify_outputs(sv, cuda):
    """Commit what spec_verify produced (uniform-k layout, C3 workload)."""
    import torch
    from test_gpu_parity import to_device
    w = wl.make_workload("c3", trial=2, B=48)
    d = to_device(w, cuda)
    tok, n = sv.spec_verify(d["target"], d["draft"], d["tokens"], None, d["uniforms"], d["temperature"],
                            k_uniform=int(w.k[0]))
    seq = np.zeros((w.B, 32), np.int32)
    L = np.full(w.B, 7, np.int32)
    dseq, dL = T(seq, cuda), T(L, cuda)
    com, coff = sv.spec_commit(tok, n, None, dseq, dL, k_uniform=int(w.k[0]))
    torch.cuda.synchronize()
    want = oracle.commit(tok.cpu().numpy(), n.cpu().numpy(), w.offsets, seq, L)
    np.testing.assert_array_equal(dseq.cpu().numpy(), want[0])
    np.testing.assert_array_equal(coff.cpu().numpy(), want[3])
    np.testing.assert_array_equal(com.cpu().numpy()[:want[3][-1]], want[2])
    assert np.all(dL.cpu().numpy() == 7 + n.cpu().numpy() + 1)


def test_adapt_k_parity_over_rounds(sv, cuda):
    """600 sequences, 60 rounds; each round's k is the previous round's
    output and n is drawn up to it (errors now and then)."""
    import torch
    g = np.random.default_rng(7)
    B, rounds_n = 600, 60
    ref = oracle.AdaptK(B, 1, 10)
    k = T(ref.k.copy(), cuda)
    hist = torch.zeros((B, 10), dtype=torch.float64, device=cuda)
    rounds = torch.zeros(B, dtype=torch.int32, device=cuda)
    skill = g.random(B)                                  # per-sequence acceptance tendency
    for r in range(rounds_n):
        ku = ref.k.copy()
        n = np.array([g.binomial(int(kb), skill[b]) for b, kb in enumerate(ku)], np.int32)
        n[g.random(B) < 0.02] = -1
        offsets = np.concatenate([[0], np.cumsum(ku)]).astype(np.int32)
        want = ref.update(n, ku)
        sv.spec_adapt_k(T(n, cuda), T(offsets, cuda), hist, rounds, k)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(k.cpu().numpy(), want, err_msg=f"round {r}")
    assert len(set(ref.k.tolist())) > 3                  # the trajectories spread over k


def test_adapt_k_boundaries_on_device(sv, cuda):
    """Rates exactly 0.8 and 0.5 (strict comparisons) for 20 rounds."""
    import torch
    B = 2
    k = T(np.array([5, 5], np.int32), cuda)
    hist = torch.zeros((B, 10), dtype=torch.float64, device=cuda)
    rounds = torch.zeros(B, dtype=torch.int32, device=cuda)
    offs = T(np.array([0, 5, 7], np.int32), cuda)        # k = 5 and 2
    n = T(np.array([4, 1], np.int32), cuda)              # 4/5 = 0.8, 1/2 = 0.5
    for _ in range(20):
        sv.spec_adapt_k(n, offs, hist, rounds, k)
    torch.cuda.synchronize()
    assert k.cpu().numpy().tolist() == [5, 5]


def random_text(g, B, max_len, alphabet):
    """Token streams with repeats: random motifs copied at random places."""
    seq = g.integers(0, alphabet, size=(B, max_len)).astype(np.int32)
    for b in range(B):
        for _ in range(4):
            m = int(g.integers(2, 12))
            src, dst = g.integers(0, max_len - m, size=2)
            seq[b, dst:dst + m] = seq[b, src:src + m]
    L = g.integers(0, max_len + 1, size=B).astype(np.int32)
    return seq, L


@pytest.mark.parametrize("B,max_len,alphabet,nmax,nmin,kmax", [
    (64, 128, 4, 3, 1, 5), (300, 2048, 200, 3, 1, 8), (40, 4096, 32000, 4, 2, 10),
    (17, 300, 3, 6, 6, 63), (5, 50, 10, 2, 1, 0)])
def test_ngram_parity(sv, cuda, B, max_len, alphabet, nmax, nmin, kmax):
    import torch
    g = np.random.default_rng(max_len + B)
    seq, L = random_text(g, B, max_len, alphabet)
    L[:2] = [0, 1]
    want_t, want_o = oracle.ngram_draft(seq, L, nmax, nmin, kmax)
    dt, do = sv.spec_ngram_draft(T(seq, cuda), T(L, cuda), ngram_max=nmax, ngram_min=nmin, k_max=kmax)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(do.cpu().numpy(), want_o)
    np.testing.assert_array_equal(dt.cpu().numpy()[:want_o[-1]], want_t)


def test_greedy_round_end_to_end(sv, cuda):
    """One greedy round on the device: n-gram drafts from each sequence's
    prefix, a 'perfect' target (its argmax at every position is the
    sequence's true next token), the verify, and the commit.  The committed
    tokens must be the longest draft prefix that agrees with the true
    continuation plus the true next token after it."""
    import torch
    g = np.random.default_rng(11)
    B, max_len, V, kmax = 64, 512, 1000, 8
    truth, _ = random_text(g, B, max_len, 50)
    L = g.integers(64, max_len - 2 * kmax, size=B).astype(np.int32)
    seq = truth.copy()
    for b in range(B):
        seq[b, L[b]:] = -1                               # the future is unknown to the drafter
    dseq, dL = T(seq, cuda), T(L, cuda)
    dtok, doff = sv.spec_ngram_draft(dseq, dL, ngram_max=3, ngram_min=1, k_max=kmax)
    torch.cuda.synchronize()
    off = doff.cpu().numpy()
    drafts = dtok.cpu().numpy()[:off[-1]]
    k = np.diff(off).astype(np.int32)
    # target row (b, i) predicts position L_b + i: argmax = truth there
    rows = []
    for b in range(B):
        for i in range(int(k[b]) + 1):
            z = g.standard_normal(V).astype(np.float32)
            z[truth[b, L[b] + i] % V] = 10.0
            rows.append(z)
    target = np.stack(rows)
    w = wl.assemble(target, np.zeros((len(drafts), V), np.float32), drafts % V,
                    g.random(len(drafts) + B, dtype=np.float32), np.zeros(B, np.float32), k)
    from test_gpu_parity import to_device
    d = to_device(w, cuda)
    out_tok, n = sv.spec_verify(d["target"], d["draft"], d["tokens"], d["offsets"], d["uniforms"],
                                d["temperature"])
    com, coff = sv.spec_commit(out_tok, n, d["offsets"], dseq, dL)
    torch.cuda.synchronize()
    n = n.cpu().numpy()
    for b in range(B):
        j = 0
        while j < k[b] and drafts[off[b] + j] % V == truth[b, L[b] + j] % V:
            j += 1
        assert n[b] == j, b
    new_L = dL.cpu().numpy()
    assert np.all(new_L == L + n + 1)
    got = dseq.cpu().numpy()
    for b in range(B):
        np.testing.assert_array_equal(got[b, L[b]:new_L[b]] % V, truth[b, L[b]:new_L[b]] % V)
