"""Randomized parity: calls of random shape against the fp64 oracle.

Each case draws a workload recipe (C1-C5's value distributions), a batch
size, a vocabulary (the workloads' own, 4099, or any size from 64 up), the
drafts per sequence, a launch form (automatic by size, early exit after one
or two leading positions, one pass with the draw in one launch or in three)
and an entry point (spec_verify, spec_verify_gathered with the drafter's
q_i(x_i), or spec_verify_noalloc), from a fixed seed, so a failure names a
case that reproduces on the CPU side exactly.  The bar is that of
tests/test_gpu_parity.py; inputs are capped at 1.5 GB of logits.
"""
import numpy as np
import pytest

import oracle
import workloads as wl
from test_gpu_parity import compare, set_form, to_device
from test_oracle_draft import gathered_q

pytestmark = pytest.mark.gpu


def _cases(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        name = str(rng.choice(["c1", "c2", "c3", "c4", "c5"]))
        V = int(rng.choice([4099, 32000, 50000, 128256, 152064, int(rng.integers(64, 200000))]))
        k = int(rng.integers(1, 13)) if name != "c5" else None
        B = int(rng.integers(1, 300))
        elt = 4 if name == "c1" else 2
        if (2 * (k or 10) + 1) * B * V * elt > 1.5e9:
            B = max(1, int(1.5e9 / ((2 * (k or 10) + 1) * V * elt)))
        form = str(rng.choice(["auto", "early1", "early2", "full", "full3"]))
        entry = str(rng.choice(["verify", "verify", "gathered", "noalloc"]))
        out.append((i, name, B, V, k, "auto" if entry == "noalloc" else form, entry))
    return out


CASES = _cases(32, 7)


@pytest.fixture(scope="module")
def sv(cuda):
    import os

    import speculative_decoding_rejection_spec_amd as sv
    if not os.path.exists(sv.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    yield sv
    sv.reset_options()


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-{c[1]}-B{c[2]}-V{c[3]}-{c[5]}-{c[6]}" for c in CASES])
def test_random_call(sv, cuda, case):
    import torch
    i, name, B, V, k, form, entry = case
    print(f"[case {i}: {name} B={B} V={V} k={k} form={form} entry={entry}]", flush=True)
    w = wl.make_workload(name, trial=2000 + i, B=B, V=V, k=k)
    sv.reset_options()
    try:
        if form == "early1":
            sv.set_early_exit(1)
        elif form == "early2":
            sv.set_early_exit(2)
        elif form in ("full", "full3"):
            set_form(sv, form)
        d = to_device(w, cuda)
        if entry == "gathered":
            qg = gathered_q(w)
            ref = oracle.verify(w, threads=16, draft_probs=qg)
            tok, n, _ = sv.spec_verify_gathered(d["target"], d["draft"], d["tokens"], torch.from_numpy(qg).to(cuda),
                                                d["offsets"], d["uniforms"], d["temperature"])
        else:
            ref = oracle.verify(w, threads=16)
            call = sv.spec_verify_noalloc if entry == "noalloc" else sv.spec_verify
            try:
                tok, n = call(d["target"], d["draft"], d["tokens"], d["offsets"], d["uniforms"], d["temperature"])
            except sv.SpecVerifyError as e:
                # (only the no-alloc scratch may refuse a valid call: too large for it)
                assert entry == "noalloc" and "scratch" in str(e), e
                pytest.skip(f"larger than the no-alloc scratch: {e}")
        torch.cuda.synchronize()
        compare(w, dict(tokens=tok.cpu().numpy(), n=n.cpu().numpy()), ref, f"case {i}")
    finally:
        sv.reset_options()


def _sample_cases(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        dtype = str(rng.choice(["f32", "bf16"]))
        V = int(rng.choice([4099, 32000, 152064, int(rng.integers(16, 200000))]))
        rows = int(rng.integers(1, 600))
        rows = max(1, min(rows, int(5e8 // (V * 4))))
        shape = str(rng.choice(["normal", "spiky", "flat"]))
        out.append((i, dtype, V, rows, shape))
    return out


SAMPLE_CASES = _sample_cases(12, 11)


@pytest.mark.parametrize("case", SAMPLE_CASES, ids=[f"{c[0]}-{c[1]}-V{c[2]}-R{c[3]}-{c[4]}" for c in SAMPLE_CASES])
def test_random_draft_sample(sv, cuda, case):
    """spec_draft_sample on random rows: logits normal (scale 2), spiky (a
    few tokens 8-20 above the rest) or flat (scale 0.05), temperatures from
    0 to 2, against the oracle's sampler (the bar of
    tests/test_gpu_drafting.py)."""
    from test_gpu_drafting import check_sample, run_sample
    i, dtype, V, rows, shape = case
    print(f"[sample case {i}: {dtype} V={V} rows={rows} {shape}]", flush=True)
    g = np.random.default_rng(3000 + i)
    z = (g.standard_normal((rows, V)) * (0.05 if shape == "flat" else 2.0)).astype(np.float32)
    if shape == "spiky":
        for r in range(rows):
            z[r, g.integers(0, V, size=3)] += g.uniform(8.0, 20.0, size=3).astype(np.float32)
    stored = wl.bf16_round(z) if dtype == "bf16" else z
    T = g.choice(np.array([0.0, 0.3, 0.7, 1.0, 2.0], np.float32), size=rows)
    u = g.random(rows, dtype=np.float32)
    tok, prob = run_sample(sv, stored, T, u, cuda)
    nflag = check_sample(stored, T, u, tok, prob, f"sample case {i}")
    assert nflag <= max(1, rows // 100)


def _book_cases(n, seed):
    rng = np.random.default_rng(seed)
    return [(i, int(rng.integers(1, 3000)), int(rng.integers(16, 3000)), int(rng.integers(2, 50000)),
             int(rng.integers(1, 7)), int(rng.integers(0, 64))) for i in range(n)]


BOOK_CASES = _book_cases(10, 13)


@pytest.mark.parametrize("case", BOOK_CASES, ids=[f"{c[0]}-B{c[1]}-L{c[2]}-a{c[3]}" for c in BOOK_CASES])
def test_random_commit_and_ngram(sv, cuda, case):
    """spec_commit of a random round (k_b up to the case's k_max, n_b from -1
    to k_b, sequences from empty to full) and spec_ngram_draft over random
    token streams with repeats (n from the case's n_max down to a random
    n_min), both bit-exact against the oracle."""
    import torch
    from test_gpu_bookkeeping import T, random_round, random_text
    i, B, max_len, alphabet, nmax, kmax = case
    print(f"[bookkeeping case {i}: B={B} max_len={max_len} alphabet={alphabet} n_max={nmax} k_max={kmax}]",
          flush=True)
    g = np.random.default_rng(4000 + i)
    k, offsets, out_tokens, out_n, seq, L = random_round(g, B, max_len, kmax=kmax)
    want = oracle.commit(out_tokens, out_n, offsets, seq, L)
    dseq, dL = T(seq, cuda), T(L, cuda)
    com, coff = sv.spec_commit(T(out_tokens, cuda), T(out_n, cuda), T(offsets, cuda), dseq, dL)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(dseq.cpu().numpy(), want[0])
    np.testing.assert_array_equal(dL.cpu().numpy(), want[1])
    np.testing.assert_array_equal(coff.cpu().numpy(), want[3])
    np.testing.assert_array_equal(com.cpu().numpy()[:want[3][-1]], want[2])

    nmin = int(g.integers(1, nmax + 1))
    seq, L = random_text(g, min(B, 400), max_len, alphabet)
    want_t, want_o = oracle.ngram_draft(seq, L, nmax, nmin, kmax)
    dt, do = sv.spec_ngram_draft(T(seq, cuda), T(L, cuda), ngram_max=nmax, ngram_min=nmin, k_max=kmax)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(do.cpu().numpy(), want_o)
    np.testing.assert_array_equal(dt.cpu().numpy()[:want_o[-1]], want_t)
