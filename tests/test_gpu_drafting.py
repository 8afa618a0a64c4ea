"""GPU parity of the drafter-side entry points against the fp64 oracle:
spec_draft_sample (the drafter's softmax + inverse-CDF step) and
spec_verify_gathered (the verify with the drafter's gathered q(x)).

Bar, as for spec_verify: tokens and accept counts bit-exact on every row or
sequence the oracle does not flag (accept band |u - alpha| < 1e-5, CDF band
|u Z - C_t| < 1e-12); flagged ones valid and under 0.1% over the large
runs; fp32 probabilities within relative 1e-6 of the fp64 value.
"""
import numpy as np
import pytest
import scipy.special

import oracle
import workloads as wl
from test_gpu_parity import compare, to_device
from test_oracle_draft import gathered_q

pytestmark = pytest.mark.gpu

FORMS = ["early", "full"]
FORM = {"name": None}


@pytest.fixture(scope="module", params=FORMS)
def sv(cuda, request):
    import os

    import speculative_decoding_rejection_spec_amd as sv
    if not os.path.exists(sv.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    sv.reset_options()
    sv.set_early_exit(1 if request.param == "early" else 0)
    FORM["name"] = request.param
    print(f"[form {request.param}]", flush=True)
    yield sv
    sv.reset_options()


def _logits_tensor(rows, dev):
    import torch
    if rows.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(rows).view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(np.ascontiguousarray(rows)).to(dev)


def run_sample(sv, rows, T, u, dev):
    import torch
    tok, prob = sv.spec_draft_sample(_logits_tensor(rows, dev), torch.from_numpy(T).to(dev),
                                     torch.from_numpy(u).to(dev))
    torch.cuda.synchronize()
    return tok.cpu().numpy(), prob.cpu().numpy()


def check_sample(rows, T, u, tok, prob, label):
    ref = oracle.draft_sample(rows, T, u, threads=16)
    flagged = (ref["flags"] & oracle.FLAG_B) != 0
    bad = np.nonzero((tok != ref["tokens"]) & ~flagged)[0]
    assert bad.size == 0, f"{label}: {bad.size} rows differ, first {bad[:5]}"
    ok = ~flagged & (ref["tokens"] >= 0)
    rel = np.abs(prob[ok] - ref["probs"][ok]) / ref["probs"][ok]
    assert rel.max() < 1e-6, (label, rel.max())
    assert np.all(tok[ref["tokens"] < 0] == -1) and np.all(np.isnan(prob[ref["tokens"] < 0]))
    return int(flagged.sum())


@pytest.mark.parametrize("dtype,V,rows", [("f32", 32000, 512), ("bf16", 128256, 256), ("bf16", 4099, 700)])
def test_draft_sample_parity(sv, cuda, dtype, V, rows):
    g = np.random.default_rng(V + rows)
    z = (g.standard_normal((rows, V)) * 2).astype(np.float32)
    stored = wl.bf16_round(z) if dtype == "bf16" else z
    T = g.choice(np.array([0.0, 0.6, 1.0, 1.5], np.float32), size=rows)
    T[:3] = [-1.0, np.nan, np.inf]                       # unusable temperatures
    u = g.random(rows, dtype=np.float32)
    tok, prob = run_sample(sv, stored, T, u, cuda)
    nflag = check_sample(stored, T, u, tok, prob, f"{dtype} V={V}")
    assert nflag <= max(1, rows // 1000)
    greedy = T == 0
    np.testing.assert_array_equal(prob[greedy], 1.0)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_draft_sample_masked_vocabulary(sv, cuda, dtype):
    """Masked (-inf) logits carry no probability: a masked prefix longer
    than a workgroup's first tile of loads, a padded tail, a block across
    segment boundaries, scattered entries."""
    V, rows = 40000, 96
    g = np.random.default_rng(53)
    z = (g.standard_normal((rows, V)) * 2).astype(np.float32)
    idx = np.arange(V)
    for r in range(rows):
        kind = r % 4
        if kind == 0:
            z[r, idx < 2600] = -np.inf
        elif kind == 1:
            z[r, idx >= V - 464] = -np.inf
        elif kind == 2:
            z[r, (idx >= 7000) & (idx < 18000)] = -np.inf
        else:
            z[r, g.random(V) < 0.3] = -np.inf
    stored = wl.bf16_round(z) if dtype == "bf16" else z
    T = g.choice(np.array([0.0, 0.6, 1.0], np.float32), size=rows)
    u = (g.integers(0, 1 << 24, size=rows) / float(1 << 24)).astype(np.float32)
    tok, prob = run_sample(sv, stored, T, u, cuda)
    check_sample(stored, T, u, tok, prob, f"masked {dtype}")
    assert np.all(np.isfinite(z[np.arange(rows), tok]))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_draft_sample_masked_extreme_uniforms(sv, cuda, dtype):
    """u = 0 picks the first token with mass (never a masked one before
    it), u = 1 - 2^-24 a token at the end of the unmasked mass (never a
    masked tail token): the oracle's tokens, every one finite in its row."""
    V, rows = 40000, 64
    g = np.random.default_rng(59)
    z = (g.standard_normal((rows, V)) * 2).astype(np.float32)
    idx = np.arange(V)
    for r in range(rows):
        kind = r % 4
        if kind == 0:
            z[r, idx < 2600] = -np.inf
        elif kind == 1:
            z[r, idx >= V - 464] = -np.inf
        elif kind == 2:
            z[r, (idx < 3000) | (idx >= V - 3000)] = -np.inf
        else:
            z[r, g.random(V) < 0.3] = -np.inf
    stored = wl.bf16_round(z) if dtype == "bf16" else z
    T = np.where(np.arange(rows) % 8 < 6, 1.0, 0.6).astype(np.float32)
    u = np.where(np.arange(rows) % 2 == 0, 0.0, 1.0 - 2.0 ** -24).astype(np.float32)
    tok, prob = run_sample(sv, stored, T, u, cuda)
    ref = oracle.draft_sample(stored, T, u, threads=16)
    np.testing.assert_array_equal(tok, ref["tokens"])
    assert np.all(np.isfinite(z[np.arange(rows), tok]))
    first = np.argmax(np.isfinite(z), axis=1)
    np.testing.assert_array_equal(tok[::2], first[::2])      # u = 0: the first unmasked token


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_draft_sample_nonfinite_rows(sv, cuda, dtype):
    """A row whose maximum is not finite (+inf, or every entry -inf) gives
    -1 and NaN, as a data error does in the verify (reading R26); the other
    rows are unaffected."""
    V, rows = 20000, 12
    g = np.random.default_rng(59)
    z = (g.standard_normal((rows, V)) * 2).astype(np.float32)
    z[1, 777] = np.inf
    z[4] = -np.inf
    z[7, 19999] = np.inf                            # in the row's last sub-chunk
    z[5] = -np.inf                                  # a greedy row with no finite logit
    T = np.array([1.0, 1.0, 0.0, 0.7, 1.0, 0.0, 1.0, 0.0, 1.0, 1.0, 0.7, 1.0], np.float32)
    stored = wl.bf16_round(z) if dtype == "bf16" else z
    u = (g.integers(0, 1 << 24, size=rows) / float(1 << 24)).astype(np.float32)
    tok, prob = run_sample(sv, stored, T, u, cuda)
    bad = [1, 4, 5, 7]
    assert np.all(tok[bad] == -1) and np.all(np.isnan(prob[bad]))
    good = [r for r in range(rows) if r not in bad]
    ref = oracle.draft_sample(stored[good], T[good], u[good])
    ok = (ref["flags"] & oracle.FLAG_B) == 0
    assert np.array_equal(tok[good][ok], ref["tokens"][ok])


def test_draft_sample_zipf_rows(sv, cuda):
    """Zipf-shaped rows like the workloads' target logits, bf16, V = 128256."""
    w = wl.make_workload("c3", trial=5, B=96)
    rows = w.target[:200]
    g = np.random.default_rng(9)
    T = g.choice(np.array([0.0, 0.7, 1.0], np.float32), size=len(rows))
    u = g.random(len(rows), dtype=np.float32)
    tok, prob = run_sample(sv, rows, T, u, cuda)
    check_sample(rows, T, u, tok, prob, "zipf")


def run_gathered(sv, w, qg, dev, emit=False):
    import torch
    d = to_device(w, dev)
    tok, n, ep = sv.spec_verify_gathered(d["target"], d["draft"], d["tokens"],
                                         torch.from_numpy(qg).to(dev), d["offsets"], d["uniforms"],
                                         d["temperature"])
    torch.cuda.synchronize()
    return dict(tokens=tok.cpu().numpy(), n=n.cpu().numpy(), emit=ep.cpu().numpy())


GATHERED_CASES = [("c1", 128, None), ("c2", 32, None), ("c3", None, None), ("c4", 64, None),
                  ("c5", None, None)]


@pytest.mark.parametrize("name,B,V", GATHERED_CASES, ids=[c[0] for c in GATHERED_CASES])
def test_gathered_parity(sv, cuda, name, B, V):
    w = wl.make_workload(name, trial=0, B=B, V=V)
    qg = gathered_q(w)
    ref = oracle.verify(w, threads=16, draft_probs=qg)
    gpu = run_gathered(sv, w, qg, cuda)
    nseq, namb = compare(w, gpu, ref, f"gathered {name}")
    print(f"gathered {name}: {nseq} sequences, {namb} ambiguous", flush=True)


def test_gathered_emit_probability(sv, cuda):
    """The emitted token's probability under its draw, against a numpy
    evaluation of the residual max(0, p_n - q_n)/Z or of p_k."""
    w = wl.make_workload("c5", trial=1, B=48, V=6000)
    qg = gathered_q(w)
    ref = oracle.verify(w, draft_probs=qg)
    gpu = run_gathered(sv, w, qg, cuda)
    t = wl.logits_as_f32(w.target).astype(np.float64)
    d = wl.logits_as_f32(w.draft).astype(np.float64)
    for b in range(w.B):
        n, T = int(gpu["n"][b]), float(w.temperature[b])
        if ref["flags"][b] & (oracle.FLAG_A | oracle.FLAG_B | oracle.FLAG_D):
            continue
        x = int(gpu["tokens"][w.target_row(b, n)])
        if T == 0:
            assert gpu["emit"][b] == 1.0
            continue
        p = scipy.special.softmax(t[w.target_row(b, n)] / T)
        if n < int(w.k[b]):
            q = scipy.special.softmax(d[w.draft_row(b, n)] / T)
            r = np.maximum(0.0, p - q)
            want = r[x] / r.sum()
        else:
            want = p[x]
        assert abs(gpu["emit"][b] - want) <= 1e-6 * want + 1e-12, (b, gpu["emit"][b], want)


def test_gathered_ignores_other_draft_rows(sv, cuda):
    """Rewriting the draft rows the verify must not read changes nothing."""
    w = wl.make_workload("c5", trial=3, B=64, V=8000)
    qg = gathered_q(w)
    base = run_gathered(sv, w, qg, cuda)
    draft = wl.logits_as_f32(w.draft).copy()
    for b in range(w.B):
        for i in range(int(w.k[b])):
            if i != base["n"][b]:
                j = int(w.offsets[b]) + i
                draft[j] = -10.0
                draft[j, w.tokens[j]] = 20.0
    w2 = wl.Workload(**{**w.__dict__, "draft": wl.bf16_round(draft)})
    got = run_gathered(sv, w2, qg, cuda)
    assert np.array_equal(got["tokens"], base["tokens"]) and np.array_equal(got["n"], base["n"])


def test_gathered_leads_past_short_sequences(sv, cuda):
    """Leading positions 2 and 3 on C5 (k_b from 1): sequences with k_b below
    the lead settle in the first round with their bonus draw still to make."""
    if FORM["name"] != "early":
        pytest.skip("early-exit form only")
    w = wl.make_workload("c5", trial=6, B=128)
    assert np.any(w.k < 3)
    qg = gathered_q(w)
    ref = oracle.verify(w, threads=16, draft_probs=qg)
    try:
        for lead in (2, 3):
            sv.set_early_exit(lead)
            compare(w, run_gathered(sv, w, qg, cuda), ref, f"gathered lead {lead}")
    finally:
        sv.set_early_exit(1)


def test_gathered_nonfinite_draft_rows(sv, cuda):
    """The gathered form reads a draft row only at the rejection: a
    non-finite maximum there is a data error, elsewhere it changes nothing
    (reading R26)."""
    w = wl.make_workload("c4", trial=2, B=32, V=4096)
    qg = gathered_q(w)
    base = oracle.verify(w, draft_probs=qg)
    draft = wl.logits_as_f32(w.draft).copy()
    for b in range(w.B):
        n = int(base["n"][b])
        if n < 0:
            continue
        pos = n if b % 2 == 0 else (n + 1 if n + 1 < int(w.k[b]) else -1)
        if pos >= 0 and pos < int(w.k[b]):
            draft[int(w.offsets[b]) + pos, 11] = np.inf
    w2 = wl.Workload(**{**w.__dict__, "draft": wl.bf16_round(draft)})
    ref = oracle.verify(w2, draft_probs=qg)
    assert (ref["n"] == -1).sum() >= 5
    compare(w2, run_gathered(sv, w2, qg, cuda), ref, "gathered non-finite draft rows")


def test_gathered_data_errors(sv, cuda):
    w = wl.make_workload("c3", trial=4, B=12, V=3000)
    qg = gathered_q(w)
    qg[w.offsets[2] + 1] = 0.0
    qg[w.offsets[5]] = np.nan
    qg[w.offsets[7] + 2] = 1.5
    gpu = run_gathered(sv, w, qg, cuda)
    ref = oracle.verify(w, draft_probs=qg)
    for b in range(w.B):
        sl = slice(w.target_row(b, 0), w.target_row(b, int(w.k[b])) + 1)
        if b in (2, 5, 7):
            assert gpu["n"][b] == -1 and np.all(gpu["tokens"][sl] == -1) and np.isnan(gpu["emit"][b])
        elif not ref["flags"][b] & (oracle.FLAG_A | oracle.FLAG_B):
            assert gpu["n"][b] == ref["n"][b] and np.array_equal(gpu["tokens"][sl], ref["tokens"][sl])


def test_gathered_many_sequences_flag_rate(sv, cuda):
    tot = amb = 0
    for name, B in (("c1", 1024), ("c3", 512)):
        w = wl.make_workload(name, trial=8, B=B)
        qg = gathered_q(w)
        n, a = compare(w, run_gathered(sv, w, qg, cuda), oracle.verify(w, threads=16, draft_probs=qg),
                       f"gathered {name}-many")
        tot += n
        amb += a
    assert amb <= 0.001 * tot
