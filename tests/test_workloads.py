"""Sanity of the seeded input generator (shared by the oracle and GPU tests)."""
import numpy as np
import torch

import workloads as wl


def test_bf16_round_matches_torch():
    g = np.random.default_rng(0)
    x = np.concatenate([g.standard_normal(100000).astype(np.float32) * 10,
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.0e38, -1e-40], np.float32)])
    ours = wl.bf16_round(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    np.testing.assert_array_equal(wl.bf16_to_f32(ours),
                                  torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_layout_and_determinism():
    a = wl.make_workload("c5", trial=3, B=20, V=1000)
    b = wl.make_workload("c5", trial=3, B=20, V=1000, threads=1)
    for f in ("target", "draft", "tokens", "uniforms", "temperature", "offsets"):
        np.testing.assert_array_equal(getattr(a, f), getattr(b, f))
    assert a.target.shape == (a.total + a.B, 1000) and a.draft.shape == (a.total, 1000)
    assert a.k.min() >= 1 and a.k.max() <= 10
    assert set(np.unique(a.temperature)) <= {0.0, np.float32(0.6), 1.0}
    assert np.all((a.tokens >= 0) & (a.tokens < 1000))
    assert np.all((a.uniforms >= 0) & (a.uniforms < 1))
    c = wl.make_workload("c5", trial=4, B=20, V=1000)
    assert not np.array_equal(a.target[:5], c.target[:5])


def test_greedy_drafts_are_draft_argmax():
    w = wl.make_workload("c2g", V=2048)
    vals = wl.logits_as_f32(w.draft)
    assert list(w.tokens) == [int(np.argmax(r)) for r in vals]


def test_sampled_drafts_follow_q():
    # Gumbel-max drafts: the drafted token's frequency tracks softmax(z/T)
    z = np.array([0.0, 1.0, 2.0, 0.5], np.float32)
    counts = np.zeros(4)
    for t in range(4000):
        rng = np.random.Generator(np.random.Philox(t))
        e = rng.standard_exponential(4)
        counts[int(np.argmax(z / 0.7 - np.log(e)))] += 1
    q = np.exp(z / 0.7) / np.exp(z / 0.7).sum()
    assert np.all(np.abs(counts / 4000 - q) < 0.03)


def test_subset_keeps_rows():
    w = wl.make_workload("c5", B=10, V=256)
    s = w.subset([3, 7])
    for j, b in enumerate([3, 7]):
        for i in range(int(w.k[b]) + 1):
            np.testing.assert_array_equal(s.target[s.target_row(j, i)], w.target[w.target_row(b, i)])
            assert s.uniforms[s.uniform_slot(j, i)] == w.uniforms[w.uniform_slot(b, i)]
        for i in range(int(w.k[b])):
            np.testing.assert_array_equal(s.draft[s.draft_row(j, i)], w.draft[w.draft_row(b, i)])
