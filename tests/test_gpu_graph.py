"""Verify calls captured in a HIP graph and replayed.

A replay runs the captured kernels with the same arguments every time, so
each call takes its epoch (the number that tells its records, tasks and
schedule entries from an earlier call's) on the device, from a counter at
the workspace's start.  Every replay below gets new inputs copied into the
captured tensors and must match the fp64 oracle on those inputs, with eager
calls on the same workspace between the replays (their epochs come from
the same counter); in each launch form through spec_verify with a caller
workspace, through spec_verify_noalloc in the early-exit form (chosen by
size) and in one pass, and through spec_verify_gathered in both.  The bar
is that of tests/test_gpu_parity.py.
"""
import pytest

import oracle
import workloads as wl
from test_gpu_parity import compare, set_form, to_device
from test_oracle_draft import gathered_q

pytestmark = pytest.mark.gpu

ORDER = [0, 1, 2, 1, 0, 2]       # the workload copied in before each replay


@pytest.fixture(scope="module")
def sv(cuda):
    import os

    import speculative_decoding_rejection_spec_amd as sv
    if not os.path.exists(sv.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    yield sv
    sv.reset_options()


def _replays(sv, dev, works, call, eager, qgs=None):
    """Captures call(static inputs) once and replays it in ORDER, each time
    after copying that workload's inputs in; eager(j) runs an eager call
    on workload j between replays.  Every output is compared with the
    oracle.  qgs: the drafter's gathered q_i(x_i) of each workload (input
    "qg"), for the gathered form."""
    import torch
    refs = [oracle.verify(w, threads=16, **({} if qgs is None else {"draft_probs": qgs[i]}))
            for i, w in enumerate(works)]
    inputs = [to_device(w, dev) for w in works]
    if qgs is not None:
        for d, q in zip(inputs, qgs):
            d["qg"] = torch.from_numpy(q).to(dev)
    static = {k: v.clone() for k, v in inputs[0].items()}
    B, total = works[0].B, int(works[0].k.sum())
    out_tok = torch.empty(total + B, dtype=torch.int32, device=dev)
    out_n = torch.empty(B, dtype=torch.int32, device=dev)

    side = torch.cuda.Stream(dev)                  # (warm-up off the capturing stream, as torch asks)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        call(static, out_tok, out_n)
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(static, out_tok, out_n)
    torch.cuda.synchronize()

    for rep, i in enumerate(ORDER):
        print(f"[replay {rep}: workload {i}]", flush=True)
        for k in static:
            static[k].copy_(inputs[i][k])
        graph.replay()
        torch.cuda.synchronize()
        compare(works[i], dict(tokens=out_tok.cpu().numpy(), n=out_n.cpu().numpy()), refs[i], f"replay {rep}")
        if rep % 2 == 1:
            j = (i + 1) % len(works)
            tok, n = eager(inputs[j])
            torch.cuda.synchronize()
            compare(works[j], dict(tokens=tok.cpu().numpy(), n=n.cpu().numpy()), refs[j], f"eager after {rep}")


@pytest.mark.parametrize("form", ["early", "full", "full3"])
def test_graph_replays_with_a_caller_workspace(sv, cuda, form):
    import torch
    set_form(sv, form)
    try:
        works = [wl.make_workload("c3", trial=t, B=24, V=50000) for t in (21, 22, 23)]
        w = works[0]
        ws = torch.empty(sv.spec_verify_workspace_size(w.B, int(w.k.sum()), w.V, torch.bfloat16),
                         dtype=torch.uint8, device=cuda)

        def call(d, out_tok, out_n):
            sv.spec_verify(d["target"], d["draft"], d["tokens"], d["offsets"], d["uniforms"], d["temperature"],
                           out_tokens=out_tok, out_n_accepted=out_n, workspace=ws)

        def eager(d):
            return sv.spec_verify(d["target"], d["draft"], d["tokens"], d["offsets"], d["uniforms"],
                                  d["temperature"], workspace=ws)

        _replays(sv, cuda, works, call, eager)
    finally:
        sv.reset_options()


@pytest.mark.parametrize("case", [("c4", 48, 152064), ("c3", 24, 50000)], ids=["early-exit", "one-pass"])
def test_graph_replays_without_allocation(sv, cuda, case):
    """spec_verify_noalloc, in the form its default tuning picks: C4-shaped
    rows at B = 48 (about 248 MB: early exit) and a small C3-shaped call
    (one pass)."""
    name, B, V = case
    sv.reset_options()
    works = [wl.make_workload(name, trial=t, B=B, V=V) for t in (31, 32, 33)]

    def call(d, out_tok, out_n):
        sv.spec_verify_noalloc(d["target"], d["draft"], d["tokens"], d["offsets"], d["uniforms"],
                               d["temperature"], out_tokens=out_tok, out_n_accepted=out_n)

    def eager(d):
        return sv.spec_verify_noalloc(d["target"], d["draft"], d["tokens"], d["offsets"], d["uniforms"],
                                      d["temperature"])

    _replays(sv, cuda, works, call, eager)


@pytest.mark.parametrize("lead", [1, 0], ids=["early-exit", "one-pass"])
def test_graph_replays_gathered(sv, cuda, lead):
    """spec_verify_gathered (the drafter's q_i(x_i) handed over), its first
    round and listed remainder or its one pass, with a caller workspace."""
    import torch
    sv.reset_options()
    sv.set_early_exit(lead)
    try:
        works = [wl.make_workload("c3", trial=t, B=24, V=50000) for t in (41, 42, 43)]
        qgs = [gathered_q(w) for w in works]
        w = works[0]
        ws = torch.empty(sv.spec_verify_workspace_size(w.B, int(w.k.sum()), w.V, torch.bfloat16),
                         dtype=torch.uint8, device=cuda)

        def call(d, out_tok, out_n):
            sv.spec_verify_gathered(d["target"], d["draft"], d["tokens"], d["qg"], d["offsets"], d["uniforms"],
                                    d["temperature"], out_tokens=out_tok, out_n_accepted=out_n, workspace=ws)

        def eager(d):
            tok, n, _ = sv.spec_verify_gathered(d["target"], d["draft"], d["tokens"], d["qg"], d["offsets"],
                                                d["uniforms"], d["temperature"], workspace=ws)
            return tok, n

        _replays(sv, cuda, works, call, eager, qgs)
    finally:
        sv.reset_options()


def test_epoch_counter_skips_zero(sv, cuda):
    """The epoch counter at the workspace's start wraps past 0 (the number
    no call takes): set to 2^32 - 2, two early-exit calls take 2^32 - 1 and
    then 1, both against the oracle, and leave 1 in both words."""
    import numpy as np
    import torch
    sv.reset_options()
    sv.set_early_exit(1)
    try:
        works = [wl.make_workload("c3", trial=t, B=24, V=50000) for t in (51, 52)]
        w = works[0]
        ws = torch.zeros(sv.spec_verify_workspace_size(w.B, int(w.k.sum()), w.V, torch.bfloat16),
                         dtype=torch.uint8, device=cuda)
        ws[:4].copy_(torch.tensor([0xFE, 0xFF, 0xFF, 0xFF], dtype=torch.uint8))
        seen = []
        for i, wk in enumerate(works):
            d = to_device(wk, cuda)
            tok, n = sv.spec_verify(d["target"], d["draft"], d["tokens"], d["offsets"], d["uniforms"],
                                    d["temperature"], workspace=ws)
            torch.cuda.synchronize()
            compare(wk, dict(tokens=tok.cpu().numpy(), n=n.cpu().numpy()), oracle.verify(wk, threads=16),
                    f"call {i}")
            seen.append(ws[:8].cpu().numpy().view(np.uint32).tolist())
        assert seen == [[0xFFFFFFFF, 0xFFFFFFFF], [1, 1]], seen
    finally:
        sv.reset_options()
