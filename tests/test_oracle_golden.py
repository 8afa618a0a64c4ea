"""Pins of the oracle on verify steps worked by hand (tests/golden/hand_cases.json):
each case gives exact-decimal probabilities (or raw logits for T = 0), the
cited step of the pages it exercises, the hand computation, and the
expected accept count, output tokens, alpha per tested position and the
residual mass Z."""
import json
import os

import numpy as np
import pytest

import oracle
import workloads as wl

HERE = os.path.dirname(os.path.abspath(__file__))
CASES = json.load(open(os.path.join(HERE, "golden", "hand_cases.json")))["cases"]


def workload_of(case):
    if "target_probs" in case:
        t = np.log(np.array(case["target_probs"], np.float64)).astype(np.float32)
        d = np.log(np.array(case["draft_probs"], np.float64)).astype(np.float32)
    else:
        t = np.array(case["target_logits"], np.float32)
        d = np.array(case["draft_logits"], np.float32)
    k = len(case["tokens"])
    return wl.assemble(t, d, np.array(case["tokens"]), np.array(case["uniforms"], np.float32),
                       np.array([case["T"]], np.float32), [k])


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_hand_case(case):
    r = oracle.verify(workload_of(case), diag=True)
    assert int(r["n"][0]) == case["n"]
    assert r["tokens"].tolist() == case["out"]
    assert r["flags"][0] == 0
    if "alpha" in case:
        n_tested = min(case["n"] + 1, len(case["tokens"]))
        np.testing.assert_allclose(r["alpha"][:n_tested], case["alpha"][:n_tested], atol=1e-6)
    if "Z" in case:
        assert abs(float(r["Z"][0]) - case["Z"]) < 1e-6


def test_cases_cite_the_pages():
    for c in CASES:
        assert c["cite"].startswith("page ") and c["work"]
