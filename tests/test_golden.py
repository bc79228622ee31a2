"""Oracle against hand-derived closed forms (tests/golden/*.json)."""
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")
_NS = {"log": math.log, "exp": math.exp, "sqrt": math.sqrt}


def ev(x):
    if isinstance(x, str):
        return float(eval(x, {"__builtins__": {}}, _NS))  # closed forms written in this repo
    return float(x)


def evs(a):
    if isinstance(a, list):
        return [evs(v) for v in a]
    return ev(a)


def load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


@pytest.mark.parametrize("case", load("junction_small.json")["cases"])
def test_junction_golden(case):
    h = None if case["h"] is None else np.array(case["h"], dtype=np.float64)
    out = oracle.junction(h, np.array(case["ids"]), np.array(case["emb"], dtype=np.float64))
    np.testing.assert_allclose(out, np.array(evs(case["expected"])), rtol=1e-15, atol=1e-15)


@pytest.mark.parametrize("case", load("loss_two_vocab.json")["cases"])
def test_loss_golden(case):
    s = np.array(evs(case["student"]))
    t = np.array(evs(case["teacher"]))
    y = np.array(case["labels"])
    r = oracle.matryoshka_loss([s, t], y, case["alpha"])
    np.testing.assert_allclose(r["ce"], evs(case["ce"]), rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(r["dist"], evs(case["dist"]), rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(r["loss"], evs(case["loss"]), rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(r["total"], evs(case["total"]), rtol=1e-14, atol=1e-15)
    g = oracle.matryoshka_grad([s, t], y, case["alpha"])
    for gm, exp in zip(g, case["grad"]):
        np.testing.assert_allclose(gm, evs(exp), rtol=1e-14, atol=1e-15)


def test_lse_argmax_accept_golden():
    d = load("lse_accept_argmax.json")
    for c in d["lse"]:
        l = np.array([ev(v) for v in c["l"]])
        assert oracle.logsumexp(l) == pytest.approx(ev(c["expected"]), rel=1e-15, abs=1e-15)
    for c in d["argmax"]:
        assert int(oracle.argmax_lowest(np.array(c["l"], dtype=np.float64))) == c["expected"]
    for c in d["accept"]:
        got = oracle.accept_prefix(np.array([c["draft"]]), np.array([c["verify"]]), c["draft_len"])
        assert int(got[0]) == c["expected"]
