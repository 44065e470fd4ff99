"""The oracle against a PQ-HSA step worked by hand (tests/golden): every
expected value there is a rational number or a logarithm derived on paper
from the output formula of the PQ-HSA page, section A, not from any code."""
import math
import os
from fractions import Fraction

import numpy as np

from oracle import pqhsa_oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pqhsa_worked_example.txt")


def _load():
    f = {}
    for line in open(GOLDEN):
        line = line.split("#", 1)[0].strip()
        if line:
            k, v = line.split(":", 1)
            f[k.strip()] = v.strip()
    return f


def _rows(s):
    return np.array([[float(x) for x in part.split()] for part in s.split("|")])


def _value(s):
    s = s.strip()
    if s.startswith("ln "):
        return math.log(float(Fraction(s[3:])))
    return float(Fraction(s))


def _setup(f):
    q = np.array([[float(x) for x in f["q"].split()]])
    C = _rows(f["centroids"])
    B = np.stack([_rows(f["codebook0"]), _rows(f["codebook1"])])
    lists = np.array([int(x) for x in f["lists"].split()])
    codes = _rows(f["codes"]).astype(np.int64)
    V = _rows(f["V"])
    # keys equal their reconstruction C[list] + concat_m B_m[code_m]
    K = C[lists] + np.concatenate([B[0][codes[:, 0]], B[1][codes[:, 1]]], axis=1)
    return q, K, V, C, B, lists, codes


def _step(f, background):
    q, K, V, C, B, lists, codes = _setup(f)
    return orc.head_group_step(q, K, V, int(f["T"]), int(f["n_indexed"]), C, B, lists, codes,
                               float(f["scale"]), int(f["n_sink"]), int(f["n_recent"]),
                               int(f["budget_bp"]), background=background)


def test_worked_example_with_background():
    f = _load()
    r = _step(f, True)
    assert r["k"] == int(f["expect_k"])
    assert r["selected"].tolist() == [int(x) for x in f["expect_selected"].split()]
    want = np.array([_value(x) for x in f["expect_O"].split()])
    np.testing.assert_allclose(r["O"][0], want, rtol=1e-14, atol=1e-14)
    lse = r["m"][0] + math.log(r["denom"][0])
    assert abs(lse - _value(f["expect_lse"])) < 1e-14


def test_worked_example_without_background():
    f = _load()
    r = _step(f, False)
    want = np.array([_value(x) for x in f["expect_O_exact_only"].split()])
    np.testing.assert_allclose(r["O"][0], want, rtol=1e-14, atol=1e-14)
    lse = r["m"][0] + math.log(r["denom"][0])
    assert abs(lse - _value(f["expect_lse_exact_only"])) < 1e-14


def test_worked_example_dense():
    f = _load()
    q, K, V, *_ = _setup(f)
    O, _, _ = orc.dense_attention(q, K, V, float(f["scale"]))
    want = np.array([_value(x) for x in f["expect_O_dense"].split()])
    np.testing.assert_allclose(O[0], want, rtol=1e-14, atol=1e-14)
