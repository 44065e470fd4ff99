"""The oracles against examples worked by hand (tests/golden): every
expected value there is a rational number or a logarithm derived on paper
from the rule its fixture cites (the PQ-HSA output formula, the append
encoder and mean update, the query-reuse merge law), not from any code."""
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


APPEND = os.path.join(os.path.dirname(__file__), "golden", "append_worked_example.txt")


def test_append_worked_example():
    from oracle import pqhsa_append as ap
    C = np.zeros((3, 128))
    B = np.zeros((16, 256, 8))
    K = np.zeros((3, 128))
    V = np.zeros((3, 128))
    mu = np.zeros((3, 128))
    n_old = np.zeros(3, np.int64)
    codes_want = np.zeros((3, 16), np.int64)
    lists_want = mu0_want = n_want = None
    for line in open(APPEND):
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        f = line.replace(":", "").split()
        tag, nums = f[0], f[1:]
        if tag == "C":
            C[int(nums[0]), int(nums[1])] = float(nums[2])
        elif tag == "B":
            B[int(nums[0]), int(nums[1]), int(nums[2])] = float(nums[3])
        elif tag == "K":
            K[int(nums[0]), int(nums[1])] = float(nums[2])
        elif tag == "V":
            V[int(nums[0]), int(nums[1])] = float(nums[2])
        elif tag == "mu":
            mu[int(nums[0]), int(nums[1])] = float(nums[2])
        elif tag == "n":
            n_old[int(nums[0])] = int(nums[1])
        elif tag == "expect_lists":
            lists_want = [int(x) for x in nums]
        elif tag == "expect_code":
            codes_want[int(nums[0]), int(nums[1])] = int(nums[2])
        elif tag == "expect_mu0":
            mu0_want = [float(x) for x in nums]
        elif tag == "expect_n":
            n_want = [int(x) for x in nums]
    lists, codes = ap.encode_tokens(K, C, B)
    assert lists.tolist() == lists_want
    assert np.array_equal(codes, codes_want)
    mu_new, n_new = ap.append_means(mu, n_old, V, lists, 3)
    np.testing.assert_allclose(mu_new[:, 0], mu0_want, rtol=0, atol=1e-14)
    assert np.all(mu_new[:, 1:] == 0.0)
    assert n_new.tolist() == n_want


MERGE = os.path.join(os.path.dirname(__file__), "golden", "reuse_merge_worked_example.txt")


def test_reuse_merge_worked_example():
    from oracle import pqhsa_reuse as ru
    parts, want = [], {}
    for line in open(MERGE):
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        k, v = line.split(":", 1)
        if k == "part":
            m, n, d = (x.strip() for x in v.split("|"))
            parts.append((-np.inf if m == "-inf" else _value(m), np.array([_value(n)]),
                          _value(d)))
        else:
            want[k] = _value(v)
    M, N, D = ru.merge_states(parts)
    assert abs(M - want["expect_m"]) < 1e-15
    assert abs(N[0] - want["expect_N"]) < 1e-13 and abs(D - want["expect_D"]) < 1e-14
    assert abs(N[0] / D - want["expect_O"]) < 1e-13
