"""Pins of the calibration-statistics oracle to things other than itself.

The oracle (oracle/saf_calib_oracle.py) follows "When Can Attention Heads Be
Statically Defined?", Section 3.1 (Equations 1 and 2) and Appendix A.1
(Equations 5-6).  The tests check it against a hand-worked example, library
routines (numpy's variance, scipy's relative entropy), the already pinned
ordinary-head forward, invariants and special cases.
"""

import json
import math
import os

import numpy as np
import pytest
from scipy.special import rel_entr

import oracle
from oracle import saf_calib_oracle as C

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _qk(N, T, D, seed, sigma=1.0):
    rng = np.random.default_rng(seed)
    return sigma * rng.standard_normal((N, T, D)), sigma * rng.standard_normal((N, T, D))


def test_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "calib_stats_worked_T2.json")))
    st = C.calibration_stats(np.array(g["q"]), np.array(g["k"]), g["scale"])
    np.testing.assert_allclose(st["ahat"], g["ahat"], rtol=0, atol=1e-15)
    assert st["s_var"] == pytest.approx(g["s_var"], rel=1e-14)
    assert st["s_kl"] == pytest.approx(g["s_kl"], rel=1e-13)


def test_attention_matrix_is_the_pinned_forward():
    q, k = _qk(1, 23, 8, 1)
    v = np.random.default_rng(2).standard_normal((23, 8))
    A = C.attention_matrix(q[0], k[0], 0.3)
    O, _ = oracle.ordinary_head_fwd(q[0], k[0], v, 0.3)
    np.testing.assert_allclose(A @ v, O, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(A.sum(axis=1), 1.0, rtol=1e-14)
    assert np.all(A[np.triu_indices(23, 1)] == 0)


def test_scores_against_library_routines():
    N, T, D = 5, 17, 4
    q, k = _qk(N, T, D, 3, sigma=1.5)
    st = C.calibration_stats(q, k, 0.5)
    As = np.stack([C.attention_matrix(q[n], k[n], 0.5) for n in range(N)])
    # Equation 1: per-entry sample variance (ddof = 1) summed over entries, / T^2
    assert st["s_var"] == pytest.approx(np.var(As, axis=0, ddof=1).sum() / T ** 2, rel=1e-12)
    # Equation 2: scipy's elementwise relative entropy over the causal rows
    causal = np.tril(np.ones((T, T), dtype=bool))
    kl = sum(rel_entr(As[n][causal], st["ahat"][causal]).sum() for n in range(N))
    assert st["s_kl"] == pytest.approx(kl / (N * T), rel=1e-12)
    np.testing.assert_allclose(st["ahat"], As.mean(axis=0), rtol=0, atol=0)


def test_single_pass_identities():
    """The identities a single pass over the sequences relies on:
    sum_n KL = sum_n sum A log A - N sum A-hat log A-hat and
    sum_n ||A - A-hat||^2 = sum_n ||A||^2 - N ||A-hat||^2."""
    N, T, D = 6, 21, 8
    q, k = _qk(N, T, D, 4, sigma=2.0)
    st = C.calibration_stats(q, k, 1 / math.sqrt(D))
    As = np.stack([C.attention_matrix(q[n], k[n], 1 / math.sqrt(D)) for n in range(N)])
    A_hat = st["ahat"]
    causal = np.tril(np.ones((T, T), dtype=bool))
    ent = sum((As[n][causal] * np.log(As[n][causal])).sum() for n in range(N))
    ent_hat = (A_hat[causal] * np.log(A_hat[causal])).sum()
    assert st["s_kl"] == pytest.approx((ent - N * ent_hat) / (N * T), rel=1e-9)
    sq = (As ** 2).sum() - N * (A_hat ** 2).sum()
    assert st["s_var"] == pytest.approx(sq / ((N - 1) * T * T), rel=1e-9)


def test_special_cases():
    q, k = _qk(1, 9, 4, 5)
    A = C.attention_matrix(q[0], k[0], 0.5)
    # one sequence: the mean is that sequence, both scores 0
    st = C.calibration_stats(q, k, 0.5)
    np.testing.assert_array_equal(st["ahat"], A)
    assert st["s_var"] == 0 and st["s_kl"] == 0
    # identical sequences: no spread
    st = C.calibration_stats(np.repeat(q, 4, axis=0), np.repeat(k, 4, axis=0), 0.5)
    np.testing.assert_allclose(st["ahat"], A, rtol=1e-15, atol=1e-16)
    assert st["s_var"] < 1e-30 and abs(st["s_kl"]) < 1e-15
    # row 0 has one key: A(0, 0) = 1 in every sequence
    q, k = _qk(3, 6, 4, 6)
    assert C.calibration_stats(q, k, 1.0)["ahat"][0, 0] == 1.0


def test_invariants():
    N, T, D = 4, 15, 8
    q, k = _qk(N, T, D, 7)
    st = C.calibration_stats(q, k, 0.25)
    # the score scale can move between q and the scale factor
    st2 = C.calibration_stats(2 * q, k, 0.125)
    np.testing.assert_allclose(st2["ahat"], st["ahat"], rtol=1e-12, atol=1e-15)
    assert st2["s_var"] == pytest.approx(st["s_var"], rel=1e-10)
    assert st2["s_kl"] == pytest.approx(st["s_kl"], rel=1e-10)
    # order of the sequences does not matter
    perm = [2, 0, 3, 1]
    st3 = C.calibration_stats(q[perm], k[perm], 0.25)
    assert st3["s_var"] == pytest.approx(st["s_var"], rel=1e-12)
    assert st3["s_kl"] == pytest.approx(st["s_kl"], rel=1e-12)
    assert st["s_var"] > 0 and st["s_kl"] > 0
    # sharper attention varies more across sequences
    hot = C.calibration_stats(3 * q, k, 0.25)
    assert hot["s_var"] > st["s_var"] and hot["s_kl"] > st["s_kl"]
    # causal: a later key's scores never change earlier rows
    k2 = k.copy()
    k2[:, -1] += 5.0
    st4 = C.calibration_stats(q, k2, 0.25)
    np.testing.assert_allclose(st4["ahat"][:-1], st["ahat"][:-1], rtol=0, atol=0)


def test_rows_partition_adds_up():
    N, T, D = 3, 19, 4
    q, k = _qk(N, T, D, 8, sigma=1.5)
    full = C.calibration_stats(q, k, 0.5)
    parts = [C.calibration_rows(q, k, 0.5, r) for r in (np.arange(0, 7), np.arange(7, 12), np.arange(12, T))]
    assert sum(p["sq"] for p in parts) / ((N - 1) * T * T) == pytest.approx(full["s_var"], rel=1e-12)
    assert sum(p["kl"] for p in parts) / (N * T) == pytest.approx(full["s_kl"], rel=1e-12)
    np.testing.assert_allclose(np.concatenate([p["ahat"] for p in parts]), full["ahat"], rtol=0, atol=0)
