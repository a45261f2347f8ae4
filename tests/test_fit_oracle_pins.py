"""Pins of the fitting oracle to things other than itself.

The oracle (oracle/saf_fit_oracle.py) follows "When Can Attention Heads Be
Statically Defined?": Algorithm 1 (target preparation and the acceptance
statistic), Section 3.2 "Fitting" (Equation 4), Appendix A.2 (initialisation,
Adam settings) and Appendix D.1 (Equation 20).  Each test below checks it
against a hand-worked example, a closed form, an independent derivation
(torch autograd of Equation 4, torch.optim.Adam) or an invariant.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import saf_fit_oracle as F
from oracle import frozen_pattern, frozen_lognorm
from synth.targets import calibration_mean

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _random_target(T, seed):
    """A random causal row-stochastic matrix (Dirichlet rows)."""
    rng = np.random.default_rng(seed)
    P = np.zeros((T, T))
    for i in range(T):
        P[i, : i + 1] = rng.dirichlet(np.full(i + 1, 0.7))
    return P


def _torch_loss(eta_abs, eta_rel, a, r):
    """Equation 4 written with torch.logsumexp over each causal row (an
    independent evaluation of the objective, for autograd)."""
    T = eta_abs.shape[0]
    i = torch.arange(T)[:, None]
    j = torch.arange(T)[None, :]
    d = (i - j).clamp(min=0)
    G = a[None, :] + r[d]
    G = torch.where(j <= i, G, torch.full_like(G, -math.inf))
    return (torch.logsumexp(G, dim=1).sum() - eta_abs @ a - eta_rel @ r) / T


def test_target_statistics_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "fit_target_worked_T3.json")))
    A = np.array(g["ahat"])
    P = F.fit_target(A, g["floor"])
    for i, row in enumerate(g["P"]):
        np.testing.assert_allclose(P[i, : i + 1], row, rtol=1e-14, atol=0)
        assert np.all(P[i, i + 1 :] == 0)
    st = F.fit_statistics(A, g["floor"])
    np.testing.assert_allclose(st["eta_abs"], g["eta_abs"], rtol=1e-14)
    np.testing.assert_allclose(st["eta_rel"], g["eta_rel"], rtol=1e-14)
    assert st["negent"] == pytest.approx(g["negent"], rel=1e-13)
    a0, r0 = F.fit_init(st["eta_rel"])
    np.testing.assert_array_equal(a0, g["init_a"])
    np.testing.assert_allclose(r0, g["init_r"], rtol=1e-13)


def test_target_ignores_upper_triangle_and_scales_rows():
    A = calibration_mean(12, 5, 0).astype(np.float64)
    B = A * np.arange(1, 13)[:, None]  # rows rescaled: P is unchanged (floor aside)
    B[np.triu_indices(12, 1)] = 1e6
    A2 = A.copy()
    A2[np.triu_indices(12, 1)] = -7.0
    np.testing.assert_allclose(F.fit_target(A2), F.fit_target(A), rtol=0, atol=0)
    # (zeros floored at 1e-30 differ by less than 1e-29 after the rescaling)
    np.testing.assert_allclose(F.fit_target(B, floor=1e-30), F.fit_target(A, floor=1e-30), rtol=1e-13, atol=1e-29)
    P = F.fit_target(A)
    np.testing.assert_allclose(P.sum(axis=1), 1.0, rtol=1e-14)
    eta_abs, eta_rel = F.marginals(P)
    # each marginal distributes the T rows' unit mass
    assert eta_abs.sum() == pytest.approx(12, rel=1e-14)
    assert eta_rel.sum() == pytest.approx(12, rel=1e-14)
    # brute-force diagonal sums
    for d in range(12):
        assert eta_rel[d] == pytest.approx(sum(P[i, i - d] for i in range(d, 12)), rel=1e-14)


def test_init_closed_forms():
    T = 9
    # uniform causal rows: eta_rel(d) = sum_{i >= d} 1/(i+1) = H_T - H_d
    P = np.tril(np.ones((T, T))) / np.arange(1, T + 1)[:, None]
    _, eta_rel = F.marginals(P)
    a, r = F.fit_init(eta_rel)
    H = [sum(1.0 / m for m in range(1, n + 1)) for n in range(T + 1)]
    for d in range(T):
        assert r[d] == pytest.approx(math.log((H[T] - H[d]) / (T - d)), rel=1e-13)
    assert np.all(a == 0)
    # identity target: all mass on the diagonal; the floor keeps the rest at 1e-9
    Pid = F.fit_target(np.eye(T))
    _, eta_rel = F.marginals(Pid)
    a, r = F.fit_init(eta_rel)
    assert abs(r[0]) < 1e-7  # log(~T / T)
    np.testing.assert_allclose(r[1:], math.log(1e-9), rtol=1e-12)


def test_gradient_is_equation_20_and_matches_autograd():
    T = 17
    P = _random_target(T, 3)
    eta_abs, eta_rel = F.marginals(P)
    rng = np.random.default_rng(4)
    a = rng.standard_normal(T)
    r = rng.standard_normal(T) - 0.1 * np.arange(T)
    ga, gr = F.fit_gradient(eta_abs, eta_rel, a, r)
    ta = torch.tensor(a, dtype=torch.float64, requires_grad=True)
    tr = torch.tensor(r, dtype=torch.float64, requires_grad=True)
    L = _torch_loss(torch.tensor(eta_abs), torch.tensor(eta_rel), ta, tr)
    L.backward()
    np.testing.assert_allclose(ga, ta.grad.numpy(), rtol=1e-10, atol=1e-15)
    np.testing.assert_allclose(gr, tr.grad.numpy(), rtol=1e-10, atol=1e-15)
    assert F.fit_loss(eta_abs, eta_rel, a, r) == pytest.approx(L.item(), rel=1e-13)
    # each gradient sums to zero: both marginals carry T units of mass
    assert abs(ga.sum()) < 1e-13 and abs(gr.sum()) < 1e-13


def test_adam_steps_match_torch_optim():
    T = 13
    P = F.fit_target(calibration_mean(T, 11, 2))
    eta_abs, eta_rel = F.marginals(P)
    steps = 30
    a, r, logz = F.fit_pattern(eta_abs, eta_rel, steps=steps)
    a0, r0 = F.fit_init(eta_rel)
    ta = torch.tensor(a0, dtype=torch.float64, requires_grad=True)
    tr = torch.tensor(r0, dtype=torch.float64, requires_grad=True)
    opt = torch.optim.Adam([ta, tr], lr=0.05, betas=(0.9, 0.999), eps=1e-8)
    ea, er = torch.tensor(eta_abs), torch.tensor(eta_rel)
    for _ in range(steps):
        opt.zero_grad()
        _torch_loss(ea, er, ta, tr).backward()
        opt.step()
    np.testing.assert_allclose(a, ta.detach().numpy(), rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(r, tr.detach().numpy(), rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(logz, frozen_lognorm(a, r, T), rtol=0, atol=0)


def test_fit_recovers_a_compact_target():
    """A target that is itself a compact pattern is recovered: kappa -> 0 and
    the fitted marginals equal the target's (Equation 20 at the optimum)."""
    T = 24
    rng = np.random.default_rng(8)
    a_true = rng.standard_normal(T)
    a_true[0] += 3.0  # a sink
    r_true = -0.3 * np.arange(T) + 0.3 * rng.standard_normal(T)
    P = frozen_pattern(a_true, r_true, T)
    eta_abs, eta_rel = F.marginals(P)
    negent = F.neg_entropy(P)
    # the recipe's 400 steps reach the optimum to ~1e-9 on this target (far
    # longer runs end in Adam's noise-driven oscillation around it)
    a, r, _ = F.fit_pattern(eta_abs, eta_rel)
    kappa = F.fit_kappa(negent, eta_abs, eta_rel, a, r)
    assert abs(kappa) < 1e-9
    mu_abs, mu_rel = F.fitted_marginals(a, r, T)
    np.testing.assert_allclose(mu_abs, eta_abs, atol=1e-7)
    np.testing.assert_allclose(mu_rel, eta_rel, atol=1e-7)
    np.testing.assert_allclose(frozen_pattern(a, r, T), P, atol=1e-7)


def test_kappa_from_statistics_equals_dense_kl():
    for seed, T in ((0, 7), (1, 30), (2, 64)):
        P = F.fit_target(calibration_mean(T, 21, seed))
        eta_abs, eta_rel = F.marginals(P)
        rng = np.random.default_rng(seed)
        a = rng.standard_normal(T)
        r = rng.standard_normal(T)
        k_dense = F.fit_kappa_dense(P, a, r)
        k_stat = F.fit_kappa(F.neg_entropy(P), eta_abs, eta_rel, a, r)
        assert k_dense > 0
        assert k_stat == pytest.approx(k_dense, rel=1e-11, abs=1e-13)
        # brute force of the row-averaged KL on the smallest case
        if T == 7:
            Q = frozen_pattern(a, r, T)
            kl = sum(P[i, j] * math.log(P[i, j] / Q[i, j]) for i in range(T) for j in range(i + 1)) / T
            assert k_dense == pytest.approx(kl, rel=1e-12)


def test_degenerate_lengths():
    # T = 1: the single weight is 1 whatever a and r; nothing moves
    a, r, logz = F.fit_pattern(np.array([1.0]), np.array([1.0]))
    assert a[0] == 0 and r[0] == 0 and logz[0] == 0
    # T = 2: one free logit; the fit reproduces row 1 of the target
    p10 = 0.3
    P = np.array([[1.0, 0.0], [p10, 1 - p10]])
    eta_abs, eta_rel = F.marginals(P)
    a, r, _ = F.fit_pattern(eta_abs, eta_rel)
    q10 = frozen_pattern(a, r, 2)[1, 0]
    assert q10 == pytest.approx(p10, abs=1e-3)


def test_fit_improves_on_init_and_acceptance_rule():
    T = 40
    A = calibration_mean(T, 31, 1)
    res = F.fit_head(A)
    a0, r0 = F.fit_init(res["eta_rel"])
    k0 = F.fit_kappa(res["negent"], res["eta_abs"], res["eta_rel"], a0, r0)
    assert res["kappa"] < k0
    assert res["accepted"] == (res["kappa"] <= 0.2)
    assert res["kappa"] == pytest.approx(F.fit_kappa_dense(F.fit_target(A), res["a"], res["r"]), rel=1e-10)


def test_planted_mistake_in_gradient_is_caught():
    """A sign error planted in the oracle's gradient breaks the autograd pin."""
    T = 8
    P = _random_target(T, 9)
    eta_abs, eta_rel = F.marginals(P)
    a = np.zeros(T)
    r = np.linspace(0, -2, T)
    ga, gr = F.fit_gradient(eta_abs, eta_rel, a, r)
    mu_abs, mu_rel = F.fitted_marginals(a, r, T)
    wrong = (eta_abs - mu_abs) / T
    ta = torch.tensor(a, dtype=torch.float64, requires_grad=True)
    tr = torch.tensor(r, dtype=torch.float64, requires_grad=True)
    _torch_loss(torch.tensor(eta_abs), torch.tensor(eta_rel), ta, tr).backward()
    assert np.allclose(ga, ta.grad.numpy(), rtol=1e-10, atol=1e-15)
    assert not np.allclose(wrong, ta.grad.numpy(), rtol=1e-3, atol=1e-6)
