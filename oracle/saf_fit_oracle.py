"""Dense float64 reference for fitting a compact pattern -- TEST INFRASTRUCTURE.

Only tests, the smoke check and the bench's CPU-baseline leg use this module.
It shares no code with the HIP library.

Source: "When Can Attention Heads Be Statically Defined?"
  * Algorithm 1 (one-time SAF recipe): the target preparation (floor the
    causal entries of the calibration mean at 1e-9, row-normalise, take the
    two marginals), the fit, and the acceptance statistic kappa, the
    row-averaged KL divergence of the fitted pattern from the target;
  * Section 3.2 "Fitting", Equation 4: the objective
        L(a, r) = (1/T) [ sum_i log Z(i) - sum_j eta_abs(j) a(j)
                          - sum_d eta_rel(d) r(d) ],
    with eta_abs(j) = sum_{i >= j} P(i, j) and eta_rel(d) = sum_{i-j=d} P(i, j);
  * Appendix A.2 "Selection, fitting, and installation": start from a = 0 and
    r(d) = log max(eta_rel(d) / (T - d), 1e-9), then J = 400 Adam steps at
    learning rate 0.05 with no early stopping; accept when kappa <= 0.2 nats;
  * Appendix D.1, Equation 20: the gradient of Equation 4 is the fitted
    pattern's marginal minus the target's, divided by T.

Indexing is 0-based as in ``saf_oracle``: ``a[j]`` weights key j, ``r[d]``
offset d = i - j, and Z(i) = N(i) is the row normaliser of Equation 3.

Adam follows Kingma & Ba (2015) with the bias-corrected moments and eps added
to the square root of the second moment, with the default moment decays
(0.9, 0.999) and eps = 1e-8; the pages name the optimiser and the learning
rate only.

Every quantity is evaluated from its dense definition; nothing here uses the
convolution structure of the normaliser.
"""

from __future__ import annotations

from typing import Dict, Optional, Tuple

import numpy as np

from .saf_oracle import frozen_lognorm, frozen_pattern

F64 = np.float64

TARGET_FLOOR = 1e-9      # Algorithm 1: floor of the causal target entries
INIT_FLOOR = 1e-9        # Appendix A.2: floor inside the initial r
FIT_STEPS = 400          # Appendix A.2: J
FIT_LR = 0.05            # Appendix A.2: gamma
FIT_TOLERANCE = 0.2      # Section 3.2 "Fitting": acceptance bound on kappa (nats)
ADAM_BETAS = (0.9, 0.999)
ADAM_EPS = 1e-8


# ---------------------------------------------------------------------------
# Target preparation (Algorithm 1: floor, row-normalise, marginals).
# ---------------------------------------------------------------------------


def fit_target(ahat, floor: float = TARGET_FLOOR) -> np.ndarray:
    """P: the causal entries of the [T, T] calibration mean floored at
    ``floor`` and each row divided by its sum; entries j > i are 0 (the upper
    triangle of ``ahat`` is never read)."""
    A = np.asarray(ahat, dtype=F64)
    T = A.shape[0]
    if A.shape != (T, T):
        raise ValueError("ahat must be [T, T]")
    causal = np.tril(np.ones((T, T), dtype=bool))
    X = np.where(causal, np.maximum(np.where(causal, A, 0.0), floor), 0.0)
    return X / X.sum(axis=1, keepdims=True)


def marginals(P) -> Tuple[np.ndarray, np.ndarray]:
    """(eta_abs, eta_rel) of a causal [T, T] matrix: column sums, and sums
    along each diagonal i - j = d (Equation 4)."""
    P = np.asarray(P, dtype=F64)
    T = P.shape[0]
    eta_abs = P.sum(axis=0)
    eta_rel = np.array([np.trace(P, offset=-d) for d in range(T)], dtype=F64)
    return eta_abs, eta_rel


def neg_entropy(P) -> float:
    """sum_i sum_{j <= i} P(i, j) log P(i, j) (0 log 0 = 0): the part of
    kappa that depends on the target alone."""
    P = np.asarray(P, dtype=F64)
    pos = P > 0
    return float((P[pos] * np.log(P[pos])).sum())


def fit_statistics(ahat, floor: float = TARGET_FLOOR) -> Dict[str, np.ndarray]:
    """The target's sufficient statistics: eta_abs, eta_rel and the summed
    negative row entropy ``negent``."""
    P = fit_target(ahat, floor)
    eta_abs, eta_rel = marginals(P)
    return {"eta_abs": eta_abs, "eta_rel": eta_rel, "negent": neg_entropy(P)}


# ---------------------------------------------------------------------------
# Objective and gradient (Equation 4, Equation 20).
# ---------------------------------------------------------------------------


def fit_loss(eta_abs, eta_rel, a, r) -> float:
    """Equation 4 at (a, r)."""
    eta_abs = np.asarray(eta_abs, dtype=F64)
    eta_rel = np.asarray(eta_rel, dtype=F64)
    T = eta_abs.shape[0]
    a = np.asarray(a, dtype=F64)[:T]
    r = np.asarray(r, dtype=F64)[:T]
    z = frozen_lognorm(a, r, T)
    return float((z.sum() - eta_abs @ a - eta_rel @ r) / T)


def fitted_marginals(a, r, T: int) -> Tuple[np.ndarray, np.ndarray]:
    """The marginals of the dense compact pattern P-hat(a, r) (Equation 3)."""
    return marginals(frozen_pattern(a, r, T))


def fit_gradient(eta_abs, eta_rel, a, r) -> Tuple[np.ndarray, np.ndarray]:
    """(dL/da, dL/dr) of Equation 4: each is (fitted marginal - target
    marginal) / T (Equation 20 for a, and the same argument for r, whose
    logits are the diagonal i - j = d)."""
    eta_abs = np.asarray(eta_abs, dtype=F64)
    eta_rel = np.asarray(eta_rel, dtype=F64)
    T = eta_abs.shape[0]
    mu_abs, mu_rel = fitted_marginals(a, r, T)
    return (mu_abs - eta_abs) / T, (mu_rel - eta_rel) / T


# ---------------------------------------------------------------------------
# The fit: initialisation and Adam (Appendix A.2).
# ---------------------------------------------------------------------------


def fit_init(eta_rel, floor: float = INIT_FLOOR) -> Tuple[np.ndarray, np.ndarray]:
    """a = 0 and r(d) = log max(eta_rel(d) / (T - d), floor): the mean target
    weight on diagonal d, which holds T - d entries."""
    eta_rel = np.asarray(eta_rel, dtype=F64)
    T = eta_rel.shape[0]
    a = np.zeros(T, dtype=F64)
    r = np.log(np.maximum(eta_rel / (T - np.arange(T, dtype=F64)), floor))
    return a, r


def adam_update(theta, g, m, v, t: int, lr: float, betas=ADAM_BETAS, eps: float = ADAM_EPS):
    """One Adam step (Kingma & Ba 2015) at step number t >= 1: the moments
    are updated in place and the new parameters returned."""
    b1, b2 = betas
    m *= b1
    m += (1.0 - b1) * g
    v *= b2
    v += (1.0 - b2) * g * g
    m_hat = m / (1.0 - b1 ** t)
    v_hat = v / (1.0 - b2 ** t)
    return theta - lr * m_hat / (np.sqrt(v_hat) + eps)


def fit_pattern(eta_abs, eta_rel, steps: int = FIT_STEPS, lr: float = FIT_LR,
                betas=ADAM_BETAS, eps: float = ADAM_EPS,
                init: Optional[Tuple[np.ndarray, np.ndarray]] = None):
    """Fit (a, r) to the target marginals: ``steps`` Adam steps on Equation 4
    from the initialisation of Appendix A.2 (or ``init``), both parameter
    vectors updated together from the gradient at the same point.

    Returns (a, r, logz), logz = log N of the fitted pattern (natural log).
    """
    eta_abs = np.asarray(eta_abs, dtype=F64)
    eta_rel = np.asarray(eta_rel, dtype=F64)
    T = eta_abs.shape[0]
    if init is None:
        a, r = fit_init(eta_rel)
    else:
        a = np.array(init[0], dtype=F64)
        r = np.array(init[1], dtype=F64)
    ma = np.zeros(T, dtype=F64)
    va = np.zeros(T, dtype=F64)
    mr = np.zeros(T, dtype=F64)
    vr = np.zeros(T, dtype=F64)
    for t in range(1, steps + 1):
        ga, gr = fit_gradient(eta_abs, eta_rel, a, r)
        a = adam_update(a, ga, ma, va, t, lr, betas, eps)
        r = adam_update(r, gr, mr, vr, t, lr, betas, eps)
    return a, r, frozen_lognorm(a, r, T)


# ---------------------------------------------------------------------------
# Acceptance (Algorithm 1).
# ---------------------------------------------------------------------------


def fit_kappa_dense(P, a, r) -> float:
    """kappa = (1/T) sum_i KL(P[i, :i+1] || P-hat[i, :i+1]), with the dense
    fitted pattern (0 log 0 = 0 on the target side)."""
    P = np.asarray(P, dtype=F64)
    T = P.shape[0]
    Q = frozen_pattern(a, r, T)
    pos = P > 0
    return float((P[pos] * (np.log(P[pos]) - np.log(Q[pos]))).sum() / T)


def fit_kappa(negent: float, eta_abs, eta_rel, a, r) -> float:
    """kappa from the sufficient statistics alone: since every target row sums
    to 1, sum_ij P log P-hat = sum_j eta_abs a + sum_d eta_rel r - sum_i log Z,
    so kappa = negent / T + L(a, r) (Equation 4)."""
    T = np.shape(eta_abs)[0]
    return float(negent / T + fit_loss(eta_abs, eta_rel, a, r))


def fit_head(ahat, steps: int = FIT_STEPS, lr: float = FIT_LR, tolerance: float = FIT_TOLERANCE):
    """Algorithm 1's per-head fitting for one calibration mean: target,
    marginals, fit, kappa and the acceptance decision kappa <= tolerance."""
    st = fit_statistics(ahat)
    a, r, logz = fit_pattern(st["eta_abs"], st["eta_rel"], steps, lr)
    kappa = fit_kappa(st["negent"], st["eta_abs"], st["eta_rel"], a, r)
    return {"a": a, "r": r, "logz": logz, "kappa": kappa, "accepted": kappa <= tolerance, **st}
