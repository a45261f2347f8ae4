"""Dense float64 reference for the calibration statistics -- TEST INFRASTRUCTURE.

Only tests, the smoke check and the bench's CPU-baseline leg use this module.
It shares no code with the HIP library.

Source: "When Can Attention Heads Be Statically Defined?"
  * Section 3.1 "Calibration and head selection": over N calibration
    sequences a head's causal attention A^(n) (Appendix A.1, Equations 5-6)
    gives the empirical mean A-hat = N^-1 sum_n A^(n), the attention-variance
    score (Equation 1)
        s_var = sum_n ||A^(n) - A-hat||_F^2 / ((N - 1) T^2)
    and the forward-KL score (Equation 2)
        s_KL = (N T)^-1 sum_n sum_i KL(A^(n)[i, :i+1] || A-hat[i, :i+1]);
  * Algorithm 1 (measure A-hat and s_var before fitting).

Everything is evaluated from these definitions: every A^(n) is formed
densely, the mean is taken, and both scores are summed entry by entry
against it.  Indexing is 0-based (row i attends to keys 0..i).  For N = 1
the variance score is reported as 0 (Equation 1 divides by N - 1 and no
spread is observable).
"""

from __future__ import annotations

from typing import Dict

import numpy as np

F64 = np.float64


def attention_matrix(q, k, scale: float) -> np.ndarray:
    """A = causal row softmax of scale * Q K^T (Appendix A.1, Equations
    5-6) for one head and one sequence: q, k are [T, D]; returns [T, T]
    with zeros above the diagonal."""
    q = np.asarray(q, dtype=F64)
    k = np.asarray(k, dtype=F64)
    T = q.shape[0]
    S = scale * (q @ k.T)
    causal = np.tril(np.ones((T, T), dtype=bool))
    S = np.where(causal, S, -np.inf)
    m = S.max(axis=1, keepdims=True)
    E = np.exp(S - m)
    return E / E.sum(axis=1, keepdims=True)


def calibration_stats(q, k, scale: float) -> Dict[str, object]:
    """A-hat, s_var and s_KL of one head from its N calibration sequences:
    q, k are [N, T, D]."""
    q = np.asarray(q, dtype=F64)
    k = np.asarray(k, dtype=F64)
    N, T, _ = q.shape
    As = np.stack([attention_matrix(q[n], k[n], scale) for n in range(N)])
    Ahat = As.mean(axis=0)
    if N > 1:
        s_var = float(((As - Ahat[None]) ** 2).sum() / ((N - 1) * T * T))
    else:
        s_var = 0.0
    causal = np.tril(np.ones((T, T), dtype=bool))
    kl = 0.0
    for n in range(N):
        P = As[n][causal]
        Q = Ahat[causal]
        pos = P > 0
        kl += float((P[pos] * (np.log(P[pos]) - np.log(Q[pos]))).sum())
    return {"ahat": Ahat, "s_var": s_var, "s_kl": kl / (N * T)}
