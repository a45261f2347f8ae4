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


def attention_rows(q, k, scale: float, rows) -> np.ndarray:
    """Rows ``rows`` of A = causal row softmax of scale * Q K^T (Appendix
    A.1, Equations 5-6) for one head and one sequence: q, k are [T, D];
    returns [len(rows), T] with zeros at keys j > i."""
    q = np.asarray(q, dtype=F64)
    k = np.asarray(k, dtype=F64)
    T = q.shape[0]
    rows = np.asarray(rows, dtype=np.int64)
    S = scale * (q[rows] @ k.T)
    S = np.where(np.arange(T)[None, :] <= rows[:, None], S, -np.inf)
    m = S.max(axis=1, keepdims=True)
    E = np.exp(S - m)
    return E / E.sum(axis=1, keepdims=True)


def attention_matrix(q, k, scale: float) -> np.ndarray:
    """The whole [T, T] causal attention matrix of one head and sequence."""
    return attention_rows(q, k, scale, np.arange(np.shape(q)[0]))


def calibration_rows(q, k, scale: float, rows) -> Dict[str, object]:
    """The part of one head's statistics that rows ``rows`` determine: the
    mean rows A-hat[rows] and the rows' terms of the two score sums,
    ``sq`` = sum_n sum_{i in rows} ||A^(n)[i] - A-hat[i]||^2 and
    ``kl`` = sum_n sum_{i in rows} KL(A^(n)[i] || A-hat[i]).  Both scores
    are sums over rows, so the rows of a partition add up to the whole."""
    q = np.asarray(q, dtype=F64)
    k = np.asarray(k, dtype=F64)
    N = q.shape[0]
    As = np.stack([attention_rows(q[n], k[n], scale, rows) for n in range(N)])
    Ahat = As.mean(axis=0)
    sq = float(((As - Ahat[None]) ** 2).sum())
    kl = 0.0
    for n in range(N):
        pos = As[n] > 0
        kl += float((As[n][pos] * (np.log(As[n][pos]) - np.log(Ahat[pos]))).sum())
    return {"ahat": Ahat, "sq": sq, "kl": kl}


def calibration_stats(q, k, scale: float) -> Dict[str, object]:
    """A-hat, s_var and s_KL of one head from its N calibration sequences:
    q, k are [N, T, D]."""
    N, T, _ = np.shape(q)
    part = calibration_rows(q, k, scale, np.arange(T))
    s_var = part["sq"] / ((N - 1) * T * T) if N > 1 else 0.0
    return {"ahat": part["ahat"], "s_var": s_var, "s_kl": part["kl"] / (N * T)}
