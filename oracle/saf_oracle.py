"""Dense float64 reference for the SAF hybrid attention layer.

TEST INFRASTRUCTURE: only tests, the smoke check and the bench's CPU-baseline
leg use this module.  It shares no code with the HIP library.

Source: "When Can Attention Heads Be Statically Defined?" (arXiv 2609.34650).

Indexing.  The pages index keys 1..T and offsets 0..T-1 (Section 3.2).  Here
everything is 0-based: ``a[j]`` is alpha(j+1) and ``r[d]`` is rho(d), so the
normaliser of query row ``i`` sums over keys ``k = 0..i`` with offset ``i-k``,
diagonal included, and row 0 holds the single weight 1.

Ordinary heads (Appendix A.1, Equations 5-7):
    S = s * Q K^T (s = 1/sqrt(d_h) unless given), A = causal row softmax of S,
    O = A V, and the row log-sum-exp L_i = log sum_{j<=i} exp(S_ij).
Frozen heads (Section 3.2, Equation 3; Section 3 "head output"):
    G_ij = a[j] + r[i-j] for j <= i, P_ij = exp(G_ij) / N(i) with
    N(i) = sum_{k<=i} exp(a[k] + r[i-k]), O = P V, and L_i = log N(i).
    The logits carry no temperature: Equation 3 has none.
Backward (Section 3.3 "Fused computation", Appendix D.2):
    ordinary heads: dV = A^T dO, dA = dO V^T, dS = A o (dA - rowsum(A o dA)),
    dQ = s dS K, dK = s dS^T Q;
    frozen heads: dV = P^T dO, and Q, K get no gradient (exact zeros), because
    a frozen head has no query/key slot.

All arithmetic is float64; inputs are upcast exactly.  Large heads are
processed in row chunks so that at most one chunk of the dense T x T matrix is
resident, but each chunk is the full dense definition.
"""

from __future__ import annotations

import math
from typing import Iterable, Optional, Sequence, Tuple

import numpy as np

F64 = np.float64
_CHUNK_ELEMS = 1 << 24  # rows per chunk = _CHUNK_ELEMS // T


def default_scale(D: int) -> float:
    """Ordinary-head score scale 1/sqrt(d_h) (Appendix A.1, Equation 5)."""
    return 1.0 / math.sqrt(D)


def _rows_chunks(T: int, rows: Optional[np.ndarray] = None):
    rows = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    step = max(1, _CHUNK_ELEMS // max(T, 1))
    for s in range(0, len(rows), step):
        yield rows[s : s + step]


def _prefix(x, T: int) -> np.ndarray:
    x = np.asarray(x, dtype=F64)
    if x.shape[-1] < T:
        raise ValueError(f"stored prior length {x.shape[-1]} is shorter than T={T}")
    return x[..., :T]


def _row_logsumexp(G: np.ndarray) -> np.ndarray:
    """log sum_j exp(G_ij) per row, shifted by the row maximum.

    Every causal row contains its diagonal, so the maximum is finite.
    """
    m = G.max(axis=1)
    return m + np.log(np.exp(G - m[:, None]).sum(axis=1))


# ---------------------------------------------------------------------------
# Frozen heads: Section 3.2, Equation 3.
# ---------------------------------------------------------------------------


def frozen_logits(a, r, T: int, rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """G[i, j] = a[j] + r[i - j] for j <= i and -inf for j > i.

    ``a`` is the absolute key-position preference, ``r`` the relative-distance
    preference (Equation 3's exponent).  Only the first T entries of each are
    used; entries beyond T never enter a causal row.
    """
    a = _prefix(a, T)
    r = _prefix(r, T)
    rows = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    j = np.arange(T)
    delta = rows[:, None] - j[None, :]
    causal = delta >= 0
    G = np.full((len(rows), T), -np.inf, dtype=F64)
    G[causal] = (a[None, :] + r[np.where(causal, delta, 0)])[causal]
    return G


def frozen_lognorm(a, r, T: int) -> np.ndarray:
    """log N(i) with N(i) = sum_{k <= i} exp(a[k] + r[i - k])  (Equation 3)."""
    out = np.empty(T, dtype=F64)
    for rows in _rows_chunks(T):
        out[rows] = _row_logsumexp(frozen_logits(a, r, T, rows))
    return out


def frozen_pattern(a, r, T: int, rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """The compact pattern P-hat of Equation 3 as a dense [rows, T] matrix."""
    rows = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    G = frozen_logits(a, r, T, rows)
    logN = _row_logsumexp(G)
    return np.exp(G - logN[:, None])


def frozen_rows_fwd(v, a, r, rows: Sequence[int]) -> Tuple[np.ndarray, np.ndarray]:
    """Output rows O[rows] = P-hat[rows] V of one frozen head, and log N(rows)."""
    v = np.asarray(v, dtype=F64)
    T = v.shape[0]
    rows = np.asarray(rows, dtype=np.int64)
    G = frozen_logits(a, r, T, rows)
    logN = _row_logsumexp(G)
    P = np.exp(G - logN[:, None])
    return P @ v, logN


def frozen_head_fwd(v, a, r) -> Tuple[np.ndarray, np.ndarray]:
    """O = P-hat V and log N for one frozen head; v is [T, D]."""
    v = np.asarray(v, dtype=F64)
    T, D = v.shape
    O = np.empty((T, D), dtype=F64)
    L = np.empty(T, dtype=F64)
    for rows in _rows_chunks(T):
        O[rows], L[rows] = frozen_rows_fwd(v, a, r, rows)
    return O, L


def frozen_head_bwd(do, a, r) -> np.ndarray:
    """dV = P-hat^T dO for one frozen head (Section 3.3, Appendix D.2)."""
    do = np.asarray(do, dtype=F64)
    T, D = do.shape
    dv = np.zeros((T, D), dtype=F64)
    for rows in _rows_chunks(T):
        P = frozen_pattern(a, r, T, rows)
        dv += P.T @ do[rows]
    return dv


def frozen_head_pattern_grad(v, do, a, r) -> Tuple[np.ndarray, np.ndarray]:
    """Gradients of a frozen head's pattern parameters, for the variant whose
    alpha and rho stay trainable (Appendix C.3.2 "Pattern content and
    trainability"; the pattern of Section 3.2, Equation 3).

    With W = P-hat (row softmax of the logits G_ij = a[j] + r[i-j], j <= i),
    O = W V and an upstream gradient dO, the chain rule through the row
    softmax (normaliser included) gives, per row i,
        dW = dO V^T,   D_i = sum_j W_ij dW_ij,   dG_ij = W_ij (dW_ij - D_i),
    and since a[j] enters every logit of column j and r[d] every logit of
    diagonal i - j = d:
        da[j] = sum_i dG_ij   (column sums),
        dr[d] = sum_i dG_{i, i-d}   (diagonal sums).
    Returns (da, dr), each of length T; entries beyond T would be zero.
    """
    T = np.shape(v)[0]
    da = np.zeros(T, dtype=F64)
    dr = np.zeros(T, dtype=F64)
    for rows in _rows_chunks(T):
        ga, gr = frozen_rows_pattern_grad(v, do, a, r, rows)
        da += ga
        dr += gr
    return da, dr


def frozen_rows_pattern_grad(v, do, a, r, rows: Sequence[int]) -> Tuple[np.ndarray, np.ndarray]:
    """The contribution of query rows ``rows`` to (da, dr) of one frozen head
    (see frozen_head_pattern_grad).  Key j only meets rows i >= j and offset d
    only rows i >= d, so for j, d >= min(rows) with rows = [min(rows), T) this
    is the full gradient entry."""
    v = np.asarray(v, dtype=F64)
    do = np.asarray(do, dtype=F64)
    T = v.shape[0]
    rows = np.asarray(rows, dtype=np.int64)
    da = np.zeros(T, dtype=F64)
    dr = np.zeros(T, dtype=F64)
    W = frozen_pattern(a, r, T, rows)
    dW = do[rows] @ v.T
    Drow = (W * dW).sum(axis=1)
    dG = W * (dW - Drow[:, None])
    da += dG.sum(axis=0)
    for n, i in enumerate(rows):
        dr[: i + 1] += dG[n, i::-1]  # dG[i, i - d] for d = 0..i
    return da, dr


# ---------------------------------------------------------------------------
# Ordinary heads: Appendix A.1, Equations 5-7.
# ---------------------------------------------------------------------------


def _ordinary_scores(q, k, scale: float, rows: np.ndarray) -> np.ndarray:
    T = k.shape[0]
    S = scale * (q[rows] @ k.T)
    S[np.arange(T)[None, :] > rows[:, None]] = -np.inf
    return S


def ordinary_rows_fwd(q, k, v, scale: float, rows: Sequence[int]) -> Tuple[np.ndarray, np.ndarray]:
    """Output rows and row log-sum-exp of causal softmax attention."""
    q = np.asarray(q, dtype=F64)
    k = np.asarray(k, dtype=F64)
    v = np.asarray(v, dtype=F64)
    rows = np.asarray(rows, dtype=np.int64)
    S = _ordinary_scores(q, k, scale, rows)
    L = _row_logsumexp(S)
    A = np.exp(S - L[:, None])
    return A @ v, L


def ordinary_head_fwd(q, k, v, scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """O = softmax_causal(s Q K^T) V and L for one head; q, k, v are [T, D]."""
    v = np.asarray(v, dtype=F64)
    T, D = v.shape
    O = np.empty((T, D), dtype=F64)
    L = np.empty(T, dtype=F64)
    for rows in _rows_chunks(T):
        O[rows], L[rows] = ordinary_rows_fwd(q, k, v, scale, rows)
    return O, L


def ordinary_head_bwd(q, k, v, do, scale: float) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """dQ, dK, dV of O = softmax_causal(s Q K^T) V given dO (chain rule)."""
    q = np.asarray(q, dtype=F64)
    k = np.asarray(k, dtype=F64)
    v = np.asarray(v, dtype=F64)
    do = np.asarray(do, dtype=F64)
    T, D = q.shape
    dq = np.zeros((T, D), dtype=F64)
    dk = np.zeros((T, D), dtype=F64)
    dv = np.zeros((T, D), dtype=F64)
    for rows in _rows_chunks(T):
        S = _ordinary_scores(q, k, scale, rows)
        A = np.exp(S - _row_logsumexp(S)[:, None])
        dv += A.T @ do[rows]
        dA = do[rows] @ v.T
        dS = A * (dA - (A * dA).sum(axis=1, keepdims=True))
        dq[rows] = scale * (dS @ k)
        dk += scale * (dS.T @ q[rows])
    return dq, dk, dv


# ---------------------------------------------------------------------------
# The hybrid layer: heads of both kinds in their original order
# (Section 3.3 "Fused computation", Appendix D.2).
# ---------------------------------------------------------------------------


def _check(q, v, frozen, a, r):
    B, H, T, D = np.shape(q)
    if len(frozen) != H:
        raise ValueError("frozen mask length must equal H")
    if np.shape(a)[0] != H or np.shape(r)[0] != H:
        raise ValueError("a and r need one row per head")
    return B, H, T, D


def _kv_group(q, k, v) -> int:
    """Query heads per key/value head.  Grouped-query attention (the pages'
    Qwen path, Appendix D.2): query head h uses key/value head h // group."""
    H, Hk = np.shape(q)[1], np.shape(k)[1]
    if np.shape(v)[1] != Hk or Hk < 1 or H % Hk != 0:
        raise ValueError("k and v need the same number of heads, dividing the query heads")
    return H // Hk


def hybrid_fwd(q, k, v, frozen, a, r, scale: Optional[float] = None,
               heads: Optional[Iterable[Tuple[int, int]]] = None):
    """Forward of the hybrid layer.

    q: [B, H, T, D]; k, v: [B, Hkv, T, D] with Hkv dividing H (Hkv = H for
    multi-head attention; otherwise query head h uses key/value head
    h // (H / Hkv), the grouped-query path of the pages' Qwen experiments);
    frozen: [H] flags; a, r: [H, Tp] with Tp >= T.
    Returns O [B, H, T, D] and L [B, H, T] in float64.  For frozen heads L is
    log N(i), the same for every batch element, and q, k are never read.
    ``heads`` restricts the work to the listed (b, h) pairs; other entries of
    the outputs are NaN.
    """
    B, H, T, D = _check(q, v, frozen, a, r)
    g = _kv_group(q, k, v)
    s = default_scale(D) if scale is None else float(scale)
    O = np.full((B, H, T, D), np.nan, dtype=F64)
    L = np.full((B, H, T), np.nan, dtype=F64)
    todo = [(b, h) for b in range(B) for h in range(H)] if heads is None else list(heads)
    for b, h in todo:
        if frozen[h]:
            O[b, h], L[b, h] = frozen_head_fwd(v[b, h // g], a[h], r[h])
        else:
            O[b, h], L[b, h] = ordinary_head_fwd(q[b, h], k[b, h // g], v[b, h // g], s)
    return O, L


def hybrid_pattern_grad(v, do, frozen, a, r):
    """Pattern-parameter gradients of every frozen head, summed over the batch.

    v, do: [B, H, T, D]; frozen: [H] flags; a, r: [H, Tp] with Tp >= T.
    Returns dA, dR of shape [H, T] (float64); rows of ordinary heads are NaN.
    """
    B, H, T, D = np.shape(v)
    if len(frozen) != H or np.shape(a)[0] != H or np.shape(r)[0] != H:
        raise ValueError("frozen mask, a and r need one entry per head")
    dA = np.full((H, T), np.nan, dtype=F64)
    dR = np.full((H, T), np.nan, dtype=F64)
    for h in range(H):
        if not frozen[h]:
            continue
        dA[h] = 0.0
        dR[h] = 0.0
        for b in range(B):
            ga, gr = frozen_head_pattern_grad(v[b, h], do[b, h], a[h], r[h])
            dA[h] += ga
            dR[h] += gr
    return dA, dR


def hybrid_bwd(q, k, v, do, frozen, a, r, scale: Optional[float] = None,
               heads: Optional[Iterable[Tuple[int, int]]] = None):
    """Backward of the hybrid layer given dO: returns dQ, dK, dV (float64).

    Frozen heads get dQ = dK = 0 exactly and dV = P-hat^T dO.  Multi-head
    attention only (k, v with H heads).
    """
    B, H, T, D = _check(q, v, frozen, a, r)
    if _kv_group(q, k, v) != 1:
        raise ValueError("the backward is defined here for multi-head attention only")
    s = default_scale(D) if scale is None else float(scale)
    dq = np.full((B, H, T, D), np.nan, dtype=F64)
    dk = np.full((B, H, T, D), np.nan, dtype=F64)
    dv = np.full((B, H, T, D), np.nan, dtype=F64)
    todo = [(b, h) for b in range(B) for h in range(H)] if heads is None else list(heads)
    for b, h in todo:
        if frozen[h]:
            dq[b, h] = 0.0
            dk[b, h] = 0.0
            dv[b, h] = frozen_head_bwd(do[b, h], a[h], r[h])
        else:
            dq[b, h], dk[b, h], dv[b, h] = ordinary_head_bwd(q[b, h], k[b, h], v[b, h], do[b, h], s)
    return dq, dk, dv
