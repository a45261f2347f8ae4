"""Parity of the calibration statistics with the float64 oracle (GPU
required).

Bars from the arithmetic.  The library forms each score s = q.k in fp32 on
MFMA from the same bf16 inputs (D products: error at most
D u sum_d |q_d k_d|, u = 2^-24), scales it by scale log2 e (one rounding), and
subtracts the row's log-sum-exp, itself a sum of at most T terms in fp32
(relative error (T + 2) u, i.e. (T + 2) u / ln 2 in log2 units).  So every
probability carries a relative error of at most
    rho = ln 2 (2 sl2 D u max|q.k|_1 + 2 u max|x|) + (T + 4) u + 2^-21
(x the log2 probability, 2^-21 for the hardware exp2), and the mean over N
sequences (A0 + s1/N from the shifted sums s1 = sum (A - A0), s2 =
sum (A - A0)^2, A0 the first sequence's value) adds N u.  The mean is
compared entry by entry at rho + N u relative.  s_var sums each entry's
squared deviations s2 - s1^2/N: a relative error rho on every probability
moves it by at most 2 rho sum_n sum |A_n - A-hat| A_n; the fp32 sums add at
most N u s2 (s2), and 2 u (sum |A - A0|)^2 <= 2 N u s2 (s1^2/N), so
3 N u sum_n sum (A_n - A0)^2 in all, plus 4 u sum A_n^2 for the final
subtraction and the fp64 partial sums.  s_KL is sum_n sum A ln A - N sum A-hat ln A-hat: each term
moves by (rho + 64 u) A (|ln A| + 1) at most (64 u for the fp32 sums of a
lane's terms before they join the fp64 partials).
"""

import math

import numpy as np
import pytest
import torch

from oracle import saf_calib_oracle as C
from synth.calib import CALIB_WORKLOADS, calibration_head, calibration_qk
from _helpers import host, say

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from fixed_pattern_hybrid_amd import binding

    return binding


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda().to(torch.bfloat16)


def _rho(q, k, scale, T, D, rows=None):
    """Relative error bound of one probability (module docstring); the
    maximum |q.k|_1 is taken over ``rows`` (all rows by default)."""
    sl2 = scale * math.log2(math.e)
    N = q.shape[0]
    qk1 = max(float((np.abs(q[n] if rows is None else q[n][rows]) @ np.abs(k[n]).T).max()) for n in range(N))
    xmax = 2 * sl2 * qk1 + math.log2(max(T, 1)) + 1
    return math.log(2) * (2 * sl2 * D * U * qk1 + 2 * U * xmax) + (T + 4) * U + 2.0 ** -21


def _sums(q, k, scale, rows):
    """The oracle's statistics of ``rows`` and the terms of the score bars."""
    N = q.shape[0]
    part = C.calibration_rows(q, k, scale, rows)
    As = np.stack([C.attention_rows(q[n], k[n], scale, rows) for n in range(N)])
    Ah = part["ahat"]

    def alnA(X):
        X = X[X > 0]
        return float((X * (np.abs(np.log(X)) + 1)).sum())

    return {"ahat": Ah, "sq": part["sq"], "kl": part["kl"],
            "dev": float((np.abs(As - Ah[None]) * As).sum()), "sq_all": float((As ** 2).sum()),
            "sq_shift": float(((As - As[:1]) ** 2).sum()),
            "ent": sum(alnA(As[n]) for n in range(N)) + N * alnA(Ah)}


def _score_bars(rho, N, T, tot):
    var_bar = 0.0
    if N > 1:
        var_bar = (2 * rho * tot["dev"] + 3 * N * U * tot["sq_shift"] + 4 * U * tot["sq_all"]) / ((N - 1) * T * T)
    kl_bar = (rho + 64 * U) * tot["ent"] / (N * T)
    return var_bar, kl_bar


def _check_head(q, k, scale, ahat_g, s_var_g, s_kl_g, what):
    """q, k: one head's [N, T, D] inputs; compare the library's outputs."""
    N, T, D = q.shape
    tot = _sums(q, k, scale, np.arange(T))
    ref_var = tot["sq"] / ((N - 1) * T * T) if N > 1 else 0.0
    ref_kl = tot["kl"] / (N * T)
    rho = _rho(q, k, scale, T, D)
    causal = np.tril(np.ones((T, T), dtype=bool))
    Ah = tot["ahat"]
    err = np.abs(ahat_g - Ah)[causal]
    bar = ((rho + N * U) * Ah)[causal] + 1e-30
    worst = float(np.max(err / bar))
    var_bar, kl_bar = _score_bars(rho, N, T, tot)
    dv = abs(s_var_g - ref_var)
    dk = abs(s_kl_g - ref_kl)
    say(f"{what}: ahat err/bar {worst:.3f} (rho {rho:.2e}); s_var {ref_var:.4e} err {dv:.2e} (bar {var_bar:.2e}); "
        f"s_kl {ref_kl:.4e} err {dk:.2e} (bar {kl_bar:.2e})")
    assert worst <= 1.0
    assert dv <= var_bar + 1e-300
    assert dk <= kl_bar + 1e-300


@pytest.mark.parametrize("N,H,T,D", [
    (3, 2, 1, 64), (2, 2, 2, 64), (4, 3, 37, 64), (1, 2, 70, 64), (5, 2, 200, 128),
    (3, 2, 300, 96), (6, 1, 129, 64), (2, 2, 513, 128),
])
def test_calib_parity(B, N, H, T, D):
    q, k = calibration_qk(N, H, T, D, seed=900 + T)
    scale = 1 / math.sqrt(D)
    ahat, s_var, s_kl = B.saf_calib_stats(_dev(q), _dev(k))
    torch.cuda.synchronize()
    ahat, s_var, s_kl = host(ahat), s_var.cpu().numpy(), s_kl.cpu().numpy()
    for h in range(H):
        _check_head(q[:, h], k[:, h], scale, ahat[h], s_var[h], s_kl[h], f"N={N} H={H} T={T} D={D} head {h}")
        assert np.all(ahat[h][np.triu_indices(T, 1)] == 0)  # untouched zeros
    if N == 1:
        assert np.all(s_var == 0)


def test_calib_scale_strides_upper_triangle(B):
    """An explicit scale, strided q/k views, a padded ahat whose entries above
    the diagonal must stay untouched, and identical sequences (no spread)."""
    N, H, T, D = 3, 2, 150, 64
    q, k = calibration_qk(N, H, T, D, seed=31)
    qd = _dev(q).permute(1, 0, 2, 3).contiguous().permute(1, 0, 2, 3)  # head-major storage
    kd = _dev(k).permute(1, 0, 2, 3).contiguous().permute(1, 0, 2, 3)
    pad = torch.full((H, T, T + 4), float("nan"), dtype=torch.float32, device="cuda")
    ahat, s_var, s_kl = B.saf_calib_stats(qd, kd, softmax_scale=0.2, ahat=pad)
    torch.cuda.synchronize()
    A = host(pad)
    upper = np.triu(np.ones((T, T + 4), dtype=bool), 1)
    upper[:, T:] = True
    assert np.all(np.isnan(A[:, upper]))
    for h in range(H):
        _check_head(q[:, h], k[:, h], 0.2, A[h, :, :T], float(s_var[h]), float(s_kl[h]), f"strided head {h}")
    # identical sequences: both scores are 0 and the mean is the attention
    qs = np.repeat(q[:1], 4, axis=0)
    ks = np.repeat(k[:1], 4, axis=0)
    ahat, s_var, s_kl = B.saf_calib_stats(_dev(qs), _dev(ks))
    torch.cuda.synchronize()
    assert float(s_var.abs().max()) < 1e-12 and float(s_kl.abs().max()) < 1e-6
    A1 = C.attention_matrix(qs[0, 0], ks[0, 0], 1 / math.sqrt(D))
    assert float(np.max(np.abs(host(ahat)[0] - A1))) < 1e-5


def test_calib_deterministic(B):
    q, k = calibration_qk(4, 2, 260, 64, seed=5)
    x = B.saf_calib_stats(_dev(q), _dev(k))
    y = B.saf_calib_stats(_dev(q), _dev(k))
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(x, y))


def test_calib_workload_sampled(B):
    """The 124M model's calibration (32 sequences of length 4096, a layer's 12
    heads of d = 64) in the launch configuration the benchmark times; the
    mean is checked on sampled rows of every head and both scores in full
    for the lowest-variance head (the oracle sums rows in chunks: the scores
    are sums over rows)."""
    wl = CALIB_WORKLOADS["gpt2_124m_4k"]
    N, H, T, D = wl.N, wl.H, wl.T, wl.D
    scale = 1 / math.sqrt(D)
    say(f"workload {wl.name}: generating inputs")
    q, k = calibration_qk(N, H, T, D, wl.seed)
    ahat, s_var, s_kl = B.saf_calib_stats(_dev(q), _dev(k))
    torch.cuda.synchronize()
    s_var, s_kl = s_var.cpu().numpy(), s_kl.cpu().numpy()
    assert np.all(np.isfinite(s_var)) and np.all(np.isfinite(s_kl)) and np.all(s_var >= 0)
    rows = np.array([0, 1, 63, 64, 127, 128, 2047, 4031, 4094, 4095])
    for h in range(H):
        qh, kh = q[:, h], k[:, h]
        part = C.calibration_rows(qh, kh, scale, rows)
        got = host(ahat[h, rows])
        Ah = part["ahat"]
        mask = np.arange(T)[None, :] <= rows[:, None]
        rel = float(np.max(np.abs(got - Ah)[mask] / np.maximum(Ah[mask], 1e-30)))
        rho = _rho(qh, kh, scale, T, D, rows)
        say(f"workload head {h}: s_var {s_var[h]:.4e} s_kl {s_kl[h]:.4e}; sampled rows of the mean rel {rel:.2e} "
            f"(bar {rho + N * U:.2e})")
        assert rel <= rho + N * U
        assert np.all(host(ahat[h])[np.triu_indices(T, 1)] == 0)
    # full scores of the lowest-variance head (the first candidate for
    # replacement)
    for h in (int(np.argmin(s_var)),):
        qh, kh = q[:, h], k[:, h]
        tot = None
        for r0 in range(0, T, 512):
            part = _sums(qh, kh, scale, np.arange(r0, min(r0 + 512, T)))
            tot = part if tot is None else {x: tot[x] + part[x] for x in ("sq", "kl", "dev", "sq_all", "sq_shift", "ent")}
        ref_var = tot["sq"] / ((N - 1) * T * T)
        ref_kl = tot["kl"] / (N * T)
        var_bar, kl_bar = _score_bars(_rho(qh, kh, scale, T, D), N, T, tot)
        say(f"workload head {h}: s_var {s_var[h]:.6e} vs {ref_var:.6e} (bar {var_bar:.1e}); "
            f"s_kl {s_kl[h]:.6e} vs {ref_kl:.6e} (bar {kl_bar:.1e})")
        assert abs(s_var[h] - ref_var) <= var_bar
        assert abs(s_kl[h] - ref_kl) <= kl_bar


def test_calib_many_heads(B):
    """300 heads (more than a head list holds) of a short sequence."""
    N, H, T, D = 2, 300, 40, 64
    q, k = calibration_qk(N, H, T, D, seed=77)
    ahat, s_var, s_kl = B.saf_calib_stats(_dev(q), _dev(k))
    torch.cuda.synchronize()
    ahat, s_var, s_kl = host(ahat), s_var.cpu().numpy(), s_kl.cpu().numpy()
    for h in (0, 256, H - 1):
        _check_head(q[:, h], k[:, h], 1 / math.sqrt(D), ahat[h], s_var[h], s_kl[h], f"many heads: head {h}")
