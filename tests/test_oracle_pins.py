"""Pins of the float64 oracle against what the pages and mathematics fix.

Each test compares the oracle with something other than itself: hand-worked
examples stored under tests/golden, closed forms derived from Equation 3,
library routines (torch's scaled_dot_product_attention and autograd on the CPU
in float64, scipy's logsumexp), invariants the equations imply, and central
finite differences.  None of these re-types the oracle's own code.
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
rng0 = np.random.default_rng(20260101)


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# --------------------------------------------------------------------------
# Hand-worked examples (tests/golden)
# --------------------------------------------------------------------------


def test_frozen_worked_example_T3():
    g = _load("frozen_pattern_worked_T3.json")
    a = np.log(np.array(g["exp_a"], dtype=np.float64))
    r = np.log(np.array(g["exp_r"], dtype=np.float64))
    num = g["P_numerators"]
    # exact rationals from the fixture
    P_exact = np.array([[float(Fraction(num[i][j], g["N"][i])) for j in range(3)] for i in range(3)])
    P = oracle.frozen_pattern(a, r, 3)
    np.testing.assert_allclose(P, P_exact, rtol=0, atol=1e-15)
    np.testing.assert_allclose(oracle.frozen_lognorm(a, r, 3), np.log(g["N"]), rtol=0, atol=1e-15)
    O, L = oracle.frozen_head_fwd(np.array(g["V"]), a, r)
    np.testing.assert_allclose(O, np.array(g["O"]), rtol=1e-14, atol=0)
    np.testing.assert_allclose(L, np.log(g["N"]), atol=1e-15)


def test_ordinary_worked_example_T3():
    g = _load("ordinary_attention_worked_T3.json")
    q = np.array(g["Q"])
    k = np.log(np.array(g["exp_K"], dtype=np.float64))[:, None]
    v = np.array(g["V"])
    O, L = oracle.ordinary_head_fwd(q, k, v, scale=1.0)
    np.testing.assert_allclose(O, np.array(g["O"]), rtol=1e-14)
    np.testing.assert_allclose(L, np.log(g["row_sums"]), atol=1e-15)


def test_pages_check_fixture_matches_config():
    from synth import CONFIGS

    g = _load("pages_mixed_head_check.json")["shape"]
    c = CONFIGS["pages_check_t129"]
    assert (c.B, c.T, c.H, c.D, c.Tp) == (g["B"], g["T"], g["H"], g["D"], g["prior_len"])
    assert list(c.frozen) == g["frozen_heads_zero_based"]


# --------------------------------------------------------------------------
# Invariants of Equation 3
# --------------------------------------------------------------------------


@pytest.mark.parametrize("T", [1, 2, 17, 64, 129])
def test_frozen_rows_causal_stochastic(T):
    a = rng0.standard_normal(T)
    r = -0.05 * np.arange(T) + 0.5 * rng0.standard_normal(T)
    P = oracle.frozen_pattern(a, r, T)
    assert P.shape == (T, T)
    assert np.all(P >= 0)
    assert np.all(np.triu(P, 1) == 0.0)
    np.testing.assert_allclose(P.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    assert P[0, 0] == 1.0


def test_gauge_invariance():
    T = 200
    a = rng0.standard_normal(T)
    r = -0.05 * np.arange(T) + 0.5 * rng0.standard_normal(T)
    P = oracle.frozen_pattern(a, r, T)
    P1 = oracle.frozen_pattern(a + 3.7, r - 1.25, T)
    lam = 0.3
    P2 = oracle.frozen_pattern(a + lam * np.arange(T), r + lam * np.arange(T), T)
    np.testing.assert_allclose(P1, P, rtol=0, atol=1e-14)
    np.testing.assert_allclose(P2, P, rtol=0, atol=1e-13)


def test_gauge_shift_of_lognorm_long():
    # (a + lam*j, r + lam*d) adds lam*i to every logit of row i, so
    # log N shifts by exactly lam*i; the weights are unchanged.
    # T = 8192 with lam = 0.04 spans the same ~330 nats as the 32K prefill's
    # peaked r (slope 0.01) does.
    T = 8192
    rng = np.random.default_rng(5)
    a = rng.standard_normal(T)
    r = np.where(np.arange(T) < 8, 3.0, -0.04 * np.arange(T))
    lam = 0.04
    L = oracle.frozen_lognorm(a, r, T)
    L2 = oracle.frozen_lognorm(a + lam * np.arange(T), r + lam * np.arange(T), T)
    np.testing.assert_allclose(L2 - L, lam * np.arange(T), rtol=0, atol=1e-9)
    assert np.all(np.isfinite(L))


# --------------------------------------------------------------------------
# Closed forms derived from Equation 3
# --------------------------------------------------------------------------


def test_closed_form_uniform_prefix_mean():
    T, D = 50, 3
    v = rng0.standard_normal((T, D))
    O, L = oracle.frozen_head_fwd(v, np.zeros(T), np.zeros(T))
    expect = np.cumsum(v, axis=0) / np.arange(1, T + 1)[:, None]
    np.testing.assert_allclose(O, expect, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(L, np.log(np.arange(1, T + 1)), atol=1e-13)


@pytest.mark.parametrize("lam,T", [(0.05, 300), (0.01, 8192), (1.7, 40)])
def test_closed_form_geometric_normaliser(lam, T):
    # a = 0, r[d] = -lam*d: N(i) = sum_{d=0..i} exp(-lam d) = (1 - e^{-lam(i+1)}) / (1 - e^{-lam})
    i = np.arange(T)
    L = oracle.frozen_lognorm(np.zeros(T), -lam * np.arange(T), T)
    expect = np.log(-np.expm1(-lam * (i + 1))) - np.log(-np.expm1(-lam))
    np.testing.assert_allclose(L, expect, rtol=0, atol=1e-11)


def test_closed_form_identity_and_window():
    T, D = 40, 5
    v = rng0.standard_normal((T, D))
    a = rng0.standard_normal(T)
    r = np.full(T, -np.inf)
    r[0] = 0.0
    O, L = oracle.frozen_head_fwd(v, a, r)
    np.testing.assert_allclose(O, v, rtol=0, atol=1e-15)
    np.testing.assert_allclose(L, a, atol=1e-15)
    w = 4
    r = np.where(np.arange(T) < w, 0.0, -np.inf)
    O, _ = oracle.frozen_head_fwd(v, np.zeros(T), r)
    for t in range(T):
        lo = max(0, t - w + 1)
        np.testing.assert_allclose(O[t], v[lo : t + 1].mean(axis=0), rtol=1e-13, atol=1e-14)


def test_row0_equals_v0_both_kinds():
    B, H, T, D = 2, 3, 9, 4
    q, k, v = (rng0.standard_normal((B, H, T, D)) for _ in range(3))
    a, r = rng0.standard_normal((H, T)), rng0.standard_normal((H, T))
    O, _ = oracle.hybrid_fwd(q, k, v, [0, 1, 0], a, r)
    np.testing.assert_allclose(O[:, :, 0], v[:, :, 0], rtol=0, atol=1e-15)


# --------------------------------------------------------------------------
# Library routines: torch SDPA / autograd (float64, CPU) and scipy
# --------------------------------------------------------------------------


def _sdpa(q, k, v, scale, mask=None, causal=False):
    return torch.nn.functional.scaled_dot_product_attention(
        q, k, v, attn_mask=mask, is_causal=causal, scale=scale
    )


def test_frozen_equals_softmax_of_bias_via_sdpa():
    # A frozen head is causal softmax attention whose logits are the additive
    # positional bias of Equation 3 and whose query-key term is zero.
    T, D = 33, 8
    a = rng0.standard_normal(T)
    r = -0.05 * np.arange(T) + 0.5 * rng0.standard_normal(T)
    v = rng0.standard_normal((T, D))
    i = np.arange(T)[:, None]
    j = np.arange(T)[None, :]
    bias = np.where(j <= i, a[j] + r[np.clip(i - j, 0, None)], -np.inf)
    out = _sdpa(
        torch.zeros(1, 1, T, D, dtype=torch.float64),
        torch.from_numpy(rng0.standard_normal((1, 1, T, D))),
        torch.from_numpy(v)[None, None],
        1.0,
        mask=torch.from_numpy(bias)[None, None],
    )[0, 0].numpy()
    O, _ = oracle.frozen_head_fwd(v, a, r)
    np.testing.assert_allclose(O, out, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("T,D", [(1, 4), (37, 16), (130, 64)])
def test_ordinary_fwd_bwd_equals_sdpa_autograd(T, D):
    q, k, v, do = (rng0.standard_normal((T, D)) for _ in range(4))
    s = 1.0 / math.sqrt(D)
    tq, tk, tv = (torch.tensor(x[None, None], requires_grad=True) for x in (q, k, v))
    out = _sdpa(tq, tk, tv, s, causal=True)
    out.backward(torch.from_numpy(do)[None, None])
    O, L = oracle.ordinary_head_fwd(q, k, v, s)
    np.testing.assert_allclose(O, out[0, 0].detach().numpy(), rtol=1e-11, atol=1e-12)
    S = s * q @ k.T
    S[np.triu_indices(T, 1)] = -np.inf
    np.testing.assert_allclose(L, logsumexp(S, axis=1), rtol=0, atol=1e-12)
    dq, dk, dv = oracle.ordinary_head_bwd(q, k, v, do, s)
    np.testing.assert_allclose(dq, tq.grad[0, 0].numpy(), rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(dk, tk.grad[0, 0].numpy(), rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(dv, tv.grad[0, 0].numpy(), rtol=1e-10, atol=1e-11)


def test_frozen_dv_equals_sdpa_autograd():
    T, D = 45, 6
    a = rng0.standard_normal(T)
    r = -0.05 * np.arange(T) + 0.5 * rng0.standard_normal(T)
    v, do = rng0.standard_normal((T, D)), rng0.standard_normal((T, D))
    i = np.arange(T)[:, None]
    j = np.arange(T)[None, :]
    bias = np.where(j <= i, a[j] + r[np.clip(i - j, 0, None)], -np.inf)
    tv = torch.tensor(v[None, None], requires_grad=True)
    out = _sdpa(torch.zeros(1, 1, T, D, dtype=torch.float64), torch.zeros(1, 1, T, D, dtype=torch.float64),
                tv, 1.0, mask=torch.from_numpy(bias)[None, None])
    out.backward(torch.from_numpy(do)[None, None])
    np.testing.assert_allclose(oracle.frozen_head_bwd(do, a, r), tv.grad[0, 0].numpy(), rtol=1e-11, atol=1e-12)


# --------------------------------------------------------------------------
# Frozen heads: no Q/K gradient, Q/K never read
# --------------------------------------------------------------------------


def test_frozen_qk_untouched_and_zero_grad():
    B, H, T, D = 2, 4, 21, 8
    q, k, v, do = (rng0.standard_normal((B, H, T, D)) for _ in range(4))
    frozen = [0, 1, 0, 1]
    a, r = rng0.standard_normal((H, 24)), rng0.standard_normal((H, 24))
    qn, kn = q.copy(), k.copy()
    qn[:, [1, 3]] = np.nan
    kn[:, [1, 3]] = np.nan
    O1, L1 = oracle.hybrid_fwd(q, k, v, frozen, a, r)
    O2, L2 = oracle.hybrid_fwd(qn, kn, v, frozen, a, r)
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)
    g1 = oracle.hybrid_bwd(q, k, v, do, frozen, a, r)
    g2 = oracle.hybrid_bwd(qn, kn, v, do, frozen, a, r)
    for x, y in zip(g1, g2):
        assert np.array_equal(x, y)
    dq, dk, dv = g1
    assert np.all(dq[:, [1, 3]] == 0.0) and np.all(dk[:, [1, 3]] == 0.0)
    assert np.all(dq[:, [0, 2], 1:] != 0.0)  # row 0 has one key: its dQ is 0
    for b in range(B):
        for h in (1, 3):
            np.testing.assert_array_equal(L1[b, h], L1[0, h])  # batch-independent log N


# --------------------------------------------------------------------------
# Brute-force central finite differences
# --------------------------------------------------------------------------


def test_finite_differences_tiny():
    B, H, T, D = 1, 2, 7, 4
    rng = np.random.default_rng(77)
    q, k, v, do = (rng.standard_normal((B, H, T, D)) for _ in range(4))
    frozen = [0, 1]
    a, r = rng.standard_normal((H, T)), rng.standard_normal((H, T))
    s = 0.7

    def loss(qq, kk, vv):
        O, _ = oracle.hybrid_fwd(qq, kk, vv, frozen, a, r, scale=s)
        return float((O * do).sum())

    dq, dk, dv = oracle.hybrid_bwd(q, k, v, do, frozen, a, r, scale=s)
    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp = x.copy()
            xm = x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = {"q": q, "k": k, "v": v}
            args_m = dict(args_p)
            args_p[name] = xp
            args_m[name] = xm
            fd[idx] = (loss(args_p["q"], args_p["k"], args_p["v"]) - loss(args_m["q"], args_m["k"], args_m["v"])) / (2 * h)
        err = np.linalg.norm(fd - g) / max(np.linalg.norm(g), 1e-8)
        assert err <= 1e-7, (name, err)
        if name in ("q", "k"):
            assert np.all(g[:, 1] == 0.0)
            assert np.all(fd[:, 1] == 0.0)


# --------------------------------------------------------------------------
# Causality and stored prior length
# --------------------------------------------------------------------------


def test_prefix_truncation_and_prior_length():
    B, H, T, D, Tp = 1, 2, 50, 8, 80
    rng = np.random.default_rng(3)
    q, k, v = (rng.standard_normal((B, H, T, D)) for _ in range(3))
    a, r = rng.standard_normal((H, Tp)), rng.standard_normal((H, Tp))
    frozen = [1, 0]
    O, L = oracle.hybrid_fwd(q, k, v, frozen, a, r)
    Tc = 23
    Oc, Lc = oracle.hybrid_fwd(q[:, :, :Tc], k[:, :, :Tc], v[:, :, :Tc], frozen, a[:, :Tc], r[:, :Tc])
    np.testing.assert_allclose(Oc, O[:, :, :Tc], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(Lc, L[:, :, :Tc], rtol=0, atol=1e-13)
    O2, L2 = oracle.hybrid_fwd(q, k, v, frozen, a[:, :T], r[:, :T])
    assert np.array_equal(O, O2) and np.array_equal(L, L2)
    with pytest.raises(ValueError):
        oracle.frozen_lognorm(a[0, :10], r[0, :10], 11)


def test_rows_subset_matches_full():
    T, D = 300, 16
    rng = np.random.default_rng(9)
    q, k, v = (rng.standard_normal((T, D)) for _ in range(3))
    a, r = rng.standard_normal(T), rng.standard_normal(T)
    rows = np.array([0, 1, 77, 255, 299])
    O, L = oracle.ordinary_head_fwd(q, k, v, 0.25)
    Or, Lr = oracle.ordinary_rows_fwd(q, k, v, 0.25, rows)
    np.testing.assert_allclose(Or, O[rows], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(Lr, L[rows], atol=1e-13)
    O, L = oracle.frozen_head_fwd(v, a, r)
    Or, Lr = oracle.frozen_rows_fwd(v, a, r, rows)
    np.testing.assert_allclose(Or, O[rows], rtol=1e-13, atol=1e-14)


def test_chunking_does_not_change_result(monkeypatch):
    from oracle import saf_oracle

    T, D = 96, 8
    rng = np.random.default_rng(11)
    q, k, v, do = (rng.standard_normal((T, D)) for _ in range(4))
    a, r = rng.standard_normal(T), rng.standard_normal(T)
    ref = (saf_oracle.ordinary_head_fwd(q, k, v, 0.3), saf_oracle.ordinary_head_bwd(q, k, v, do, 0.3),
           saf_oracle.frozen_head_fwd(v, a, r), saf_oracle.frozen_head_bwd(do, a, r))
    monkeypatch.setattr(saf_oracle, "_CHUNK_ELEMS", 7 * T)  # 7-row chunks, ragged tail
    got = (saf_oracle.ordinary_head_fwd(q, k, v, 0.3), saf_oracle.ordinary_head_bwd(q, k, v, do, 0.3),
           saf_oracle.frozen_head_fwd(v, a, r), saf_oracle.frozen_head_bwd(do, a, r))
    for x, y in zip(ref, got):
        for xx, yy in zip(x if isinstance(x, tuple) else (x,), y if isinstance(y, tuple) else (y,)):
            np.testing.assert_allclose(yy, xx, rtol=1e-13, atol=1e-13)


# --------------------------------------------------------------------------
# Trainable-pattern gradients (da, dr of frozen heads)
# --------------------------------------------------------------------------


def test_pattern_grad_finite_differences():
    # L = sum_b <dO_b, O_b(a, r)> differentiated by central differences of the
    # (separately pinned) forward, entry by entry, batch summed.
    B, T, D = 2, 9, 5
    rng = np.random.default_rng(101)
    v, do = rng.standard_normal((B, 1, T, D)), rng.standard_normal((B, 1, T, D))
    a, r = rng.standard_normal((1, T)), rng.standard_normal((1, T))

    def loss(aa, rr):
        O, _ = oracle.hybrid_fwd(v, v, v, [1], aa, rr)
        return float((O * do).sum())

    dA, dR = oracle.hybrid_pattern_grad(v, do, [1], a, r)
    h = 1e-6
    for x, g in ((a, dA), (r, dR)):
        fd = np.zeros(T)
        for j in range(T):
            xp, xm = x.copy(), x.copy()
            xp[0, j] += h
            xm[0, j] -= h
            lp = loss(xp, r) if x is a else loss(a, xp)
            lm = loss(xm, r) if x is a else loss(a, xm)
            fd[j] = (lp - lm) / (2 * h)
        assert np.linalg.norm(fd - g[0]) <= 1e-7 * np.linalg.norm(fd), (fd, g[0])


def test_pattern_grad_equals_autograd_of_bias():
    # A frozen head is softmax attention with logits a[j] + r[i-j]; torch
    # autograd (float64, CPU) through sdpa with that additive mask gives the
    # gradient of the mask, whose column and diagonal sums are da and dr.
    T, D = 40, 6
    rng = np.random.default_rng(102)
    a = rng.standard_normal(T)
    r = -0.05 * np.arange(T) + 0.5 * rng.standard_normal(T)
    v, do = rng.standard_normal((T, D)), rng.standard_normal((T, D))
    ta = torch.tensor(a, requires_grad=True)
    tr = torch.tensor(r, requires_grad=True)
    i = torch.arange(T)[:, None]
    j = torch.arange(T)[None, :]
    causal = j <= i
    bias = torch.where(causal, ta[j.expand(T, T)] + tr[(i - j).clamp(min=0)], torch.tensor(-math.inf, dtype=torch.float64))
    out = _sdpa(torch.zeros(1, 1, T, D, dtype=torch.float64), torch.zeros(1, 1, T, D, dtype=torch.float64),
                torch.from_numpy(v)[None, None], 1.0, mask=bias[None, None])
    out.backward(torch.from_numpy(do)[None, None])
    da, dr = oracle.frozen_head_pattern_grad(v, do, a, r)
    np.testing.assert_allclose(da, ta.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dr, tr.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_pattern_grad_closed_form_T2():
    # T = 2: row 0 has weight 1 (no gradient); row 1 has weights w, 1 - w with
    # w = sigmoid((a0 + r1) - (a1 + r0)).  With g_j = dO_1 . V_j:
    # dG_10 = w (1 - w)(g0 - g1) = -dG_11, so da = [c, -c] and dr = [-c, c].
    a = np.array([0.3, -1.1])
    r = np.array([0.7, 0.2])
    v = np.array([[1.0, 2.0], [-0.5, 0.25]])
    do = np.array([[3.0, -1.0], [0.5, 1.5]])
    w = 1.0 / (1.0 + math.exp(-((a[0] + r[1]) - (a[1] + r[0]))))
    g0, g1 = do[1] @ v[0], do[1] @ v[1]
    c = w * (1 - w) * (g0 - g1)
    da, dr = oracle.frozen_head_pattern_grad(v, do, a, r)
    np.testing.assert_allclose(da, [c, -c], rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(dr, [-c, c], rtol=1e-14, atol=1e-15)


def test_pattern_grad_invariants():
    # Adding a constant to every a (or every r) leaves each row softmax
    # unchanged, so both gradients sum to zero; the last key only meets the
    # last row and the largest offset only the corner entry (i, j) = (T-1, 0).
    T, D = 64, 8
    rng = np.random.default_rng(103)
    v, do = rng.standard_normal((T, D)), rng.standard_normal((T, D))
    a, r = rng.standard_normal(T), rng.standard_normal(T)
    da, dr = oracle.frozen_head_pattern_grad(v, do, a, r)
    scale = np.abs(da).sum() + np.abs(dr).sum()
    assert abs(da.sum()) <= 1e-13 * scale and abs(dr.sum()) <= 1e-13 * scale
    P = oracle.frozen_pattern(a, r, T)
    O = P @ v
    dW = do @ v.T
    Dl = (do * O).sum(axis=1)  # sum_j W dW = dO . O
    np.testing.assert_allclose(da[T - 1], P[T - 1, T - 1] * (dW[T - 1, T - 1] - Dl[T - 1]), rtol=1e-12)
    np.testing.assert_allclose(dr[T - 1], P[T - 1, 0] * (dW[T - 1, 0] - Dl[T - 1]), rtol=1e-12)
    # ordinary heads get no pattern gradient (NaN rows), batch sums add up
    vb, dob = rng.standard_normal((3, 2, T, D)), rng.standard_normal((3, 2, T, D))
    ab, rb = rng.standard_normal((2, T + 5)), rng.standard_normal((2, T + 5))
    dA, dR = oracle.hybrid_pattern_grad(vb, dob, [0, 1], ab, rb)
    assert np.all(np.isnan(dA[0])) and np.all(np.isnan(dR[0]))
    sa = sum(oracle.frozen_head_pattern_grad(vb[b, 1], dob[b, 1], ab[1], rb[1])[0] for b in range(3))
    np.testing.assert_allclose(dA[1], sa, rtol=1e-13, atol=1e-14)


def test_pattern_grad_chunking(monkeypatch):
    from oracle import saf_oracle

    T, D = 70, 4
    rng = np.random.default_rng(104)
    v, do = rng.standard_normal((T, D)), rng.standard_normal((T, D))
    a, r = rng.standard_normal(T), rng.standard_normal(T)
    ref = saf_oracle.frozen_head_pattern_grad(v, do, a, r)
    monkeypatch.setattr(saf_oracle, "_CHUNK_ELEMS", 9 * T)
    got = saf_oracle.frozen_head_pattern_grad(v, do, a, r)
    for x, y in zip(ref, got):
        np.testing.assert_allclose(y, x, rtol=1e-13, atol=1e-14)


def test_pattern_grad_tail_rows_give_tail_entries():
    # Key j and offset d are only met by rows i >= j (resp. i >= d): the rows
    # [T0, T) alone give the full entries j, d >= T0.
    T, D, T0 = 90, 4, 71
    rng = np.random.default_rng(105)
    v, do = rng.standard_normal((T, D)), rng.standard_normal((T, D))
    a, r = rng.standard_normal(T), rng.standard_normal(T)
    da, dr = oracle.frozen_head_pattern_grad(v, do, a, r)
    ta, tr_ = oracle.frozen_rows_pattern_grad(v, do, a, r, np.arange(T0, T))
    np.testing.assert_allclose(ta[T0:], da[T0:], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(tr_[T0:], dr[T0:], rtol=1e-12, atol=1e-14)


# --------------------------------------------------------------------------
# Grouped-query attention (key/value heads shared by groups of query heads)
# --------------------------------------------------------------------------


def test_gqa_equals_multi_head_with_repeated_kv():
    B, H, Hk, T, D = 2, 8, 2, 37, 8
    rng = np.random.default_rng(201)
    q = rng.standard_normal((B, H, T, D))
    k, v = rng.standard_normal((B, Hk, T, D)), rng.standard_normal((B, Hk, T, D))
    a, r = rng.standard_normal((H, T)), rng.standard_normal((H, T))
    frozen = [0, 1, 0, 0, 1, 1, 1, 1]  # group 1 fully frozen, group 0 mixed
    O, L = oracle.hybrid_fwd(q, k, v, frozen, a, r)
    Or, Lr = oracle.hybrid_fwd(q, np.repeat(k, H // Hk, axis=1), np.repeat(v, H // Hk, axis=1), frozen, a, r)
    np.testing.assert_array_equal(O, Or)
    np.testing.assert_array_equal(L, Lr)
    with pytest.raises(ValueError):
        oracle.hybrid_fwd(q, k[:, :1], v, frozen, a, r)
    with pytest.raises(ValueError):
        oracle.hybrid_fwd(q, rng.standard_normal((B, 3, T, D)), rng.standard_normal((B, 3, T, D)), frozen, a, r)
    with pytest.raises(ValueError):
        oracle.hybrid_bwd(q, k, v, q, frozen, a, r)


def test_gqa_ordinary_equals_sdpa_enable_gqa():
    B, H, Hk, T, D = 1, 6, 3, 45, 16
    rng = np.random.default_rng(202)
    q = rng.standard_normal((B, H, T, D))
    k, v = rng.standard_normal((B, Hk, T, D)), rng.standard_normal((B, Hk, T, D))
    a, r = rng.standard_normal((H, T)), rng.standard_normal((H, T))
    O, _ = oracle.hybrid_fwd(q, k, v, [0] * H, a, r)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), is_causal=True, enable_gqa=True
    ).numpy()
    np.testing.assert_allclose(O, ref, rtol=1e-11, atol=1e-12)
