"""Parity of compact-pattern fitting with the float64 oracle (GPU required).

Target statistics.  Every entry of P = max(A, floor) / s_i is a product of
positive fp32 values: the row sum s_i over at most T floored entries (at most
T - 1 roundings), its reciprocal and the product (one rounding each); each
marginal then sums at most T such entries.  With u = 2^-24 the standard bound
for sums of positive terms gives a relative error of at most 2 (T + 2) u per
entry of eta_abs and eta_rel.  negent sums each row's p log2 p in fp32 (row
terms all <= 0, so no cancellation between them) and converts with one
subtraction of log2 s_i; the bar is 4 (T + 4) u relative to |negent| plus
2^-20 per row for the absolute error of the hardware log2 near 1.

The fit.  The library runs Adam in fp32 on gradients from fp32 marginals; the
oracle in fp64.  Adam normalises each gradient entry by its own running RMS,
so entries whose gradient is near zero move by rounding-driven amounts of up
to the learning rate; parameters therefore cannot be compared entry by entry
after many steps.  What the fit hands on is the pattern P-hat (installed in a
bf16 layer, whose weights carry relative rounding 2^-9) and kappa (compared
with 0.2).  The bars: P-hat within 2^-10 absolute (half a bf16 ulp at 1), and
kappa and the loss within 1e-4 absolute (the acceptance decision is compared
only where the oracle's kappa is farther than 1e-3 from 0.2).  An fp32
evaluation of the same dense formulas on the CPU stays 100x inside these bars
(kappa within 5e-9, P-hat within 2e-4 at T <= 512).  The library's kappa and
log N are also checked against the oracle's dense evaluation at the library's
own parameters (1e-5 and the frozen-head log N bar).

The first steps are compared entry by entry where the step is well
conditioned.  An Adam step moves an entry by lr * g / (|g| + eps) at the
first step (and a moment-weighted version later); its sensitivity to a
relative error rho of g is lr * rho * eps / (|g| + eps).  Entries whose
oracle gradient stays at or above 100 eps at every step (so the factor is
below 1/100) and whose relative gradient error stays below ~0.05 (fp32
marginals differ by ~1e-6 relative from the oracle's, against |mu - eta| >=
100 eps T) move within steps * lr * 1e-3 of the oracle.  Entries with a
gradient near eps may differ by up to the step itself, so the bar for them
is steps * lr * 2.
"""

import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import saf_fit_oracle as F
from synth.targets import FIT_WORKLOADS, calibration_mean
from _helpers import LSE_FRZ_ABS, host, say

pytestmark = pytest.mark.gpu

U = 2.0 ** -24
PHAT_ABS = 2.0 ** -10
KAPPA_ABS = 1e-4
KAPPA_SELF_ABS = 1e-5


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from fixed_pattern_hybrid_amd import binding

    return binding


def _means(n, T, seed):
    return np.stack([calibration_mean(T, seed, h) for h in range(n)])


def _check_stats(T, ea, er, ne, st, what):
    ea = np.asarray(ea, np.float64)
    er = np.asarray(er, np.float64)
    rel = 2 * (T + 2) * U
    e1 = np.max(np.abs(ea - st["eta_abs"]) / np.maximum(st["eta_abs"], 1e-300))
    e2 = np.max(np.abs(er - st["eta_rel"]) / np.maximum(st["eta_rel"], 1e-300))
    e3 = abs(float(ne) - st["negent"])
    nb = 4 * (T + 4) * U * abs(st["negent"]) + T * 2.0 ** -20
    say(f"{what}: eta_abs rel {e1:.2e} eta_rel rel {e2:.2e} (bar {rel:.2e}) negent abs {e3:.2e} (bar {nb:.2e})")
    assert e1 <= rel and e2 <= rel and e3 <= nb


# ---------------------------------------------------------------------------
# Target statistics.
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("T", [1, 2, 3, 37, 256, 300, 513, 1100])
def test_fit_targets_parity(B, T):
    n = 3
    A = _means(n, T, 100 + T)
    ea, er, ne = B.saf_fit_targets(torch.from_numpy(A).cuda())
    torch.cuda.synchronize()
    ea, er, ne = host(ea), host(er), host(ne)
    for h in range(n):
        _check_stats(T, ea[h], er[h], ne[h], F.fit_statistics(A[h]), f"targets T={T} head {h}")


def test_fit_targets_upper_triangle_strides_and_floor(B):
    """Entries above the diagonal are never read (NaN there changes nothing),
    rows may be padded, and zero entries are floored."""
    T, n = 130, 2
    A = _means(n, T, 5)
    A[1] = np.eye(T, dtype=np.float32)  # all off-diagonal mass from the floor
    ref = [F.fit_statistics(A[h]) for h in range(n)]
    base = B.saf_fit_targets(torch.from_numpy(A).cuda())
    pad = np.full((n, T, T + 12), np.nan, dtype=np.float32)
    pad[:, :, :T] = np.where(np.tril(np.ones((T, T), bool)), A, np.nan)
    dpad = torch.from_numpy(pad).cuda()[:, :, :T]
    got = B.saf_fit_targets(dpad)
    torch.cuda.synchronize()
    for x, y in zip(base, got):
        assert torch.equal(x, y)  # bitwise
    for h in range(n):
        _check_stats(T, host(got[0])[h], host(got[1])[h], host(got[2])[h], ref[h], f"padded head {h}")
    # one head's mean given alone (head stride 0 path)
    one = B.saf_fit_targets(torch.from_numpy(A[0]).cuda())
    torch.cuda.synchronize()
    assert torch.equal(one[0][0], base[0][0]) and torch.equal(one[2][0], base[2][0])


@pytest.mark.parametrize("T", [256, 300, 1024])
def test_fit_targets_vector_and_scalar_reads(B, T):
    """Rows that start 16-byte aligned take the 16-byte-read marginal
    kernels, other layouts the 4-byte ones: a tensor and its copy with rows
    padded to an odd stride both match the oracle."""
    n = 2
    A = _means(n, T, 40 + T)
    aligned = torch.from_numpy(A).cuda()
    pad = np.zeros((n, T, T + 1), dtype=np.float32)
    pad[:, :, :T] = A
    odd = torch.from_numpy(pad).cuda()[:, :, :T]
    got_a = B.saf_fit_targets(aligned)
    got_o = B.saf_fit_targets(odd)
    torch.cuda.synchronize()
    for h in range(n):
        ref = F.fit_statistics(A[h])
        for got, what in ((got_a, "16-byte"), (got_o, "4-byte")):
            _check_stats(T, host(got[0])[h], host(got[1])[h], host(got[2])[h], ref, f"{what} reads T={T} head {h}")


def test_fit_targets_head_stride_off_alignment(B):
    """Rows 16-byte aligned within each head but heads 8 bytes apart from a
    16-byte boundary: the 4-byte-read kernels run, and every head matches
    the oracle and the same means stored contiguously."""
    T, n = 256, 3
    A = _means(n, T, 77)
    flat = torch.zeros(n * (T * T + 2), dtype=torch.float32, device="cuda")
    view = flat.as_strided((n, T, T), (T * T + 2, T, 1))
    view.copy_(torch.from_numpy(A).cuda())
    got = B.saf_fit_targets(view)
    dense = B.saf_fit_targets(torch.from_numpy(A).cuda())
    torch.cuda.synchronize()
    for h in range(n):
        ref = F.fit_statistics(A[h])
        _check_stats(T, host(got[0])[h], host(got[1])[h], host(got[2])[h], ref, f"head stride T*T+2, head {h}")
        _check_stats(T, host(dense[0])[h], host(dense[1])[h], host(dense[2])[h], ref, f"contiguous, head {h}")


def test_fit_targets_deterministic(B):
    A = torch.from_numpy(_means(2, 700, 9)).cuda()
    x = B.saf_fit_targets(A)
    y = B.saf_fit_targets(A)
    torch.cuda.synchronize()
    assert all(torch.equal(p, q) for p, q in zip(x, y))


# ---------------------------------------------------------------------------
# The fit.
# ---------------------------------------------------------------------------


def _fit_inputs(A):
    """Oracle statistics rounded to fp32: the same values feed both sides."""
    sts = [F.fit_statistics(x) for x in A]
    ea = np.stack([s["eta_abs"] for s in sts]).astype(np.float32)
    er = np.stack([s["eta_rel"] for s in sts]).astype(np.float32)
    ne = np.array([s["negent"] for s in sts], dtype=np.float32)
    return ea, er, ne


def _run_fit(B, ea, er, ne, steps):
    out = B.saf_fit_pattern(torch.from_numpy(ea).cuda(), torch.from_numpy(er).cuda(),
                            torch.from_numpy(ne).cuda(), steps=steps)
    torch.cuda.synchronize()
    return {k: (host(v) if v is not None else None) for k, v in out.items()}


def _oracle_fit(ea, er, ne, steps):
    a, r, logz = F.fit_pattern(ea.astype(np.float64), er.astype(np.float64), steps=steps)
    loss = F.fit_loss(ea.astype(np.float64), er.astype(np.float64), a, r)
    return a, r, logz, loss, float(ne) / ea.shape[0] + loss


@pytest.mark.parametrize("T", [1, 2, 5, 64, 300, 513])
def test_fit_init_parity(B, T):
    n = 3
    A = _means(n, T, 200 + T)
    ea, er, ne = _fit_inputs(A)
    g = _run_fit(B, ea, er, ne, 0)
    for h in range(n):
        a, r, logz, loss, kappa = _oracle_fit(ea[h], er[h], ne[h], 0)
        assert np.all(g["a"][h] == 0)
        er_ = np.max(np.abs(g["r"][h] - r) / (1 + np.abs(r)))
        ez = np.max(np.abs(g["logz"][h] - logz))
        say(f"init T={T} head {h}: r {er_:.2e} logz {ez:.2e} loss {abs(g['loss'][h]-loss):.2e} "
            f"kappa {abs(g['kappa'][h]-kappa):.2e}")
        assert er_ <= 8 * U
        assert ez <= LSE_FRZ_ABS
        assert abs(g["loss"][h] - loss) <= KAPPA_SELF_ABS
        assert abs(g["kappa"][h] - kappa) <= KAPPA_SELF_ABS


def _oracle_steps(ea, er, steps):
    """The oracle's first ``steps`` Adam steps, and which entries kept
    |gradient| >= 100 eps at every step (well conditioned)."""
    ea = ea.astype(np.float64)
    er = er.astype(np.float64)
    T = ea.shape[0]
    a, r = F.fit_init(er)
    m = [np.zeros(T) for _ in range(4)]
    ok_a = np.ones(T, bool)
    ok_r = np.ones(T, bool)
    for t in range(1, steps + 1):
        ga, gr = F.fit_gradient(ea, er, a, r)
        ok_a &= np.abs(ga) >= 100 * F.ADAM_EPS
        ok_r &= np.abs(gr) >= 100 * F.ADAM_EPS
        a = F.adam_update(a, ga, m[0], m[1], t, F.FIT_LR)
        r = F.adam_update(r, gr, m[2], m[3], t, F.FIT_LR)
    return a, r, ok_a, ok_r


def _check_steps(g, h, ea, er, steps, what):
    a, r, ok_a, ok_r = _oracle_steps(ea, er, steps)
    tight = steps * F.FIT_LR * 1e-3
    loose = steps * F.FIT_LR * 2
    da = np.abs(g["a"][h] - a)
    dr = np.abs(g["r"][h] - r)
    wa = float(np.max(da[ok_a], initial=0.0))
    wr = float(np.max(dr[ok_r], initial=0.0))
    say(f"{what}: well-conditioned a {wa:.2e} ({ok_a.sum()}/{ok_a.size}) r {wr:.2e} ({ok_r.sum()}/{ok_r.size}) "
        f"(bar {tight:.1e}); all a {da.max():.2e} r {dr.max():.2e} (bar {loose:.1e})")
    assert wa <= tight and wr <= tight
    assert da.max() <= loose and dr.max() <= loose


@pytest.mark.parametrize("steps", [1, 2, 4])
def test_fit_first_steps_entrywise(B, steps):
    T, n = 300, 3
    A = _means(n, T, 300 + steps)
    ea, er, ne = _fit_inputs(A)
    g = _run_fit(B, ea, er, ne, steps)
    for h in range(n):
        _check_steps(g, h, ea[h], er[h], steps, f"first {steps} steps head {h}")
        a, r, logz, loss, kappa = _oracle_fit(ea[h], er[h], ne[h], steps)
        assert abs(g["kappa"][h] - kappa) <= KAPPA_SELF_ABS


def _check_fitted(T, g, h, P, ref, what):
    """Bars on what the fit hands on (see the module docstring)."""
    a, r, logz, loss, kappa = ref
    Pg = oracle.frozen_pattern(g["a"][h].astype(np.float64), g["r"][h].astype(np.float64), T)
    Po = oracle.frozen_pattern(a, r, T)
    dP = float(np.max(np.abs(Pg - Po)))
    dk = abs(float(g["kappa"][h]) - kappa)
    dl = abs(float(g["loss"][h]) - loss)
    # the library's own kappa and log N at its parameters
    k_self = F.fit_kappa_dense(P, g["a"][h].astype(np.float64), g["r"][h].astype(np.float64))
    z_self = oracle.frozen_lognorm(g["a"][h].astype(np.float64), g["r"][h].astype(np.float64), T)
    dks = abs(float(g["kappa"][h]) - k_self)
    dzs = float(np.max(np.abs(g["logz"][h] - z_self)))
    say(f"{what}: kappa {kappa:.5f} |dP| {dP:.2e} |dkappa| {dk:.2e} |dloss| {dl:.2e} "
        f"self: kappa {dks:.2e} logz {dzs:.2e}")
    assert dP <= PHAT_ABS
    assert dk <= KAPPA_ABS and dl <= KAPPA_ABS
    assert dks <= KAPPA_SELF_ABS
    assert dzs <= LSE_FRZ_ABS
    if abs(kappa - F.FIT_TOLERANCE) > 1e-3:
        assert (g["kappa"][h] <= F.FIT_TOLERANCE) == (kappa <= F.FIT_TOLERANCE)


@pytest.mark.parametrize("T", [64, 300, 513])
def test_fit_recipe_parity(B, T):
    n = 4
    A = _means(n, T, 400 + T)
    ea, er, ne = _fit_inputs(A)
    g = _run_fit(B, ea, er, ne, F.FIT_STEPS)
    for h in range(n):
        P = F.fit_target(A[h])
        ref = _oracle_fit(ea[h], er[h], ne[h], F.FIT_STEPS)
        _check_fitted(T, g, h, P, ref, f"recipe T={T} head {h}")


def test_fit_recipe_parity_T1024(B):
    """The whole recipe (J = 400 Adam steps, lr 0.05; Appendix A.2) at
    T = 1024 for two heads, against the oracle's own 400-step fit (about 20 s
    of float64 work per head): the same bars as at the shorter lengths."""
    T, n = 1024, 2
    A = _means(n, T, 1024)
    ea, er, ne = _fit_inputs(A)
    g = _run_fit(B, ea, er, ne, F.FIT_STEPS)
    for h in range(n):
        P = F.fit_target(A[h])
        ref = _oracle_fit(ea[h], er[h], ne[h], F.FIT_STEPS)
        _check_fitted(T, g, h, P, ref, f"recipe T={T} head {h}")


def test_fit_recovers_compact_target(B):
    """A target that is itself a compact pattern is recovered to fp32
    precision (kappa -> 0, Equation 20 at the optimum)."""
    T = 256
    rng = np.random.default_rng(12)
    a_true = rng.standard_normal(T)
    a_true[0] += 4.0
    r_true = -0.05 * np.arange(T) + 0.3 * rng.standard_normal(T)
    P = oracle.frozen_pattern(a_true, r_true, T)
    ea, er = F.marginals(P)
    ne = F.neg_entropy(P)
    g = _run_fit(B, ea[None].astype(np.float32), er[None].astype(np.float32),
                 np.array([ne], np.float32), F.FIT_STEPS)
    Pg = oracle.frozen_pattern(g["a"][0].astype(np.float64), g["r"][0].astype(np.float64), T)
    dP = float(np.max(np.abs(Pg - P)))
    say(f"compact target: kappa {g['kappa'][0]:.2e} |P-hat - P| {dP:.2e}")
    assert abs(g["kappa"][0]) <= KAPPA_SELF_ABS
    assert dP <= 1e-4


def test_fit_degenerate_lengths(B):
    # T = 1: nothing moves, the single weight is 1, kappa = 0
    g = _run_fit(B, np.ones((2, 1), np.float32), np.ones((2, 1), np.float32), np.zeros(2, np.float32), 400)
    assert np.all(g["a"] == 0) and np.all(g["r"] == 0) and np.all(g["logz"] == 0)
    assert np.all(np.abs(g["kappa"]) <= 1e-7)
    # T = 2: one free logit; the fit reproduces row 1 of the target
    P = np.array([[1.0, 0.0], [0.3, 0.7]])
    ea, er = F.marginals(P)
    g = _run_fit(B, ea[None].astype(np.float32), er[None].astype(np.float32),
                 np.array([F.neg_entropy(P)], np.float32), 400)
    q10 = oracle.frozen_pattern(g["a"][0].astype(np.float64), g["r"][0].astype(np.float64), 2)[1, 0]
    assert abs(q10 - 0.3) <= 1e-3


def test_fit_deterministic_and_steps_zero_outputs(B):
    A = _means(2, 200, 77)
    ea, er, ne = _fit_inputs(A)
    x = _run_fit(B, ea, er, ne, 37)
    y = _run_fit(B, ea, er, ne, 37)
    for k in ("a", "r", "logz", "loss", "kappa"):
        assert np.array_equal(x[k], y[k])
    # kappa is optional: without negent the call still fits
    out = B.saf_fit_pattern(torch.from_numpy(ea).cuda(), torch.from_numpy(er).cuda(), None, steps=37)
    torch.cuda.synchronize()
    assert out["kappa"] is None
    assert np.array_equal(host(out["a"]), x["a"]) and np.array_equal(host(out["loss"]), x["loss"])


def test_fit_workload_sampled(B):
    """The 124M, 25% fitting workload (36 heads at T = 4096, the recipe's 400
    steps) in the launch configuration the benchmark times; sampled heads are
    checked against the oracle: target statistics entry by entry, the first
    two steps entry by entry, and at 400 steps the library's kappa and log N
    against the oracle's dense evaluation at its parameters, and the
    gradient's reduction (Equation 20)."""
    wl = FIT_WORKLOADS["gpt2_124m_25pct"]
    n, T = wl.n_heads, wl.T
    say(f"workload {wl.name}: generating {n} calibration means")
    A = np.stack([calibration_mean(T, wl.seed, h) for h in range(n)])
    dA = torch.from_numpy(A).cuda()
    ea, er, ne = B.saf_fit_targets(dA)
    full = B.saf_fit_pattern(ea, er, ne, steps=F.FIT_STEPS)
    two = B.saf_fit_pattern(ea, er, ne, steps=2)
    torch.cuda.synchronize()
    del dA
    g = {k: host(v) for k, v in full.items()}
    g2 = {k: host(v) for k, v in two.items()}
    ea_h, er_h, ne_h = host(ea), host(er), host(ne)
    assert np.all(np.isfinite(g["a"])) and np.all(np.isfinite(g["r"])) and np.all(np.isfinite(g["kappa"]))
    for h in (0, n - 1):
        st = F.fit_statistics(A[h])
        _check_stats(T, ea_h[h], er_h[h], ne_h[h], st, f"workload head {h}")
        # first two steps from the library's own statistics (fp32 inputs to both)
        _check_steps(g2, h, ea_h[h], er_h[h], 2, f"workload head {h} two steps")
        P = F.fit_target(A[h])
        ag = g["a"][h].astype(np.float64)
        rg = g["r"][h].astype(np.float64)
        k_self = F.fit_kappa_dense(P, ag, rg)
        z_self = oracle.frozen_lognorm(ag, rg, T)
        dks = abs(float(g["kappa"][h]) - k_self)
        dzs = float(np.max(np.abs(g["logz"][h] - z_self)))
        ga0, gr0 = F.fit_gradient(st["eta_abs"], st["eta_rel"], *F.fit_init(st["eta_rel"]))
        ga, gr = F.fit_gradient(st["eta_abs"], st["eta_rel"], ag, rg)
        red = math.sqrt((ga ** 2).sum() + (gr ** 2).sum()) / math.sqrt((ga0 ** 2).sum() + (gr0 ** 2).sum())
        say(f"workload head {h}: kappa {g['kappa'][h]:.5f} self kappa {dks:.2e} logz {dzs:.2e} "
            f"gradient norm ratio {red:.2e}")
        assert dks <= KAPPA_SELF_ABS
        assert dzs <= LSE_FRZ_ABS
        assert red < 0.1


def test_fit_many_heads(B):
    """More heads than a head list holds (300): the fit indexes heads by grid
    position; three heads checked over the first steps and at init."""
    n, T = 300, 64
    A = np.stack([calibration_mean(T, 606, h) for h in range(n)])
    ea, er, ne = _fit_inputs(A)
    g = _run_fit(B, ea, er, ne, 3)
    for h in (0, 257, n - 1):
        _check_steps(g, h, ea[h], er[h], 3, f"many heads: head {h}")
