"""Parity of the frozen heads' pattern gradients (trainable-pattern variant)
with the float64 oracle (GPU required).

The HIP path takes O and lse from its own forward (the inputs a caller would
pass); the oracle recomputes everything from v, dO, a and r.  Small shapes
compare every entry; the workload shapes compare the entries that the last 64
rows alone determine (the last keys and the largest offsets) and properties
that hold at any size; one whole head is compared at the 124M layer's length
with a single batch element.

Bars.  The library forms D_b[i] = dO . O from the forward's stored output O,
which carries that forward's rounding: for bf16, the weights rounded to bf16
for the second product and the output rounded to bf16 (for fp32 only the fp32
output rounding).  Taking each rounding error as independent and uniform
within half an ulp, D_b[i] has variance
    sum_j h(W_ij)^2 / 3 * dW_b[i][j]^2  +  sum_d h(O_b[i][d])^2 / 3 * dO_b[i][d]^2
(h = half an ulp; the first sum is absent for fp32), and an entry of da or dr,
a W-weighted sum of D_b over rows, the corresponding weighted variance.  The
test allows 4 standard deviations of that term (its L2 norm over the entries,
from the oracle's W, O and dW; emulating the rounding on the CPU reproduces
the library's errors to three digits, at 0.1 to 1.4 standard deviations) plus
rel-L2 1e-2 of the reference for the remaining arithmetic (bf16; W from the
forward's log N within 1e-4, fp32 products and sums) or 1e-4 (fp32: each term
dG carries ~1e-6 relative error, and the column / diagonal sums cancel: sum of
|terms| over |sum| is 4 to 11 on these shapes).  The pure rounding term is the
whole error when the true gradient is 0, as at T = 1.
"""

import numpy as np
import pytest
import torch

import oracle
from synth import CONFIGS, make_inputs
from _helpers import BF16_GRAD_RELL2, host, rel_l2, say, upload
from _helpers import forward_rounding_sigma as _forward_rounding_sigma
from _helpers import half_ulp as _half_ulp

pytestmark = pytest.mark.gpu

PG_F32_RELL2 = 1e-4


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from fixed_pattern_hybrid_amd import binding

    return binding


def _fwd_then_pgrad(B, inp, dev, strided=False, sentinel=7.0):
    q, k, v, do = dev["q"], dev["k"], dev["v"], dev["do"]
    if strided:
        v = v.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
        do = do.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    fz = [int(x) for x in inp.frozen]
    O, L = B.saf_hybrid_attn_fwd(q, k, v, fz, dev["a"], dev["r"])
    da = torch.full_like(dev["a"], sentinel)
    dr = torch.full_like(dev["r"], sentinel)
    B.saf_pattern_grad(v, O, do, L, fz, dev["a"], dev["r"], da=da, dr=dr)
    torch.cuda.synchronize()
    return host(da), host(dr), fz


def run_pgrad_parity(B, cfg, strided=False):
    say(f"case {cfg.name} B={cfg.B} H={cfg.H} T={cfg.T} D={cfg.D} Tp={cfg.Tp} frozen={cfg.frozen} "
        f"{cfg.dtype} strided={strided}")
    inp = make_inputs(cfg, with_do=True)
    dev = upload(inp)
    da, dr, fz = _fwd_then_pgrad(B, inp, dev, strided)
    ref_a, ref_r = oracle.hybrid_pattern_grad(inp.v, inp.do, fz, inp.a, inp.r)
    bar = BF16_GRAD_RELL2 if cfg.dtype == "bf16" else PG_F32_RELL2
    T = cfg.T
    for h in range(cfg.H):
        if not fz[h]:
            # ordinary heads' rows are not written
            assert np.all(da[h] == 7.0) and np.all(dr[h] == 7.0), h
            continue
        sa, sr = _forward_rounding_sigma(cfg, inp, h)
        for n, got, ref, sig in (("da", da[h, :T], ref_a[h], sa), ("dr", dr[h, :T], ref_r[h], sr)):
            err = float(np.linalg.norm(got.astype(np.float64) - ref))
            lim = bar * float(np.linalg.norm(ref)) + 4.0 * sig
            say(f"  h{h}: {n} rel-L2 {rel_l2(got, ref):.3e} (L2 error {err:.3e} = {err / max(sig, 1e-30):.2f} "
                f"rounding sd, allowed {lim:.3e})")
            assert err <= lim, (h, n, err, lim)
        assert np.all(da[h, T:] == 0.0) and np.all(dr[h, T:] == 0.0)  # beyond T
        assert np.all(np.isfinite(da[h])) and np.all(np.isfinite(dr[h]))


SMALL = [
    CONFIGS["tiny"],
    CONFIGS["pages_check_t129"],
    CONFIGS["pages_check_t129"].with_(dtype="f32", name="pages-check_fp32"),
    CONFIGS["pages_check_t129"].with_(frozen=(0, 1, 2, 3), B=3, name="pages-check_all-frozen_B3"),
]


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: c.name)
def test_pgrad_small_cases(B, cfg):
    run_pgrad_parity(B, cfg)


@pytest.mark.parametrize("T", [1, 2, 17, 64, 65, 127, 128, 129, 200, 257, 400])
def test_pgrad_ragged_lengths(B, T):
    cfg = CONFIGS["pages_check_t129"].with_(T=T, prior_len=T + 5, B=3, H=3, frozen=(1, 2), name=f"pg_T{T}")
    run_pgrad_parity(B, cfg)


@pytest.mark.parametrize("D", [64, 96, 128])
def test_pgrad_head_dims(B, D):
    cfg = CONFIGS["pages_check_t129"].with_(D=D, T=300, H=4, B=5, frozen=(0, 3), qkv_scale=0.5,
                                            prior_len=None, name=f"pg_D{D}")
    run_pgrad_parity(B, cfg)


@pytest.mark.parametrize("D", [16, 64, 128])
def test_pgrad_fp32(B, D):
    cfg = CONFIGS["tiny"].with_(D=D, T=70, B=2, H=3, frozen=(0, 2), name=f"pg_fp32_D{D}")
    run_pgrad_parity(B, cfg)


def test_pgrad_strided_and_deterministic(B):
    cfg = CONFIGS["pages_check_t129"].with_(B=4, T=333, prior_len=None, name="pg_strided")
    run_pgrad_parity(B, cfg, strided=True)
    inp = make_inputs(cfg, with_do=True)
    dev = upload(inp)
    r1 = _fwd_then_pgrad(B, inp, dev)
    r2 = _fwd_then_pgrad(B, inp, dev)
    assert np.array_equal(r1[0], r2[0]) and np.array_equal(r1[1], r2[1]), "must be bitwise reproducible"


def test_pgrad_no_frozen_head_is_a_no_op(B):
    cfg = CONFIGS["pages_check_t129"].with_(frozen=(), name="pg_none")
    inp = make_inputs(cfg, with_do=True)
    dev = upload(inp)
    da, dr, fz = _fwd_then_pgrad(B, inp, dev)
    assert np.all(da == 7.0) and np.all(dr == 7.0)


def test_pgrad_workload_one_batch_element_full_head(B):
    # The 124M layer's shape (T = 4096, d = 64, heads 9-11 frozen) with one
    # batch element, so that the oracle computes a whole head: every entry of
    # da and dr of head 9.
    cfg = CONFIGS["gpt2_124m_4k_25pct"].with_(B=1, name="gpt2-124m-layer_B1")
    say(f"workload {cfg.name}")
    inp = make_inputs(cfg, with_do=True)
    dev = upload(inp)
    da, dr, fz = _fwd_then_pgrad(B, inp, dev)
    h = 9
    ref_a, ref_r = oracle.frozen_head_pattern_grad(inp.v[0, h], inp.do[0, h], inp.a[h], inp.r[h])
    sa, sr = _forward_rounding_sigma(cfg, inp, h)
    T = cfg.T
    for n, got, ref, sig in (("da", da[h, :T], ref_a, sa), ("dr", dr[h, :T], ref_r, sr)):
        err = float(np.linalg.norm(got.astype(np.float64) - ref))
        lim = BF16_GRAD_RELL2 * float(np.linalg.norm(ref)) + 4.0 * sig
        say(f"  h{h}: {n} rel-L2 {rel_l2(got, ref):.3e} (L2 error {err:.3e} = {err / max(sig, 1e-30):.2f} "
            f"rounding sd, allowed {lim:.3e})")
        assert err <= lim, (n, err, lim)


@pytest.mark.parametrize("key", ["gpt2_124m_4k_25pct", "1b_8k_rank_share"])
def test_pgrad_workload_tail_entries(B, key):
    # Keys j >= T - 64 meet only rows [T - 64, T): compare their da entries
    # for every frozen head (summed over the batch; the matching dr entries,
    # offsets >= T - 64, are ~e^-200 here and carry no information).  Both
    # gradients sum to sum_b sum_i (D_b[i] - stored D_b[i]) (each row of W sums
    # to 1), i.e. to 0 up to the forward's rounding inside D, whose variance is
    # at most sum_d dO_id^2 (h(max_j |V_jd|)^2 + (2^-9 max_j |V_jd|)^2) / 3 per
    # row (|O_id| <= max_j |V_jd|, sum_j W_ij^2 <= 1): allow 4 standard
    # deviations plus fp32 summation (1e-6 of the absolute sum).
    cfg = CONFIGS[key]
    say(f"workload {cfg.name}")
    inp = make_inputs(cfg, with_do=True)
    dev = upload(inp)
    da, dr, fz = _fwd_then_pgrad(B, inp, dev)
    T = cfg.T
    rows = np.arange(T - 64, T)
    for h in range(cfg.H):
        if not fz[h]:
            continue
        ta = np.zeros(T)
        for b in range(cfg.B):
            ta += oracle.frozen_rows_pattern_grad(inp.v[b, h], inp.do[b, h], inp.a[h], inp.r[h], rows)[0]
        ea = rel_l2(da[h, T - 64:T], ta[T - 64:])
        var = 0.0
        for b in range(cfg.B):
            vmax = np.abs(np.asarray(inp.v[b, h], np.float64)).max(axis=0)
            do2 = (np.asarray(inp.do[b, h], np.float64) ** 2).sum(axis=0)
            var += float((do2 * (_half_ulp(vmax, 8) ** 2 + (2.0 ** -9 * vmax) ** 2) / 3).sum())
        sum_a, sum_r = float(da[h, :T].astype(np.float64).sum()), float(dr[h, :T].astype(np.float64).sum())
        lim_a = 4.0 * np.sqrt(var) + 1e-6 * float(np.abs(da[h, :T]).sum())
        lim_r = 4.0 * np.sqrt(var) + 1e-6 * float(np.abs(dr[h, :T]).sum())
        say(f"  h{h}: tail da rel-L2 {ea:.3e}; sums da {sum_a:.3e} dr {sum_r:.3e} (allowed {lim_a:.3e}, "
            f"{lim_r:.3e}; absolute sums {np.abs(da[h, :T]).sum():.3e}, {np.abs(dr[h, :T]).sum():.3e})")
        assert ea <= BF16_GRAD_RELL2, (h, ea)
        assert abs(sum_a) <= lim_a and abs(sum_r) <= lim_r, (h, sum_a, sum_r, lim_a, lim_r)
        assert np.all(np.isfinite(da[h])) and np.all(np.isfinite(dr[h]))
