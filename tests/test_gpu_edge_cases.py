"""Edge cases of the compact pattern (Section 3.2, Equation 3) through the
whole layer: forward, backward and the pattern gradients, bf16 and fp32
(GPU required).

Equation 3 allows -inf preferences: a key or an offset that never receives
weight.  The cases below put them where the kernels' tiling, factored weights
and band-sum normalisers could mishandle them:

* the identity pattern (r[0] = 0, every other offset -inf): W = I, so the
  output equals V and dV equals dO; the pattern gradients vanish;
* hard sliding windows (r[d] = 0 for d < w, -inf beyond): O is the window
  mean of V;
* a whole 256-offset segment of r at -inf (the band-sum normaliser's unit)
  and a run of keys whose a is -inf, at T > 512;
* NaN beyond T in a and r (stored prior length > T: never read) and NaN in
  the a, r rows of ordinary heads (never read);
* lengths T = 1 and T = 4097 (one past a 64-row tile multiple at the 124M
  layer's head dimension).

Expected values come only from the oracle; bars are the parity bars of the
layer (forward max-abs beyond the output's rounding and rel-L2, gradient
rel-L2, frozen dQ/dK exactly +0.0) and, for the pattern gradients, the
rounding bar of the pattern-gradient tests.
"""

import numpy as np
import pytest
import torch

import oracle
from synth import CONFIGS, make_inputs
from _helpers import (
    BF16_FWD_MAXABS, BF16_FWD_RELL2, BF16_GRAD_RELL2, F32_MAXABS, F32_RELL2, LSE_FRZ_ABS, LSE_ORD_ABS,
    forward_rounding_sigma, host, max_abs, out_max_abs, rel_l2, say, upload,
)

pytestmark = pytest.mark.gpu

PG_F32_RELL2 = 1e-4
NEG = -np.inf


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from fixed_pattern_hybrid_amd import binding

    return binding


def _layer_vs_oracle(B, cfg, inp, pattern_grad=True):
    """Forward, backward and (if any head is frozen) pattern gradients of the
    library against the oracle on one set of inputs."""
    say(f"case {cfg.name} B={cfg.B} H={cfg.H} T={cfg.T} D={cfg.D} Tp={cfg.Tp} frozen={cfg.frozen} {cfg.dtype}")
    bf16 = cfg.dtype == "bf16"
    o_max, o_rel = (BF16_FWD_MAXABS, BF16_FWD_RELL2) if bf16 else (F32_MAXABS, F32_RELL2)
    g_rel = BF16_GRAD_RELL2 if bf16 else F32_RELL2
    dev = upload(inp)
    fz = [int(x) for x in inp.frozen]
    O, L = B.saf_hybrid_attn_fwd(dev["q"], dev["k"], dev["v"], fz, dev["a"], dev["r"])
    dq, dk, dv = B.saf_hybrid_attn_bwd(dev["q"], dev["k"], dev["v"], O, dev["do"], L, fz, dev["a"], dev["r"])
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.hybrid_fwd(inp.q, inp.k, inp.v, fz, inp.a, inp.r)
    ref_dq, ref_dk, ref_dv = oracle.hybrid_bwd(inp.q, inp.k, inp.v, inp.do, fz, inp.a, inp.r)
    got_o, got_l = host(O), host(L)
    e_raw, e_o, e_r = max_abs(got_o, ref_o), out_max_abs(got_o, ref_o, cfg.dtype), rel_l2(got_o, ref_o)
    say(f"  O: raw max-abs {e_raw:.3e}, beyond output rounding {e_o:.3e}, rel-L2 {e_r:.3e}")
    assert e_o <= o_max and e_r <= o_rel, (e_o, e_r)
    for h in range(cfg.H):
        lim = LSE_FRZ_ABS if fz[h] else LSE_ORD_ABS
        e_l = max_abs(got_l[:, h], ref_l[:, h])
        assert e_l <= lim, (h, e_l)
    for n, g, rr in (("dQ", dq, ref_dq), ("dK", dk, ref_dk), ("dV", dv, ref_dv)):
        gh = host(g)
        assert np.all(np.isfinite(gh)), n
        if np.linalg.norm(rr) > 0:
            e = rel_l2(gh, rr)
            say(f"  {n}: rel-L2 {e:.3e}")
            assert e <= g_rel, (n, e)
    gq, gk = host(dq), host(dk)
    for h in range(cfg.H):
        if fz[h]:
            assert np.all(gq[:, h] == 0.0) and np.all(gk[:, h] == 0.0)
            assert not np.any(np.signbit(gq[:, h])) and not np.any(np.signbit(gk[:, h]))
    assert np.all(np.isfinite(got_o)) and np.all(np.isfinite(got_l))
    if not pattern_grad or not any(fz):
        return O, L, dq, dk, dv
    da = torch.full_like(dev["a"], 7.0)
    dr = torch.full_like(dev["r"], 7.0)
    B.saf_pattern_grad(dev["v"], O, dev["do"], L, fz, dev["a"], dev["r"], da=da, dr=dr)
    torch.cuda.synchronize()
    da, dr = host(da), host(dr)
    ref_a, ref_r = oracle.hybrid_pattern_grad(inp.v, inp.do, fz, inp.a, inp.r)
    bar = BF16_GRAD_RELL2 if bf16 else PG_F32_RELL2
    T = cfg.T
    for h in range(cfg.H):
        if not fz[h]:
            assert np.all(da[h] == 7.0) and np.all(dr[h] == 7.0), h
            continue
        sa, sr = forward_rounding_sigma(cfg, inp, h)
        for n, got, ref, sig in (("da", da[h, :T], ref_a[h], sa), ("dr", dr[h, :T], ref_r[h], sr)):
            assert np.all(np.isfinite(got)), (h, n)
            err = float(np.linalg.norm(got.astype(np.float64) - ref))
            lim = bar * float(np.linalg.norm(ref)) + 4.0 * sig
            say(f"  h{h}: {n} L2 error {err:.3e} (allowed {lim:.3e}, |ref| {np.linalg.norm(ref):.3e})")
            assert err <= lim, (h, n, err, lim)
        assert np.all(da[h, T:] == 0.0) and np.all(dr[h, T:] == 0.0)
    return O, L, dq, dk, dv


def _cfg(dtype, T=300, B_=2, H=4, frozen=(1, 3), D=64, Tp=None, name="edge"):
    base = CONFIGS["tiny"] if dtype == "f32" else CONFIGS["pages_check_t129"]
    return base.with_(T=T, B=B_, H=H, D=D, frozen=frozen, prior_len=Tp, name=f"{name}_{dtype}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_identity_pattern(B, dtype):
    cfg = _cfg(dtype, T=300, name="identity")
    inp = make_inputs(cfg, with_do=True)
    for h in cfg.frozen:
        inp.r[h, 1:] = NEG
        inp.r[h, 0] = 0.0
    O, L, dq, dk, dv = _layer_vs_oracle(B, cfg, inp)
    # W = I: the frozen heads pass V through and return dO as dV; log N(i) = a[i]
    for h in cfg.frozen:
        o, v = host(O[:, h]), inp.v[:, h]
        assert max_abs(o, v) <= (2.0 ** -8 * np.abs(v).max() if dtype == "bf16" else F32_MAXABS)
        assert rel_l2(host(dv[:, h]), inp.do[:, h]) <= (4e-3 if dtype == "bf16" else F32_RELL2)
        assert max_abs(host(L[:, h]), np.broadcast_to(inp.a[h, :cfg.T], (cfg.B, cfg.T))) <= LSE_FRZ_ABS


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("w", [1, 5, 64, 200])
def test_sliding_window_pattern(B, dtype, w):
    cfg = _cfg(dtype, T=333, name=f"window{w}")
    inp = make_inputs(cfg, with_do=True)
    for h in cfg.frozen:
        inp.r[h, :w] = 0.0
        inp.r[h, w:] = NEG
    inp.a[3] = 0.0  # head 3: a plain window mean; head 1 keeps random a
    O = _layer_vs_oracle(B, cfg, inp)[0]
    # head 3: O[i] is the mean of V over keys max(0, i - w + 1) .. i
    v = inp.v[:, 3].astype(np.float64)
    c = np.cumsum(np.concatenate([np.zeros((cfg.B, 1, cfg.D)), v], axis=1), axis=1)
    i = np.arange(cfg.T)
    lo = np.maximum(0, i - w + 1)
    mean = (c[:, i + 1] - c[:, lo]) / (i - lo + 1)[None, :, None]
    tol = BF16_FWD_MAXABS if dtype == "bf16" else F32_MAXABS
    assert out_max_abs(host(O[:, 3]), mean, dtype) <= tol


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_minus_inf_segments_beyond_512(B, dtype):
    # r at -inf over offsets [256, 512) (a whole segment of the normaliser's
    # band sums), a at -inf over keys [600, 700); every row keeps a finite
    # term (its diagonal, or for rows in [600, 700) an offset below 256)
    cfg = _cfg(dtype, T=1000, B_=2, H=3, frozen=(0, 2), name="inf_segments")
    inp = make_inputs(cfg, with_do=True)
    for h in cfg.frozen:
        inp.r[h, 256:512] = NEG
        inp.a[h, 600:700] = NEG
    inp.r[2, 700:] = NEG  # head 2: no offset beyond 699 either
    _layer_vs_oracle(B, cfg, inp)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_nan_where_never_read(B, dtype):
    # entries [T, Tp) of a and r and the rows of ordinary heads are never
    # read: NaN there must not change any result
    cfg = _cfg(dtype, T=200, Tp=256, H=4, frozen=(0, 2), name="nan_unread")
    inp = make_inputs(cfg, with_do=True)
    _layer_vs_oracle(B, cfg, inp)

    def run(inp):
        dev = upload(inp)
        fz = [int(x) for x in inp.frozen]
        O, L = B.saf_hybrid_attn_fwd(dev["q"], dev["k"], dev["v"], fz, dev["a"], dev["r"])
        g = B.saf_hybrid_attn_bwd(dev["q"], dev["k"], dev["v"], O, dev["do"], L, fz, dev["a"], dev["r"])
        da, dr = torch.zeros_like(dev["a"]), torch.zeros_like(dev["r"])
        B.saf_pattern_grad(dev["v"], O, dev["do"], L, fz, dev["a"], dev["r"], da=da, dr=dr)
        torch.cuda.synchronize()
        return (O, L) + tuple(g) + (da[(0, 2), :cfg.T], dr[(0, 2), :cfg.T])

    ref = run(inp)
    inp.a[:, cfg.T:] = np.nan
    inp.r[:, cfg.T:] = np.nan
    for h in (1, 3):
        inp.a[h] = np.nan
        inp.r[h] = np.nan
    for x, y in zip(run(inp), ref):
        assert torch.equal(x, y)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_single_token(B, dtype):
    # T = 1: W[0][0] = 1 for every frozen head, softmax of one score for
    # ordinary heads, so O = V and dV = dO everywhere, dQ = dK = 0
    cfg = _cfg(dtype, T=1, Tp=3, B_=3, H=4, frozen=(0, 3), name="single_token")
    inp = make_inputs(cfg, with_do=True)
    O, L, dq, dk, dv = _layer_vs_oracle(B, cfg, inp)
    assert max_abs(host(O), inp.v) <= (0.0 if dtype == "bf16" else 1e-5)
    assert max_abs(host(dv), inp.do) <= (0.0 if dtype == "bf16" else 1e-5)


def test_length_4097_layer_shape(B):
    # one past a tile multiple at the 124M layer's head dimension, with an
    # ordinary and a frozen head (every element compared)
    cfg = CONFIGS["gpt2_124m_4k_25pct"].with_(B=1, H=2, T=4097, frozen=(1,), name="T4097")
    inp = make_inputs(cfg, with_do=True)
    _layer_vs_oracle(B, cfg, inp)


def test_length_4097_fp32(B):
    cfg = CONFIGS["tiny"].with_(B=1, H=2, T=4097, frozen=(0,), name="T4097_fp32")
    inp = make_inputs(cfg, with_do=True)
    _layer_vs_oracle(B, cfg, inp, pattern_grad=False)
