"""Seeded fuzz of the hybrid layer against the float64 oracle (GPU required).

The pages validate their fused kernels with a fuzz of 50 random operations
against an eager reference (Appendix D.2, Table 27).  This test draws 50
operations from one seeded generator: batch, head count, ragged length,
head dimension, dtype, frozen mask, stored prior length, tensor strides
(contiguous or [B, T, H, D] storage), the packed Q/K layout, grouped-query
key/value heads (forward only), the caller's stored log N, an explicit
softmax scale and the pattern gradients.  Each operation is compared with
the oracle at the layer's parity bars; the test stops at the first failure
and names the operation.  More seeds on request: SAF_FUZZ_SEEDS=7,99,2026
(and SAF_FUZZ_OPS, default 150) runs that many operations per seed in
test_fuzz_more_seeds, which is skipped otherwise.
"""

import os

import numpy as np
import pytest
import torch

import oracle
from synth import CONFIGS, make_inputs
from _helpers import (
    BF16_FWD_MAXABS, BF16_FWD_RELL2, BF16_GRAD_RELL2, F32_MAXABS, F32_RELL2, LSE_FRZ_ABS, LSE_ORD_ABS,
    forward_rounding_sigma, host, max_abs, out_max_abs, rel_l2, say, to_dev,
)

N_OPS = 50
FUZZ_SEED = 20260  # generator of the operations (inputs use their own seeds)
PG_F32_RELL2 = 1e-4


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from fixed_pattern_hybrid_amd import binding

    return binding


def draw_ops(n=N_OPS, seed=FUZZ_SEED):
    """The fuzzed operations: a list of dicts (pure host logic)."""
    g = np.random.default_rng(seed)
    ops = []
    for x in range(n):
        dtype = "f32" if g.random() < 0.25 else "bf16"
        D = int(g.choice([64, 96, 128] if dtype == "bf16" else [16, 32, 64, 96, 128]))
        H = int(g.integers(1, 7))
        gqa = H > 1 and g.random() < 0.2
        Hkv = H
        if gqa:
            divs = [d for d in range(1, H) if H % d == 0]
            Hkv = int(g.choice(divs))
        T = int(g.choice([1, 2, 63, 64, 65, 128, 129]) if g.random() < 0.3 else g.integers(1, 321))
        ops.append(dict(
            idx=x, dtype=dtype, D=D, H=H, Hkv=Hkv, B=int(g.integers(1, 4)), T=T,
            Tp=T + int(g.choice([0, 0, 1, 63])),
            frozen=tuple(int(h) for h in range(H) if g.random() < 0.4),
            strided=bool(g.random() < 0.3), packed=bool(g.random() < 0.25),
            logz=bool(g.random() < 0.25), scale=(None if g.random() < 0.7 else float(g.uniform(0.05, 0.3))),
            pgrad=bool(g.random() < 0.35), seed=int(g.integers(0, 2 ** 31)),
            qkv_scale=float(g.choice([0.125, 0.5, 1.0])),
        ))
    return ops


def test_fuzz_ops_cover_the_options():
    # host-only check of the draw itself (runs without a GPU): every option occurs
    ops = draw_ops()
    assert len(ops) == N_OPS
    for key in ("strided", "packed", "logz", "pgrad"):
        assert any(o[key] for o in ops) and not all(o[key] for o in ops), key
    assert any(o["Hkv"] < o["H"] for o in ops)
    assert any(o["dtype"] == "f32" for o in ops) and any(o["dtype"] == "bf16" for o in ops)
    assert {64, 96, 128} <= {o["D"] for o in ops}
    assert any(len(o["frozen"]) == 0 for o in ops) and any(len(o["frozen"]) == o["H"] for o in ops)
    assert any(o["T"] == 1 for o in ops) and any(o["Tp"] > o["T"] for o in ops)


def _restride(t):
    """The same values in [B, T, H, D] storage, seen as [B, H, T, D]."""
    return t.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)


def run_op(B, op):
    dtype = op["dtype"]
    bf16 = dtype == "bf16"
    base = CONFIGS["pages_check_t129"] if bf16 else CONFIGS["tiny"]
    gqa = op["Hkv"] < op["H"]
    cfg = base.with_(B=op["B"], H=op["H"], T=op["T"], D=op["D"], frozen=op["frozen"], prior_len=op["Tp"],
                     kv_heads=op["Hkv"] if gqa else None, qkv_scale=op["qkv_scale"], bwd=not gqa,
                     name=f"fuzz{op['idx']}")
    inp = make_inputs(cfg, seed=op["seed"], with_do=not gqa)
    tdt = torch.bfloat16 if bf16 else torch.float32
    q, k, v = (to_dev(getattr(inp, n), tdt) for n in ("q", "k", "v"))
    do = to_dev(inp.do, tdt) if not gqa else None
    a, r = torch.from_numpy(inp.a).cuda(), torch.from_numpy(inp.r).cuda()
    fz = [int(x) for x in inp.frozen]
    ordh = [h for h in range(cfg.H) if not fz[h]]
    if op["strided"]:
        q, k, v = _restride(q), _restride(k), _restride(v)
        if do is not None:
            do = _restride(do)
    logz = B.saf_pattern_lognorm(a, r, cfg.T) if op["logz"] else None
    scale = op["scale"]
    if op["packed"]:
        qp = q[:, ordh] if ordh else None
        kp = (k if gqa else k[:, ordh]) if ordh else None
        O, L = B.saf_hybrid_attn_fwd(qp, kp, v, fz, a, r, softmax_scale=scale, logz=logz, qk_packed=True)
    else:
        O, L = B.saf_hybrid_attn_fwd(q, k, v, fz, a, r, softmax_scale=scale, logz=logz)
    grads = None
    if not gqa:
        if op["packed"]:
            dqp, dkp, dv = B.saf_hybrid_attn_bwd(qp, kp, v, O, do, L, fz, a, r, softmax_scale=scale, qk_packed=True)
            dq = torch.zeros_like(q)
            dk = torch.zeros_like(k)
            if ordh:
                dq[:, ordh] = dqp
                dk[:, ordh] = dkp
        else:
            dq, dk, dv = B.saf_hybrid_attn_bwd(q, k, v, O, do, L, fz, a, r, softmax_scale=scale)
        grads = (dq, dk, dv)
    pg = None
    if op["pgrad"] and not gqa and any(fz):
        da, dr = torch.full_like(a, 7.0), torch.full_like(r, 7.0)
        B.saf_pattern_grad(v, O, do, L, fz, a, r, da=da, dr=dr)
        pg = (da, dr)
    torch.cuda.synchronize()

    # expected values from the oracle only
    o_max, o_rel = (BF16_FWD_MAXABS, BF16_FWD_RELL2) if bf16 else (F32_MAXABS, F32_RELL2)
    ref_o, ref_l = oracle.hybrid_fwd(inp.q, inp.k, inp.v, fz, inp.a, inp.r, scale=scale)
    got_o, got_l = host(O), host(L)
    e_o, e_r = out_max_abs(got_o, ref_o, dtype), rel_l2(got_o, ref_o)
    say(f"  O raw max-abs {max_abs(got_o, ref_o):.3e} beyond rounding {e_o:.3e} rel-L2 {e_r:.3e}")
    assert e_o <= o_max and e_r <= o_rel, ("O", e_o, e_r)
    for h in range(cfg.H):
        e_l = max_abs(got_l[:, h], ref_l[:, h])
        assert e_l <= (LSE_FRZ_ABS if fz[h] else LSE_ORD_ABS), ("lse", h, e_l)
    if grads is not None:
        g_rel = BF16_GRAD_RELL2 if bf16 else F32_RELL2
        refs = oracle.hybrid_bwd(inp.q, inp.k, inp.v, inp.do, fz, inp.a, inp.r, scale=scale)
        for n, gt, rr in zip(("dQ", "dK", "dV"), grads, refs):
            gh = host(gt)
            assert np.all(np.isfinite(gh)), n
            if np.linalg.norm(rr) > 0:
                e = rel_l2(gh, rr)
                say(f"  {n} rel-L2 {e:.3e}")
                assert e <= g_rel, (n, e)
        if not op["packed"]:
            gq, gk = host(grads[0]), host(grads[1])
            for h in range(cfg.H):
                if fz[h]:
                    assert np.all(gq[:, h] == 0.0) and not np.any(np.signbit(gq[:, h])), ("dQ zero", h)
                    assert np.all(gk[:, h] == 0.0) and not np.any(np.signbit(gk[:, h])), ("dK zero", h)
    if pg is not None:
        da, dr = host(pg[0]), host(pg[1])
        ref_a, ref_r = oracle.hybrid_pattern_grad(inp.v, inp.do, fz, inp.a, inp.r)
        bar = BF16_GRAD_RELL2 if bf16 else PG_F32_RELL2
        for h in range(cfg.H):
            if not fz[h]:
                assert np.all(da[h] == 7.0) and np.all(dr[h] == 7.0), ("pattern grad wrote an ordinary row", h)
                continue
            sa, sr = forward_rounding_sigma(cfg, inp, h)
            for n, gt, rr, sig in (("da", da[h, :cfg.T], ref_a[h], sa), ("dr", dr[h, :cfg.T], ref_r[h], sr)):
                err = float(np.linalg.norm(gt.astype(np.float64) - rr))
                lim = bar * float(np.linalg.norm(rr)) + 4.0 * sig
                assert err <= lim, (n, h, err, lim)
            assert np.all(da[h, cfg.T:] == 0.0) and np.all(dr[h, cfg.T:] == 0.0)


@pytest.mark.gpu
def test_fuzz_50_operations(B):
    for op in draw_ops():
        say(f"fuzz op {op['idx']}: {op}")
        try:
            run_op(B, op)
        except AssertionError as e:
            raise AssertionError(f"fuzz operation {op['idx']} failed: {op}: {e}") from e


@pytest.mark.gpu
def test_fuzz_more_seeds(B):
    seeds = [int(x) for x in os.environ.get("SAF_FUZZ_SEEDS", "").split(",") if x.strip()]
    if not seeds:
        pytest.skip("set SAF_FUZZ_SEEDS to fuzz with more generator seeds")
    n = int(os.environ.get("SAF_FUZZ_OPS", "150"))
    for seed in seeds:
        for op in draw_ops(n=n, seed=seed):
            say(f"fuzz seed {seed} op {op['idx']}: {op}")
            try:
                run_op(B, op)
            except AssertionError as e:
                raise AssertionError(f"fuzz seed {seed} operation {op['idx']} failed: {op}: {e}") from e
