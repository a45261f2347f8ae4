"""Parity of the fused-dQ backward schedule (saf_attn_params.fused_dq = 1)
with the float64 oracle and with the two-pass schedule (GPU required).

The fused schedule computes dQ inside the key-block programs and adds each
program's contribution into an fp32 accumulator with atomic adds, so only
the summation order of dQ differs from the two-pass backward: dQ, dK and dV
are held to the layer's gradient bar against the oracle (rel-L2 1e-2), and
to the two passes within a few bf16 units (both round the same fp32
gradients to bf16; dK and dV differ only through delta's summation order).
Frozen heads' dQ and dK stay exactly +0.0.
"""

import numpy as np
import pytest
import torch

import oracle
from synth import CONFIGS, make_inputs
from _helpers import BF16_GRAD_RELL2, host, rel_l2, say, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from fixed_pattern_hybrid_amd import binding

    return binding


def _both(B, cfg, strided=False, packed=False):
    say(f"fused-dQ case {cfg.name} B={cfg.B} H={cfg.H} T={cfg.T} frozen={cfg.frozen} strided={strided} "
        f"packed={packed}")
    inp = make_inputs(cfg, with_do=True)
    dev = upload(inp)
    q, k, v, do = dev["q"], dev["k"], dev["v"], dev["do"]
    if strided:
        q, k, v, do = (t.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3) for t in (q, k, v, do))
    fz = [int(x) for x in inp.frozen]
    ordh = [h for h in range(cfg.H) if not fz[h]]
    O, L = B.saf_hybrid_attn_fwd(q, k, v, fz, dev["a"], dev["r"])
    two = B.saf_hybrid_attn_bwd(q, k, v, O, do, L, fz, dev["a"], dev["r"])
    if packed:
        qp, kp = q[:, ordh].contiguous(), k[:, ordh].contiguous()
        dqp, dkp, dvf = B.saf_hybrid_attn_bwd(qp, kp, v, O, do, L, fz, dev["a"], dev["r"], qk_packed=True,
                                              fused_dq=True)
        dqf = torch.zeros_like(q)
        dkf = torch.zeros_like(k)
        dqf[:, ordh] = dqp
        dkf[:, ordh] = dkp
        fused = (dqf, dkf, dvf)
    else:
        fused = B.saf_hybrid_attn_bwd(q, k, v, O, do, L, fz, dev["a"], dev["r"], fused_dq=True)
    torch.cuda.synchronize()
    return inp, fz, two, fused


def _check(cfg, inp, fz, two, fused, oracle_full=True):
    if oracle_full:
        refs = oracle.hybrid_bwd(inp.q, inp.k, inp.v, inp.do, fz, inp.a, inp.r)
        for n, g, rr in zip(("dQ", "dK", "dV"), fused, refs):
            gh = host(g)
            assert np.all(np.isfinite(gh)), n
            if np.linalg.norm(rr) > 0:
                e = rel_l2(gh, rr)
                say(f"  fused {n}: rel-L2 {e:.3e}")
                assert e <= BF16_GRAD_RELL2, (n, e)
    # scale of the comparison: the largest entry of the two-pass result, but
    # at least that of dV (where the true dQ, dK vanish, as at T = 1, both
    # sides hold only rounding noise of the gradients' own magnitude)
    floor = max(float(np.abs(host(two[2])).max()), 1e-30)
    for n, x, y in zip(("dQ", "dK", "dV"), fused, two):
        xh, yh = host(x), host(y)
        scale = max(float(np.abs(yh).max()), floor)
        d = float(np.abs(xh - yh).max()) / scale
        say(f"  fused vs two-pass {n}: max |diff| / max |x| = {d:.3e}")
        assert d <= 2.0 ** -6, (n, d)  # a few bf16 units of the largest entry
    gq, gk = host(fused[0]), host(fused[1])
    for h in range(cfg.H):
        if fz[h]:
            assert np.all(gq[:, h] == 0.0) and not np.any(np.signbit(gq[:, h]))
            assert np.all(gk[:, h] == 0.0) and not np.any(np.signbit(gk[:, h]))


SMALL = [
    CONFIGS["pages_check_t129"],
    CONFIGS["pages_check_t129"].with_(frozen=(), name="pages-check_no-frozen"),
    CONFIGS["pages_check_t129"].with_(frozen=(0, 1, 2, 3), name="pages-check_all-frozen"),
    CONFIGS["pages_check_t129"].with_(T=1, prior_len=3, name="T1"),
    CONFIGS["pages_check_t129"].with_(T=64, B=3, name="T64"),
    CONFIGS["pages_check_t129"].with_(T=65, B=1, H=2, frozen=(1,), name="T65"),
    CONFIGS["pages_check_t129"].with_(T=300, B=5, H=4, frozen=(0, 3), qkv_scale=0.5, prior_len=None,
                                      name="T300"),
    CONFIGS["pages_check_t129"].with_(T=513, B=2, H=6, frozen=(1, 2, 5), prior_len=None, name="T513"),
]


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: c.name)
def test_fused_dq_small_cases(B, cfg):
    _check(cfg, *_both(B, cfg))


def test_fused_dq_strided_and_packed(B):
    cfg = CONFIGS["pages_check_t129"].with_(T=333, B=3, prior_len=None, name="fused_strided")
    _check(cfg, *_both(B, cfg, strided=True))
    cfg = CONFIGS["pages_check_t129"].with_(T=257, B=2, prior_len=None, frozen=(0, 2), name="fused_packed")
    _check(cfg, *_both(B, cfg, packed=True))


def test_fused_dq_dk_dv_reproducible(B):
    cfg = CONFIGS["pages_check_t129"].with_(T=700, B=2, H=4, prior_len=None, name="fused_repro")
    inp, fz, _, f1 = _both(B, cfg)
    dev = upload(inp)
    O, L = B.saf_hybrid_attn_fwd(dev["q"], dev["k"], dev["v"], fz, dev["a"], dev["r"])
    f2 = B.saf_hybrid_attn_bwd(dev["q"], dev["k"], dev["v"], O, dev["do"], L, fz, dev["a"], dev["r"],
                               fused_dq=True)
    torch.cuda.synchronize()
    assert torch.equal(f1[1], f2[1]) and torch.equal(f1[2], f2[2])  # no atomics in dK, dV


def test_fused_dq_rejected_where_not_built(B):
    cfg = CONFIGS["pages_check_t129"].with_(D=128, T=64, name="fused_d128")
    inp = make_inputs(cfg, with_do=True)
    dev = upload(inp)
    fz = [int(x) for x in inp.frozen]
    O, L = B.saf_hybrid_attn_fwd(dev["q"], dev["k"], dev["v"], fz, dev["a"], dev["r"])
    with pytest.raises(B.SafError) as ei:
        B.saf_hybrid_attn_bwd(dev["q"], dev["k"], dev["v"], O, dev["do"], L, fz, dev["a"], dev["r"],
                              fused_dq=True)
    assert ei.value.status == B.SAF_EUNSUPPORTED


@pytest.mark.parametrize("key,heads", [("gpt2_124m_4k_25pct", [(7, 0), (3, 10), (0, 8)]),
                                       ("gpt2_124m_4k_50pct_interleaved", [(5, 11)])])
def test_fused_dq_workload_sampled_heads(B, key, heads):
    cfg = CONFIGS[key]
    say(f"workload {cfg.name} (fused dQ)")
    inp, fz, two, fused = _both(B, cfg)
    _check(cfg, inp, fz, two, fused, oracle_full=False)
    s = 1.0 / np.sqrt(cfg.D)
    for b, h in heads:
        if fz[h]:
            continue
        rdq, rdk, rdv = oracle.ordinary_head_bwd(inp.q[b, h], inp.k[b, h], inp.v[b, h], inp.do[b, h], s)
        for n, g, rr in (("dQ", fused[0], rdq), ("dK", fused[1], rdk), ("dV", fused[2], rdv)):
            e = rel_l2(host(g[b, h]), rr)
            say(f"  b{b}h{h} {n} rel-L2 {e:.3e}")
            assert e <= BF16_GRAD_RELL2, (n, e)
