"""The torch.autograd glue (fixed_pattern_hybrid_amd.autograd) against the
library's entry points called directly (GPU required).

The glue computes nothing itself, so its gradients must equal, bit for bit,
those of saf_hybrid_attn_bwd and saf_pattern_grad called with the same
output gradient; one case also checks dV against the float64 oracle, which
pins the order in which the glue hands the gradients back.
"""

import numpy as np
import pytest
import torch

import oracle
from synth import CONFIGS, make_inputs
from _helpers import BF16_GRAD_RELL2, F32_RELL2, host, rel_l2, say, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from fixed_pattern_hybrid_amd import binding

    return binding


@pytest.fixture(scope="module")
def AG(B):
    from fixed_pattern_hybrid_amd import autograd

    return autograd


def _leaf(t, grad):
    return t.detach().clone().requires_grad_(grad)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_gradients_equal_direct_calls(B, AG, dtype):
    base = CONFIGS["pages_check_t129"] if dtype == "bf16" else CONFIGS["tiny"]
    cfg = base.with_(B=3, T=150, prior_len=None, frozen=(1, 3), H=4, name=f"autograd_{dtype}")
    inp = make_inputs(cfg, with_do=True)
    dev = upload(inp)
    fz = [int(x) for x in inp.frozen]
    say(f"case {cfg.name} B={cfg.B} H={cfg.H} T={cfg.T} D={cfg.D} frozen={cfg.frozen}")
    q, k, v, a, r = (_leaf(dev[n], True) for n in ("q", "k", "v", "a", "r"))
    O = AG.hybrid_attention(q, k, v, a, r, fz)
    # the gradient of sum(O * G) with respect to O is G in O's dtype
    G = dev["do"].float()
    (O.float() * G).sum().backward()
    g = G.to(O.dtype)

    O2, L2 = B.saf_hybrid_attn_fwd(dev["q"], dev["k"], dev["v"], fz, dev["a"], dev["r"])
    dq, dk, dv = B.saf_hybrid_attn_bwd(dev["q"], dev["k"], dev["v"], O2, g, L2, fz, dev["a"], dev["r"])
    da, dr = B.saf_pattern_grad(dev["v"], O2, g, L2, fz, dev["a"], dev["r"])
    torch.cuda.synchronize()
    assert torch.equal(O.detach(), O2)
    for name, got, want in (("dq", q.grad, dq), ("dk", k.grad, dk), ("dv", v.grad, dv),
                            ("da", a.grad, da), ("dr", r.grad, dr)):
        assert got is not None and got.shape == want.shape, name
        assert torch.equal(got, want), f"{name} differs from the direct call"

    ref_dv = oracle.hybrid_bwd(inp.q, inp.k, inp.v, host(g), fz, inp.a, inp.r)[2]
    e = rel_l2(host(v.grad), ref_dv)
    say(f"  dV rel-L2 against the oracle {e:.3e}")
    assert e <= (BF16_GRAD_RELL2 if dtype == "bf16" else F32_RELL2)


def test_pattern_gradients_only(B, AG):
    # q, k, v without gradients: only the pattern gradients are formed
    cfg = CONFIGS["pages_check_t129"].with_(B=2, T=97, prior_len=None, name="autograd_pattern_only")
    inp = make_inputs(cfg, with_do=True)
    dev = upload(inp)
    fz = [int(x) for x in inp.frozen]
    q, k, v = (_leaf(dev[n], False) for n in ("q", "k", "v"))
    a, r = _leaf(dev["a"], True), _leaf(dev["r"], True)
    O = AG.hybrid_attention(q, k, v, a, r, fz)
    O.backward(dev["do"])
    O2, L2 = B.saf_hybrid_attn_fwd(dev["q"], dev["k"], dev["v"], fz, dev["a"], dev["r"])
    da, dr = B.saf_pattern_grad(dev["v"], O2, dev["do"], L2, fz, dev["a"], dev["r"])
    torch.cuda.synchronize()
    assert q.grad is None and k.grad is None and v.grad is None
    assert torch.equal(a.grad, da) and torch.equal(r.grad, dr)
    # ordinary heads' rows of the pattern gradients stay zero
    for h in range(cfg.H):
        if not fz[h]:
            assert not a.grad[h].any() and not r.grad[h].any()


def test_bf16_autocast(B, AG):
    # fp32 q, k, v under bf16 autocast run the bf16 path; their gradients are
    # those of the bf16 call, cast back to fp32
    cfg = CONFIGS["tiny"].with_(B=2, T=129, H=4, frozen=(1, 3), prior_len=192, name="autograd_autocast")
    inp = make_inputs(cfg, with_do=True)
    dev = upload(inp)  # fp32 tensors
    fz = [int(x) for x in inp.frozen]
    q, k, v = (_leaf(dev[n], True) for n in ("q", "k", "v"))
    with torch.autocast("cuda", dtype=torch.bfloat16):
        O = AG.hybrid_attention(q, k, v, dev["a"], dev["r"], fz)
    assert O.dtype == torch.bfloat16
    g = dev["do"].to(torch.bfloat16)
    O.backward(g)
    qb, kb_, vb = (dev[n].to(torch.bfloat16) for n in ("q", "k", "v"))
    O2, L2 = B.saf_hybrid_attn_fwd(qb, kb_, vb, fz, dev["a"], dev["r"])
    dq, dk, dv = B.saf_hybrid_attn_bwd(qb, kb_, vb, O2, g, L2, fz, dev["a"], dev["r"])
    torch.cuda.synchronize()
    assert torch.equal(O.detach(), O2)
    for got, want in ((q.grad, dq), (k.grad, dk), (v.grad, dv)):
        assert got.dtype == torch.float32 and torch.equal(got, want.float())


def test_grouped_query_backward_is_refused(B, AG):
    cfg = CONFIGS["pages_check_t129"].with_(H=8, kv_heads=2, B=1, T=64, prior_len=None, frozen=(1,),
                                            name="autograd_gqa")
    inp = make_inputs(cfg, with_do=True)
    dev = upload(inp)
    fz = [int(x) for x in inp.frozen]
    q, k, v = (_leaf(dev[n], True) for n in ("q", "k", "v"))
    O = AG.hybrid_attention(q, k, v, dev["a"], dev["r"], fz)
    with pytest.raises(NotImplementedError):
        O.backward(dev["do"])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(O), host(B.saf_hybrid_attn_fwd(dev["q"], dev["k"], dev["v"], fz,
                                                                       dev["a"], dev["r"])[0]))
