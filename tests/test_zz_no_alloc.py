"""The no-allocation forward (saf_hybrid_attn_fwd_noalloc) against the
workspace forward (GPU required).

The no-allocation entry point runs the same kernels with the normaliser
partials in the library's static scratch array instead of a caller
workspace, so its outputs must equal the workspace forward's bit for bit.
Two calls in a row, the second on a smaller input, check that the scratch
left by the first call does not leak into the second.
"""

import ctypes

import numpy as np
import pytest
import torch

from synth import CONFIGS, make_inputs
from _helpers import say, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from fixed_pattern_hybrid_amd import binding

    return binding


def _noalloc_via_abi(B, q, k, v, fz, a, r, out, lse):
    """One saf_hybrid_attn_fwd_noalloc call straight through the C ABI."""
    prm = B.Params(q, fz, a.shape[1])
    prm.set_strides(q=q, k=k, v=v, o=out)
    st = B.LIB.saf_hybrid_attn_fwd_noalloc(prm.ref(), q.data_ptr(), k.data_ptr(), v.data_ptr(), a.data_ptr(),
                                           r.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                           torch.cuda.current_stream().cuda_stream)
    return st


CASES = [
    # larger first, then smaller: the second call finds the first call's
    # partials in the scratch
    CONFIGS["pages_check_t129"].with_(B=3, H=6, T=2500, prior_len=2600, frozen=(1, 4, 5), name="noalloc_big"),
    CONFIGS["pages_check_t129"].with_(B=2, H=4, T=300, prior_len=None, frozen=(0, 3), name="noalloc_small"),
]


def test_noalloc_forward_matches_workspace_forward_twice(B):
    outs = []
    for cfg in CASES:
        say(f"noalloc case {cfg.name} B={cfg.B} H={cfg.H} T={cfg.T} frozen={cfg.frozen}")
        inp = make_inputs(cfg, with_do=False)
        dev = upload(inp)
        fz = [int(x) for x in inp.frozen]
        o_ws, l_ws = B.saf_hybrid_attn_fwd(dev["q"], dev["k"], dev["v"], fz, dev["a"], dev["r"])
        o_na = torch.full_like(o_ws, float("nan"))
        l_na = torch.full_like(l_ws, float("nan"))
        st = _noalloc_via_abi(B, dev["q"], dev["k"], dev["v"], fz, dev["a"], dev["r"], o_na, l_na)
        torch.cuda.synchronize()
        assert st == B.SAF_OK, B.status_string(st)
        assert torch.equal(o_na, o_ws) and torch.equal(l_na, l_ws), cfg.name
        outs.append((o_na, l_na))
    assert all(bool(torch.isfinite(o.float()).all()) for o, _ in outs)


def test_noalloc_binding_and_other_layouts(B):
    # the binding's wrapper, the packed Q/K layout, the stored log N (no
    # scratch needed) and the fp32 path (no scratch needed)
    cfg = CONFIGS["pages_check_t129"].with_(B=2, H=4, T=700, prior_len=None, frozen=(1, 2), D=128,
                                            name="noalloc_d128")
    inp = make_inputs(cfg, with_do=False)
    dev = upload(inp)
    fz = [int(x) for x in inp.frozen]
    ordh = [h for h in range(cfg.H) if not fz[h]]
    o_ws, l_ws = B.saf_hybrid_attn_fwd(dev["q"], dev["k"], dev["v"], fz, dev["a"], dev["r"])
    o, l = torch.empty_like(o_ws), torch.empty_like(l_ws)
    B.saf_hybrid_attn_fwd_noalloc(dev["q"], dev["k"], dev["v"], fz, dev["a"], dev["r"], out=o, lse=l)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ws) and torch.equal(l, l_ws)
    qp, kp = dev["q"][:, ordh].contiguous(), dev["k"][:, ordh].contiguous()
    B.saf_hybrid_attn_fwd_noalloc(qp, kp, dev["v"], fz, dev["a"], dev["r"], out=o, lse=l, qk_packed=True)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ws) and torch.equal(l, l_ws)
    logz = B.saf_pattern_lognorm(dev["a"], dev["r"], cfg.T)
    o_z, l_z = B.saf_hybrid_attn_fwd(dev["q"], dev["k"], dev["v"], fz, dev["a"], dev["r"], logz=logz)
    B.saf_hybrid_attn_fwd_noalloc(dev["q"], dev["k"], dev["v"], fz, dev["a"], dev["r"], out=o, lse=l, logz=logz)
    torch.cuda.synchronize()
    assert torch.equal(o, o_z) and torch.equal(l, l_z)
    c32 = CONFIGS["tiny"].with_(T=200, B=2, name="noalloc_fp32")
    inp = make_inputs(c32, with_do=False)
    dev = upload(inp)
    fz = [int(x) for x in inp.frozen]
    o_ws, l_ws = B.saf_hybrid_attn_fwd(dev["q"], dev["k"], dev["v"], fz, dev["a"], dev["r"])
    o, l = torch.empty_like(o_ws), torch.empty_like(l_ws)
    B.saf_hybrid_attn_fwd_noalloc(dev["q"], dev["k"], dev["v"], fz, dev["a"], dev["r"], out=o, lse=l)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ws) and torch.equal(l, l_ws)


def test_noalloc_rejects_shapes_beyond_its_scratch(B):
    # bf16, two frozen heads at T = 2^17: 2 x 32 partial groups x 2^17 rows x
    # 8 bytes = 64 MiB > 32 MiB.  Rejected before anything is enqueued, so
    # the (small, valid) buffers are never touched.
    T = 1 << 17
    x = torch.zeros(64, dtype=torch.bfloat16, device="cuda")
    a = torch.zeros(16, dtype=torch.float32, device="cuda")
    fz = [0, 1, 1, 0]
    prm = B.Params(torch.empty((1, 4, T, 64), dtype=torch.bfloat16, device="meta"), fz, T)
    for n in ("q", "k", "v", "o"):
        setattr(prm.p, n + "_stride", B._i64x3(4 * T * 64, T * 64, 64))
    st = B.LIB.saf_hybrid_attn_fwd_noalloc(prm.ref(), x.data_ptr(), x.data_ptr(), x.data_ptr(), a.data_ptr(),
                                           a.data_ptr(), x.data_ptr(), a.data_ptr(), None)
    assert st == B.SAF_ESCRATCH
    torch.cuda.synchronize()
    assert bool((x == 0).all()) and bool((a == 0).all())


def test_noalloc_forward_under_graph_capture(B):
    # The caller the entry point is for: a forward captured into a HIP graph.
    # Every replay must equal the eager result, also after eager no-allocation
    # calls on other inputs have overwritten the shared scratch in between.
    cfg = CONFIGS["pages_check_t129"].with_(B=2, H=6, T=700, prior_len=None, frozen=(0, 3, 5), name="noalloc_graph")
    other = cfg.with_(T=900, name="noalloc_graph_other")
    inp, inp2 = make_inputs(cfg, with_do=False), make_inputs(other, seed=7, with_do=False)
    dev, dev2 = upload(inp), upload(inp2)
    fz = [int(x) for x in inp.frozen]
    O0, L0 = B.saf_hybrid_attn_fwd(dev["q"], dev["k"], dev["v"], fz, dev["a"], dev["r"])
    O, L = torch.empty_like(O0), torch.empty_like(L0)
    O2, L2 = torch.empty_like(dev2["v"]), torch.empty((other.B, other.H, other.T), device="cuda")

    def step():
        B.saf_hybrid_attn_fwd_noalloc(dev["q"], dev["k"], dev["v"], fz, dev["a"], dev["r"], out=O, lse=L)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # first call on the device outside capture (symbol address, LDS attribute)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(3):
        O.fill_(float("nan"))
        L.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        say(f"  replay {rep}")
        assert torch.equal(O, O0) and torch.equal(L, L0)
        # eager no-allocation call on other inputs: overwrites the scratch
        B.saf_hybrid_attn_fwd_noalloc(dev2["q"], dev2["k"], dev2["v"], fz, dev2["a"], dev2["r"], out=O2, lse=L2)
        torch.cuda.synchronize()
