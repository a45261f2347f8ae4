"""Parity of the HIP path with the float64 oracle (GPU required).

Small shapes compare every element; the workload shapes compare sampled heads
(and, for the 32K prefill, sampled rows) that the oracle computes one by one,
plus properties that hold at any size.  Inputs come from the seeded
generator in ``synth``; expected values come only from ``oracle``.
"""

import numpy as np
import pytest
import torch

import oracle
from synth import CONFIGS, get_config, make_inputs
from _helpers import (
    BF16_FWD_MAXABS, BF16_FWD_RELL2, BF16_GRAD_RELL2, F32_MAXABS, F32_RELL2, LSE_FRZ_ABS,
    LSE_ORD_ABS, host, max_abs, out_max_abs, rel_l2, say, upload,
)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from fixed_pattern_hybrid_amd import binding

    return binding


def _bars(cfg):
    if cfg.dtype == "bf16":
        return dict(o_max=BF16_FWD_MAXABS, o_rel=BF16_FWD_RELL2, g_rel=BF16_GRAD_RELL2, g_max=None)
    return dict(o_max=F32_MAXABS, o_rel=F32_RELL2, g_rel=F32_RELL2, g_max=None)


def _check_head(tag, cfg, got_o, ref_o, got_l, ref_l, frozen_h):
    bars = _bars(cfg)
    e_max, e_rel = out_max_abs(got_o, ref_o, cfg.dtype), rel_l2(got_o, ref_o)
    e_l = max_abs(got_l, ref_l)
    say(f"  {tag}: O max-abs {max_abs(got_o, ref_o):.3e} (beyond output rounding {e_max:.3e}) "
        f"rel-L2 {e_rel:.3e} lse max-abs {e_l:.3e}")
    assert e_max <= bars["o_max"], (tag, e_max)
    assert e_rel <= bars["o_rel"], (tag, e_rel)
    assert e_l <= (LSE_FRZ_ABS if frozen_h else LSE_ORD_ABS), (tag, e_l)


def run_full_parity(B, cfg, seed=None, strided=False, poison_frozen_qk=False, scale=None):
    """Forward and backward on every element of a small case."""
    say(f"case {cfg.name} B={cfg.B} H={cfg.H} T={cfg.T} D={cfg.D} Tp={cfg.Tp} frozen={cfg.frozen} "
        f"{cfg.dtype} strided={strided} poison={poison_frozen_qk} seed={seed}")
    inp = make_inputs(cfg, seed, with_do=True)
    dev = upload(inp)
    q, k, v, do = dev["q"], dev["k"], dev["v"], dev["do"]
    if strided:
        # [B, T, H, D] storage seen as [B, H, T, D] (non-contiguous Q/K/V views)
        q = q.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
        k = k.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
        v = v.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
        assert not q.is_contiguous()
    fz = [int(x) for x in inp.frozen]
    if poison_frozen_qk:
        q = q.clone()
        k = k.clone()
        for h in range(cfg.H):
            if fz[h]:
                q[:, h] = float("nan")
                k[:, h] = float("nan")
    O, L = B.saf_hybrid_attn_fwd(q, k, v, fz, dev["a"], dev["r"], softmax_scale=scale)
    dq, dk, dv = B.saf_hybrid_attn_bwd(q, k, v, O, do, L, fz, dev["a"], dev["r"], softmax_scale=scale)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.hybrid_fwd(inp.q, inp.k, inp.v, fz, inp.a, inp.r, scale=scale)
    ref_dq, ref_dk, ref_dv = oracle.hybrid_bwd(inp.q, inp.k, inp.v, inp.do, fz, inp.a, inp.r, scale=scale)
    got = {n: host(t) for n, t in dict(o=O, l=L, dq=dq, dk=dk, dv=dv).items()}
    bars = _bars(cfg)
    e = {
        "O": (out_max_abs(got["o"], ref_o, cfg.dtype), rel_l2(got["o"], ref_o)),
        "dQ": (max_abs(got["dq"], ref_dq), rel_l2(got["dq"], ref_dq)),
        "dK": (max_abs(got["dk"], ref_dk), rel_l2(got["dk"], ref_dk)),
        "dV": (max_abs(got["dv"], ref_dv), rel_l2(got["dv"], ref_dv)),
    }
    say(f"  O: raw max-abs {max_abs(got['o'], ref_o):.3e}")
    for n, (m, r) in e.items():
        say(f"  {n}: max-abs {m:.3e} rel-L2 {r:.3e}")
    assert e["O"][0] <= bars["o_max"] and e["O"][1] <= bars["o_rel"], e["O"]
    refs = {"dQ": ref_dq, "dK": ref_dk, "dV": ref_dv}
    for n in ("dQ", "dK", "dV"):
        if np.linalg.norm(refs[n]) > 0:
            assert e[n][1] <= bars["g_rel"], (n, e[n])
    for h in range(cfg.H):
        lim = LSE_FRZ_ABS if fz[h] else LSE_ORD_ABS
        assert max_abs(got["l"][:, h], ref_l[:, h]) <= lim, (h, max_abs(got["l"][:, h], ref_l[:, h]))
        if fz[h]:
            # exact +0.0 for frozen heads' query/key gradients
            assert np.all(got["dq"][:, h] == 0.0) and np.all(got["dk"][:, h] == 0.0)
            assert not np.any(np.signbit(got["dq"][:, h])) and not np.any(np.signbit(got["dk"][:, h]))
    for t in got.values():
        assert np.all(np.isfinite(t))
    return O, L, dq, dk, dv


SMALL = [
    CONFIGS["tiny"],
    CONFIGS["pages_check_t129"],
    CONFIGS["pages_check_t129"].with_(dtype="f32", name="pages-check_fp32"),
    CONFIGS["pages_check_t129"].with_(frozen=(), name="pages-check_no-frozen"),
    CONFIGS["pages_check_t129"].with_(frozen=(0, 1, 2, 3), name="pages-check_all-frozen"),
]


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: c.name)
def test_small_cases(B, cfg):
    run_full_parity(B, cfg)


@pytest.mark.parametrize("T", [1, 17, 64, 65, 127, 200, 257])
def test_ragged_lengths(B, T):
    cfg = CONFIGS["pages_check_t129"].with_(T=T, prior_len=T + 5, B=2, H=3, frozen=(1,), name=f"ragged_T{T}")
    run_full_parity(B, cfg)


@pytest.mark.parametrize("D", [64, 96, 128])
@pytest.mark.parametrize("mask", [(), (0,), (1, 3), (0, 1, 2, 3)])
def test_head_dims_and_masks(B, D, mask):
    cfg = CONFIGS["pages_check_t129"].with_(D=D, T=150, H=4, B=5, frozen=mask, qkv_scale=0.5,
                                            name=f"D{D}_mask{''.join(map(str, mask))}")
    run_full_parity(B, cfg)


@pytest.mark.parametrize("H,T", [(40, 100), (256, 24)])
def test_many_heads(B, H, T):
    # head lists up to the maximum head count; every third head frozen
    cfg = CONFIGS["pages_check_t129"].with_(H=H, T=T, B=3, prior_len=None, frozen=tuple(range(1, H, 3)),
                                            name=f"heads{H}")
    run_full_parity(B, cfg)


@pytest.mark.parametrize("D", [16, 32, 64, 96, 128])
def test_fp32_path(B, D):
    cfg = CONFIGS["tiny"].with_(D=D, T=70, B=2, H=3, frozen=(2,), name=f"fp32_D{D}")
    run_full_parity(B, cfg)


def test_strided_views(B):
    run_full_parity(B, CONFIGS["pages_check_t129"].with_(B=3, T=300, prior_len=None, name="strided"), strided=True)


def test_explicit_scale(B):
    run_full_parity(B, CONFIGS["pages_check_t129"].with_(name="scale0.3"), scale=0.3)


def test_frozen_qk_poison_and_determinism(B):
    cfg = CONFIGS["pages_check_t129"].with_(T=260, B=4, prior_len=None, name="poison")
    r1 = run_full_parity(B, cfg)
    r2 = run_full_parity(B, cfg, poison_frozen_qk=True)
    r3 = run_full_parity(B, cfg)
    for x, y, z in zip(r1, r2, r3):
        assert torch.equal(x, z), "results must be bitwise reproducible"
        fx = torch.nan_to_num(x)
        fy = torch.nan_to_num(y)
        assert torch.equal(fx, fy), "frozen heads' Q/K must not be read"


def test_stage_events_do_not_change_results(B):
    cfg = CONFIGS["pages_check_t129"].with_(T=333, B=2, prior_len=None, name="events")
    inp = make_inputs(cfg)
    dev = upload(inp)
    fz = [int(x) for x in inp.frozen]
    O1, L1 = B.saf_hybrid_attn_fwd(dev["q"], dev["k"], dev["v"], fz, dev["a"], dev["r"])
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    for e in evs:
        e.record()
    O2, L2 = B.saf_hybrid_attn_fwd(dev["q"], dev["k"], dev["v"], fz, dev["a"], dev["r"], events=evs)
    torch.cuda.synchronize()
    assert torch.equal(O1, O2) and torch.equal(L1, L2)
    assert evs[0].elapsed_time(evs[2]) >= 0.0


def test_graph_capture_replays_match_eager(B):
    # The entry points allocate nothing and issue no memsets, so a caller can
    # capture forward + backward into a HIP graph; every replay (with eager
    # work and synchronisation between replays) must equal the eager result.
    cfg = CONFIGS["pages_check_t129"].with_(B=3, T=300, prior_len=None, name="graph")
    inp = make_inputs(cfg, with_do=True)
    dev = upload(inp)
    q, k, v, do, a, r = dev["q"], dev["k"], dev["v"], dev["do"], dev["a"], dev["r"]
    fz = [int(x) for x in inp.frozen]
    O0, L0 = B.saf_hybrid_attn_fwd(q, k, v, fz, a, r)
    G0 = B.saf_hybrid_attn_bwd(q, k, v, O0, do, L0, fz, a, r)
    torch.cuda.synchronize()

    O, L = torch.empty_like(O0), torch.empty_like(L0)
    dq, dk, dv = (torch.empty_like(x) for x in G0)
    prm = B.Params(v, fz, a.shape[1])
    wsf = torch.empty(max(B.workspace_bytes(prm, False), 256), dtype=torch.uint8, device="cuda")
    wsb = torch.empty(max(B.workspace_bytes(prm, True), 256), dtype=torch.uint8, device="cuda")

    def step():
        B.saf_hybrid_attn_fwd(q, k, v, fz, a, r, out=O, lse=L, workspace=wsf)
        B.saf_hybrid_attn_bwd(q, k, v, O, do, L, fz, a, r, dq=dq, dk=dk, dv=dv, workspace=wsb)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(3):
        for t in (O, L, dq, dk, dv):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        say(f"  replay {rep}")
        assert torch.equal(O, O0) and torch.equal(L, L0)
        for got, ref in zip((dq, dk, dv), G0):
            assert torch.equal(got, ref)
        B.saf_hybrid_attn_fwd(q, k, v, fz, a, r)  # eager work between replays
        torch.cuda.synchronize()


def test_concurrent_calls_on_two_streams(B):
    # No mutable global state on the workspace entry points: two layers'
    # forward + backward enqueued on two streams at once (each with its own
    # workspace) give exactly their sequential results.
    cfgs = [CONFIGS["pages_check_t129"].with_(B=3, T=600, prior_len=None, name="stream_a"),
            CONFIGS["pages_check_t129"].with_(B=2, H=6, T=900, prior_len=None, frozen=(0, 2, 3), name="stream_b")]
    runs = []
    for c in cfgs:
        inp = make_inputs(c, with_do=True)
        dev = upload(inp)
        fz = [int(x) for x in inp.frozen]
        O, L = B.saf_hybrid_attn_fwd(dev["q"], dev["k"], dev["v"], fz, dev["a"], dev["r"])
        G = B.saf_hybrid_attn_bwd(dev["q"], dev["k"], dev["v"], O, dev["do"], L, fz, dev["a"], dev["r"])
        torch.cuda.synchronize()
        runs.append((dev, fz, (O, L) + tuple(G)))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [None, None]
    for rep in range(3):
        for s_ in streams:
            s_.wait_stream(torch.cuda.current_stream())
        for x, (dev, fz, _) in enumerate(runs):
            with torch.cuda.stream(streams[x]):
                O, L = B.saf_hybrid_attn_fwd(dev["q"], dev["k"], dev["v"], fz, dev["a"], dev["r"],
                                             stream=streams[x])
                G = B.saf_hybrid_attn_bwd(dev["q"], dev["k"], dev["v"], O, dev["do"], L, fz, dev["a"], dev["r"],
                                          stream=streams[x])
                outs[x] = (O, L) + tuple(G)
        torch.cuda.synchronize()
        for x in range(2):
            for got, ref in zip(outs[x], runs[x][2]):
                assert torch.equal(got, ref), (rep, x)


# --------------------------------------------------------------------------
# Pattern entry points
# --------------------------------------------------------------------------


def test_lognorm_closed_form_and_gauge(B):
    T = 32768
    lam = 0.01
    a = torch.zeros(1, T, dtype=torch.float32, device="cuda")
    r = (-lam * torch.arange(T, dtype=torch.float64)).float().cuda()[None]
    got = host(B.saf_pattern_lognorm(a, r, T))[0]
    i = np.arange(T)
    expect = np.log(-np.expm1(-lam * (i + 1))) - np.log(-np.expm1(-lam))
    say(f"  geometric closed form max-abs {max_abs(got, expect):.3e}")
    assert max_abs(got, expect) <= LSE_FRZ_ABS
    rng = np.random.default_rng(1)
    a0 = rng.standard_normal(T).astype(np.float32)
    r0 = np.where(i < 8, 3.0, -0.01 * i).astype(np.float32)
    a1 = (a0 + lam * i).astype(np.float32)
    r1 = (r0 + lam * i).astype(np.float32)
    L0 = host(B.saf_pattern_lognorm(torch.from_numpy(a0[None]).cuda(), torch.from_numpy(r0[None]).cuda(), T))[0]
    L1 = host(B.saf_pattern_lognorm(torch.from_numpy(a1[None]).cuda(), torch.from_numpy(r1[None]).cuda(), T))[0]
    # shifting a and r by lam*j and lam*d adds lam*i to log N; the oracle sees
    # the same fp32-rounded shifted inputs
    rows = np.unique(np.concatenate([np.arange(0, T, 97), [1, 7, 8, 9, T - 1]]))
    zero_v = np.zeros((T, 1))
    ref0 = oracle.frozen_rows_fwd(zero_v, a0, r0, rows)[1]
    ref1 = oracle.frozen_rows_fwd(zero_v, a1, r1, rows)[1]
    say(f"  peaked r: max-abs {max_abs(L0[rows], ref0):.3e}; shifted: {max_abs(L1[rows], ref1):.3e}")
    assert max_abs(L0[rows], ref0) <= LSE_FRZ_ABS
    assert max_abs(L1[rows], ref1) <= 4 * LSE_FRZ_ABS  # values reach ~330 here
    assert np.all(np.isfinite(L1))
    assert max_abs(L1 - L0, lam * i) <= 4 * LSE_FRZ_ABS


@pytest.mark.parametrize("T,Tp", [(1, 1), (129, 192), (1000, 1000)])
def test_pattern_dense_matches_oracle(B, T, Tp):
    rng = np.random.default_rng(T)
    a = rng.standard_normal(Tp).astype(np.float32)
    r = (-0.05 * np.arange(Tp) + 0.5 * rng.standard_normal(Tp)).astype(np.float32)
    W = host(B.saf_pattern_dense(torch.from_numpy(a).cuda(), torch.from_numpy(r).cuda(), T))
    ref = oracle.frozen_pattern(a, r, T)
    say(f"  T={T}: max-abs {max_abs(W, ref):.3e}")
    assert max_abs(W, ref) <= 1e-5
    assert np.all(np.triu(W, 1) == 0.0)
    np.testing.assert_allclose(W.sum(axis=1), 1.0, atol=1e-5)


def test_lognorm_special_patterns(B):
    T = 300
    i = np.arange(T)
    rng = np.random.default_rng(4)
    a = rng.standard_normal(T).astype(np.float32)
    ident = np.full(T, -np.inf, dtype=np.float32)
    ident[0] = 0.0
    window = np.where(i < 5, 0.0, -np.inf).astype(np.float32)
    got = host(B.saf_pattern_lognorm(torch.from_numpy(np.stack([a, np.zeros(T, np.float32)])).cuda(),
                                     torch.from_numpy(np.stack([ident, window])).cuda(), T))
    assert max_abs(got[0], a) <= 1e-6  # identity pattern: log N(i) = a[i]
    assert max_abs(got[1], np.log(np.minimum(i + 1, 5))) <= 1e-6


# --------------------------------------------------------------------------
# Workload shapes: sampled heads / rows against the oracle
# --------------------------------------------------------------------------

SAMPLES = {
    "gpt2_124m_4k_25pct": [(7, 0), (3, 10)],
    "gpt2_124m_4k_50pct_interleaved": [(0, 0), (5, 11)],
    "1b_8k_rank_share": [(1, 3), (0, 15)],
}


@pytest.mark.parametrize("key", list(SAMPLES))
def test_workload_sampled_heads(B, key):
    cfg = CONFIGS[key]
    say(f"workload {cfg.name}")
    inp = make_inputs(cfg)
    dev = upload(inp)
    fz = [int(x) for x in inp.frozen]
    O, L = B.saf_hybrid_attn_fwd(dev["q"], dev["k"], dev["v"], fz, dev["a"], dev["r"])
    dq, dk, dv = B.saf_hybrid_attn_bwd(dev["q"], dev["k"], dev["v"], O, dev["do"], L, fz, dev["a"], dev["r"])
    torch.cuda.synchronize()
    # properties at full size
    for h in range(cfg.H):
        if fz[h]:
            assert int(torch.count_nonzero(dq[:, h])) == 0 and int(torch.count_nonzero(dk[:, h])) == 0
    for t in (O, L, dq, dk, dv):
        assert bool(torch.isfinite(t.float()).all())
    s = 1.0 / np.sqrt(cfg.D)
    for b, h in SAMPLES[key]:
        say(f"  head b={b} h={h} frozen={fz[h]}")
        if fz[h]:
            ro, rl = oracle.frozen_head_fwd(inp.v[b, h], inp.a[h], inp.r[h])
            rdv = oracle.frozen_head_bwd(inp.do[b, h], inp.a[h], inp.r[h])
            rdq = rdk = None
        else:
            ro, rl = oracle.ordinary_head_fwd(inp.q[b, h], inp.k[b, h], inp.v[b, h], s)
            rdq, rdk, rdv = oracle.ordinary_head_bwd(inp.q[b, h], inp.k[b, h], inp.v[b, h], inp.do[b, h], s)
        _check_head(f"b{b}h{h}", cfg, host(O[b, h]), ro, host(L[b, h]), rl, fz[h])
        for n, g, rr in (("dQ", dq, rdq), ("dK", dk, rdk), ("dV", dv, rdv)):
            if rr is None:
                continue
            e = rel_l2(host(g[b, h]), rr)
            say(f"    {n} rel-L2 {e:.3e}")
            assert e <= BF16_GRAD_RELL2, (n, e)


def test_workload_prefill_32k_sampled_rows(B):
    cfg = CONFIGS["prefill_32k"]
    say(f"workload {cfg.name}")
    inp = make_inputs(cfg)
    dev = upload(inp)
    fz = [int(x) for x in inp.frozen]
    O, L = B.saf_hybrid_attn_fwd(dev["q"], dev["k"], dev["v"], fz, dev["a"], dev["r"])
    torch.cuda.synchronize()
    assert bool(torch.isfinite(O.float()).all()) and bool(torch.isfinite(L).all())
    T = cfg.T
    rows = np.unique(np.concatenate([[0, 1, 7, 8, 9, 127, 128, 4095, T - 2, T - 1],
                                     np.random.default_rng(0).integers(0, T, 40)]))
    s = 1.0 / np.sqrt(cfg.D)
    for h in (0, 5, 9, 11):
        if fz[h]:
            ro, rl = oracle.frozen_rows_fwd(inp.v[0, h], inp.a[h], inp.r[h], rows)
        else:
            ro, rl = oracle.ordinary_rows_fwd(inp.q[0, h], inp.k[0, h], inp.v[0, h], s, rows)
        _check_head(f"h{h} rows", cfg, host(O[0, h])[rows], ro, host(L[0, h])[rows], rl, fz[h])
    # log N of one frozen head on every 61st row
    h = 10
    rows = np.arange(0, T, 61)
    rl = oracle.frozen_rows_fwd(np.zeros((T, 1)), inp.a[h], inp.r[h], rows)[1]
    e = max_abs(host(L[0, h])[rows], rl)
    say(f"  h{h} log N on {len(rows)} rows max-abs {e:.3e}")
    assert e <= LSE_FRZ_ABS


@pytest.mark.parametrize("T", [8193, 16385])
def test_forward_normaliser_key_groups(B, T):
    """Normaliser partials over key groups of 512 (T = 8193: two chunks of
    256 keys per group) and 768 (T = 16385: three chunks) keys; sampled rows
    of both head kinds and log N of the frozen head."""
    cfg = CONFIGS["pages_check_t129"].with_(T=T, B=1, H=2, frozen=(1,), prior_len=None, bwd=False,
                                            name=f"keygroups_T{T}")
    say(f"case {cfg.name}")
    inp = make_inputs(cfg, with_do=False)
    dev = upload(inp)
    fz = [int(x) for x in inp.frozen]
    O, L = B.saf_hybrid_attn_fwd(dev["q"], dev["k"], dev["v"], fz, dev["a"], dev["r"])
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, 1, 255, 256, 511, 512, 767, 768, 1023, 1024, T - 2, T - 1],
                                     np.random.default_rng(T).integers(0, T, 30)]))
    s = 1.0 / np.sqrt(cfg.D)
    ro, rl = oracle.ordinary_rows_fwd(inp.q[0, 0], inp.k[0, 0], inp.v[0, 0], s, rows)
    _check_head("h0 rows", cfg, host(O[0, 0])[rows], ro, host(L[0, 0])[rows], rl, 0)
    ro, rl = oracle.frozen_rows_fwd(inp.v[0, 1], inp.a[1], inp.r[1], rows)
    _check_head("h1 rows", cfg, host(O[0, 1])[rows], ro, host(L[0, 1])[rows], rl, 1)
    rows = np.arange(0, T, 97)
    rl = oracle.frozen_rows_fwd(np.zeros((T, 1)), inp.a[1], inp.r[1], rows)[1]
    e = max_abs(host(L[0, 1])[rows], rl)
    say(f"  h1 log N on {len(rows)} rows max-abs {e:.3e}")
    assert e <= LSE_FRZ_ABS


# --------------------------------------------------------------------------
# Grouped-query forward (key/value heads shared by groups of query heads)
# --------------------------------------------------------------------------


def run_gqa_fwd_parity(B, cfg, strided=False):
    say(f"case {cfg.name} B={cfg.B} H={cfg.H} Hkv={cfg.Hkv} T={cfg.T} D={cfg.D} frozen={cfg.frozen} "
        f"{cfg.dtype} strided={strided}")
    inp = make_inputs(cfg, with_do=False)
    dev = upload(inp)
    q, k, v = dev["q"], dev["k"], dev["v"]
    if strided:
        k = k.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
        v = v.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    fz = [int(x) for x in inp.frozen]
    O, L = B.saf_hybrid_attn_fwd(q, k, v, fz, dev["a"], dev["r"])
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.hybrid_fwd(inp.q, inp.k, inp.v, fz, inp.a, inp.r)
    for h in range(cfg.H):
        _check_head(f"h{h}", cfg, host(O[:, h]), ref_o[:, h], host(L[:, h]), ref_l[:, h], fz[h])


@pytest.mark.parametrize("Hkv,mask", [(2, (1, 4, 5, 6, 7)), (2, ()), (2, tuple(range(8))), (1, (0, 3)),
                                      (4, (2, 3)), (8, (5,))])
def test_gqa_forward_groups_and_masks(B, Hkv, mask):
    cfg = CONFIGS["pages_check_t129"].with_(H=8, kv_heads=Hkv, B=3, T=300, prior_len=None, frozen=mask,
                                            bwd=False, name=f"gqa_kv{Hkv}_mask{len(mask)}")
    run_gqa_fwd_parity(B, cfg)


@pytest.mark.parametrize("D", [64, 96, 128])
def test_gqa_forward_head_dims(B, D):
    cfg = CONFIGS["pages_check_t129"].with_(H=8, kv_heads=2, D=D, B=2, T=257, prior_len=None, frozen=(3, 6),
                                            bwd=False, qkv_scale=0.5, name=f"gqa_D{D}")
    run_gqa_fwd_parity(B, cfg)


def test_gqa_forward_fp32_and_strided(B):
    run_gqa_fwd_parity(B, CONFIGS["tiny"].with_(H=8, kv_heads=4, T=70, B=2, frozen=(1, 6), bwd=False,
                                               name="gqa_fp32"))
    # d = 96 and 128: the fp32 rows are split over thread pairs
    for D in (96, 128):
        run_gqa_fwd_parity(B, CONFIGS["tiny"].with_(D=D, H=8, kv_heads=2, T=133, B=2, frozen=(0, 5),
                                                   bwd=False, name=f"gqa_fp32_D{D}"))
    run_gqa_fwd_parity(B, CONFIGS["pages_check_t129"].with_(H=8, kv_heads=2, B=2, T=200, prior_len=None,
                                                            frozen=(0, 5), bwd=False, name="gqa_strided"),
                       strided=True)


def test_gqa_rejected_by_backward(B):
    cfg = CONFIGS["pages_check_t129"].with_(H=8, kv_heads=2, B=1, T=64, prior_len=None, frozen=(1,),
                                            name="gqa_bwd")
    inp = make_inputs(cfg, with_do=True)
    dev = upload(inp)
    fz = [int(x) for x in inp.frozen]
    O, L = B.saf_hybrid_attn_fwd(dev["q"], dev["k"], dev["v"], fz, dev["a"], dev["r"])
    prm = B.Params(dev["q"], fz, dev["a"].shape[1], kv_heads=2)
    prm.set_strides(q=dev["q"], k=dev["k"], v=dev["v"], o=O, do=dev["do"], dq=O, dk=O, dv=O)
    ws = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    st = B.LIB.saf_hybrid_attn_bwd(prm.ref(), dev["q"].data_ptr(), dev["k"].data_ptr(), dev["v"].data_ptr(),
                                   O.data_ptr(), dev["do"].data_ptr(), L.data_ptr(), dev["a"].data_ptr(),
                                   dev["r"].data_ptr(), O.data_ptr(), O.data_ptr(), O.data_ptr(),
                                   ws.data_ptr(), ws.numel(), None)
    assert st == B.SAF_EUNSUPPORTED


def test_workload_qwen3_gqa_prefill_sampled_heads(B):
    cfg = CONFIGS["qwen3_4b_prefill_B4_T4096_30pct"]
    say(f"workload {cfg.name}")
    inp = make_inputs(cfg)
    dev = upload(inp)
    fz = [int(x) for x in inp.frozen]
    O, L = B.saf_hybrid_attn_fwd(dev["q"], dev["k"], dev["v"], fz, dev["a"], dev["r"])
    torch.cuda.synchronize()
    assert bool(torch.isfinite(O.float()).all()) and bool(torch.isfinite(L).all())
    g = cfg.H // cfg.Hkv
    s = 1.0 / np.sqrt(cfg.D)
    # an ordinary head and a frozen head of the partly frozen group 5, and a
    # head of a fully frozen group
    for b, h in ((3, 20), (0, 23), (2, 31), (1, 0)):
        say(f"  head b={b} h={h} (kv head {h // g}) frozen={fz[h]}")
        if fz[h]:
            ro, rl = oracle.frozen_head_fwd(inp.v[b, h // g], inp.a[h], inp.r[h])
        else:
            ro, rl = oracle.ordinary_head_fwd(inp.q[b, h], inp.k[b, h // g], inp.v[b, h // g], s)
        _check_head(f"b{b}h{h}", cfg, host(O[b, h]), ro, host(L[b, h]), rl, fz[h])


# --------------------------------------------------------------------------
# Precomputed normalisers (the stored log Z of the frozen heads)
# --------------------------------------------------------------------------


@pytest.mark.parametrize("key,kv", [("pages_check_t129", None), ("tiny", None), ("pages_check_t129", 2)])
def test_forward_with_precomputed_lognorm(B, key, kv):
    cfg = CONFIGS[key].with_(T=300 if key != "tiny" else 128, prior_len=None, B=2, H=8,
                             frozen=(1, 2, 6), name=f"logz_{key}_kv{kv}", kv_heads=kv, bwd=kv is None)
    say(f"case {cfg.name} dtype={cfg.dtype}")
    inp = make_inputs(cfg, with_do=kv is None)
    dev = upload(inp)
    fz = [int(x) for x in inp.frozen]
    logz = B.saf_pattern_lognorm(dev["a"], dev["r"], cfg.T)  # [H, T]
    O, L = B.saf_hybrid_attn_fwd(dev["q"], dev["k"], dev["v"], fz, dev["a"], dev["r"], logz=logz)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.hybrid_fwd(inp.q, inp.k, inp.v, fz, inp.a, inp.r)
    for h in range(cfg.H):
        _check_head(f"h{h}", cfg, host(O[:, h]), ref_o[:, h], host(L[:, h]), ref_l[:, h], fz[h])
        if fz[h]:
            for b in range(cfg.B):
                assert torch.equal(L[b, h], logz[h]), "frozen lse rows are the given log N"
    if kv is None:
        # the backward reads the copied normalisers from lse
        dq, dk, dv = B.saf_hybrid_attn_bwd(dev["q"], dev["k"], dev["v"], O, dev["do"], L, fz, dev["a"], dev["r"])
        torch.cuda.synchronize()
        ref_dq, ref_dk, ref_dv = oracle.hybrid_bwd(inp.q, inp.k, inp.v, inp.do, fz, inp.a, inp.r)
        bar = _bars(cfg)["g_rel"]
        for n, g, rr in (("dQ", dq, ref_dq), ("dK", dk, ref_dk), ("dV", dv, ref_dv)):
            e = rel_l2(host(g), rr)
            say(f"  {n} rel-L2 {e:.3e}")
            assert e <= bar, (n, e)


@pytest.mark.parametrize("spike", [60.0, 70.0])
def test_frozen_wide_range_patterns(B, spike):
    # a and r spiking at unrelated positions (a[0] = r[5] = spike): in log2
    # units the sum of their maxima exceeds the normaliser of rows like i = 1
    # by about spike * log2(e) -- 87 (factored weights, close to their 90
    # limit) or 101 (beyond it: those blocks take the per-weight
    # exponential).  Both must match the oracle.
    cfg = CONFIGS["pages_check_t129"].with_(T=400, prior_len=None, B=3, name=f"wide_range_{spike:g}")
    inp = make_inputs(cfg, with_do=True)
    for h in (1, 3):
        inp.a[h, 0] = spike
        inp.r[h, 5] = spike
        inp.a[h, 200] = -40.0
    dev = upload(inp)
    fz = [int(x) for x in inp.frozen]
    O, L = B.saf_hybrid_attn_fwd(dev["q"], dev["k"], dev["v"], fz, dev["a"], dev["r"])
    dq, dk, dv = B.saf_hybrid_attn_bwd(dev["q"], dev["k"], dev["v"], O, dev["do"], L, fz, dev["a"], dev["r"])
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.hybrid_fwd(inp.q, inp.k, inp.v, fz, inp.a, inp.r)
    ref_dv = oracle.hybrid_bwd(inp.q, inp.k, inp.v, inp.do, fz, inp.a, inp.r)[2]
    for h in (1, 3):
        _check_head(f"h{h}", cfg, host(O[:, h]), ref_o[:, h], host(L[:, h]), ref_l[:, h], True)
        e = rel_l2(host(dv[:, h]), ref_dv[:, h])
        say(f"  h{h} dV rel-L2 {e:.3e}")
        assert e <= BF16_GRAD_RELL2


# ---------------------------------------------------------------------------
# Packed Q/K layout: replaced heads have no query or key slot (Section 3.3,
# Appendix D.2).  The same kernels run with a head-to-slot map, so the
# results must equal the full layout's bit for bit.
# ---------------------------------------------------------------------------


def _packed_vs_full(B, cfg):
    inp = make_inputs(cfg, with_do=cfg.bwd)
    dev = upload(inp)
    fz = [int(x) for x in inp.frozen]
    ordh = [h for h in range(cfg.H) if not fz[h]]
    gqa = cfg.kv_heads not in (0, None, cfg.H)
    qp = dev["q"][:, ordh].contiguous() if ordh else None
    kp = (dev["k"] if gqa else dev["k"][:, ordh].contiguous()) if ordh else None
    say(f"packed Q/K: {cfg.name} frozen={tuple(h for h in range(cfg.H) if fz[h])}")
    O, L = B.saf_hybrid_attn_fwd(dev["q"], dev["k"], dev["v"], fz, dev["a"], dev["r"])
    Op, Lp = B.saf_hybrid_attn_fwd(qp, kp, dev["v"], fz, dev["a"], dev["r"], qk_packed=True)
    torch.cuda.synchronize()
    assert torch.equal(O, Op) and torch.equal(L, Lp)
    if not cfg.bwd:
        return
    dq, dk, dv = B.saf_hybrid_attn_bwd(dev["q"], dev["k"], dev["v"], O, dev["do"], L, fz, dev["a"], dev["r"])
    dqp, dkp, dvp = B.saf_hybrid_attn_bwd(qp, kp, dev["v"], O, dev["do"], L, fz, dev["a"], dev["r"],
                                          qk_packed=True)
    torch.cuda.synchronize()
    assert tuple(dqp.shape) == (cfg.B, len(ordh), cfg.T, cfg.D)
    assert torch.equal(dv, dvp)
    if ordh:
        assert torch.equal(dq[:, ordh], dqp) and torch.equal(dk[:, ordh], dkp)


@pytest.mark.parametrize("key,frozen", [("pages_check_t129", (3,)), ("pages_check_t129", (0, 2)),
                                        ("pages_check_t129", (0, 1, 2, 3)), ("pages_check_t129", ()),
                                        ("tiny", (1,)), ("tiny", (0, 1, 2, 3))])
def test_packed_qk_layout_matches_full(B, key, frozen):
    cfg = CONFIGS[key].with_(frozen=frozen, name=f"{key}_packed{len(frozen)}")
    _packed_vs_full(B, cfg)


def test_packed_q_grouped_query_forward(B):
    cfg = CONFIGS["pages_check_t129"].with_(H=8, kv_heads=2, B=2, T=200, prior_len=None, frozen=(1, 4, 5),
                                            bwd=False, name="gqa_packed_q")
    _packed_vs_full(B, cfg)
