"""Host-side checks of the C ABI: the library loads, exports every function
declared in include/saf_hybrid.h, its parameter block matches the binding, and
invalid arguments are rejected before anything touches the GPU."""

import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "saf_hybrid.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b(saf_\w+)\s*\(", src, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def b():
    from fixed_pattern_hybrid_amd import binding

    return binding


def test_header_declares_expected_entry_points():
    names = _declared_functions()
    for n in ("saf_hybrid_attn_fwd", "saf_hybrid_attn_bwd", "saf_pattern_dense"):
        assert n in names


def test_library_exports_every_declared_symbol(b):
    for n in _declared_functions():
        assert hasattr(b.LIB, n), n
    assert set(_declared_functions()) == set(b.EXPORTED)


def test_param_block_layout_matches_c(tmp_path, b):
    src = tmp_path / "sz.c"
    src.write_text(
        '#include <stdio.h>\n#include <stddef.h>\n#include "saf_hybrid.h"\n'
        "int main(void){printf(\"%zu %zu %zu %zu %zu %zu %zu\\n\", sizeof(saf_attn_params),"
        " offsetof(saf_attn_params, q_stride), offsetof(saf_attn_params, dv_stride),"
        " offsetof(saf_attn_params, frozen), offsetof(saf_attn_params, n_stage_events),"
        " offsetof(saf_attn_params, kv_heads), offsetof(saf_attn_params, logz));return 0;}\n"
    )
    exe = tmp_path / "sz"
    subprocess.run(["gcc", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", f"-I{ROOT}/include",
                    str(src), "-o", str(exe)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True).stdout.split()]
    P = b.SafParams
    want = [ctypes.sizeof(P), P.q_stride.offset, P.dv_stride.offset, P.frozen.offset, P.n_stage_events.offset,
            P.kv_heads.offset, P.logz.offset]
    assert got == want


def test_status_strings(b):
    for s in (0, -1, -2, -3, -4, 7):
        assert isinstance(b.status_string(s), str) and b.status_string(s)
    assert b.version()[0] >= 1


def _params(b, **kw):
    H = kw.get("H", 4)
    p = b.SafParams()
    p.struct_bytes = ctypes.sizeof(b.SafParams)
    p.B, p.H, p.T, p.D = kw.get("B", 1), H, kw.get("T", 16), kw.get("D", 64)
    p.prior_len = kw.get("prior_len", p.T)
    p.dtype = kw.get("dtype", b.SAF_BF16)
    p.softmax_scale = kw.get("scale", 0.0)
    for n in ("q", "k", "v", "o", "do", "dq", "dk", "dv"):
        setattr(p, n + "_stride", b._i64x3(p.H * p.T * p.D, p.T * p.D, p.D))
    arr = (ctypes.c_uint8 * H)(*kw.get("frozen", [0] * H))
    p.frozen = ctypes.cast(arr, ctypes.POINTER(ctypes.c_uint8))
    return p, arr


FAKE = 0x10000  # a 16-byte aligned non-null address; never dereferenced on these paths


@pytest.mark.parametrize(
    "mut,expect",
    [
        ({"struct_bytes": 3}, -1),
        ({"B": 0}, -1),
        ({"T": 0}, -1),
        ({"H": 300}, -2),
        ({"D": 80}, -2),
        ({"dtype": 5}, -2),
        ({"prior_len": 8}, -1),
        ({"kv_heads": 3}, -1),
        ({"kv_heads": -1}, -1),
        ({"kv_heads": 8}, -1),
        ({"softmax_scale": float("nan")}, -1),
        ({"qk_packed": 2}, -1),
        ({"qk_packed": -1}, -1),
    ],
)
def test_fwd_rejects_bad_params(b, mut, expect):
    p, arr = _params(b)
    for k, v in mut.items():
        setattr(p, k, v)
    st = b.LIB.saf_hybrid_attn_fwd(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None)
    assert st == expect


def test_fwd_rejects_bad_pointers_and_strides(b):
    p, arr = _params(b)
    call = lambda *x: b.LIB.saf_hybrid_attn_fwd(ctypes.byref(p), *x, None, 0, None)  # noqa: E731
    assert call(None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE) == -1  # q null, ordinary heads present
    assert call(FAKE + 2, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE) == -1  # misaligned
    assert call(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == -1  # lse null
    p.q_stride = b._i64x3(0, 0, 12)  # t stride not a multiple of 16 bytes
    assert call(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE) == -1
    p.q_stride = b._i64x3(0, 0, (1 << 24) + 8)  # t stride beyond SAF_MAX_T_STRIDE
    assert call(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE) == -2
    p.q_stride = b._i64x3(0, 0, 1 << 24)  # largest accepted t stride: the v tensor fails next
    assert call(FAKE, FAKE, FAKE + 2, FAKE, FAKE, FAKE, FAKE) == -1
    p2, arr2 = _params(b, frozen=[1, 1, 1, 1])  # all frozen: q/k unused, a/r required
    st = b.LIB.saf_hybrid_attn_fwd(ctypes.byref(p2), None, None, FAKE, None, FAKE, FAKE, FAKE, None, 0, None)
    assert st == -1
    p3, arr3 = _params(b, frozen=[0, 2, 0, 0])  # flags must be 0/1
    st = b.LIB.saf_hybrid_attn_fwd(ctypes.byref(p3), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None)
    assert st == -1


def test_bwd_workspace_checks(b):
    p, arr = _params(b, B=2, H=4, T=100)
    need = b.LIB.saf_hybrid_attn_workspace_bytes(ctypes.byref(p), 1)
    assert need >= 2 * 4 * 100 * 4 and need % 256 == 0
    assert b.LIB.saf_hybrid_attn_workspace_bytes(ctypes.byref(p), 0) == 0
    args = [FAKE] * 11
    assert b.LIB.saf_hybrid_attn_bwd(ctypes.byref(p), *args, None, need, None) == -3
    assert b.LIB.saf_hybrid_attn_bwd(ctypes.byref(p), *args, FAKE, need - 1, None) == -3
    assert b.LIB.saf_hybrid_attn_bwd(ctypes.byref(p), *args, FAKE + 16, need, None) == -3
    bad, _ = _params(b, D=48)
    assert b.LIB.saf_hybrid_attn_workspace_bytes(ctypes.byref(bad), 1) == 0


def test_grid_size_limits(b):
    args = [FAKE] * 7
    # bf16: B*H*T within 2^40 but B*H*ceil(T/128) programs beyond 2^31 - 1
    p, arr = _params(b, B=65535, H=256, T=32768, prior_len=32768)
    assert b.LIB.saf_hybrid_attn_fwd(ctypes.byref(p), *args, None, 0, None) == -2
    assert b.LIB.saf_hybrid_attn_workspace_bytes(ctypes.byref(p), 1) == 0
    # fp32: B*H beyond the 65535 limit of the grid's second dimension
    p2, arr2 = _params(b, B=300, H=256, T=16, dtype=b.SAF_F32)
    assert b.LIB.saf_hybrid_attn_fwd(ctypes.byref(p2), *args, None, 0, None) == -2
    # just inside both limits: rejected only later, on the fake pointers' alignment
    p3, arr3 = _params(b, B=255, H=256, T=16, dtype=b.SAF_F32)
    assert b.LIB.saf_hybrid_attn_fwd(ctypes.byref(p3), FAKE + 2, *args[1:], None, 0, None) == -1


def test_fwd_workspace_checks(b):
    # normaliser partials (float2 per frozen head, key group, row), then the
    # maxima of the frozen heads' a and r over 256-entry segments
    def fwd_ws(n_frz, groups, T):
        return _ru(n_frz * groups * T * 8) + _ru(2 * n_frz * -(-T // 256) * 4)

    T = 2100  # nine key groups of 256
    p, arr = _params(b, B=2, H=4, T=T, frozen=[0, 1, 0, 1])
    need = b.LIB.saf_hybrid_attn_workspace_bytes(ctypes.byref(p), 0)
    assert need == fwd_ws(2, 9, T)
    for T2, groups in ((256, 1), (257, 2), (8192, 32), (8193, 17), (32768, 32), (1 << 20, 32)):
        p2, arr2 = _params(b, B=1, H=4, T=T2, frozen=[0, 1, 0, 1])
        assert b.LIB.saf_hybrid_attn_workspace_bytes(ctypes.byref(p2), 0) == fwd_ws(2, groups, T2)
    args = [FAKE] * 7
    assert b.LIB.saf_hybrid_attn_fwd(ctypes.byref(p), *args, None, need, None) == -3
    assert b.LIB.saf_hybrid_attn_fwd(ctypes.byref(p), *args, FAKE, need - 1, None) == -3
    assert b.LIB.saf_hybrid_attn_fwd(ctypes.byref(p), *args, FAKE + 16, need, None) == -3
    p32, arr32 = _params(b, B=2, H=4, T=T, frozen=[0, 1, 0, 1], dtype=b.SAF_F32)
    assert b.LIB.saf_hybrid_attn_workspace_bytes(ctypes.byref(p32), 0) == 0
    p.logz = FAKE  # precomputed normalisers: no partials
    assert b.LIB.saf_hybrid_attn_workspace_bytes(ctypes.byref(p), 0) == 0
    p.logz = FAKE + 2
    assert b.LIB.saf_hybrid_attn_fwd(ctypes.byref(p), *args, FAKE, need, None) == -1
    p.logz = None
    pord, arro = _params(b, B=2, H=4, T=T)
    assert b.LIB.saf_hybrid_attn_workspace_bytes(ctypes.byref(pord), 0) == 0


def test_pattern_entry_points_reject(b):
    assert b.LIB.saf_pattern_dense(0, 4, FAKE, FAKE, FAKE, None) == -1
    assert b.LIB.saf_pattern_dense(8, 4, FAKE, FAKE, FAKE, None) == -1
    assert b.LIB.saf_pattern_dense(40000, 40000, FAKE, FAKE, FAKE, None) == -1
    assert b.LIB.saf_pattern_dense(8, 8, None, FAKE, FAKE, None) == -1
    assert b.LIB.saf_pattern_lognorm(0, 8, 8, FAKE, FAKE, FAKE, None) == -1
    assert b.LIB.saf_pattern_lognorm(2, 8, 7, FAKE, FAKE, FAKE, None) == -1
    assert b.LIB.saf_pattern_lognorm(2, 8, 8, FAKE, FAKE, FAKE + 1, None) == -1


def test_binding_has_no_cpu_fallback():
    src = open(os.path.join(ROOT, "fixed_pattern_hybrid_amd", "binding.py")).read()
    assert "oracle" not in src and "import numpy" not in src


def test_binding_rejects_mismatched_tensors(b):
    # The library sees only pointers and strides; the binding must refuse
    # tensors whose shape, dtype or device differs from v's before any call.
    import torch

    B_, H, T, D = 2, 3, 16, 64
    mk = lambda *s, dt=torch.bfloat16: torch.zeros(*s, dtype=dt)  # noqa: E731
    q, k, v = mk(B_, H, T, D), mk(B_, H, T, D), mk(B_, H, T, D)
    a, r = mk(H, T, dt=torch.float32), mk(H, T, dt=torch.float32)
    fz = [0, 1, 0]
    with pytest.raises(ValueError, match="shape"):
        b.saf_hybrid_attn_fwd(mk(B_, H, T - 1, D), k, v, fz, a, r)
    with pytest.raises(ValueError, match="dtype"):
        b.saf_hybrid_attn_fwd(q, k, v, fz, a, r, out=mk(B_, H, T, D, dt=torch.float16))
    with pytest.raises(ValueError, match="shape"):
        b.saf_hybrid_attn_fwd(q, k, v, fz, a, r, lse=mk(B_, H, T + 1, dt=torch.float32))
    with pytest.raises(ValueError, match="a and r"):
        b.saf_hybrid_attn_fwd(q, k, v, fz, a[:2], r[:2])
    with pytest.raises(ValueError, match="one entry per head"):
        b.Params(v, [0, 1], T)
    lse = mk(B_, H, T, dt=torch.float32)
    with pytest.raises(ValueError, match="shape"):
        b.saf_hybrid_attn_bwd(q, k, v, v, v, lse, fz, a, r, dq=mk(B_, H, T, D // 2))
    with pytest.raises(ValueError, match="dtype"):
        b.saf_hybrid_attn_bwd(q, k, v, v, mk(B_, H, T, D, dt=torch.float32), lse, fz, a, r)
    # well-formed host tensors pass every shape check and stop at the device check
    with pytest.raises(ValueError, match="GPU"):
        b.saf_hybrid_attn_fwd(q, k, v, fz, a, r)
    with pytest.raises(ValueError, match="GPU"):
        b.saf_hybrid_attn_bwd(q, k, v, v, v, lse, fz, a, r)


def test_binding_packed_layout_rejects_mismatched_tensors(b):
    # Packed Q/K layout: B, T and D come from v, so a caller's out, q or k
    # of another shape must be refused before the library is called.
    import torch

    B_, H, T, D = 1, 4, 64, 64
    fz = [0, 1, 0, 1]
    n_ord = 2
    mk = lambda *s, dt=torch.bfloat16: torch.zeros(*s, dtype=dt)  # noqa: E731
    q, k = mk(B_, n_ord, T, D), mk(B_, n_ord, T, D)
    v = mk(B_, H, T, D)
    a, r = mk(H, T, dt=torch.float32), mk(H, T, dt=torch.float32)
    # an out longer than v (the case that would read q/k/v and write lse
    # past their ends)
    with pytest.raises(ValueError, match="out has shape"):
        b.saf_hybrid_attn_fwd(q, k, v, fz, a, r, out=mk(B_, H, 4 * T, D), qk_packed=True)
    with pytest.raises(ValueError, match="out has shape"):
        b.saf_hybrid_attn_fwd(q, k, v, fz, a, r, out=mk(B_ + 1, H, T, D), qk_packed=True)
    with pytest.raises(ValueError, match="out has dtype"):
        b.saf_hybrid_attn_fwd(q, k, v, fz, a, r, out=mk(B_, H, T, D, dt=torch.float32), qk_packed=True)
    with pytest.raises(ValueError, match="q has shape"):
        b.saf_hybrid_attn_fwd(mk(B_, H, T, D), k, v, fz, a, r, qk_packed=True)
    with pytest.raises(ValueError, match="k has shape"):
        b.saf_hybrid_attn_fwd(q, mk(B_, n_ord, T + 1, D), v, fz, a, r, qk_packed=True)
    lse = mk(B_, H, T, dt=torch.float32)
    with pytest.raises(ValueError, match="q has shape"):
        b.saf_hybrid_attn_bwd(mk(B_, H, T, D), k, v, v, v, lse, fz, a, r, qk_packed=True)
    with pytest.raises(ValueError, match="dq has shape"):
        b.saf_hybrid_attn_bwd(q, k, v, v, v, lse, fz, a, r, dq=mk(B_, n_ord, T // 2, D), qk_packed=True)
    with pytest.raises(ValueError, match="shape"):
        b.saf_hybrid_attn_bwd(q, k, v, mk(B_, H, 2 * T, D), v, lse, fz, a, r, qk_packed=True)
    # consistent host tensors pass every shape check and stop at the device check
    with pytest.raises(ValueError, match="GPU"):
        b.saf_hybrid_attn_fwd(q, k, v, fz, a, r, out=mk(B_, H, T, D), qk_packed=True)
    with pytest.raises(ValueError, match="GPU"):
        b.saf_hybrid_attn_bwd(q, k, v, v, v, lse, fz, a, r, qk_packed=True)


def test_noalloc_forward_rejects_before_any_hip_call(b):
    # The no-allocation forward validates like the workspace forward and
    # refuses shapes whose normaliser partials exceed its static scratch,
    # all before touching the GPU (here there is none).
    import ctypes

    assert b.NOALLOC_SCRATCH_BYTES == 32 << 20
    assert "scratch" in b.status_string(b.SAF_ESCRATCH)
    FAKE = 1 << 20  # 16-byte aligned, never dereferenced on these paths
    T = 1 << 17
    fz = (ctypes.c_uint8 * 4)(0, 1, 1, 0)
    p = b.SafParams()
    p.struct_bytes = ctypes.sizeof(b.SafParams)
    p.B, p.H, p.T, p.D, p.prior_len, p.dtype = 1, 4, T, 64, T, b.SAF_BF16
    p.frozen = ctypes.cast(fz, ctypes.POINTER(ctypes.c_uint8))
    for name in ("q", "k", "v", "o"):
        setattr(p, name + "_stride", b._i64x3(4 * T * 64, T * 64, 64))
    need = b.LIB.saf_hybrid_attn_workspace_bytes(ctypes.byref(p), 0)
    assert need > b.NOALLOC_SCRATCH_BYTES  # 2 frozen heads x 32 groups x 2^17 rows x 8 B
    args = [FAKE] * 7
    assert b.LIB.saf_hybrid_attn_fwd_noalloc(ctypes.byref(p), *args, None) == b.SAF_ESCRATCH
    # argument errors come first, as in the workspace forward
    bad = list(args)
    bad[6] = FAKE + 2  # misaligned lse
    assert b.LIB.saf_hybrid_attn_fwd_noalloc(ctypes.byref(p), *bad, None) == b.SAF_EINVAL
    p.D = 80
    assert b.LIB.saf_hybrid_attn_fwd_noalloc(ctypes.byref(p), *args, None) == b.SAF_EUNSUPPORTED


def test_pattern_grad_workspace_and_rejects(b):
    # bf16: D_b of frozen rows, then per program (frozen head, batch group of
    # 2, key block of 128, query chunk of 512) 128 column and 640 diagonal
    # partial sums
    B_, H, T = 3, 4, 600
    p, arr = _params(b, B=B_, H=H, T=T, frozen=[0, 1, 1, 0])
    ru = lambda x: -(-x // 256) * 256  # noqa: E731
    progs = 2 * 2 * 5 * 2
    want = ru(2 * B_ * T * 4) + ru(progs * 128 * 4) + ru(progs * 640 * 4)
    need = b.LIB.saf_pattern_grad_workspace_bytes(ctypes.byref(p))
    assert need == want
    p32, a32 = _params(b, B=B_, H=H, T=T, frozen=[0, 1, 1, 0], dtype=b.SAF_F32)
    assert b.LIB.saf_pattern_grad_workspace_bytes(ctypes.byref(p32)) == ru(2 * B_ * T * 4)
    pord, ao = _params(b, B=B_, H=H, T=T)
    assert b.LIB.saf_pattern_grad_workspace_bytes(ctypes.byref(pord)) == 0
    bad, ab = _params(b, D=48)
    assert b.LIB.saf_pattern_grad_workspace_bytes(ctypes.byref(bad)) == 0
    args = [FAKE] * 8  # v, o, dout, lse, a, r, da, dr
    g = b.LIB.saf_pattern_grad
    assert g(ctypes.byref(p), *args, None, need, None) == -3
    assert g(ctypes.byref(p), *args, FAKE, need - 1, None) == -3
    assert g(ctypes.byref(p), *args, FAKE + 16, need, None) == -3
    for k in range(8):
        a2 = list(args)
        a2[k] = None
        assert g(ctypes.byref(p), *a2, FAKE, need, None) == -1, k
    a2 = list(args)
    a2[6] = FAKE + 2  # da misaligned
    assert g(ctypes.byref(p), *a2, FAKE, need, None) == -1
    bad2, ab2 = _params(b, B=B_, H=H, T=T, frozen=[0, 1, 1, 0], prior_len=T - 1)
    assert g(ctypes.byref(bad2), *args, FAKE, need, None) == -1
    # more than 2^31 - 1 programs (B*H*T within the layer's limits)
    big, abig = _params(b, B=256, H=256, T=1 << 20, frozen=[1] * 256)
    assert g(ctypes.byref(big), *args, FAKE, 1 << 62, None) == -2
    # no frozen head: valid, nothing to do, no workspace needed
    assert g(ctypes.byref(pord), *args, None, 0, None) == 0


def test_binding_pattern_grad_checks(b):
    import torch

    B_, H, T, D = 2, 3, 16, 64
    mk = lambda *s, dt=torch.bfloat16: torch.zeros(*s, dtype=dt)  # noqa: E731
    v, o, do = mk(B_, H, T, D), mk(B_, H, T, D), mk(B_, H, T, D)
    a, r = mk(H, T, dt=torch.float32), mk(H, T, dt=torch.float32)
    lse = mk(B_, H, T, dt=torch.float32)
    fz = [0, 1, 0]
    with pytest.raises(ValueError, match="shape"):
        b.saf_pattern_grad(v, mk(B_, H, T - 1, D), do, lse, fz, a, r)
    with pytest.raises(ValueError, match="shape"):
        b.saf_pattern_grad(v, o, do, lse, fz, a, r, da=mk(H, T + 1, dt=torch.float32))
    with pytest.raises(ValueError, match="dtype"):
        b.saf_pattern_grad(v, o, do, lse, fz, a, r, dr=mk(H, T, dt=torch.float64))
    with pytest.raises(ValueError, match="GPU"):
        b.saf_pattern_grad(v, o, do, lse, fz, a, r)


def test_grouped_query_params(b):
    # kv_heads divides H: accepted by the forward (rejected here only by the
    # misaligned lse pointer), refused by the backward and the pattern
    # gradients (grouped-query layouts are a prefill path)
    p, arr = _params(b, B=2, H=8, T=64, frozen=[0, 0, 0, 1, 0, 0, 1, 1])
    p.kv_heads = 2
    args = [FAKE] * 6
    assert b.LIB.saf_hybrid_attn_fwd(ctypes.byref(p), *args, FAKE + 2, FAKE, 1 << 20, None) == -1
    assert b.LIB.saf_hybrid_attn_bwd(ctypes.byref(p), *([FAKE] * 11), FAKE, 1 << 20, None) == -2
    assert b.LIB.saf_pattern_grad(ctypes.byref(p), *([FAKE] * 8), FAKE, 1 << 20, None) == -2
    p.kv_heads = 8  # = H: multi-head; rejected only by the misaligned lse pointer
    bargs = [FAKE] * 11
    bargs[5] = FAKE + 2
    assert b.LIB.saf_hybrid_attn_bwd(ctypes.byref(p), *bargs, FAKE, 1 << 20, None) == -1


def test_binding_grouped_query_checks(b):
    import torch

    B_, H, Hk, T, D = 2, 8, 2, 16, 64
    mk = lambda *s, dt=torch.bfloat16: torch.zeros(*s, dtype=dt)  # noqa: E731
    q, k, v = mk(B_, H, T, D), mk(B_, Hk, T, D), mk(B_, Hk, T, D)
    a, r = mk(H, T, dt=torch.float32), mk(H, T, dt=torch.float32)
    fz = [0] * H
    with pytest.raises(ValueError, match="divide"):
        b.saf_hybrid_attn_fwd(q, mk(B_, 3, T, D), mk(B_, 3, T, D), fz, a, r)
    with pytest.raises(ValueError, match="shape"):
        b.saf_hybrid_attn_fwd(q, k, mk(B_, Hk * 2, T, D), fz, a, r)
    with pytest.raises(ValueError, match="a and r"):
        b.saf_hybrid_attn_fwd(q, k, v, fz, a[:Hk], r[:Hk])
    with pytest.raises(ValueError, match="GPU"):
        b.saf_hybrid_attn_fwd(q, k, v, fz, a, r)


def _ru(x, a=256):
    return -(-x // a) * a


def test_fit_workspace_sizes(b):
    L = b.LIB
    assert L.saf_fit_targets_workspace_bytes(0, 10) == 0
    assert L.saf_fit_targets_workspace_bytes(3, 0) == 0
    assert L.saf_fit_targets_workspace_bytes(16385, 10) == 0
    # row sums and entropies [n][T], partial marginals [n][2][ceil(T/512)][T]
    assert L.saf_fit_targets_workspace_bytes(3, 1000) == 2 * _ru(3000 * 4) + _ru(3000 * 5 * 2 * 4)
    assert L.saf_fit_targets_workspace_bytes(36, 4096) == 2 * _ru(36 * 4096 * 4) + _ru(36 * 4096 * 5 * 8 * 4)
    # second parameter buffer and four moment vectors, five arrays of
    # 256-entry segment maxima (a and r of both buffers, -log N), then float2
    # partials of chunk groups (4 chunks of 256) for the normalisers and both
    # marginals, each 256-byte aligned
    def fit_ws(n, T):
        nseg = -(-T // 256)
        maxg = -(-nseg // 4)
        part = n * maxg * T * 8
        return 6 * _ru(n * T * 4) + 5 * _ru(n * nseg * 4) + _ru(part) + _ru(2 * part)
    assert L.saf_fit_pattern_workspace_bytes(3, 1000) == fit_ws(3, 1000)
    assert L.saf_fit_pattern_workspace_bytes(36, 4096) == fit_ws(36, 4096)
    assert fit_ws(36, 4096) == 6 * _ru(36 * 4096 * 4) + 5 * _ru(36 * 16 * 4) + 3 * 36 * 4 * 4096 * 8
    assert L.saf_fit_pattern_workspace_bytes(1, 1) == 13 * 256
    assert L.saf_fit_pattern_workspace_bytes(0, 5) == 0
    assert L.saf_fit_pattern_workspace_bytes(2, (1 << 20) + 1) == 0


def test_fit_targets_rejects_before_launch(b):
    L = b.LIB
    n, T = 2, 100
    need = L.saf_fit_targets_workspace_bytes(n, T)
    ok = dict(n=n, T=T, ahat=FAKE, hs=T * T, rs=T, floor=1e-9, ea=FAKE, er=FAKE, ne=FAKE, ws=FAKE, wsb=need)

    def call(**kw):
        x = {**ok, **kw}
        return L.saf_fit_targets(x["n"], x["T"], x["ahat"], x["hs"], x["rs"], x["floor"], x["ea"], x["er"],
                                 x["ne"], x["ws"], x["wsb"], None)

    assert call(n=0) == -1
    assert call(T=0) == -1
    assert call(floor=0.0) == -1
    assert call(floor=float("inf")) == -1
    assert call(floor=float("nan")) == -1
    assert call(ahat=None) == -1
    assert call(ahat=FAKE + 2) == -1  # 4-byte alignment
    assert call(rs=T - 1) == -1
    assert call(hs=-4) == -1
    assert call(ea=None) == -1
    assert call(ne=FAKE + 2) == -1
    assert call(ws=None) == -3
    assert call(wsb=need - 1) == -3
    assert call(ws=FAKE + 16) == -3


def test_fit_pattern_rejects_before_launch(b):
    L = b.LIB
    n, T = 2, 100
    need = L.saf_fit_pattern_workspace_bytes(n, T)
    ok = dict(n=n, T=T, ea=FAKE, er=FAKE, ne=FAKE, steps=400, lr=0.05, b1=0.9, b2=0.999, eps=1e-8,
              a=FAKE, r=FAKE, z=FAKE, loss=FAKE, kappa=FAKE, ws=FAKE, wsb=need)

    def call(**kw):
        x = {**ok, **kw}
        return L.saf_fit_pattern(x["n"], x["T"], x["ea"], x["er"], x["ne"], x["steps"], x["lr"], x["b1"],
                                 x["b2"], x["eps"], x["a"], x["r"], x["z"], x["loss"], x["kappa"], x["ws"],
                                 x["wsb"], None)

    assert call(n=0) == -1
    assert call(T=0) == -1
    assert call(steps=-1) == -1
    assert call(lr=0.0) == -1
    assert call(lr=float("nan")) == -1
    assert call(b1=1.0) == -1
    assert call(b2=-0.1) == -1
    assert call(eps=0.0) == -1
    assert call(ea=None) == -1
    assert call(z=FAKE + 1) == -1
    assert call(ne=None) == -1  # kappa needs negent
    assert call(loss=FAKE + 2) == -1
    assert call(ws=None) == -3
    assert call(wsb=need - 1) == -3
    assert call(ws=FAKE + 64) == -3


def test_fit_binding_checks_without_gpu(b):
    import torch

    with pytest.raises(ValueError):
        b.saf_fit_targets(torch.zeros(4, 4))  # not a GPU tensor
    with pytest.raises(ValueError):
        b.saf_fit_pattern(torch.zeros(2, 4), torch.zeros(2, 4))


def test_calib_workspace_and_rejects(b):
    L = b.LIB
    # row log-sum-exps [N][H][T] fp32, then [H][nqb (nqb + 1)][3] fp64 partials
    nqb = -(-300 // 128)
    assert L.saf_calib_stats_workspace_bytes(4, 3, 300) == _ru(4 * 3 * 300 * 4) + _ru(3 * nqb * (nqb + 1) * 3 * 8)
    assert L.saf_calib_stats_workspace_bytes(0, 3, 300) == 0
    assert L.saf_calib_stats_workspace_bytes(4, 0, 300) == 0
    assert L.saf_calib_stats_workspace_bytes(4, 3, 0) == 0
    N, H, T, D = 2, 2, 100, 64
    need = L.saf_calib_stats_workspace_bytes(N, H, T)
    st = (ctypes.c_int64 * 3)(H * T * D, T * D, D)
    ok = dict(N=N, H=H, T=T, D=D, scale=0.0, q=FAKE, qs=st, k=FAKE, ks=st, a=FAKE, ah=T * T, ar=T,
              sv=FAKE, sk=FAKE, ws=FAKE, wsb=need)

    def call(**kw):
        x = {**ok, **kw}
        return L.saf_calib_stats(x["N"], x["H"], x["T"], x["D"], x["scale"], x["q"], x["qs"], x["k"], x["ks"],
                                 x["a"], x["ah"], x["ar"], x["sv"], x["sk"], x["ws"], x["wsb"], None)

    assert call(N=0) == -1
    assert call(T=0) == -1
    assert call(D=80) == -2
    assert call(scale=float("nan")) == -1
    assert call(q=None) == -1
    assert call(k=FAKE + 8) == -1  # 16-byte alignment
    bad = (ctypes.c_int64 * 3)(H * T * D, T * D, D + 4)  # row stride not a multiple of 8
    assert call(qs=bad) == -1
    short = (ctypes.c_int64 * 3)(H * T * D, T * D, 32)  # rows shorter than D
    assert call(ks=short) == -1
    assert call(a=FAKE + 2) == -1
    assert call(ar=T - 1) == -1
    assert call(ah=-4) == -1
    assert call(sv=FAKE + 4) == -1  # fp64 alignment
    assert call(sk=None) == -1
    assert call(ws=None) == -3
    assert call(wsb=need - 1) == -3
