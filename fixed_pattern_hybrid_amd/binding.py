"""ctypes binding of libsaf_hybrid.so (argument marshalling only).

Every computation runs in the HIP library; this module only turns torch
tensors into pointers, strides and a parameter block, allocates outputs and
the workspace with torch, and raises on a non-zero status.  If the library is
missing, importing this module raises -- there is no fallback.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsaf_hybrid.so")

SAF_OK = 0
SAF_EINVAL = -1
SAF_EUNSUPPORTED = -2
SAF_EWORKSPACE = -3
SAF_EHIP = -4
SAF_ESCRATCH = -5
NOALLOC_SCRATCH_BYTES = 32 << 20
SAF_F32 = 0
SAF_BF16 = 1

EXPORTED = (
    "saf_hybrid_attn_fwd",
    "saf_hybrid_attn_fwd_noalloc",
    "saf_hybrid_attn_bwd",
    "saf_hybrid_attn_workspace_bytes",
    "saf_pattern_dense",
    "saf_pattern_grad",
    "saf_pattern_grad_workspace_bytes",
    "saf_pattern_lognorm",
    "saf_fit_targets",
    "saf_fit_targets_workspace_bytes",
    "saf_fit_pattern",
    "saf_fit_pattern_workspace_bytes",
    "saf_calib_stats",
    "saf_calib_stats_workspace_bytes",
    "saf_status_string",
    "saf_version",
)

_i64x3 = ctypes.c_int64 * 3


class SafParams(ctypes.Structure):
    """Mirror of ``saf_attn_params`` in include/saf_hybrid.h."""

    _fields_ = [
        ("struct_bytes", ctypes.c_uint32),
        ("B", ctypes.c_int32),
        ("H", ctypes.c_int32),
        ("T", ctypes.c_int32),
        ("D", ctypes.c_int32),
        ("prior_len", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("q_stride", _i64x3),
        ("k_stride", _i64x3),
        ("v_stride", _i64x3),
        ("o_stride", _i64x3),
        ("do_stride", _i64x3),
        ("dq_stride", _i64x3),
        ("dk_stride", _i64x3),
        ("dv_stride", _i64x3),
        ("frozen", ctypes.POINTER(ctypes.c_uint8)),
        ("stage_events", ctypes.c_void_p),
        ("n_stage_events", ctypes.c_int32),
        ("kv_heads", ctypes.c_int32),
        ("logz", ctypes.c_void_p),
        ("qk_packed", ctypes.c_int32),
        ("fused_dq", ctypes.c_int32),
    ]


class SafError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: status {status} ({status_string(status)})")


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m fixed_pattern_hybrid_amd.build` "
            "(the HIP library is required; there is no CPU fallback)"
        )
    lib = ctypes.CDLL(LIB_PATH)
    vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32
    pp = ctypes.POINTER(SafParams)
    lib.saf_hybrid_attn_fwd.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.saf_hybrid_attn_fwd.restype = ctypes.c_int
    lib.saf_hybrid_attn_fwd_noalloc.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.saf_hybrid_attn_fwd_noalloc.restype = ctypes.c_int
    lib.saf_hybrid_attn_bwd.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.saf_hybrid_attn_bwd.restype = ctypes.c_int
    lib.saf_hybrid_attn_workspace_bytes.argtypes = [pp, ctypes.c_int]
    lib.saf_hybrid_attn_workspace_bytes.restype = sz
    lib.saf_pattern_grad.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.saf_pattern_grad.restype = ctypes.c_int
    lib.saf_pattern_grad_workspace_bytes.argtypes = [pp]
    lib.saf_pattern_grad_workspace_bytes.restype = sz
    lib.saf_pattern_dense.argtypes = [i32, i32, vp, vp, vp, vp]
    lib.saf_pattern_dense.restype = ctypes.c_int
    lib.saf_pattern_lognorm.argtypes = [i32, i32, i32, vp, vp, vp, vp]
    lib.saf_pattern_lognorm.restype = ctypes.c_int
    f32, i64 = ctypes.c_float, ctypes.c_int64
    lib.saf_fit_targets.argtypes = [i32, i32, vp, i64, i64, f32, vp, vp, vp, vp, sz, vp]
    lib.saf_fit_targets.restype = ctypes.c_int
    lib.saf_fit_targets_workspace_bytes.argtypes = [i32, i32]
    lib.saf_fit_targets_workspace_bytes.restype = sz
    lib.saf_fit_pattern.argtypes = [i32, i32, vp, vp, vp, i32, f32, f32, f32, f32,
                                    vp, vp, vp, vp, vp, vp, sz, vp]
    lib.saf_fit_pattern.restype = ctypes.c_int
    lib.saf_fit_pattern_workspace_bytes.argtypes = [i32, i32]
    lib.saf_fit_pattern_workspace_bytes.restype = sz
    lib.saf_calib_stats.argtypes = [i32, i32, i32, i32, f32, vp, ctypes.POINTER(ctypes.c_int64), vp,
                                    ctypes.POINTER(ctypes.c_int64), vp, i64, i64, vp, vp, vp, sz, vp]
    lib.saf_calib_stats.restype = ctypes.c_int
    lib.saf_calib_stats_workspace_bytes.argtypes = [i32, i32, i32]
    lib.saf_calib_stats_workspace_bytes.restype = sz
    lib.saf_status_string.argtypes = [ctypes.c_int]
    lib.saf_status_string.restype = ctypes.c_char_p
    lib.saf_version.argtypes = []
    lib.saf_version.restype = ctypes.c_int32
    return lib


LIB = _load()


def status_string(status: int) -> str:
    return LIB.saf_status_string(int(status)).decode()


def version() -> Tuple[int, int]:
    v = LIB.saf_version()
    return (v >> 16, v & 0xFFFF)


def _check(status: int, what: str) -> None:
    if status != SAF_OK:
        raise SafError(status, what)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stride3(t: Optional[torch.Tensor]):
    if t is None:
        return _i64x3(0, 0, 0)
    if t.dim() != 4 or t.stride(3) != 1:
        raise ValueError("expected a [B, H, T, D] tensor with unit stride on D")
    return _i64x3(t.stride(0), t.stride(1), t.stride(2))


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return SAF_BF16
    if t.dtype == torch.float32:
        return SAF_F32
    raise ValueError(f"unsupported dtype {t.dtype}")


def _check_like(name: str, t, ref: torch.Tensor, shape=None, dtype=None) -> None:
    """t must match ref's device and the given (default: ref's) shape and dtype.

    The library sees only pointers and strides, so a smaller or differently
    typed tensor would be read or written past its end; this is where that
    is caught.
    """
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    want_shape = tuple(ref.shape) if shape is None else tuple(shape)
    want_dtype = ref.dtype if dtype is None else dtype
    if tuple(t.shape) != want_shape:
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {want_shape}")
    if t.dtype != want_dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {want_dtype}")
    if t.device != ref.device:
        raise ValueError(f"{name} is on {t.device}, expected {ref.device}")


def _check_layer_inputs(v: torch.Tensor, a: torch.Tensor, r: torch.Tensor, **tensors) -> None:
    if v.dim() != 4:
        raise ValueError("v must be [B, H, T, D]")
    _dtype_code(v)
    H = v.shape[1]
    if a.dim() != 2 or a.shape[0] != H:
        raise ValueError("a and r must both be [H, Tp]")
    _check_like("r", r, a)
    if a.dtype != torch.float32 or not a.is_contiguous() or not r.is_contiguous():
        raise ValueError("a and r must be contiguous float32 [H, Tp]")
    if a.device != v.device:
        raise ValueError("a and r must be on the device of v")
    for name, t in tensors.items():
        _check_like(name, t, v)


def _require_gpu(v: torch.Tensor) -> None:
    if not v.is_cuda:
        raise ValueError("tensors must be on a GPU")


def _stream_handle(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


class Params:
    """Owns a SafParams block and the host arrays it points to."""

    def __init__(self, v: torch.Tensor, frozen: Sequence[int], prior_len: int,
                 softmax_scale: Optional[float] = None, events=None, kv_heads: int = 0):
        """v: any [B, H, T, D] tensor of the call (query heads); kv_heads: key/value
        heads of a grouped-query call (0: as many as query heads)."""
        B, H, T, D = v.shape
        if len(frozen) != H:
            raise ValueError("frozen mask needs one entry per head")
        self.frozen_arr = (ctypes.c_uint8 * H)(*[int(x) for x in frozen])
        self.p = SafParams()
        self.p.struct_bytes = ctypes.sizeof(SafParams)
        self.p.B, self.p.H, self.p.T, self.p.D = B, H, T, D
        self.p.prior_len = int(prior_len)
        self.p.dtype = _dtype_code(v)
        self.p.softmax_scale = 0.0 if softmax_scale is None else float(softmax_scale)
        self.p.frozen = ctypes.cast(self.frozen_arr, ctypes.POINTER(ctypes.c_uint8))
        self.p.kv_heads = int(kv_heads)
        self.events_arr = None
        if events:
            handles = [int(e.cuda_event) for e in events]
            self.events_arr = (ctypes.c_void_p * len(handles))(*handles)
            self.p.stage_events = ctypes.cast(self.events_arr, ctypes.c_void_p)
            self.p.n_stage_events = len(handles)

    def set_strides(self, **tensors):
        for name, t in tensors.items():
            setattr(self.p, name + "_stride", _stride3(t))

    def ref(self):
        return ctypes.byref(self.p)


def workspace_bytes(params: Params, for_bwd: bool) -> int:
    return int(LIB.saf_hybrid_attn_workspace_bytes(params.ref(), 1 if for_bwd else 0))


def _n_ordinary(frozen) -> int:
    return len(frozen) - sum(int(x) for x in frozen)


def _fwd_call(prm, q, k, v, a, r, out, lse, ws, ws_n, stream, noalloc):
    if noalloc:
        st = LIB.saf_hybrid_attn_fwd_noalloc(prm.ref(), q, k, _ptr(v), _ptr(a), _ptr(r), _ptr(out),
                                             _ptr(lse), _stream_handle(stream))
        _check(st, "saf_hybrid_attn_fwd_noalloc")
    else:
        st = LIB.saf_hybrid_attn_fwd(prm.ref(), q, k, _ptr(v), _ptr(a), _ptr(r), _ptr(out), _ptr(lse),
                                     _ptr(ws), ws_n, _stream_handle(stream))
        _check(st, "saf_hybrid_attn_fwd")


def _fwd_packed(q, k, v, frozen, a, r, softmax_scale, out, lse, workspace, stream, events, logz,
                noalloc=False):
    """saf_hybrid_attn_fwd with q (and k, for multi-head K/V) holding only
    the ordinary heads, in increasing head order."""
    if not isinstance(v, torch.Tensor) or v.dim() != 4:
        raise ValueError("v must be a [B, Hkv, T, D] tensor")
    H, n_ord = len(frozen), _n_ordinary(frozen)
    B, Hkv, T, D = v.shape
    if Hkv < 1 or H % Hkv != 0:
        raise ValueError(f"v has {Hkv} heads, which must divide the {H} heads of the frozen mask")
    if out is None:
        out = torch.empty((B, H, T, D), dtype=v.dtype, device=v.device)
    # B, T and D of the call come from v: a caller's out must have exactly
    # v's batch, length and head dimension with all H heads
    _check_like("out", out, v, shape=(B, H, T, D))
    _check_layer_inputs(out, a, r)
    if n_ord > 0:
        _check_like("q", q, out, shape=(B, n_ord, T, D))
        _check_like("k", k, out, shape=(B, n_ord if Hkv == H else Hkv, T, D))
    if lse is None:
        lse = torch.empty((B, H, T), dtype=torch.float32, device=v.device)
    _check_like("lse", lse, out, shape=(B, H, T), dtype=torch.float32)
    if not lse.is_contiguous():
        raise ValueError("lse must be contiguous float32 [B, H, T]")
    if logz is not None:
        _check_like("logz", logz, out, shape=(H, T), dtype=torch.float32)
        if not logz.is_contiguous():
            raise ValueError("logz must be contiguous float32 [H, T]")
    _require_gpu(v)
    prm = Params(out, frozen, a.shape[1], softmax_scale, events, kv_heads=0 if Hkv == H else Hkv)
    prm.p.qk_packed = 1
    prm.set_strides(v=v, o=out, **({"q": q, "k": k} if n_ord > 0 else {}))
    prm.p.logz = _ptr(logz)
    ws, ws_n = None, 0
    if noalloc:
        pass
    elif workspace is not None:
        _check_like("workspace", workspace, v, shape=workspace.shape, dtype=workspace.dtype)
        ws, ws_n = workspace, workspace.numel() * workspace.element_size()
    else:
        ws_n = workspace_bytes(prm, False)
        ws = torch.empty(ws_n, dtype=torch.uint8, device=v.device) if ws_n else None
    qp, kp = (_ptr(q), _ptr(k)) if n_ord > 0 else (None, None)
    _fwd_call(prm, qp, kp, v, a, r, out, lse, ws, ws_n, stream, noalloc)
    return out, lse


def saf_hybrid_attn_fwd(q, k, v, frozen, a, r, softmax_scale=None, out=None, lse=None,
                        workspace=None, stream=None, events=None, logz=None, qk_packed=False,
                        _noalloc=False):
    """Forward of the hybrid layer; returns (O, lse).

    q: [B, H, T, D]; k, v: [B, Hkv, T, D] with Hkv dividing H (grouped-query
    attention when Hkv < H); bf16 or fp32 CUDA tensors (unit stride on D);
    frozen: length-H sequence of 0/1; a, r: fp32 [H, Tp] contiguous.
    logz: optional fp32 [H, T] precomputed log N of the frozen heads (as
    saf_pattern_lognorm(a, r, T) returns it); the call then skips the
    normaliser computation and copies it into lse.
    qk_packed: q (and k with multi-head K/V) hold only the ordinary heads in
    increasing head order ([B, n_ordinary, T, D]); out is [B, H, T, D].
    """
    if qk_packed:
        return _fwd_packed(q, k, v, frozen, a, r, softmax_scale, out, lse, workspace, stream, events, logz,
                           _noalloc)
    if not isinstance(k, torch.Tensor) or k.dim() != 4 or q.dim() != 4:
        raise ValueError("q, k and v must be [B, H, T, D] tensors")
    if k.shape[0] != q.shape[0] or k.shape[2:] != q.shape[2:]:
        raise ValueError(f"k has shape {tuple(k.shape)}, expected (B, Hkv, T, D) matching q {tuple(q.shape)}")
    Hk = k.shape[1]
    if Hk < 1 or q.shape[1] % Hk != 0:
        raise ValueError(f"k and v have {Hk} heads, which must divide the {q.shape[1]} query heads")
    _check_like("v", v, k)
    _check_layer_inputs(q, a, r, **({} if out is None else {"out": out}))
    _check_like("k", k, q, shape=(q.shape[0], Hk) + tuple(q.shape[2:]))
    B, H, T, D = q.shape
    if out is None:
        out = torch.empty((B, H, T, D), dtype=v.dtype, device=v.device)
    if lse is None:
        lse = torch.empty((B, H, T), dtype=torch.float32, device=v.device)
    _check_like("lse", lse, v, shape=(B, H, T), dtype=torch.float32)
    if not lse.is_contiguous():
        raise ValueError("lse must be contiguous float32 [B, H, T]")
    if workspace is not None:
        _check_like("workspace", workspace, v, shape=workspace.shape, dtype=workspace.dtype)
    if logz is not None:
        _check_like("logz", logz, q, shape=(H, T), dtype=torch.float32)
        if not logz.is_contiguous():
            raise ValueError("logz must be contiguous float32 [H, T]")
    _require_gpu(v)
    prm = Params(q, frozen, a.shape[1], softmax_scale, events, kv_heads=0 if Hk == H else Hk)
    prm.set_strides(q=q, k=k, v=v, o=out)
    prm.p.logz = _ptr(logz)
    ws, ws_n = None, 0
    if _noalloc:
        pass
    elif workspace is not None:
        ws, ws_n = workspace, workspace.numel() * workspace.element_size()
    else:
        ws_n = workspace_bytes(prm, False)
        ws = torch.empty(ws_n, dtype=torch.uint8, device=v.device) if ws_n else None
    _fwd_call(prm, _ptr(q), _ptr(k), v, a, r, out, lse, ws, ws_n, stream, _noalloc)
    return out, lse


def saf_hybrid_attn_fwd_noalloc(q, k, v, frozen, a, r, out, lse, softmax_scale=None, stream=None,
                                events=None, logz=None, qk_packed=False):
    """saf_hybrid_attn_fwd without a workspace (the library's static scratch
    of the current device; for callers that cannot allocate).  The caller
    passes the outputs out ([B, H, T, D]) and lse (fp32 [B, H, T]); nothing
    is allocated.  Shapes needing more than NOALLOC_SCRATCH_BYTES of scratch
    raise SafError (SAF_ESCRATCH).  Calls overlapping on one GPU race."""
    if out is None or lse is None:
        raise ValueError("saf_hybrid_attn_fwd_noalloc needs caller-provided out and lse")
    return saf_hybrid_attn_fwd(q, k, v, frozen, a, r, softmax_scale=softmax_scale, out=out, lse=lse,
                               stream=stream, events=events, logz=logz, qk_packed=qk_packed, _noalloc=True)


def saf_hybrid_attn_bwd(q, k, v, o, dout, lse, frozen, a, r, softmax_scale=None,
                        dq=None, dk=None, dv=None, workspace=None, stream=None, events=None,
                        qk_packed=False, fused_dq=False):
    """Backward of the hybrid layer; returns (dQ, dK, dV).  qk_packed: q, k,
    dq and dk hold only the ordinary heads ([B, n_ordinary, T, D]).
    fused_dq: one key-block pass also accumulates dQ with fp32 atomic adds
    (bf16, D = 64; dQ not bitwise reproducible) instead of a separate
    query-block pass."""
    packed = bool(qk_packed)
    n_ord = _n_ordinary(frozen)
    if packed:
        given = {n: t for n, t in dict(dv=dv).items() if t is not None}
        _check_layer_inputs(v, a, r, o=o, dout=dout, **given)
        B, H, T, D = v.shape
        pshape = (B, n_ord, T, D)
        for name, t in dict(q=q, k=k, dq=dq, dk=dk).items():
            if t is not None or (name in ("q", "k") and n_ord > 0):
                _check_like(name, t, v, shape=pshape)
    else:
        given = {n: t for n, t in dict(dq=dq, dk=dk, dv=dv).items() if t is not None}
        _check_layer_inputs(v, a, r, q=q, k=k, o=o, dout=dout, **given)
    B, H, T, D = v.shape
    _check_like("lse", lse, v, shape=(B, H, T), dtype=torch.float32)
    if not lse.is_contiguous():
        raise ValueError("lse must be contiguous float32 [B, H, T]")
    if workspace is not None:
        _check_like("workspace", workspace, v, shape=workspace.shape, dtype=workspace.dtype)
    _require_gpu(v)
    hq = n_ord if packed else H
    mk = lambda n: torch.empty((B, n, T, D), dtype=v.dtype, device=v.device)  # noqa: E731
    dq = mk(hq) if dq is None else dq
    dk = mk(hq) if dk is None else dk
    dv = mk(H) if dv is None else dv
    prm = Params(v, frozen, a.shape[1], softmax_scale, events)
    prm.p.qk_packed = 1 if packed else 0
    prm.p.fused_dq = 1 if fused_dq else 0
    qk = {} if (packed and n_ord == 0) else dict(q=q, k=k, dq=dq, dk=dk)
    prm.set_strides(v=v, o=o, do=dout, dv=dv, **qk)
    if packed and n_ord == 0:
        q = k = None
        dq_p = dk_p = None
    else:
        dq_p, dk_p = dq, dk
    ws_n = workspace_bytes(prm, True)
    if workspace is None:
        workspace = torch.empty(ws_n, dtype=torch.uint8, device=v.device)
    st = LIB.saf_hybrid_attn_bwd(prm.ref(), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse),
                                 _ptr(a), _ptr(r), _ptr(dq_p), _ptr(dk_p), _ptr(dv), _ptr(workspace),
                                 workspace.numel() * workspace.element_size(), _stream_handle(stream))
    _check(st, "saf_hybrid_attn_bwd")
    return dq, dk, dv


def pattern_grad_workspace_bytes(params: Params) -> int:
    return int(LIB.saf_pattern_grad_workspace_bytes(params.ref()))


def saf_pattern_grad(v, o, dout, lse, frozen, a, r, da=None, dr=None, workspace=None,
                     stream=None, events=None):
    """Gradients of the frozen heads' a and r (trainable-pattern variant);
    returns (da, dr), fp32 [H, Tp].  Rows of ordinary heads are left as given
    (zeros when the outputs are allocated here)."""
    _check_layer_inputs(v, a, r, o=o, dout=dout)
    B, H, T, D = v.shape
    _check_like("lse", lse, v, shape=(B, H, T), dtype=torch.float32)
    if not lse.is_contiguous():
        raise ValueError("lse must be contiguous float32 [B, H, T]")
    for name, t in (("da", da), ("dr", dr)):
        if t is not None:
            _check_like(name, t, a)
            if not t.is_contiguous():
                raise ValueError(f"{name} must be contiguous float32 [H, Tp]")
    if workspace is not None:
        _check_like("workspace", workspace, v, shape=workspace.shape, dtype=workspace.dtype)
    _require_gpu(v)
    da = torch.zeros_like(a) if da is None else da
    dr = torch.zeros_like(r) if dr is None else dr
    prm = Params(v, frozen, a.shape[1], None, events)
    prm.set_strides(v=v, o=o, do=dout)
    ws_n = pattern_grad_workspace_bytes(prm)
    if workspace is not None:
        ws, ws_n = workspace, workspace.numel() * workspace.element_size()
    else:
        ws = torch.empty(ws_n, dtype=torch.uint8, device=v.device) if ws_n else None
    st = LIB.saf_pattern_grad(prm.ref(), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(a), _ptr(r),
                              _ptr(da), _ptr(dr), _ptr(ws), ws_n, _stream_handle(stream))
    _check(st, "saf_pattern_grad")
    return da, dr


def saf_pattern_dense(a_h: torch.Tensor, r_h: torch.Tensor, T: int, stream=None) -> torch.Tensor:
    """Dense [T, T] fp32 compact pattern of one frozen head."""
    if a_h.dtype != torch.float32 or r_h.dtype != torch.float32 or a_h.dim() != 1 or r_h.dim() != 1:
        raise ValueError("a and r must be float32 vectors [Tp]")
    if not a_h.is_contiguous() or not r_h.is_contiguous() or a_h.device != r_h.device or not a_h.is_cuda:
        raise ValueError("a and r must be contiguous vectors on one GPU")
    Tp = min(a_h.numel(), r_h.numel())
    w = torch.empty((T, T), dtype=torch.float32, device=a_h.device)
    _check(LIB.saf_pattern_dense(T, Tp, _ptr(a_h), _ptr(r_h), _ptr(w), _stream_handle(stream)),
           "saf_pattern_dense")
    return w


def saf_pattern_lognorm(a: torch.Tensor, r: torch.Tensor, T: int, stream=None) -> torch.Tensor:
    """log N(i) for every row of a, r ([n, Tp] fp32): returns [n, T]."""
    if a.dtype != torch.float32 or r.dtype != torch.float32 or a.shape != r.shape or a.dim() != 2:
        raise ValueError("a and r must be float32 [n, Tp]")
    if a.device != r.device or not a.is_cuda:
        raise ValueError("a and r must be on one GPU")
    a = a.contiguous()
    r = r.contiguous()
    n, Tp = a.shape
    out = torch.empty((n, T), dtype=torch.float32, device=a.device)
    _check(LIB.saf_pattern_lognorm(n, T, Tp, _ptr(a), _ptr(r), _ptr(out), _stream_handle(stream)),
           "saf_pattern_lognorm")
    return out


# ---------------------------------------------------------------------------
# Compact-pattern fitting.
# ---------------------------------------------------------------------------

FIT_FLOOR = 1e-9   # target floor of the pages' recipe
FIT_STEPS = 400    # Adam steps of the pages' recipe
FIT_LR = 0.05      # Adam learning rate of the pages' recipe


def fit_targets_workspace_bytes(n_heads: int, T: int) -> int:
    return int(LIB.saf_fit_targets_workspace_bytes(int(n_heads), int(T)))


def fit_pattern_workspace_bytes(n_heads: int, T: int) -> int:
    return int(LIB.saf_fit_pattern_workspace_bytes(int(n_heads), int(T)))


def _fit_vec(name: str, t: torch.Tensor, shape, device) -> None:
    if t.dtype != torch.float32 or tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous float32 {tuple(shape)}")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}")


def _workspace(nbytes: int, device, workspace: Optional[torch.Tensor]) -> torch.Tensor:
    if workspace is None:
        return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
    if workspace.dtype != torch.uint8 or workspace.numel() < nbytes or workspace.device != device:
        raise ValueError(f"workspace must be uint8 with at least {nbytes} bytes on {device}")
    return workspace


def saf_fit_targets(ahat: torch.Tensor, floor: float = FIT_FLOOR, workspace=None, stream=None):
    """Sufficient statistics of calibration means ``ahat`` (fp32 [n, T, T]
    or [T, T], last dimension contiguous): returns (eta_abs [n, T],
    eta_rel [n, T], negent [n])."""
    if ahat.dtype != torch.float32 or ahat.dim() not in (2, 3) or not ahat.is_cuda:
        raise ValueError("ahat must be a float32 [n, T, T] or [T, T] GPU tensor")
    a3 = ahat if ahat.dim() == 3 else ahat.unsqueeze(0)
    n, T, T2 = a3.shape
    if T != T2 or a3.stride(2) != 1:
        raise ValueError("ahat must be square with a contiguous last dimension")
    dev = a3.device
    eta_abs = torch.empty((n, T), dtype=torch.float32, device=dev)
    eta_rel = torch.empty((n, T), dtype=torch.float32, device=dev)
    negent = torch.empty((n,), dtype=torch.float32, device=dev)
    nbytes = fit_targets_workspace_bytes(n, T)
    ws = _workspace(nbytes, dev, workspace)
    head_stride = a3.stride(0) if n > 1 else 0
    _check(LIB.saf_fit_targets(n, T, _ptr(a3), head_stride, a3.stride(1), float(floor),
                               _ptr(eta_abs), _ptr(eta_rel), _ptr(negent), _ptr(ws), ws.numel(),
                               _stream_handle(stream)), "saf_fit_targets")
    return eta_abs, eta_rel, negent


def saf_fit_pattern(eta_abs: torch.Tensor, eta_rel: torch.Tensor, negent: Optional[torch.Tensor] = None,
                    steps: int = FIT_STEPS, lr: float = FIT_LR, betas=(0.9, 0.999), eps: float = 1e-8,
                    workspace=None, stream=None):
    """Fit compact patterns to target marginals ([n, T] each): returns a dict
    with a, r, logz ([n, T]) and loss, kappa ([n]; kappa only when negent
    is given)."""
    if eta_abs.dim() != 2 or not eta_abs.is_cuda:
        raise ValueError("eta_abs must be a float32 [n, T] GPU tensor")
    n, T = eta_abs.shape
    dev = eta_abs.device
    _fit_vec("eta_abs", eta_abs, (n, T), dev)
    _fit_vec("eta_rel", eta_rel, (n, T), dev)
    if negent is not None:
        _fit_vec("negent", negent, (n,), dev)
    out = {k: torch.empty((n, T), dtype=torch.float32, device=dev) for k in ("a", "r", "logz")}
    out["loss"] = torch.empty((n,), dtype=torch.float32, device=dev)
    out["kappa"] = torch.empty((n,), dtype=torch.float32, device=dev) if negent is not None else None
    nbytes = fit_pattern_workspace_bytes(n, T)
    ws = _workspace(nbytes, dev, workspace)
    _check(LIB.saf_fit_pattern(n, T, _ptr(eta_abs), _ptr(eta_rel), _ptr(negent), int(steps), float(lr),
                               float(betas[0]), float(betas[1]), float(eps), _ptr(out["a"]), _ptr(out["r"]),
                               _ptr(out["logz"]), _ptr(out["loss"]), _ptr(out["kappa"]), _ptr(ws),
                               ws.numel(), _stream_handle(stream)), "saf_fit_pattern")
    return out


# ---------------------------------------------------------------------------
# Calibration statistics.
# ---------------------------------------------------------------------------


def calib_stats_workspace_bytes(N: int, H: int, T: int) -> int:
    return int(LIB.saf_calib_stats_workspace_bytes(int(N), int(H), int(T)))


def saf_calib_stats(q: torch.Tensor, k: torch.Tensor, softmax_scale: Optional[float] = None,
                    ahat: Optional[torch.Tensor] = None, workspace=None, stream=None):
    """Mean attention and the two scores of H heads over N calibration
    sequences: q, k bf16 [N, H, T, D] on one GPU.  Returns (ahat [H, T, T]
    fp32, s_var [H] fp64, s_kl [H] fp64); a freshly allocated ahat is zero
    above the diagonal (the library writes only causal entries)."""
    for name, t in (("q", q), ("k", k)):
        if t.dtype != torch.bfloat16 or t.dim() != 4 or not t.is_cuda or t.stride(3) != 1:
            raise ValueError(f"{name} must be a bfloat16 [N, H, T, D] GPU tensor with contiguous D")
    if q.shape != k.shape or q.device != k.device:
        raise ValueError("q and k must have the same shape and device")
    N, H, T, D = q.shape
    dev = q.device
    if ahat is None:
        ahat = torch.zeros((H, T, T), dtype=torch.float32, device=dev)
    if ahat.dtype != torch.float32 or ahat.dim() != 3 or tuple(ahat.shape[:2]) != (H, T) or ahat.shape[2] < T \
            or ahat.stride(2) != 1 or ahat.device != dev:
        raise ValueError("ahat must be float32 [H, T, >= T] with a contiguous last dimension")
    s_var = torch.empty((H,), dtype=torch.float64, device=dev)
    s_kl = torch.empty((H,), dtype=torch.float64, device=dev)
    ws = _workspace(calib_stats_workspace_bytes(N, H, T), dev, workspace)
    qs = (ctypes.c_int64 * 3)(q.stride(0), q.stride(1), q.stride(2))
    ks = (ctypes.c_int64 * 3)(k.stride(0), k.stride(1), k.stride(2))
    scale = 0.0 if softmax_scale is None else float(softmax_scale)
    _check(LIB.saf_calib_stats(N, H, T, D, scale, _ptr(q), qs, _ptr(k), ks, _ptr(ahat), ahat.stride(0),
                               ahat.stride(1), _ptr(s_var), _ptr(s_kl), _ptr(ws), ws.numel(),
                               _stream_handle(stream)), "saf_calib_stats")
    return ahat, s_var, s_kl
