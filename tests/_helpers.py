"""Shared helpers of the GPU tests: upload seeded inputs, error metrics."""

from __future__ import annotations

import sys

import numpy as np
import torch

BF16_FWD_MAXABS = 1e-2   # forward output, bf16
BF16_FWD_RELL2 = 5e-3
BF16_GRAD_RELL2 = 1e-2   # dQ, dK, dV, bf16
F32_RELL2 = 1e-5         # fp32 path (outputs and gradients)
F32_MAXABS = 1e-5
LSE_ORD_ABS = 1e-3       # ordinary heads' row log-sum-exp
LSE_FRZ_ABS = 1e-4       # frozen heads' log N


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel_l2(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-8))


def max_abs(got, ref) -> float:
    return float(np.max(np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64))))


def bf16_half_ulp(x) -> np.ndarray:
    """Half a unit in the last place of bfloat16 at |x| (8-bit significand)."""
    ax = np.maximum(np.abs(np.asarray(x, np.float64)), 2.0 ** -126)
    return 0.5 * 2.0 ** (np.floor(np.log2(ax)) - 7)


def out_max_abs(got, ref, dtype: str) -> float:
    """Forward max-abs error of an output stored as ``dtype``.

    For bf16 outputs the half-ulp of the stored value is subtracted first: an
    exact result rounded to bf16 already differs from the float64 value by up
    to that much (0.0156 for |O| in [4, 8)), so the bar applies to the error
    beyond the storage format's own rounding.  fp32: plain max-abs.
    """
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(got - ref)
    if dtype == "bf16":
        err = err - bf16_half_ulp(np.maximum(np.abs(got), np.abs(ref)))
    return float(max(np.max(err), 0.0))


def torch_dtype(cfg):
    return torch.bfloat16 if cfg.dtype == "bf16" else torch.float32


def to_dev(x: np.ndarray, dtype) -> torch.Tensor:
    """Upload exactly (inputs already hold storage-dtype values)."""
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda").to(dtype)


def upload(inp):
    dt = torch_dtype(inp.cfg)
    dev = {n: to_dev(getattr(inp, n), dt) for n in ("q", "k", "v")}
    if inp.do is not None:
        dev["do"] = to_dev(inp.do, dt)
    dev["a"] = torch.from_numpy(inp.a).cuda()
    dev["r"] = torch.from_numpy(inp.r).cuda()
    return dev


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy()
