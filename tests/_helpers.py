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


def half_ulp(x, bits):
    """Half a unit in the last place at |x| for a significand of ``bits`` bits."""
    ax = np.maximum(np.abs(np.asarray(x, np.float64)), 2.0 ** -126)
    return 0.5 * 2.0 ** (np.floor(np.log2(ax)) - (bits - 1))


def forward_rounding_sigma(cfg, inp, h):
    """L2 norms over the entries of the standard deviations of da and dr of
    frozen head h caused by the forward's rounding inside D_b[i] = dO . O.

    The library forms D from the forward's stored output, which carries that
    forward's rounding: for bf16 the weights rounded to bf16 before the second
    product and the output rounded to bf16 (fp32: only the output rounding).
    Each rounding error is modelled as independent and uniform within half an
    ulp, so D_b[i] has variance
        sum_j h(W_ij)^2 / 3 * dW_b[i][j]^2 + sum_d h(O_b[i][d])^2 / 3 * dO_b[i][d]^2
    and an entry of da or dr, a W-weighted sum of D over rows, the matching
    weighted variance.  For fp32 the weights are not rounded, but each is an
    fp32 exponential of an fp32 exponent x = a[j] + r[i-j] - log N(i) (log2
    units): its relative error is modelled as uniform within
    e_ij = (|a[j] + r[i-j]| + |log N(i)| + 1) * log2(e) * 2^-24 (the exponent's
    rounding plus one ulp of the exponential), which takes the place of h(W_ij)
    (for bf16 it is below 2^-9 of the rounding and omitted).  Expected values
    come from the oracle's W, O and dW.
    """
    import oracle

    bits = 8 if cfg.dtype == "bf16" else 24  # significand bits of the storage type
    T = cfg.T
    P = oracle.frozen_pattern(inp.a[h], inp.r[h], T)
    if cfg.dtype != "bf16":
        G = oracle.frozen_logits(inp.a[h], inp.r[h], T)
        logN = oracle.frozen_lognorm(inp.a[h], inp.r[h], T)
        with np.errstate(invalid="ignore"):
            e_w = np.where(P > 0, (np.abs(np.where(P > 0, G, 0.0)) + np.abs(logN)[:, None] + 1.0)
                           * np.log2(np.e) * 2.0 ** -24, 0.0)
    va = np.zeros(T)
    vr = np.zeros(T)
    for b in range(cfg.B):
        v = np.asarray(inp.v[b, h], np.float64)
        do = np.asarray(inp.do[b, h], np.float64)
        O = P @ v
        var_d = (do ** 2 * half_ulp(O, bits) ** 2 / 3).sum(axis=1)
        if cfg.dtype == "bf16":
            var_d += (np.where(P > 0, half_ulp(P, bits), 0.0) ** 2 / 3 * (do @ v.T) ** 2).sum(axis=1)
        else:
            var_d += ((P * e_w) ** 2 / 3 * (do @ v.T) ** 2).sum(axis=1)
        Wv = P ** 2 * var_d[:, None]
        va += Wv.sum(axis=0)
        for i in range(T):
            vr[: i + 1] += Wv[i, i::-1]
    return float(np.sqrt(va.sum())), float(np.sqrt(vr.sum()))
