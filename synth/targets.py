"""Seeded synthetic calibration means: the inputs of compact-pattern fitting.

A calibration mean is a causal, row-stochastic [T, T] matrix: the average
attention of one head over calibration sequences (Section 3.1, Equation 1).
Without trained weights or data, each head's mean is drawn from a structured
family with the features the pages describe for low-variance heads: an
attention sink on the first key, a decay with query-key distance, and
multiplicative noise that no compact pattern reproduces exactly.

For head ``head`` of a target set with seed ``seed`` the generator is numpy's
PCG64 seeded with [seed, head], so any head can be regenerated alone.  Draw
order: the head's shape parameters (sink, decay, noise level, zero fraction),
then a [T, T] block of standard normals (noise), then a [T, T] block of
uniforms (zeroed entries).  Weights are

    w[i, j] = (1 + i - j) ** (-decay) * (1 + sink * [j == 0]) * exp(noise * n[i, j])

for j <= i, with entries whose uniform falls below ``zero_frac`` set to 0
(except the diagonal), each row divided by its sum in float64, and the
result stored as float32 with zeros above the diagonal.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Tuple

import numpy as np


@dataclass(frozen=True)
class TargetSpec:
    """Ranges of the per-head shape parameters (drawn uniformly)."""

    sink: Tuple[float, float] = (0.0, 30.0)
    decay: Tuple[float, float] = (0.3, 1.5)
    noise: Tuple[float, float] = (0.05, 0.9)
    zero_frac: Tuple[float, float] = (0.0, 0.3)


DEFAULT_SPEC = TargetSpec()


def calibration_mean(T: int, seed: int, head: int, spec: TargetSpec = DEFAULT_SPEC) -> np.ndarray:
    """One head's synthetic calibration mean, float32 [T, T]."""
    rng = np.random.default_rng([seed, head])
    sink = rng.uniform(*spec.sink)
    decay = rng.uniform(*spec.decay)
    noise = rng.uniform(*spec.noise)
    zero_frac = rng.uniform(*spec.zero_frac)
    n = rng.standard_normal((T, T))
    u = rng.random((T, T))
    i = np.arange(T)[:, None]
    j = np.arange(T)[None, :]
    causal = j <= i
    dist = np.where(causal, i - j, 0).astype(np.float64)
    w = (1.0 + dist) ** (-decay) * np.where(j == 0, 1.0 + sink, 1.0) * np.exp(noise * n)
    w = np.where(causal & ((u >= zero_frac) | (i == j)), w, 0.0)
    w /= w.sum(axis=1, keepdims=True)
    return w.astype(np.float32)


def calibration_means(T: int, n_heads: int, seed: int, spec: TargetSpec = DEFAULT_SPEC) -> np.ndarray:
    """Heads 0..n_heads-1 of a target set, float32 [n_heads, T, T]."""
    out = np.empty((n_heads, T, T), dtype=np.float32)
    for h in range(n_heads):
        out[h] = calibration_mean(T, seed, h, spec)
    return out
