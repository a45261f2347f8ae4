"""Seeded synthetic calibration means: the inputs of compact-pattern fitting.

A calibration mean is a causal, row-stochastic [T, T] matrix: the average
attention of one head over calibration sequences (Section 3.1, Equation 1).
Without trained weights or data, each head's mean is drawn from a structured
family with the features the pages describe for low-variance heads: an
attention sink on the first key, a decay with query-key distance, and
multiplicative noise that no compact pattern reproduces exactly.

For head ``head`` of a target set with seed ``seed`` the generator is numpy's
PCG64 seeded with [seed, head], so any head can be regenerated alone.  Draw
order: the head's shape parameters (sink, decay, noise level, zero
fraction), then T(T+1)/2 standard normals (noise) and T(T+1)/2 uniforms
(zeroed entries), each over the causal entries (i, j <= i) in row-major
order.  Weights are

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
    decay_by_dist = (1.0 + np.arange(T, dtype=np.float64)) ** (-decay)
    ii, jj = np.tril_indices(T)  # causal entries, row-major
    n = rng.standard_normal(ii.size)
    u = rng.random(ii.size)
    w = decay_by_dist[ii - jj] * np.exp(noise * n)
    w[jj == 0] *= 1.0 + sink
    w[(u < zero_frac) & (ii != jj)] = 0.0
    starts = ii.searchsorted(np.arange(T))  # first entry of each row
    w /= np.add.reduceat(w, starts)[ii]
    out = np.zeros((T, T), dtype=np.float32)
    out[ii, jj] = w
    return out


def calibration_means(T: int, n_heads: int, seed: int, spec: TargetSpec = DEFAULT_SPEC) -> np.ndarray:
    """Heads 0..n_heads-1 of a target set, float32 [n_heads, T, T]."""
    out = np.empty((n_heads, T, T), dtype=np.float32)
    for h in range(n_heads):
        out[h] = calibration_mean(T, seed, h, spec)
    return out


@dataclass(frozen=True)
class FitWorkload:
    """A set of heads to fit: n_heads calibration means of length T."""

    name: str
    n_heads: int
    T: int
    seed: int


# The 124M model at 4K context with 25% of its 12 x 12 heads replaced: 36
# fits at T = 4096 (the setting of the pages' fitting-cost table, Table 13).
FIT_WORKLOADS = {
    "gpt2_124m_25pct": FitWorkload("gpt2-124m-fit_H36_T4096_25pct", 36, 4096, 1337),
    "small": FitWorkload("fit-small_H4_T300", 4, 300, 7),
}
