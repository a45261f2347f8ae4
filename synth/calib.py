"""Seeded synthetic calibration activations: queries and keys of H heads over
N sequences, the inputs of the calibration statistics.

Without a trained model, each head mixes a component shared by every
sequence with a per-sequence one, in a head-specific proportion, and has a
head-specific sharpness, so that the heads span attention that barely
changes across sequences (low variance, the candidates for replacement) to
attention that changes a lot:

    q^(n) = sigma_h (c_h u + sqrt(1 - c_h^2) e^(n)),   k likewise,

with u, e^(n) standard normal [T, D] blocks.  Values are rounded to
bfloat16 (the storage type).  Generator: numpy PCG64 seeded with [seed, h]
for head h; draw order per head: sigma_h ~ U(0.5, 2.0), c_h ~ U(0, 1), the
shared q block, the shared k block, then for n = 0..N-1 the sequence's q
block and k block.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .gen import bf16_round


@dataclass(frozen=True)
class CalibWorkload:
    name: str
    N: int
    H: int
    T: int
    D: int
    seed: int


# The 124M model's calibration: 32 held-out sequences of length 4096
# (Appendix C.3), 12 heads of d = 64 per layer.
CALIB_WORKLOADS = {
    "gpt2_124m_4k": CalibWorkload("gpt2-124m-calib_N32_H12_T4096_d64", 32, 12, 4096, 64, 1351),
    "small": CalibWorkload("calib-small_N4_H3_T300_d64", 4, 3, 300, 64, 17),
}


def calibration_head(N: int, T: int, D: int, seed: int, h: int):
    """q, k of head h: float32 [N, T, D] each, holding bfloat16 values."""
    rng = np.random.default_rng([seed, h])
    sigma = rng.uniform(0.5, 2.0)
    c = rng.uniform(0.0, 1.0)
    uq = rng.standard_normal((T, D))
    uk = rng.standard_normal((T, D))
    q = np.empty((N, T, D), dtype=np.float32)
    k = np.empty((N, T, D), dtype=np.float32)
    w = np.sqrt(1.0 - c * c)
    for n in range(N):
        q[n] = sigma * (c * uq + w * rng.standard_normal((T, D)))
        k[n] = sigma * (c * uk + w * rng.standard_normal((T, D)))
    return bf16_round(q), bf16_round(k)


def calibration_qk(N: int, H: int, T: int, D: int, seed: int):
    """q, k of H heads: float32 [N, H, T, D] each, holding bfloat16 values."""
    q = np.empty((N, H, T, D), dtype=np.float32)
    k = np.empty((N, H, T, D), dtype=np.float32)
    for h in range(H):
        q[:, h], k[:, h] = calibration_head(N, T, D, seed, h)
    return q, k
