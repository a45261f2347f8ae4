"""Seeded generation of Q, K, V, dO, a and r.

The generator is numpy's PCG64 (``default_rng(seed)``).  Draw order is fixed:
Q, K, V, dO (each a full block of float32 standard normals: [B, H, T, D] for
Q and dO, [B, Hkv, T, D] for K and V), then a ([H, Tp]), then the noise of r
([H, Tp]).  Rows of ordinary heads are drawn
too and simply ignored by the layer, so the frozen set can change without
changing any other value.  Values are scaled, then rounded to the storage
dtype.  a and r stay float32, as the pages keep their prior buffers in fp32.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

from .configs import Config


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns the 16-bit patterns as uint16.  Inputs must be finite.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    rounded = (u + 0x7FFF + lsb) >> 16
    return rounded.astype(np.uint16)


def bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns (uint16) to float32 values exactly."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest bfloat16 value, returned as float32."""
    return bits_to_f32(bf16_bits(x))


@dataclass
class Inputs:
    """One workload's inputs, as float32 arrays holding storage-dtype values.

    For dtype "bf16" every element of q, k, v, do is exactly representable in
    bfloat16; ``*_bits`` views give the uint16 patterns for upload.
    """

    cfg: Config
    q: np.ndarray  # [B, H, T, D]
    k: np.ndarray  # [B, Hkv, T, D]
    v: np.ndarray  # [B, Hkv, T, D]
    do: Optional[np.ndarray]  # [B, H, T, D] or None for forward-only workloads
    a: np.ndarray  # [H, Tp] float32
    r: np.ndarray  # [H, Tp] float32
    frozen: np.ndarray  # [H] uint8

    def bits(self, name: str) -> np.ndarray:
        return bf16_bits(getattr(self, name))


def _r_vector(cfg: Config, rng: np.random.Generator) -> np.ndarray:
    H, Tp = cfg.H, cfg.Tp
    d = np.arange(Tp, dtype=np.float64)
    if cfg.r_kind == "linear_noise":
        noise = rng.standard_normal((H, Tp), dtype=np.float32)
        r = (-cfg.r_slope * d)[None, :] + cfg.r_noise * noise.astype(np.float64)
    elif cfg.r_kind == "peaked":
        base = np.where(d < 8, 3.0, -0.01 * d)
        r = np.broadcast_to(base, (H, Tp)).copy()
    else:
        raise ValueError(f"unknown r_kind {cfg.r_kind!r}")
    return r.astype(np.float32)


def make_inputs(cfg: Config, seed: Optional[int] = None, with_do: Optional[bool] = None) -> Inputs:
    """Draw the inputs of ``cfg`` (seed defaults to ``cfg.seed``)."""
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    shape = (cfg.B, cfg.H, cfg.T, cfg.D)
    kv_shape = (cfg.B, cfg.Hkv, cfg.T, cfg.D)
    want_do = cfg.bwd if with_do is None else with_do

    def draw(shape=shape):
        x = rng.standard_normal(shape, dtype=np.float32)
        if cfg.qkv_scale != 1.0:
            x *= np.float32(cfg.qkv_scale)
        if cfg.dtype == "bf16":
            x = bf16_round(x).reshape(shape)
        elif cfg.dtype != "f32":
            raise ValueError(f"unknown dtype {cfg.dtype!r}")
        return x

    q = draw()
    k = draw(kv_shape)
    v = draw(kv_shape)
    do = draw() if want_do else None
    a = rng.standard_normal((cfg.H, cfg.Tp), dtype=np.float32)
    r = _r_vector(cfg, rng)
    frozen = np.array(cfg.frozen_mask, dtype=np.uint8)
    return Inputs(cfg=cfg, q=q, k=k, v=v, do=do, a=a, r=r, frozen=frozen)
