"""Workload shapes for the SAF hybrid attention layer.

Each entry fixes the tensor shapes, which heads are frozen, the storage dtype
and the distributions of the synthetic inputs.  The shapes follow the pages:

* the 124M GPT layer (12 heads of dimension 64, T=4096, micro-batch 8) of
  "When Can Attention Heads Be Statically Defined?", Section 4 and Table 11;
* the 1B model's per-GPU share at 8K context (16 heads, B=2 per rank),
  Appendix C.5 / Table 23 -- head dimension 128 is used here;
* the mixed-head numerical check of Appendix D.2 (B=2, T=129, H=4, d=64,
  stored prior length 192, heads 1 and 3 frozen, zero-based);
* the Qwen3-4B grouped-query prefill of Appendix C.6.2 / Table 26 (32 query
  heads sharing 8 key/value heads, d=128, B in {4, 8}, T in {2048, 4096,
  8192}, forward only).

Token content does not change attention cost, so Gaussian inputs of these
shapes stand in for the pages' FineWeb-Edu activations.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, Optional, Tuple


@dataclass(frozen=True)
class Config:
    name: str
    B: int
    H: int
    T: int
    D: int
    frozen: Tuple[int, ...]
    dtype: str  # "f32" or "bf16": storage and MFMA operand type of Q,K,V,dO
    seed: int
    qkv_scale: float = 1.0  # Q, K, V, dO = N(0,1) * qkv_scale
    r_kind: str = "linear_noise"  # "linear_noise" or "peaked"
    r_slope: float = 0.05  # r[d] = -r_slope * d + N(0, r_noise)
    r_noise: float = 0.5  # standard deviation of the r noise
    prior_len: Optional[int] = None  # stored length Tp of a and r (>= T); None -> T
    bwd: bool = True  # whether the workload includes the backward pass
    note: str = ""
    kv_heads: Optional[int] = None  # key/value heads (grouped-query); None -> H

    @property
    def Hkv(self) -> int:
        return self.H if self.kv_heads is None else self.kv_heads

    @property
    def Tp(self) -> int:
        return self.T if self.prior_len is None else self.prior_len

    @property
    def frozen_mask(self) -> Tuple[int, ...]:
        return tuple(1 if h in self.frozen else 0 for h in range(self.H))

    def with_(self, **kw) -> "Config":
        d = dict(self.__dict__)
        d.update(kw)
        return Config(**d)


CONFIGS: Dict[str, Config] = {}


def _add(key: str, cfg: Config) -> None:
    CONFIGS[key] = cfg


# Tiny fp32 layer: one frozen head (the last of four).
_add(
    "tiny",
    Config(
        name="tiny_B1_H4_T128_d64_fp32_head3frozen",
        B=1, H=4, T=128, D=64, frozen=(3,), dtype="f32", seed=1337,
        qkv_scale=1.0, r_kind="linear_noise", r_slope=0.05, r_noise=0.5,
    ),
)

# 124M GPT layer at 4K context, 25% of heads frozen (the last three).
_add(
    "gpt2_124m_4k_25pct",
    Config(
        name="gpt2-124m-layer_B8_H12_T4096_d64_bf16_25pct-frozen",
        B=8, H=12, T=4096, D=64, frozen=(9, 10, 11), dtype="bf16", seed=1338,
        qkv_scale=0.125, r_kind="linear_noise", r_slope=0.05, r_noise=0.5,
    ),
)

# Same shape, 50% of heads frozen, interleaved.
_add(
    "gpt2_124m_4k_50pct_interleaved",
    Config(
        name="gpt2-124m-layer_B8_H12_T4096_d64_bf16_50pct-frozen-interleaved",
        B=8, H=12, T=4096, D=64, frozen=(0, 2, 4, 6, 8, 10), dtype="bf16",
        seed=1339, qkv_scale=0.125, r_kind="linear_noise", r_slope=0.05,
        r_noise=0.5,
    ),
)

# 1B-style layer at 8K, one GPU's share of the pages' four-GPU run.
_add(
    "1b_8k_rank_share",
    Config(
        name="1b-layer-rank-share_B2_H16_T8192_d128_bf16_25pct-frozen",
        B=2, H=16, T=8192, D=128, frozen=(12, 13, 14, 15), dtype="bf16",
        seed=1340, qkv_scale=1.0, r_kind="linear_noise", r_slope=0.02,
        r_noise=0.5,
    ),
)

# Long causal prefill, forward only, sharply peaked relative preference.
_add(
    "prefill_32k",
    Config(
        name="prefill_B1_H12_T32768_d64_bf16_25pct-frozen_peaked-r",
        B=1, H=12, T=32768, D=64, frozen=(9, 10, 11), dtype="bf16", seed=1341,
        qkv_scale=1.0, r_kind="peaked", bwd=False,
    ),
)

# The mixed-head check of Appendix D.2: stored prior length exceeds T and
# T is not a multiple of any tile size.
_add(
    "pages_check_t129",
    Config(
        name="pages-check_B2_H4_T129_d64_Tp192_heads1,3frozen",
        B=2, H=4, T=129, D=64, frozen=(1, 3), dtype="bf16", seed=1342,
        qkv_scale=1.0, r_kind="linear_noise", r_slope=0.05, r_noise=0.5,
        prior_len=192,
    ),
)

# Qwen3-4B attention layer, grouped-query prefill (forward only): 32 query
# heads over 8 key/value heads; 30% of the query heads frozen (the last ten,
# so two key/value groups are entirely frozen and one partly).
_add(
    "qwen3_4b_prefill_B4_T4096_30pct",
    Config(
        name="qwen3-4b-prefill_B4_H32_KV8_T4096_d128_bf16_30pct-frozen",
        B=4, H=32, T=4096, D=128, frozen=tuple(range(22, 32)), dtype="bf16",
        seed=1343, qkv_scale=1.0, r_kind="linear_noise", r_slope=0.02,
        r_noise=0.5, bwd=False, kv_heads=8,
    ),
)

# Order used when a workload is named by position (tiny case first, the
# headline 124M/4K/25% shape second).
ORDER = (
    "tiny",
    "gpt2_124m_4k_25pct",
    "gpt2_124m_4k_50pct_interleaved",
    "1b_8k_rank_share",
    "prefill_32k",
)


def get_config(key) -> Config:
    if isinstance(key, int):
        return CONFIGS[ORDER[key]]
    return CONFIGS[key]
