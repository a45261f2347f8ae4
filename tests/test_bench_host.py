"""Host-side checks of bench.py: its flop accounting and its one-GPU guard.

The flop counts follow the FlashAttention-2 convention the throughput is
quoted in: per causal pair (i >= j), an ordinary head costs 4d forward (QK^T
and PV) and 10d backward (S and dP recomputed once in the key-block pass,
dV, dK, and dQ), a frozen head 2d forward (WV) and 2d backward (W^T dO).
The expected totals below were worked out by hand from the workload shapes.
"""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from synth import CONFIGS  # noqa: E402


@pytest.mark.parametrize(
    "key,fwd,total",
    [
        # B=8 H=12 T=4096 d=64, 3 frozen heads
        ("gpt2_124m_4k_25pct", 1.804e11, 5.9285e11),
        # same shape, 6 frozen heads
        ("gpt2_124m_4k_50pct_interleaved", 1.547e11, 4.6397e11),
        # B=2 H=16 T=8192 d=128, 4 frozen heads
        ("1b_8k_rank_share", 4.811e11, 1.5807e12),
        # B=1 H=4 T=128 d=64, 1 frozen head
        ("tiny", 7.397e6, 2.431e7),
    ],
)
def test_flop_accounting(key, fwd, total):
    f = bench.flops(CONFIGS[key])
    assert f["fwd"] == pytest.approx(fwd, rel=5e-4)
    assert f["total"] == pytest.approx(total, rel=5e-4)
    # the kernels' shares add up to the whole
    assert f["fwd_ord"] + f["fwd_frz"] == f["fwd"]
    assert f["bwd_kv"] + f["bwd_q"] == f["bwd"]


def test_flop_accounting_per_pair():
    cfg = CONFIGS["gpt2_124m_4k_25pct"]
    P = cfg.T * (cfg.T + 1) // 2
    f = bench.flops(cfg, n_ord=1, n_frz=0, B=1)
    assert f["total"] == 14 * cfg.D * P
    f = bench.flops(cfg, n_ord=0, n_frz=1, B=1)
    assert f["total"] == 4 * cfg.D * P


def test_fused_dq_atomic_bytes():
    # 124M layer: 32 key blocks of 128, 64 query tiles of 64; key block kb
    # meets tiles 2kb .. 63, i.e. 64 - 2kb tiles: 1056 in all, for each of
    # the 8 x 9 ordinary (b, h); each adds a 64 x 64 fp32 block
    cfg = CONFIGS["gpt2_124m_4k_25pct"]
    assert bench.pairs_tiles_bytes(cfg) == 8 * 9 * 1056 * 64 * 64 * 4


def test_calibration_flop_accounting():
    # shifted-sum update per entry: log2 A (FMA), A log2 A (FMA), A - A0,
    # s1 += d, s2 += d*d (FMA): 2 + 2 + 1 + 1 + 2 flops, the exponential not
    # counted
    assert bench.CALIB_FLOPS_PER_UPDATE == 8


def test_fit_scaling_targets_closed_form():
    # the fit T-scaling leg's targets equal the oracle's statistics of a
    # uniform causal mean (column sums, diagonal sums, sum P ln P)
    import numpy as np

    from oracle.saf_fit_oracle import fit_statistics

    for T in (1, 7, 64):
        A = np.tril(np.ones((T, T))) / np.arange(1, T + 1)[:, None]
        st = fit_statistics(A)
        eta, negent = bench.uniform_causal_targets(T)
        np.testing.assert_allclose(eta, st["eta_abs"], rtol=1e-12, atol=0)
        np.testing.assert_allclose(eta, st["eta_rel"], rtol=1e-12, atol=0)
        assert abs(negent - st["negent"]) <= 1e-10 * max(1.0, abs(negent))


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert p.returncode == 2
    line = json.loads(p.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"]
