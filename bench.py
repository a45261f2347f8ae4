"""Throughput of the SAF hybrid attention layer (forward + backward) on one GPU.

A step is one forward and one backward of the hybrid layer over one batch of
seeded synthetic inputs resident in HBM (workload: the 124M GPT layer shape,
B=8, H=12 with the last 3 heads frozen, T=4096, d=64, bf16).  The headline
value is algorithmic TFLOP/s under the FlashAttention-2 counting convention:
per causal pair, ordinary heads count 4d (forward) + 10d (backward) flops and
frozen heads 2d + 2d.

Prints ONE JSON line.  Also reports, for the dominant kernel, its roofline
position from HIP events that the library records around each of its kernels
on the launch stream, and the float64 CPU oracle timed on a bounded sample.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
PEAK_F32_TFLOPS = 157.3  # MI355X fp32 vector (FMA = 2 flops)
# Fitting cost the pages print for the 124M model at 4K with 25% of heads
# replaced (Table 13, "Fit alpha, rho" column, mean over three seeds; GH200).
PAGES_FIT_S_124M_25PCT = 3.20


def pairs(T: int) -> int:
    return T * (T + 1) // 2


def flops(cfg, n_ord=None, n_frz=None, B=None):
    """Algorithmic flops of one forward and one backward (FA2 convention),
    split over the kernels that perform them."""
    P = pairs(cfg.T)
    d = cfg.D
    B = cfg.B if B is None else B
    n_frz = len(cfg.frozen) if n_frz is None else n_frz
    n_ord = cfg.H - n_frz if n_ord is None else n_ord
    f = {
        "fwd_ord": P * d * 4 * B * n_ord,     # S = QK^T, O = PV
        "fwd_frz": P * d * 2 * B * n_frz,     # O = WV
        "bwd_kv_ord": P * d * 8 * B * n_ord,  # S, dP recomputed once; dV, dK
        "bwd_kv_frz": P * d * 2 * B * n_frz,  # dV = W^T dO
        "bwd_q": P * d * 2 * B * n_ord,       # dQ
    }
    f["fwd"] = f["fwd_ord"] + f["fwd_frz"]        # one mixed-head launch
    f["bwd_kv"] = f["bwd_kv_ord"] + f["bwd_kv_frz"]  # one mixed-head launch
    f["bwd"] = f["bwd_kv"] + f["bwd_q"]
    f["total"] = f["fwd"] + f["bwd"]
    return f


DEFAULT_CONFIG = "gpt2_124m_4k_25pct"
# HBM traffic of each layer kernel at the headline workload, from rocprofv3
# FETCH_SIZE / WRITE_SIZE counters (one summary per kernel under profiles/),
# and the sources each kernel is compiled from: a summary counts only while
# those sources hash to the value recorded in it.
TRAFFIC_FILES = {n: os.path.join(ROOT, "profiles", f"traffic_{n}_gpt2-124m-layer_B8_T4096_d64_25pct.txt")
                 for n in ("fwd", "bwd_q", "bwd_kv")}
KERNEL_NAMES = {"fwd": "fwd_kernel<64>", "bwd_q": "bwd_q_kernel<64>", "bwd_kv": "bwd_kv_kernel<64>"}
_COMMON_SOURCES = ("saf_device.h", "saf_tile.h", "saf_internal.h")
KERNEL_SOURCES = {"fwd": ("kern_fwd.hip",) + _COMMON_SOURCES,
                  "bwd_q": ("kern_bwd.hip",) + _COMMON_SOURCES,
                  "bwd_kv": ("kern_bwd.hip",) + _COMMON_SOURCES}
# algorithmic HBM bytes per launch at the headline workload (each tensor
# read or written once; see algorithmic_bytes)


# Measured v_exp_f32 issue time on gfx950: 3.9 ns per wave instruction per
# SIMD (64 exponentials), 1024 SIMDs.
EXP_PER_S = 64 / 3.9e-9 * 1024


def exp_counts(cfg, with_bwd: bool):
    """Exponentials per step as this design computes them, for patterns
    whose ranges pass the factored-weight test (the synthetic ones do):
    ordinary heads take one per causal pair and (b, h) in the forward and one
    in each of the backward's two recomputing passes; frozen heads build
    their weights and normalisers from factored exponentials (one multiply
    per pair), except the backward's dV at d != 64, one per pair shared by a
    batch group of two.  Also the time they take at the measured rate."""
    P = pairs(cfg.T)
    n_frz = len(cfg.frozen)
    n_ord = cfg.H - n_frz
    groups = (cfg.B + 1) // 2
    fwd = P * cfg.B * n_ord
    bwd = (2 * P * cfg.B * n_ord + (0 if cfg.D == 64 else P * groups * n_frz)) if with_bwd else 0
    n = fwd + bwd
    return {"count": n, "fwd": fwd, "bwd": bwd, "bound_ms": round(n / EXP_PER_S * 1e3, 4)}


def kernel_source_sha(name: str = "bwd_kv") -> str:
    """Hash of the sources layer kernel `name` (fwd, bwd_q, bwd_kv) is
    compiled from."""
    import hashlib

    h = hashlib.sha256()
    for src in KERNEL_SOURCES[name]:
        with open(os.path.join(ROOT, "fixed_pattern_hybrid_amd", "csrc", src), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(name: str):
    """HBM bytes per launch of layer kernel `name` from its committed counter
    summary, or None when that was taken on other kernel sources (or is
    absent)."""
    path = TRAFFIC_FILES.get(name)
    if path is None or not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                key, val = line.split(":", 1)
                kv[key.strip()] = val.strip()
    if kv.get("kernel") != KERNEL_NAMES[name] or kv.get("source_sha") != kernel_source_sha(name):
        return None
    try:
        return int(float(kv["traffic_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def algorithmic_bytes(cfg):
    """Minimum HBM bytes per launch of each layer kernel (bf16 tensors read
    or written once): forward -- Q, K of ordinary heads, V, O, lse, a, r;
    query-block pass -- Q, K, V, O, dO of ordinary heads, lse, delta, dQ;
    key-block pass -- Q, K, V, dO of ordinary heads, dO of frozen heads, lse,
    delta, dK, dV, the frozen heads' zero dQ/dK rows, a, r."""
    n_frz = len(cfg.frozen)
    n_ord = cfg.H - n_frz
    e = 2 if cfg.dtype == "bf16" else 4
    t_ord = cfg.B * n_ord * cfg.T * cfg.D * e  # one tensor's ordinary heads
    t_frz = cfg.B * n_frz * cfg.T * cfg.D * e
    row = cfg.B * cfg.H * cfg.T * 4            # one fp32 value per (b, h, t)
    ar = 2 * n_frz * cfg.T * 4
    return {
        "fwd": 2 * t_ord + 2 * (t_ord + t_frz) + row + ar,
        "bwd_q": 6 * t_ord + 2 * row,
        "bwd_kv": 4 * t_ord + t_frz + 2 * row + 2 * (t_ord + t_frz) + 2 * t_frz + ar,
    }


def calib_copy(n_mib: int = 1024, reps: int = 5):
    """A plain device copy of known size, for scaling FETCH_SIZE/WRITE_SIZE."""
    import torch

    n = n_mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calib_copy_bytes_read": n * 4, "calib_copy_bytes_written": n * 4, "reps": reps}), flush=True)


def per_head_costs(B, cfg, reps: int = 10):
    """Per-head fwd and fwd+bwd cost at the workload's shape with every head
    ordinary versus every head frozen, timed in A-B-B-A order."""
    import numpy as np
    import torch

    from synth import make_inputs

    res = {}
    for kind, fz_set in (("ordinary", ()), ("frozen", tuple(range(cfg.H)))):
        c = cfg.with_(frozen=fz_set)
        inp = make_inputs(c)
        dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda().to(torch.bfloat16)  # noqa: E731
        t = dict(q=dev(inp.q), k=dev(inp.k), v=dev(inp.v), do=dev(inp.do),
                 a=torch.from_numpy(inp.a).cuda(), r=torch.from_numpy(inp.r).cuda(),
                 fz=[int(x) for x in inp.frozen])
        t["o"] = torch.empty_like(t["v"])
        t["lse"] = torch.empty((c.B, c.H, c.T), dtype=torch.float32, device="cuda")
        t["g"] = [torch.empty_like(t["v"]) for _ in range(3)]
        prm = B.Params(t["v"], t["fz"], inp.a.shape[1])
        t["ws"] = torch.empty(max(B.workspace_bytes(prm, True), B.workspace_bytes(prm, False), 256),
                              dtype=torch.uint8, device="cuda")
        res[kind] = t

    def run(t, with_bwd):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            B.saf_hybrid_attn_fwd(t["q"], t["k"], t["v"], t["fz"], t["a"], t["r"], out=t["o"], lse=t["lse"],
                                  workspace=t["ws"])
            if with_bwd:
                B.saf_hybrid_attn_bwd(t["q"], t["k"], t["v"], t["o"], t["do"], t["lse"], t["fz"], t["a"], t["r"],
                                      dq=t["g"][0], dk=t["g"][1], dv=t["g"][2], workspace=t["ws"])
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    def q(xs, p):
        return float(np.percentile(np.asarray(xs) / cfg.H, p))

    # the frozen heads' forward with their normalisers given (stored with the
    # pattern, as the pages keep log Z beside alpha and rho)
    fr = res["frozen"]
    fr["logz"] = B.saf_pattern_lognorm(fr["a"], fr["r"], cfg.T)

    def run_fwd_logz(t):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            B.saf_hybrid_attn_fwd(t["q"], t["k"], t["v"], t["fz"], t["a"], t["r"], out=t["o"], lse=t["lse"],
                                  workspace=t["ws"], logz=t["logz"])
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    out = {}
    for with_bwd, tag in ((False, "fwd"), (True, "fwd_bwd")):
        run(res["ordinary"], with_bwd)
        run(res["frozen"], with_bwd)
        samples = {"ordinary": [], "frozen": []}
        for order in (("ordinary", "frozen"), ("frozen", "ordinary")) * 4:
            for kind in order:
                samples[kind].append(run(res[kind], with_bwd))
        o_ms, f_ms = q(samples["ordinary"], 50), q(samples["frozen"], 50)
        o_iqr = [round(q(samples["ordinary"], 25), 5), round(q(samples["ordinary"], 75), 5)]
        f_iqr = [round(q(samples["frozen"], 25), 5), round(q(samples["frozen"], 75), 5)]
        out[tag] = {"ordinary_ms_per_head": round(o_ms, 5), "frozen_ms_per_head": round(f_ms, 5),
                    "frozen_over_ordinary": round(f_ms / o_ms, 3),
                    "ordinary_iqr": o_iqr, "frozen_iqr": f_iqr,
                    # frozen median below the ordinary one with disjoint interquartile ranges
                    "frozen_cheaper": bool(f_ms < o_ms and f_iqr[1] < o_iqr[0])}
    run(res["ordinary"], False)
    run_fwd_logz(fr)
    sz = {"ordinary": [], "frozen": []}
    for order in (("ordinary", "frozen"), ("frozen", "ordinary")) * 4:
        for kind in order:
            sz[kind].append(run(res["ordinary"], False) if kind == "ordinary" else run_fwd_logz(fr))
    o_ms, f_ms = q(sz["ordinary"], 50), q(sz["frozen"], 50)
    out["fwd_stored_lognorm"] = {"ordinary_ms_per_head": round(o_ms, 5), "frozen_ms_per_head": round(f_ms, 5),
                                 "frozen_over_ordinary": round(f_ms / o_ms, 3),
                                 "note": "forward only, the frozen heads' log N given (no normaliser pass)"}
    # zero-replacement control: the same all-ordinary call against itself in
    # A-B-B-A order; the comparison above is trusted only if this stays ~1.00
    ctl = {"a": [], "b": []}
    for order in (("a", "b"), ("b", "a")) * 4:
        for x in order:
            ctl[x].append(run(res["ordinary"], True))
    out["zero_replacement_control"] = round(float(np.median(ctl["b"]) / np.median(ctl["a"])), 4)
    out["note"] = (f"same shape (B={cfg.B}, T={cfg.T}, d={cfg.D}), all {cfg.H} heads ordinary vs all frozen; "
                   "median and quartiles of 8 A/B/B/A-ordered samples of 10 calls each")
    return out


def trainable_pattern_leg(B, cfg, t, stream, reps: int = 20):
    """Cost of the frozen heads' pattern gradients (the variant whose a and r
    keep training): saf_pattern_grad after the timed steps, with its kernels
    bracketed by the library's stage events.  Not part of the headline step."""
    import numpy as np
    import torch

    names = ["pg_delta", "pg_kv", "pg_reduce"] if cfg.dtype == "bf16" else ["pg_delta", "pg_f32"]
    da, dr = torch.zeros_like(t["a"]), torch.zeros_like(t["r"])
    prm = B.Params(t["v"], t["fz"], t["a"].shape[1])
    prm.set_strides(v=t["v"], o=t["o"], do=t["do"])
    ws = torch.empty(max(B.pattern_grad_workspace_bytes(prm), 256), dtype=torch.uint8, device="cuda")

    def call(evs=None):
        B.saf_pattern_grad(t["v"], t["o"], t["do"], t["lse"], t["fz"], t["a"], t["r"], da=da, dr=dr,
                           workspace=ws, stream=stream, events=evs)

    for _ in range(3):
        call()
    evs = []
    for _ in range(reps):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
        for x in e:
            x.record(stream)
        evs.append(e)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for s_ in range(reps):
        call(evs[s_])
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    kms = {n: float(np.mean([evs[s_][x].elapsed_time(evs[s_][x + 1]) for s_ in range(reps)]))
           for x, n in enumerate(names)}
    n_frz = len(cfg.frozen)
    fl = pairs(cfg.T) * cfg.D * 2 * cfg.B * n_frz  # dW = dO V^T over the causal pairs
    kern = "pg_kv" if cfg.dtype == "bf16" else "pg_f32"
    ach = fl / (kms[kern] * 1e-3) / 1e12
    return {"ms": round(ms, 4), "kernel_ms": {n: round(x, 4) for n, x in kms.items()},
            "roofline": {"bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4), "kernel": kern,
                         "flops_per_launch": fl},
            "note": "gradients of a and r for the frozen heads (trainable-pattern variant), one call per "
                    "step after the layer's backward; not included in value"}


def uniform_causal_targets(T: int):
    """Fit targets of uniform causal attention, P[i][j] = 1/(i+1) for j <= i:
    eta_abs[j] = eta_rel[j] = sum_{i >= j} 1/(i+1) = H_T - H_j (H the harmonic
    numbers) and sum P ln P = -sum_i ln(i+1) = -ln T!."""
    import numpy as np

    H = np.concatenate([[0.0], np.cumsum(1.0 / np.arange(1, T + 1, dtype=np.float64))])
    return H[T] - H[:T], -math.lgamma(T + 1.0)


def fit_scaling_leg(B, stream, n_heads: int = 12, Ts=(4096, 8192, 16384, 32768, 65536), steps: int = 400):
    """Cost of the compact-pattern fit as T grows: the recipe's 400 Adam
    steps on n_heads heads whose targets are the marginals of uniform causal
    attention (P[i][j] = 1/(i+1), so eta_abs[j] = eta_rel[j] = H_T - H_j in
    closed form, H the harmonic numbers, and sum P ln P = -ln T!, which gives
    kappa, the mean row KL of the fitted pattern from P; a compact pattern
    with a and r of equal slope is uniform, so kappa -> 0).  Every step evaluates the row
    normalisers and both fitted marginals exactly, over every causal pair, so
    the time grows as T^2; the target values do not change that work."""
    import numpy as np
    import torch

    rows = []
    for T in Ts:
        eta64, negent64 = uniform_causal_targets(T)
        eta = torch.from_numpy(eta64.astype(np.float32)).cuda()
        eta_abs = eta.expand(n_heads, T).contiguous()
        eta_rel = eta_abs.clone()
        negent = torch.full((n_heads,), negent64, dtype=torch.float32, device="cuda")
        ws = torch.empty(max(B.fit_pattern_workspace_bytes(n_heads, T), 256), dtype=torch.uint8, device="cuda")

        def fit(J):
            return B.saf_fit_pattern(eta_abs, eta_rel, negent, steps=J, workspace=ws, stream=stream)

        out = fit(steps)
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        ev[0].record(stream)
        fit(steps)
        ev[1].record(stream)
        fit(0)
        ev[2].record(stream)
        torch.cuda.synchronize()
        t_fit = ev[0].elapsed_time(ev[1])
        t_step = (t_fit - ev[1].elapsed_time(ev[2])) / steps
        pairs_ = T * (T + 1) // 2
        rows.append({"T": T, "fit_ms": round(t_fit, 3), "adam_step_ms": round(t_step, 5),
                     "causal_pairs_per_s": float(f"{3 * pairs_ * n_heads / (t_step * 1e-3):.4g}"),
                     "kappa_max": float(f"{float(out['kappa'].max()):.4g}")})
        del ws, out
    return {"heads": n_heads, "adam_steps": steps, "targets": "uniform causal attention (closed form)",
            "rows": rows,
            "note": "exact band sums per step (no FFT): time ~ T^2; kappa_max over the heads after the fit"}


def pattern_fit_leg(B, stream, reps: int = 5):
    """Fitting compact patterns for the 124M model's 25% replaced heads (36
    calibration means at T = 4096): target statistics, then the recipe's 400
    Adam steps, with every mean already resident in HBM.  Reported apart from
    the layer step; the pages time this one-time intervention separately."""
    import numpy as np
    import torch

    from synth.targets import FIT_WORKLOADS, calibration_mean

    wl = FIT_WORKLOADS["gpt2_124m_25pct"]
    n, T = wl.n_heads, wl.T
    A = torch.empty((n, T, T), dtype=torch.float32, device="cuda")
    for h in range(n):
        A[h].copy_(torch.from_numpy(calibration_mean(T, wl.seed, h)))
    wst = torch.empty(max(B.fit_targets_workspace_bytes(n, T), 256), dtype=torch.uint8, device="cuda")
    wsf = torch.empty(max(B.fit_pattern_workspace_bytes(n, T), 256), dtype=torch.uint8, device="cuda")
    steps = 400

    def targets():
        return B.saf_fit_targets(A, workspace=wst, stream=stream)

    def fit(st, J):
        return B.saf_fit_pattern(*st, steps=J, workspace=wsf, stream=stream)

    st = targets()
    res = fit(st, steps)
    torch.cuda.synchronize()

    def timed(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    t_all = timed(lambda: fit(targets(), steps))
    t_targets = timed(targets)
    t_fit = timed(lambda: fit(st, steps))
    t_fit0 = timed(lambda: fit(st, 0))
    t_step = (t_fit - t_fit0) / steps
    # algorithmic work: one read of each causal triangle; per Adam step one
    # multiply-add per causal pair for the normaliser and for each marginal
    pairs_ = T * (T + 1) // 2
    tbytes = n * pairs_ * 4
    step_flops = 3 * 2 * pairs_ * n
    ach_t = tbytes / (t_targets * 1e-3) / 1e9
    ach_s = step_flops / (t_step * 1e-3) / 1e12
    kappa = res["kappa"].cpu().numpy()
    return {
        "workload": wl.name, "heads": n, "T": T, "adam_steps": steps,
        "ms": round(t_all, 3), "targets_ms": round(t_targets, 4), "fit_ms": round(t_fit, 3),
        "adam_step_ms": round(t_step, 5),
        "accepted": int((kappa <= 0.2).sum()), "kappa_median": round(float(np.median(kappa)), 4),
        "pages_fit_s": PAGES_FIT_S_124M_25PCT,
        "speedup_vs_pages": round(PAGES_FIT_S_124M_25PCT * 1e3 / t_all, 1),
        "roofline": {"bound": "alu", "achieved": round(ach_s, 2), "peak": PEAK_F32_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(ach_s / PEAK_F32_TFLOPS, 4), "kernel": "lognorm + fit_step (one Adam step)",
                     "flops_per_step": step_flops},
        "targets_roofline": {"bound": "hbm", "achieved": round(ach_t, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                             "frac": round(ach_t / PEAK_HBM_GBS, 4), "bytes_per_call": tbytes},
        "note": "pages' figure: GH200, FFT fitter, three-seed mean (Table 13); another machine and "
                "implementation, context only",
    }


# Calibration time the pages print for the 124M model at 4K (Table 13,
# "Capture and mean" column, 25% rate, three-seed mean; GH200): running the
# model on 32 sequences, capturing every head's attention and averaging it.
PAGES_CALIB_S_124M = 51.56

# fp32 flops counted per (head, sequence, causal entry) update of the
# calibration statistics, as calib_stats_kernel performs it: the score's log2
# probability (1 FMA = 2), the A log2 A sum (1 FMA = 2), the deviation from the
# first sequence's value (1 subtraction), its sum (1 addition) and its square
# sum (1 FMA = 2).  The exponential is not counted.
CALIB_FLOPS_PER_UPDATE = 2 + 2 + 1 + 1 + 2


def calibration_leg(B, stream, reps: int = 3):
    """Calibration statistics of the 124M model: mean attention, variance and
    forward-KL scores of its 144 heads (12 layers x 12) over 32 sequences of
    4096 tokens, from queries and keys resident in HBM.  The synthetic
    activations of one layer's 12 heads are used for every layer (the work
    does not depend on the values).  Reported apart from the layer step."""
    import numpy as np
    import torch

    from synth.calib import CALIB_WORKLOADS, calibration_qk

    wl = CALIB_WORKLOADS["gpt2_124m_4k"]
    N, H, T, D = wl.N, wl.H, wl.T, wl.D
    layers = 12
    q1, k1 = calibration_qk(N, H, T, D, wl.seed)
    q = torch.from_numpy(q1).cuda().to(torch.bfloat16).repeat(1, layers, 1, 1)
    k = torch.from_numpy(k1).cuda().to(torch.bfloat16).repeat(1, layers, 1, 1)
    del q1, k1
    Ht = H * layers
    ahat = torch.zeros((Ht, T, T), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(B.calib_stats_workspace_bytes(N, Ht, T), 256), dtype=torch.uint8, device="cuda")

    def call():
        return B.saf_calib_stats(q, k, ahat=ahat, workspace=ws, stream=stream)

    _, s_var, s_kl = call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    pairs_ = T * (T + 1) // 2
    updates = Ht * N * pairs_  # (head, sequence, causal entry) updates of the statistics
    flops = CALIB_FLOPS_PER_UPDATE * updates
    ach = flops / (ms * 1e-3) / 1e12
    order = np.argsort(s_var.cpu().numpy()[:H])
    return {
        "workload": wl.name, "heads": Ht, "sequences": N, "T": T, "D": D,
        "ms": round(ms, 3), "updates_per_s": round(updates / (ms * 1e-3), 1),
        "lowest_variance_heads_of_layer": [int(x) for x in order[:3]],
        "pages_capture_and_mean_s": PAGES_CALIB_S_124M,
        "roofline": {"bound": "alu", "achieved": round(ach, 2), "peak": PEAK_F32_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(ach / PEAK_F32_TFLOPS, 4), "kernel": "calib_lse + calib_stats (whole call)",
                     "flops_per_call": flops},
        "note": "pages' figure: GH200, whole-model forward passes with attention capture (Table 13); "
                "here the statistics from resident queries and keys only; context, not a target",
    }


# Attention-operation prefill speedups the pages print for the Qwen3-4B
# grouped-query path over all-ordinary attention (Table 26, in parentheses),
# keyed by (B, T, replaced fraction in percent).
PAGES_GQA_SPEEDUP = {
    (4, 2048, 10): 1.16, (4, 2048, 20): 1.18, (4, 2048, 30): 1.21, (4, 2048, 50): 1.29, (4, 2048, 75): 1.38,
    (4, 4096, 10): 1.16, (4, 4096, 20): 1.19, (4, 4096, 30): 1.23, (4, 4096, 50): 1.28, (4, 4096, 75): 1.38,
    (4, 8192, 10): 1.15, (4, 8192, 20): 1.19, (4, 8192, 30): 1.23, (4, 8192, 50): 1.30, (4, 8192, 75): 1.37,
    (8, 2048, 10): 1.15, (8, 2048, 20): 1.17, (8, 2048, 30): 1.21, (8, 2048, 50): 1.28, (8, 2048, 75): 1.37,
    (8, 4096, 10): 1.15, (8, 4096, 20): 1.19, (8, 4096, 30): 1.18, (8, 4096, 50): 1.27, (8, 4096, 75): 1.37,
    (8, 8192, 10): 1.15, (8, 8192, 20): 1.18, (8, 8192, 30): 1.22, (8, 8192, 50): 1.30, (8, 8192, 75): 1.40,
}


def fwd_speedup_vs_ordinary(B, cfg, q, k, v, a, r, fz, reps: int = 10):
    """Forward time with every head ordinary over the time with the workload's
    frozen heads, same inputs and shape, timed in A-B-B-A order."""
    import numpy as np
    import torch

    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    logz = B.saf_pattern_lognorm(a, r, cfg.T)  # the stored normalisers of fixed patterns
    kinds = {"ordinary": ([0] * cfg.H, None), "hybrid": (fz, None), "hybrid_logz": (fz, logz)}

    def run(kind):
        f, lz = kind
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            B.saf_hybrid_attn_fwd(q, k, v, f, a, r, out=o, lse=lse, logz=lz)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    for kd in kinds.values():
        run(kd)
    samples = {n: [] for n in kinds}
    for order in (("ordinary", "hybrid", "hybrid_logz"), ("hybrid_logz", "hybrid", "ordinary")) * 2:
        for n in order:
            samples[n].append(run(kinds[n]))
    t_o = float(np.median(samples["ordinary"]))
    t_h = float(np.median(samples["hybrid"]))
    t_z = float(np.median(samples["hybrid_logz"]))
    frac = 100.0 * len(cfg.frozen) / cfg.H
    col = min((10, 20, 30, 50, 75), key=lambda c: abs(c - frac))  # the pages' nearest column
    return {"ordinary_ms": round(t_o, 4), "hybrid_ms": round(t_h, 4), "speedup": round(t_o / t_h, 3),
            "hybrid_stored_lognorm_ms": round(t_z, 4), "speedup_stored_lognorm": round(t_o / t_z, 3),
            "replaced_percent": round(frac, 1),
            "pages_speedup": PAGES_GQA_SPEEDUP.get((cfg.B, cfg.T, col)) if cfg.Hkv != cfg.H else None,
            "pages_column_percent": col,
            "note": "forward of the same shape with every head ordinary vs with the workload's frozen heads "
                    "(normalisers computed by the call, or given as the stored log Z); pages_speedup: the "
                    "attention-operation speedup the pages print for this B, T and fraction (a different "
                    "machine and baseline kernel; context only)"}


# Whole-update speedups the pages report for replacing 25% of the heads
# (optimiser update: forward, backward, clipping and AdamW of the whole model),
# quoted as context beside the layer ratio measured here.  Different scope,
# different machine: not a target.
PAGES_UPDATE_SPEEDUPS = [
    {"speedup": 1.056, "model": "124M GPT (12 layers x 12 heads, d=64)", "T": 4096, "replaced": "25%",
     "hardware": "1x NVIDIA GH200, bf16", "scope": "whole optimiser update (B=8 x 15 accumulation steps)",
     "source": "Section 5, Table 2a (2249.49 -> 2129.42 ms per update)"},
    {"speedup": 1.068, "model": "1B (32 layers x 16 heads, hidden 1536)", "T": 8192, "replaced": "25%",
     "hardware": "4x NVIDIA GH200 (data parallel, gradient all-reduce included), bf16",
     "scope": "whole optimiser update (B=2 per GPU x 8 accumulation steps)",
     "source": "Appendix C.5, Table 23 (4258.67 -> 3986.67 ms per update)"},
]


def fused_dq_leg(B, cfg, q, k, v, do, a, r, fz, o, lse, stream, two_pass_ms, reps: int = 20):
    """The backward's other schedule, fused dQ (one key-block pass that also
    adds each program's dQ into an fp32 accumulator with atomic adds, no
    query-block pass), timed at the same shape with its kernels bracketed by
    the library's stage events.  Not part of the headline step, whose
    backward is the deterministic two-pass schedule."""
    import numpy as np
    import torch

    g = [torch.empty_like(v) for _ in range(3)]
    prm = B.Params(v, fz, a.shape[1])
    prm.p.fused_dq = 1
    ws = torch.empty(max(B.workspace_bytes(prm, True), 256), dtype=torch.uint8, device=v.device)
    has_ord = not all(fz)
    names = ["bwd_pre", "bwd_kvq", "dq_convert"] if has_ord else ["bwd_kvq"]

    def call(evs=None):
        B.saf_hybrid_attn_bwd(q, k, v, o, do, lse, fz, a, r, dq=g[0], dk=g[1], dv=g[2], workspace=ws,
                              stream=stream, events=evs, fused_dq=True)

    for _ in range(3):
        call()
    evs = []
    for _ in range(reps):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
        for x in e:
            x.record(stream)
        evs.append(e)
    torch.cuda.synchronize()
    for s_ in range(reps):
        call(evs[s_])
    torch.cuda.synchronize()
    kms = {n: float(np.mean([evs[s_][x].elapsed_time(evs[s_][x + 1]) for s_ in range(reps)]))
           for x, n in enumerate(names)}
    tot = float(np.mean([evs[s_][0].elapsed_time(evs[s_][-1]) for s_ in range(reps)]))
    return {"bwd_ms": round(tot, 4), "kernel_ms": {n: round(x, 4) for n, x in kms.items()},
            "two_pass_bwd_ms": round(two_pass_ms, 4), "fused_over_two_pass": round(tot / two_pass_ms, 3),
            "atomic_bytes": pairs_tiles_bytes(cfg),
            "note": "fused-dQ backward schedule (fused_dq = 1): dQ accumulated with fp32 atomic adds inside the "
                    "key-block pass; the headline uses the two-pass schedule"}


def pairs_tiles_bytes(cfg):
    """fp32 bytes the fused schedule adds atomically: one 64-query x D block
    per (ordinary (b, h), 128-key block, 64-query tile at or after it)."""
    nkb = (cfg.T + 127) // 128
    nqt = (cfg.T + 63) // 64
    tiles = sum(nqt - 2 * kb for kb in range(nkb))
    return cfg.B * (cfg.H - len(cfg.frozen)) * tiles * 64 * cfg.D * 4


def layer_vs_all_ordinary(B, cfg, q, k, v, do, a, r, fz, reps: int = 10):
    """fwd+bwd of the layer with every head ordinary over the same call with
    the workload's frozen heads (same inputs and shape), 8 samples of `reps`
    calls each in A-B-B-A order."""
    import numpy as np
    import torch

    o = torch.empty_like(v)
    lse = torch.empty(v.shape[:3], dtype=torch.float32, device=v.device)
    g = [torch.empty_like(v) for _ in range(3)]
    prm = B.Params(v, [0] * cfg.H, a.shape[1])
    ws = torch.empty(max(B.workspace_bytes(prm, True), B.workspace_bytes(B.Params(v, fz, a.shape[1]), False),
                         256), dtype=torch.uint8, device=v.device)
    masks = {"ordinary": [0] * cfg.H, "hybrid": fz}

    def run(mask):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            B.saf_hybrid_attn_fwd(q, k, v, mask, a, r, out=o, lse=lse, workspace=ws)
            B.saf_hybrid_attn_bwd(q, k, v, o, do, lse, mask, a, r, dq=g[0], dk=g[1], dv=g[2], workspace=ws)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    for m in masks.values():
        run(m)
    samples = {n: [] for n in masks}
    for order in (("ordinary", "hybrid"), ("hybrid", "ordinary")) * 4:
        for n in order:
            samples[n].append(run(masks[n]))
    t_o, t_h = float(np.median(samples["ordinary"])), float(np.median(samples["hybrid"]))
    return {"ordinary_ms": round(t_o, 4), "hybrid_ms": round(t_h, 4), "speedup": round(t_o / t_h, 3),
            "note": f"one fwd+bwd of this layer with all {cfg.H} heads ordinary over the same call with heads "
                    f"{list(cfg.frozen)} frozen; median of 8 A/B/B/A-ordered samples of {reps} calls"}


def cpu_baseline(cfg, inp, budget_s: float = 20.0):
    """Time the float64 oracle on whole heads of the workload (host cores)."""
    import numpy as np

    import oracle

    try:
        from threadpoolctl import threadpool_info

        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    s = 1.0 / np.sqrt(cfg.D)
    fz = [int(x) for x in inp.frozen]
    g = cfg.H // cfg.Hkv  # query heads per key/value head
    # alternate ordinary / frozen heads, batch element by batch element, until
    # the budget is used
    ords = [h for h in range(cfg.H) if not fz[h]]
    frzs = [h for h in range(cfg.H) if fz[h]]
    order = []
    for b in range(cfg.B):
        for x in range(max(len(ords), len(frzs))):
            if x < len(ords):
                order.append((b, ords[x]))
            if x < len(frzs):
                order.append((b, frzs[x]))
    done_ord = done_frz = 0
    t0 = time.perf_counter()
    for b, h in order:
        if fz[h]:
            oracle.frozen_head_fwd(inp.v[b, h // g], inp.a[h], inp.r[h])
            if inp.do is not None:
                oracle.frozen_head_bwd(inp.do[b, h], inp.a[h], inp.r[h])
            done_frz += 1
        else:
            oracle.ordinary_head_fwd(inp.q[b, h], inp.k[b, h // g], inp.v[b, h // g], s)
            if inp.do is not None:
                oracle.ordinary_head_bwd(inp.q[b, h], inp.k[b, h], inp.v[b, h], inp.do[b, h], s)
            done_ord += 1
        if time.perf_counter() - t0 >= budget_s and done_ord and done_frz:
            break
    dt = time.perf_counter() - t0
    f = flops(cfg, n_ord=done_ord, n_frz=done_frz, B=1)
    fl = f["total"] if inp.do is not None else f["fwd"]
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:  # pragma: no cover
        pass
    return {
        "value": fl / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "cpu_model": model,
        "kind": "oracle",
        "sample": f"float64 dense oracle, fwd+bwd of {done_ord} ordinary + {done_frz} frozen whole "
                  f"(batch, head) slices of the {cfg.B * cfg.H} in the workload (T={cfg.T}, d={cfg.D}) in "
                  f"{dt:.1f} s; value = their algorithmic flops / time, i.e. the sample's rate taken as the "
                  f"whole workload's (an extrapolation: the whole call was not run)",
        "seconds": round(dt, 2),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # at least 200 ms of timed work at the headline shape (0.84 ms per step)
    ap.add_argument("--steps", type=int, default=250)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default=DEFAULT_CONFIG,
                    help="workload (synth.CONFIGS key); the default is the headline metric's; others: "
                         "gpt2_124m_4k_50pct_interleaved, 1b_8k_rank_share, prefill_32k, qwen3_4b_prefill_B4_T4096_30pct, "
                         "pages_check_t129, tiny")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--no-per-head", action="store_true")
    ap.add_argument("--no-pattern-grad", action="store_true",
                    help="skip the trainable-pattern leg (gradients of a and r, reported apart from value)")
    ap.add_argument("--no-fit", action="store_true",
                    help="skip the pattern-fitting leg (36 fits at T=4096, reported apart from value)")
    ap.add_argument("--fit-only", action="store_true", help="run only the pattern-fitting leg")
    ap.add_argument("--fit-scaling", action="store_true",
                    help="run only the fit's T-scaling leg (12 heads, T = 4096 .. 65536, 400 Adam steps each)")
    ap.add_argument("--no-calib", action="store_true",
                    help="skip the calibration-statistics leg (144 heads, 32 x 4096 tokens, apart from value)")
    ap.add_argument("--calib-only", action="store_true", help="run only the calibration-statistics leg")
    ap.add_argument("--calib-copy", action="store_true",
                    help="only run a plain copy of known size (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this library runs on one GPU only; multi-GPU sharding is not built "
                                   "(--gpus must be 1)"}))
        sys.exit(2)

    if args.calib_copy:
        calib_copy()
        return

    import numpy as np
    import torch

    from fixed_pattern_hybrid_amd import binding as B
    from synth import CONFIGS, make_inputs

    if args.fit_only:
        print(json.dumps({"pattern_fit": pattern_fit_leg(B, torch.cuda.current_stream())}), flush=True)
        return
    if args.fit_scaling:
        print(json.dumps({"fit_scaling": fit_scaling_leg(B, torch.cuda.current_stream())}), flush=True)
        return
    if args.calib_only:
        print(json.dumps({"calibration": calibration_leg(B, torch.cuda.current_stream())}), flush=True)
        return

    cfg = CONFIGS[args.config]
    inp = make_inputs(cfg)
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda().to(dt)  # noqa: E731
    q, k, v = dev(inp.q), dev(inp.k), dev(inp.v)
    do = dev(inp.do) if inp.do is not None else None
    a, r = torch.from_numpy(inp.a).cuda(), torch.from_numpy(inp.r).cuda()
    fz = [int(x) for x in inp.frozen]
    Bn, H, T, D = cfg.B, cfg.H, cfg.T, cfg.D
    o = torch.empty_like(q)
    lse = torch.empty((Bn, H, T), dtype=torch.float32, device="cuda")
    dq, dk, dv = (torch.empty_like(v), torch.empty_like(v), torch.empty_like(v)) if do is not None else (None,) * 3
    prm = B.Params(q, fz, a.shape[1], kv_heads=0 if cfg.Hkv == H else cfg.Hkv)
    ws = torch.empty(max(B.workspace_bytes(prm, True), B.workspace_bytes(prm, False), 256),
                     dtype=torch.uint8, device="cuda")
    has_frz = any(fz)
    has_ord = not all(fz)
    names_f = (["lognorm"] if has_frz else []) + ["fwd"]
    if cfg.dtype == "bf16":
        names_b = (["bwd_q"] if has_ord else []) + ["bwd_kv"]
    else:
        names_b = ["bwd_pre", "bwd_kv"] + (["bwd_q"] if has_ord else [])
    n_fwd_ev = len(names_f) + 1
    n_bwd_ev = len(names_b) + 1
    stream = torch.cuda.current_stream()

    def mk_events(n):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        for e in evs:
            e.record(stream)  # creates the underlying HIP event
        return evs

    def step(fe=None, be=None):
        B.saf_hybrid_attn_fwd(q, k, v, fz, a, r, out=o, lse=lse, workspace=ws, stream=stream, events=fe)
        if do is not None:
            B.saf_hybrid_attn_bwd(q, k, v, o, do, lse, fz, a, r, dq=dq, dk=dk, dv=dv, workspace=ws,
                                  stream=stream, events=be)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    K = args.steps
    fevs = [mk_events(n_fwd_ev) for _ in range(K)]
    bevs = [mk_events(n_bwd_ev) for _ in range(K)]
    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    t_start.record(stream)
    for s in range(K):
        step(fevs[s], bevs[s])
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms = t_start.elapsed_time(t_end) / K

    # per-kernel durations from the library's stage events
    per = {n: [] for n in names_f + names_b}
    for s in range(K):
        for x, n in enumerate(names_f):
            per[n].append(fevs[s][x].elapsed_time(fevs[s][x + 1]))
        if do is not None:
            for x, n in enumerate(names_b):
                per[n].append(bevs[s][x].elapsed_time(bevs[s][x + 1]))
    kern_ms = {n: float(np.mean(v_)) for n, v_ in per.items() if v_}
    # per-step durations: from the first forward event to the last one of the
    # step (the backward's when it runs)
    step_ms = [fevs[s][0].elapsed_time(bevs[s][-1] if do is not None else fevs[s][-1]) for s in range(K)]

    f = flops(cfg)
    total = f["total"] if do is not None else f["fwd"]
    value = total / (ms * 1e-3) / 1e12
    tokens = Bn * T / (ms * 1e-3)
    # dominant kernel and its algorithmic flops per launch
    dom = max(kern_ms, key=kern_ms.get)
    dom_flops = f.get(dom)
    roof = None
    if dom_flops is not None:
        ach = dom_flops / (kern_ms[dom] * 1e-3) / 1e12
        headline = args.config == DEFAULT_CONFIG
        traffic = measured_traffic(dom) if headline else None
        roof = {"bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(ach / PEAK_BF16_TFLOPS, 4), "traffic": traffic, "kernel": dom,
                "kernel_ms": round(kern_ms[dom], 4)}
    metric = ("hybrid-attn fwd+bwd TFLOP/s & MFMA util, 124M/4K shape, 25% heads frozen"
              if args.config == DEFAULT_CONFIG else
              f"hybrid-attn {'fwd+bwd' if do is not None else 'fwd'} TFLOP/s, workload {cfg.name}")
    out = {
        "metric": metric,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": cfg.name, "B": Bn, "H": H, "T": T, "D": D, "frozen_heads": list(cfg.frozen),
                   "pass": "fwd+bwd" if do is not None else "fwd",
                   **({"kv_heads": cfg.Hkv} if cfg.Hkv != H else {})},
        "mfma_util": round(value / PEAK_BF16_TFLOPS, 4),
        "tokens_per_s": round(tokens, 1),
        "kernel_ms": {n: round(x, 4) for n, x in kern_ms.items()},
        "fwd_ms": round(sum(kern_ms[n] for n in names_f), 4),
        "bwd_ms": round(sum(kern_ms[n] for n in names_b), 4) if do is not None else None,
        "step_ms_median": round(float(np.median(step_ms)), 4),
        "step_ms_min": round(float(np.min(step_ms)), 4),
        "step_ms_p90": round(float(np.percentile(step_ms, 90)), 4),
        "exp": exp_counts(cfg, do is not None),
        "wall_s_timed": round(wall, 3),
        "roofline": roof,
    }
    if args.config == DEFAULT_CONFIG:
        # HBM traffic of every layer kernel (counter summaries) against its
        # algorithmic bytes, and the bandwidth it implies at this run's times
        alg = algorithmic_bytes(cfg)
        hbm = {}
        for n in ("fwd", "bwd_q", "bwd_kv"):
            if n not in kern_ms:
                continue
            tb = measured_traffic(n)
            hbm[n] = {"algorithmic_bytes": alg[n], "traffic_bytes": tb,
                      "traffic_over_algorithmic": round(tb / alg[n], 3) if tb else None,
                      "traffic_GBps": round(tb / (kern_ms[n] * 1e-3) / 1e9, 1) if tb else None,
                      "frac_of_hbm_peak": round(tb / (kern_ms[n] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4) if tb else None}
        out["hbm_traffic"] = hbm
    if not args.no_pattern_grad and do is not None and has_frz:
        tp = trainable_pattern_leg(B, cfg, dict(v=v, o=o, do=do, lse=lse, a=a, r=r, fz=fz), stream)
        tp["over_layer_step"] = round(tp["ms"] / ms, 4)
        out["trainable_pattern"] = tp
    if do is not None and cfg.dtype == "bf16" and D == 64 and has_ord:
        out["bwd_fused_dq"] = fused_dq_leg(B, cfg, q, k, v, do, a, r, fz, o, lse, stream, out["bwd_ms"])
    if not args.no_per_head and do is not None:
        out["per_head"] = per_head_costs(B, cfg)
        if has_frz and has_ord:
            out["layer_vs_all_ordinary"] = layer_vs_all_ordinary(B, cfg, q, k, v, do, a, r, fz)
    if args.config == DEFAULT_CONFIG:
        out["context"] = {"pages_update_speedups": PAGES_UPDATE_SPEEDUPS,
                          "note": "the pages' whole-model update speedups at 25% replaced heads, on their "
                                  "hardware; context for layer_vs_all_ordinary, not a target"}
    if not args.no_per_head and do is None and has_frz:
        out["attention_op_speedup"] = fwd_speedup_vs_ordinary(B, cfg, q, k, v, a, r, fz)
    if not args.no_fit and args.config == DEFAULT_CONFIG:
        out["pattern_fit"] = pattern_fit_leg(B, stream)
    if not args.no_calib and args.config == DEFAULT_CONFIG:
        out["calibration"] = calibration_leg(B, stream)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, inp, args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
