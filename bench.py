"""Benchmark of one Muon optimizer step (Aurora + Contra-Muon + u/w-floor).

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--recipe aurora|classic] [--gpus 1]

A step is one libmuon `muon_update` over the whole matrix batch of the
workload (default: every matrix of the 28-layer 3.8B-style decoder, 168
matrices, 2.82B parameters, bf16 grads/weights, fp32 momentum), inputs
resident in HBM, momentum and weights updated in place. Prints one JSON line.

value = counted Newton-Schulz TFLOP/s of the whole step (4 s^2 L + 2 s^3 per
iteration per matrix, s <= L, 12 iterations, 2 passes for non-square
matrices; 5 iterations and one pass with --recipe classic) = counted flops /
step time.

`roofline` is the matrix-core engine alone (summed HIP-event time of its
launches on the library's stream over the timed steps) against the bf16 dense
peak, on the ALGORITHMIC flops of the products the library runs: each
product's flops with the upper half of a symmetric result counted once and no
padding. A block of r iterations of a rectangular matrix needs
3 s^2 L + (4 r - 3) s^3 (Gram s^2 L, 4 r - 3 short-side products of s^3,
X' = Q X 2 s^2 L); a square matrix runs one-iteration blocks, 3 s^2 L + s^3
per iteration. Beside it, three rates that are NOT hardware utilisation: the
standard-iteration rate (3 s^2 L + s^3 per iteration for every matrix, the
work of the plain iteration with symmetric halves skipped), the counted rate
(4 s^2 L + 2 s^3, the headline convention) and the executed rate (flops the
tiles issue, including padding and whole diagonal tiles; a hardware
matrix-core counter gives the same figure). Since the blocks need fewer flops
than the plain iteration, the first two can exceed the peak. Also: the
streaming kernels of the step against the page-level byte budget (momentum
14, power iteration 12, tail 8 bytes per bf16 element).
`clocks` samples the GPU clocks during the timed steps; `cpu_baseline` times
the float64 oracle on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "Aurora-Muon optimizer-step ms & MFMA TFLOP/s (% peak), 3.8B bf16 matrix set"
METRIC_CLASSIC = "Classic Muon (NS5) optimizer-step ms & MFMA TFLOP/s (% peak), 3.8B bf16 matrix set"
PEAK_BF16_TFLOPS = 2516.6       # MI355X dense bf16 matrix-core peak
PEAK_FP32_TFLOPS = 157.3


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def measured_traffic(workload: str):
    """HBM bytes per engine launch from the committed byte-counter record, or
    None when there is none for this workload or the engine source changed
    since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"ns_engine_{workload}_traffic.json")
    src = os.path.join(ROOT, "muon_newton_schulz_update_amd", "csrc", "ns_gemm.hip")
    try:
        rec = json.load(open(path))
        cur = hashlib.sha256(open(src, "rb").read()).hexdigest()
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != cur:
        return None
    return rec.get("traffic_bytes_per_launch")


def step_flops(shapes, cfg) -> float:
    from muon_newton_schulz_update_amd.inputs import counted_ns_flops
    tot = 0.0
    for r, c in shapes:
        passes = 1 if (r == c or cfg.pp_iterations == 0) else cfg.pp_iterations
        tot += counted_ns_flops(r, c, cfg.ns_steps, passes)
    return tot


def algorithmic_flops(shapes, cfg) -> float:
    """3 s^2 L + s^3 per iteration per matrix: the plain iteration's products
    with the symmetric halves of A = X X^T and A A^T counted once."""
    tot = 0.0
    for r, c in shapes:
        s, L = min(r, c), max(r, c)
        passes = 1 if (r == c or cfg.pp_iterations == 0) else cfg.pp_iterations
        tot += passes * cfg.ns_steps * (3.0 * s * s * L + float(s) ** 3)
    return tot


def stream_budget_bytes(shapes, grad_bytes, weight_bytes, cfg) -> float:
    """Page-level HBM bytes of the streaming kernels per step: momentum pass
    (read G, read and write fp32 M, write X, read W for its norm), power
    iteration (six reads of X when the Contra term is on) and tail (read U
    and X, read and write W); X and U in the grad's type. 34 B per element
    for bf16 grads and weights."""
    xb = grad_bytes
    per = grad_bytes + 8 + xb + (weight_bytes or 0)
    if cfg.contra != 0:
        per += 6 * xb
    per += xb + (xb if cfg.contra != 0 else 0) + 2 * (weight_bytes or 0)
    return float(sum(r * c for r, c in shapes)) * per


class ClockSampler:
    """Samples the GPU's current clocks with the ROCm SMI tool on a thread
    while the timed steps run (values in MHz, as the tool reports them)."""

    def __init__(self, period_s: float = 1.0):
        import threading
        self.samples = []
        self.source = None
        self.error = None
        self._stop = threading.Event()
        self._period = period_s
        self._t = threading.Thread(target=self._run, daemon=True)

    def _sample(self):
        import re
        import subprocess
        for cmd in (["rocm-smi", "--showgpuclocks", "--json"], ["amd-smi", "metric", "-c", "--json"]):
            try:
                r = subprocess.run(cmd, capture_output=True, text=True, timeout=10)
            except Exception as e:          # tool missing or hung
                self.error = f"{cmd[0]}: {e}"
                continue
            if r.returncode != 0:
                self.error = f"{cmd[0]} rc {r.returncode}"
                continue
            try:
                d = json.loads(r.stdout)
            except ValueError:
                self.error = f"{cmd[0]}: no JSON"
                continue
            found = {}

            def walk(o, key=""):
                if isinstance(o, dict):
                    for k, v in o.items():
                        walk(v, f"{key}/{k}".lower())
                elif isinstance(o, (str, int, float)):
                    m = re.search(r"(\d+(?:\.\d+)?)\s*mhz", str(o).lower())
                    val = float(m.group(1)) if m else (float(o) if isinstance(o, (int, float)) else None)
                    if val is None:
                        return
                    for name in ("sclk", "gfx", "mclk", "fclk", "socclk"):
                        if name in key and name not in found:
                            found[name] = val
            walk(d)
            if found:
                self.source = cmd[0]
                return found
        return None

    def _run(self):
        while not self._stop.is_set():
            f = self._sample()
            if f:
                self.samples.append(f)
            self._stop.wait(self._period)

    def __enter__(self):
        self._t.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        self._t.join(timeout=15)

    def summary(self):
        if not self.samples:
            return {"source": None, "error": self.error}
        out = {"source": self.source, "samples": len(self.samples)}
        for k in sorted({k for s in self.samples for k in s}):
            v = sorted(s[k] for s in self.samples if k in s)
            out[f"{k}_mhz"] = {"min": v[0], "median": v[len(v) // 2], "max": v[-1]}
        return out


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(name: str, grads, moms, weights, cfg, budget_s: float) -> dict:
    """Time the float64 oracle on a bounded sample of the workload's matrices."""
    import numpy as np
    from oracle import muon_oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        cores = os.cpu_count() or 1
    oc = O.OracleConfig(ns_steps=cfg.ns_steps, ns_a=cfg.ns_a, ns_b=cfg.ns_b, ns_c=cfg.ns_c,
                        pp_iterations=cfg.pp_iterations, pp_beta=cfg.pp_beta,
                        mu=float(np.float32(cfg.mu)), nesterov=bool(cfg.nesterov),
                        power_steps=cfg.power_steps, contra=float(np.float32(cfg.contra)),
                        target_uw=float(np.float32(cfg.target_uw)), lr=float(np.float32(cfg.lr)),
                        momentum="sgd" if cfg.flags & 1 else "ema", wide_rows=bool(cfg.flags & 2))
    # smallest matrices first so the sample stays bounded
    order = sorted(range(len(grads)), key=lambda i: grads[i].numel())
    done, flops, t_total = [], 0.0, 0.0
    for i in order:
        g = grads[i].float().cpu().double().numpy()
        m = moms[i].float().cpu().double().numpy()
        w = None if weights is None else weights[i].float().cpu().double().numpy()
        t0 = time.perf_counter()
        O.muon_update(g, m, w, oc)
        dt = time.perf_counter() - t0
        t_total += dt
        flops += step_flops([tuple(grads[i].shape)], cfg)
        done.append(tuple(grads[i].shape))
        if t_total >= budget_s:
            break
    from collections import Counter
    kinds = ", ".join(f"{n} x {r}x{c}" for (r, c), n in Counter(done).items())
    return {"value": flops / t_total / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{len(done)} matrices of {name} ({kinds}), smallest first, float64 numpy, "
                      f"{t_total:.1f} s",
            "host_cpus": os.cpu_count(), "cpu_model": cpu_model()}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="llama3p8b_all_layers")
    ap.add_argument("--recipe", default="aurora", choices=["aurora", "classic"],
                    help="aurora: the Aurora + Contra + floor step (the headline metric); classic: the "
                         "five-step Muon recipe (momentum after its warm-up, NS5, no Aurora/Contra/floor)")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work (0 = skip)")
    ap.add_argument("--no-profile", action="store_true", help="skip per-launch event timing")
    ap.add_argument("--no-clocks", action="store_true", help="do not sample GPU clocks with the SMI tool")
    ap.add_argument("--fp8-gram", action="store_true",
                    help="research option, not the headline: the first Gram of each pass on fp8 operands "
                         "(MUON_FLAG_FP8_GRAM); the line's dtype says so")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="before the steps, run one plain device copy, one read-only sum and one fill "
                         "of this many MiB (known-size references for hardware byte counters)")
    a = ap.parse_args()

    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: libmuon has no multi-GPU path (every matrix's step is "
              "independent, so a multi-GPU run would shard whole matrices across ranks)",
              file=sys.stderr)
        return 2

    import torch
    import muon_newton_schulz_update_amd as mu
    from muon_newton_schulz_update_amd import inputs as gen

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    dev = torch.device("cuda:0")
    w = gen.WORKLOADS[a.workload]
    cfg = mu.make_config(a.recipe, **dict(w.config))
    if a.fp8_gram:
        cfg.flags |= mu.MUON_FLAG_FP8_GRAM
    log(f"[bench] generating {a.workload}: {len(w.shapes)} matrices")
    grads, moms, weights = gen.make_batch(a.workload, dev)
    torch.cuda.synchronize()
    shapes = [tuple(g.shape) for g in grads]
    params = sum(r * c for r, c in shapes)
    flops = step_flops(shapes, cfg)

    h = mu.get_handle(0)
    h.reserve([(r, c, w.grad_dtype) for r, c in shapes])
    if a.copy_calibration_mib > 0:
        n = a.copy_calibration_mib * (1 << 20) // 4
        src = torch.ones(n, device=dev, dtype=torch.float32)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        tot = src.sum()              # reads the buffer once (a few bytes of partial sums written)
        torch.cuda.synchronize()
        dst.fill_(2.0)               # writes it once
        torch.cuda.synchronize()
        log(f"[bench] calibration: copy of {a.copy_calibration_mib} MiB, then a sum reading it "
            f"({float(tot):.0f}) and a fill writing it")
        del src, dst

    def step():
        mu.muon_update(grads, moms, weights, cfg, handle=h)

    for i in range(a.warmup):
        step()
        torch.cuda.synchronize()
        log(f"[bench] warmup {i + 1}/{a.warmup} done")

    prof = not a.no_profile
    if prof:
        h.profile_reset()
        h.profile_enable(True)
    torch.cuda.synchronize()
    sampler = ClockSampler() if not a.no_clocks else None
    if sampler:
        sampler.__enter__()
    t0 = time.perf_counter()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record()
    for i in range(a.steps):
        step()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if sampler:
        sampler.__exit__(None, None, None)
    ms_ev = ev0.elapsed_time(ev1)
    log(f"[bench] timed {a.steps} steps: wall {wall * 1e3:.1f} ms, events {ms_ev:.1f} ms")
    p = None
    if prof:
        h.profile_enable(False)
        p = h.profile_read()

    ms_per_step = ms_ev / a.steps
    value = flops / (ms_per_step * 1e-3) / 1e12
    out = {
        "metric": METRIC if a.recipe == "aurora" else METRIC_CLASSIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("bf16" if w.grad_dtype == torch.bfloat16 else "f32") + ("+fp8 first Gram" if a.fp8_gram else ""),
        "data": "synthetic",
        "config": {"workload": a.workload, "recipe": a.recipe, "matrices": len(shapes), "matrix_params": params,
                   "counted_ns_tflop_per_step": round(flops / 1e12, 3),
                   "standard_iteration_tflop_per_step": round(algorithmic_flops(shapes, cfg) / 1e12, 3),
                   "matrix_params_per_s": round(params / (ms_per_step * 1e-3), 1),
                   "pct_bf16_peak_whole_step": round(100 * value / PEAK_BF16_TFLOPS, 2),
                   "parallelism": "single GPU"},
    }
    if p is not None and p["gemm_launches"] > 0:
        peak = PEAK_BF16_TFLOPS if w.grad_dtype == torch.bfloat16 else PEAK_FP32_TFLOPS
        gemm_s = p["gemm_ms"] * 1e-3
        achieved = p["gemm_algorithmic_flop"] / gemm_s / 1e12
        standard = algorithmic_flops(shapes, cfg) * a.steps / gemm_s / 1e12
        counted = p["gemm_counted_flop"] / gemm_s / 1e12
        executed = p["gemm_executed_flop"] / gemm_s / 1e12
        esz = 2 if w.grad_dtype == torch.bfloat16 else 4
        wsz = (2 if w.weight_dtype == torch.bfloat16 else 4) if w.weights else 0
        budget = stream_budget_bytes(shapes, esz, wsz, cfg) * a.steps
        out["roofline"] = {
            "bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4),
            # the byte-counter record was taken on the Aurora step's launches
            "traffic": measured_traffic(a.workload) if a.recipe == "aurora" and not a.fp8_gram else None,
            "kernel": "k_ns_gemm (A = XX^T, B' = bA + cA^2 + aI, short-side products, X' = QX launches together)",
            "flops": "algorithmic flops of the products run: symmetric halves once, no padding",
            "algorithmic_tflop_per_step": round(p["gemm_algorithmic_flop"] / a.steps / 1e12, 3),
            "standard_iteration_tflops": round(standard, 2),
            "launches": int(p["gemm_launches"]),
            "avg_launch_ms": round(p["gemm_ms"] / p["gemm_launches"], 4),
            "counted_tflops": round(counted, 2), "frac_counted": round(counted / peak, 4),
            "executed_tflops": round(executed, 2), "frac_executed": round(executed / peak, 4),
            "stream_kernels_ms_per_step": round(p["stream_ms"] / a.steps, 3),
            "stream_kernels_own_gbps": round(p["stream_bytes"] / (p["stream_ms"] * 1e-3) / 1e9, 1)
            if p["stream_ms"] > 0 else None,
            "stream_budget_gb_per_step": round(budget / a.steps / 1e9, 3),
            "stream_budget_gbps": round(budget / (p["stream_ms"] * 1e-3) / 1e9, 1) if p["stream_ms"] > 0 else None,
            "stream_budget_frac_hbm": round(budget / (p["stream_ms"] * 1e-3) / 8e12, 4) if p["stream_ms"] > 0
            else None,
            "aurora_vector_ms_per_step": round(p["aux_ms"] / a.steps, 3),
            "aurora_vector_gbps": round(p["aux_bytes"] / (p["aux_ms"] * 1e-3) / 1e9, 1) if p["aux_ms"] > 0 else None,
        }
    if sampler:
        out["clocks"] = sampler.summary()
    if a.cpu_budget > 0:
        log("[bench] timing the float64 oracle on a sample")
        grads0, moms0, weights0 = gen.make_batch(a.workload, dev)   # pristine inputs
        out["cpu_baseline"] = cpu_baseline(a.workload, grads0, moms0, weights0, cfg, a.cpu_budget)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
