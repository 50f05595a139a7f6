#!/usr/bin/env python3
"""Benchmark of the affine group-quantized matmul hot path on one MI355X.

Headline: lm_head decode qmv (x [32,1,1024] bf16, W [151936,1024] 4-bit, group 64), as
effective HBM GB/s = algorithmic bytes (packed W + scales + biases + x + y) per call /
time.  The same JSON line carries the prefill qmm_t figure (x [4,512,4096] bf16,
W [14336,4096] 4-bit, group 128) in TFLOP/s, the per-kernel roofline (kernel duration
from HIP events on the launch stream) and the CPU oracle timed on a bounded sample.

Inputs are resident in HBM before timing starts; each step uses the next of several
weight/activation copies whose total exceeds the 256 MB Infinity Cache, so weights come
from HBM every call.  Usage: python bench.py [--steps K] [--warmup W] [--gpus 1]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PROFILES = os.path.join(ROOT, "profiles")


def _source_hash(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "bit_affine_quantized_qmv_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _traffic(summary_name, kernel_sources, launches_per_dispatch=1):
    """HBM bytes per launch from a committed rocprofv3 --pmc summary, if it was taken on
    the current kernel source (else None)."""
    path = os.path.join(PROFILES, summary_name)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("source_hash") != _source_hash(kernel_sources):
        return None
    return d.get("hbm_bytes_per_launch")


def _time_kernel(fn, steps, warmup, torch):
    """Run fn(i) warmup + steps times; returns (wall ms per step, mean kernel ms)."""
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        starts[i].record()
        fn(warmup + i)
        ends[i].record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    kern = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    kern.sort()
    return wall_ms, sum(kern) / len(kern), kern[len(kern) // 2]


def _cpu_threads():
    try:
        from threadpoolctl import threadpool_info
        n = max((p.get("num_threads") or 1) for p in threadpool_info()) if threadpool_info() else 1
        return int(n)
    except Exception:
        return os.cpu_count() or 1


def _oracle_rate(run_sample, budget_s):
    """Time the oracle on growing samples until ~budget_s of CPU work; returns (units/s, desc)."""
    done_units, spent, desc = 0.0, 0.0, ""
    i = 0
    while spent < budget_s:
        units, seconds, desc = run_sample(i)
        done_units += units
        spent += seconds
        i += 1
        if units == 0:
            break
    return (done_units / spent if spent > 0 else 0.0), desc, i


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--copies", type=int, default=4, help="weight copies rotated per step")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle timing per leg")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["qmv", "qmm_t", "all"], default="all")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import bit_affine_quantized_qmv_amd as q
    import synth

    q.load()
    dev = torch.device("cuda:0")
    out = {}

    # ------------------------------------------------------------ lm_head decode qmv
    cfg = synth.LM_HEAD
    n, k, m, bits, gs = cfg["n"], cfg["k"], cfg["m"], cfg["bits"], cfg["group_size"]
    w = synth.normal_weight(n, k, cfg["w_std"], seed=cfg["w_seed"])
    qw0 = q.quantize(w.to(dev), gs, bits, cfg["dtype"])
    torch.cuda.synchronize()
    copies = max(1, args.copies)
    qws = [qw0] + [q.QuantizedWeight(qw0.w_packed.clone(), qw0.scales.clone(), qw0.biases.clone(),
                                     n, k, gs, bits) for _ in range(copies - 1)]
    x0 = synth.normal_x((m, 1, k), cfg["dtype"], seed=cfg["x_seed"]).to(dev)
    xs = [x0.clone() for _ in range(copies)]
    ys = [torch.empty(m, 1, n, dtype=x0.dtype, device=dev) for _ in range(copies)]
    qmv_bytes = n * k * bits // 8 + 2 * n * (k // gs) * 2 + m * k * 2 + m * n * 2
    wall, kern_mean, kern_med = _time_kernel(
        lambda i: q.qmv(xs[i % copies], qws[i % copies], out=ys[i % copies]), args.steps, args.warmup, torch)
    forced = _time_kernel(lambda i: q.qmv(xs[i % copies], qws[i % copies], q.QMM_FLAG_FORCE_STRIDED,
                                          out=ys[i % copies]), max(5, args.steps // 10), 3, torch)
    qmv_value = qmv_bytes / (wall * 1e-3) / 1e9
    achieved = qmv_bytes / (kern_mean * 1e-3) / 1e9
    line = {
        "metric": "qmv effective HBM GB/s (lm_head decode)",
        "value": round(qmv_value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,0.02) weights quantized on the GPU, N(0,1) activations)",
        "config": {"workload": "lm_head decode qmv: x [32,1,1024] bf16, W [151936,1024] 4-bit "
                               "group 64 bf16 scales/biases, folded to one 2D call",
                   "algorithmic_bytes_per_call": qmv_bytes, "weight_copies_rotated": copies,
                   "pct_hbm_peak": round(100 * qmv_value / HBM_PEAK_GBS, 2)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": _traffic("qmv_lm_head_traffic.json",
                                         ["decode.hip", "device_common.hpp"]),
                     "kernel": "qmv_decode_kernel", "kernel_ms_mean": round(kern_mean, 5),
                     "kernel_ms_median": round(kern_med, 5)},
        "context": {"forced_per_batch_element_ms": round(forced[1], 4),
                    "forced_vs_folded": round(forced[1] / kern_mean, 2),
                    "pages_apple_m4max_ms": {"batched_grid_z": 60.0, "flattened": 2.2}},
    }
    out["qmv"] = line
    del qws, xs, ys, w

    # ------------------------------------------------------------ prefill qmm_t
    if args.only in ("all", "qmm_t"):
        pc = synth.PREFILL
        pn, pk, bb, ss = pc["n"], pc["k"], pc["b"], pc["s"]
        pw = synth.normal_weight(pn, pk, pc["w_std"], seed=pc["w_seed"])
        pq0 = q.quantize(pw.to(dev), pc["group_size"], pc["bits"], pc["dtype"])
        torch.cuda.synchronize()
        pcopies = 3
        pqs = [pq0] + [q.QuantizedWeight(pq0.w_packed.clone(), pq0.scales.clone(), pq0.biases.clone(),
                                         pn, pk, pc["group_size"], pc["bits"]) for _ in range(pcopies - 1)]
        px0 = synth.normal_x((bb, ss, pk), pc["dtype"], seed=pc["x_seed"]).to(dev)
        pxs = [px0.clone() for _ in range(pcopies)]
        pys = [torch.empty(bb, ss, pn, dtype=px0.dtype, device=dev) for _ in range(pcopies)]
        flops = 2.0 * bb * ss * pn * pk
        psteps = max(10, args.steps // 4)
        pwall, pk_mean, pk_med = _time_kernel(
            lambda i: q.qmm_t(pxs[i % pcopies], pqs[i % pcopies], out=pys[i % pcopies]), psteps,
            max(3, args.warmup // 4), torch)
        buf = synth.normal_x((bb, 2 * ss, pk), pc["dtype"], seed=pc["buf_seed"]).to(dev)
        view = buf[:, 0:ss, :]
        vwall, vk_mean, _ = _time_kernel(lambda i: q.qmm_t(view, pqs[i % pcopies], out=pys[i % pcopies]),
                                         max(5, psteps // 2), 2, torch)
        tflops = flops / (pwall * 1e-3) / 1e12
        ach = flops / (pk_mean * 1e-3) / 1e12
        out["qmm_t"] = {
            "metric": "qmm_t TFLOP/s (prefill)", "value": round(tflops, 1), "unit": "TFLOP/s",
            "steps": psteps, "ms_per_step": round(pwall, 5), "dtype": "bf16",
            "config": {"workload": "prefill qmm_t: x [4,512,4096] bf16, W [14336,4096] 4-bit group 128 "
                                   "bf16 scales/biases, y [4,512,14336]",
                       "flops_per_call": flops, "pct_mfma_peak": round(100 * tflops / MFMA_BF16_PEAK_TFLOPS, 2),
                       "narrowed_view_kernel_ms": round(vk_mean, 5)},
            "roofline": {"bound": "mfma", "achieved": round(ach, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(ach / MFMA_BF16_PEAK_TFLOPS, 4),
                         "traffic": _traffic("qmm_t_prefill_traffic.json",
                                             ["prefill.hip", "device_common.hpp"]),
                         "kernel": "qmm_prefill_kernel", "kernel_ms_mean": round(pk_mean, 5),
                         "kernel_ms_median": round(pk_med, 5)},
        }
        del pqs, pxs, pys, buf, pw

    # ------------------------------------------------------------ CPU oracle baselines
    if not args.no_cpu_baseline:
        import oracle as O
        threads = _cpu_threads()
        qw_h = {"w": qw0.w_packed.cpu().numpy().view(np.uint32),
                "s": qw0.scales.cpu().view(torch.int16).numpy().view(np.uint16),
                "b": qw0.biases.cpu().view(torch.int16).numpy().view(np.uint16)}
        x_h = x0.float().cpu().numpy().astype(np.float64).reshape(m, k)
        chunk = 4096

        def qmv_sample(i):
            lo = (i * chunk) % n
            hi = min(n, lo + chunk)
            t0 = time.perf_counter()
            codes = O.unpack(qw_h["w"][lo:hi], bits, k)
            wd = O.dequant(codes, qw_h["s"][lo:hi], qw_h["b"][lo:hi], gs, "bf16")
            O.matmul_rows(x_h, wd)
            dt = time.perf_counter() - t0
            rows = hi - lo
            nbytes = rows * k * bits // 8 + 2 * rows * (k // gs) * 2 + m * k * 2 + m * rows * 2
            return nbytes / 1e9, dt, "%d-row slices of W with all 32 activation rows" % chunk

        rate, desc, nsamp = _oracle_rate(qmv_sample, args.cpu_budget)
        out["qmv"]["cpu_baseline"] = {"value": round(rate, 3), "unit": "GB/s", "cores": threads,
                                      "kind": "oracle",
                                      "sample": "%s (%d slices: unpack, dequantize, float64 product)"
                                                % (desc, nsamp)}
        if "qmm_t" in out:
            pc = synth.PREFILL
            pq_h = {"w": pq0.w_packed.cpu().numpy().view(np.uint32),
                    "s": pq0.scales.cpu().view(torch.int16).numpy().view(np.uint16),
                    "b": pq0.biases.cpu().view(torch.int16).numpy().view(np.uint16)}
            px_h = px0.float().cpu().numpy().astype(np.float64).reshape(-1, pc["k"])
            wrows = 2048
            state = {}

            def qmm_sample(i):
                t0 = time.perf_counter()
                if "wd" not in state:
                    codes = O.unpack(pq_h["w"][:wrows], pc["bits"], pc["k"])
                    state["wd"] = O.dequant(codes, pq_h["s"][:wrows], pq_h["b"][:wrows],
                                            pc["group_size"], "bf16")
                r0 = (i * 64) % px_h.shape[0]
                O.matmul_rows(px_h[r0:r0 + 64], state["wd"])
                dt = time.perf_counter() - t0
                return 2.0 * 64 * wrows * pc["k"] / 1e12, dt, \
                    "64-row activation blocks against the first %d weight rows" % wrows

            prate, pdesc, pn_s = _oracle_rate(qmm_sample, args.cpu_budget)
            out["qmm_t"]["cpu_baseline"] = {"value": round(prate, 5), "unit": "TFLOP/s",
                                            "cores": threads, "kind": "oracle",
                                            "sample": "%s (%d blocks; unpack+dequantize once, "
                                                      "float64 product)" % (pdesc, pn_s)}

    line = out["qmv"]
    if "qmm_t" in out:
        line["qmm_t"] = out["qmm_t"]
    print(json.dumps(line))


if __name__ == "__main__":
    main()
