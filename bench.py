#!/usr/bin/env python3
"""Benchmark of the affine group-quantized matmul hot path on one MI355X.

Headline: lm_head decode qmv (x [32,1,1024] bf16, W [151936,1024] 4-bit, group 64), as
effective HBM GB/s = algorithmic bytes (packed W + scales + biases + x + y) per call /
time.  The same JSON line carries the prefill qmm_t figure (x [4,512,4096] bf16,
W [14336,4096] 4-bit, group 128) in TFLOP/s, the per-kernel roofline, the small decode
configurations with the launch floor, a paired comparison of the per-batch-element
launch against the folded one, and the CPU oracle timed on a bounded sample.

Timing: the K timed steps are captured once into a HIP graph; one replay of that graph is
the timed region.  `ms_per_step` is its host wall time (synchronize on both sides) / K;
the roofline's `kernel_ms` is the device time between two events recorded on the launch
stream around the same replay / K, i.e. the average duration of back-to-back launches.
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


QMV_SOURCES = ["decode.cpp", "decode_b4.hip", "decode_impl.hpp", "decode_kernels.hpp", "decode_parts.hpp",
               "device_common.hpp", "kernels.hpp"]
QMM_T_SOURCES = ["prefill.hip", "dequant_impl.hpp", "device_common.hpp", "kernels.hpp"]


def _source_hash(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "bit_affine_quantized_qmv_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _traffic(summary_name, kernel_sources):
    """HBM bytes per launch from a committed rocprofv3 --pmc summary (a line
    'traffic-json: {...}' in profiles/<summary_name>), if its counters were taken on the
    current kernel source; else None."""
    path = os.path.join(PROFILES, summary_name)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        for ln in f:
            if ln.startswith("traffic-json:"):
                d = json.loads(ln.split(":", 1)[1])
                if d.get("source_hash") != _source_hash(kernel_sources):
                    return None
                return d.get("hbm_bytes_per_launch")
    return None


def _profile_field(summary_name, tag, kernel_sources, field):
    """One value from a committed rocprofv3 --pmc summary (a line '<tag>: {...}' in
    profiles/<summary_name>), if its counters were taken on the current kernel source."""
    path = os.path.join(PROFILES, summary_name)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        for ln in f:
            if ln.startswith(tag + ":"):
                d = json.loads(ln.split(":", 1)[1])
                if d.get("source_hash") != _source_hash(kernel_sources):
                    return None
                return d.get(field)
    return None


def _time_steps(fn, steps, warmup, torch, use_graph=True):
    """Times `steps` calls fn(0), ..., fn(steps - 1).

    The calls are captured once into a HIP graph; after one untimed replay, one replay is
    timed two ways: wall_ms = host wall clock with torch.cuda.synchronize() on both sides,
    kernel_ms = elapsed time of two events recorded on the launch stream around it (the
    average device duration of the back-to-back launches, launch gaps included), both per
    step.  eager_ms: the same calls launched from Python (host marshalling included;
    context only).  Without a graph, both figures come from eager launches.
    """
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        fn(i)
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t0) * 1e3 / steps
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    graph_ok = use_graph
    if use_graph:
        try:
            g = torch.cuda.CUDAGraph()
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                fn(0)                      # launch-side caches are filled outside capture
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            with torch.cuda.graph(g):
                for i in range(steps):
                    fn(i)
            g.replay()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            start.record()
            g.replay()
            end.record()
            torch.cuda.synchronize()
            wall_ms = (time.perf_counter() - t0) * 1e3 / steps
            del g
        except Exception:          # timing only: fall back to eager launches
            graph_ok = False
    if not graph_ok:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        start.record()
        for i in range(steps):
            fn(i)
        end.record()
        torch.cuda.synchronize()
        wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    kernel_ms = start.elapsed_time(end) / steps
    return {"wall_ms": wall_ms, "kernel_ms": kernel_ms, "graph": graph_ok, "eager_ms": eager_ms}


def _host_info():
    """The host the oracle is timed on: CPU model, usable cores, numpy and its BLAS."""
    import numpy as np
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = ""
    try:
        b = np.show_config(mode="dicts")["Build Dependencies"]["blas"]
        blas = "%s %s" % (b.get("name", ""), b.get("version", ""))
    except Exception:
        pass
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    return {"cpu_model": model, "nproc": cores, "numpy": np.__version__, "blas": blas.strip()}


def _blas_threads():
    """Threads of the BLAS pool numpy's products run on (loaded pools only)."""
    try:
        from threadpoolctl import threadpool_info
        pools = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        return max(int(p.get("num_threads") or 1) for p in pools) if pools else 1
    except Exception:
        return 1


def _oracle_rate(run_sample, budget_s):
    """Time the oracle on successive samples until ~budget_s of CPU work; returns
    (units/s, sample description, samples run)."""
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


def _leg(metric, amount, t, bound, unit, peak, kernel, config):
    """One measured leg: `amount` algorithmic bytes (GB/s legs) or flops (TFLOP/s legs) per call,
    over the graph-replay step time (value) and the device time of the same replay (roofline)."""
    scale = 1e9 if unit == "GB/s" else 1e12
    value = amount / (t["wall_ms"] * 1e-3) / scale
    achieved = amount / (t["kernel_ms"] * 1e-3) / scale
    return {"metric": metric, "value": round(value, 1), "unit": unit, "ms_per_step": round(t["wall_ms"], 5),
            "config": config,
            "roofline": {"bound": bound, "achieved": round(achieved, 1), "peak": peak, "unit": unit,
                         "frac": round(achieved / peak, 4), "traffic": None, "kernel": kernel,
                         "kernel_ms": round(t["kernel_ms"], 5)}}


def _next_legs(args, q, torch, dev, synth, res, nsteps, nwarm):
    """Gathered-weight decode, standalone dequantize and the unaligned-K prefill."""
    # gathered qmv over an expert stack, every expert read once per call
    ec = synth.EXPERTS
    e, n, k, bits, gs = ec["e"], ec["n"], ec["k"], ec["bits"], ec["group_size"]
    we = synth.normal_weight(e * n, k, ec["w_std"], seed=ec["w_seed"])
    st = q.quantize(we.to(dev), gs, bits, ec["dtype"])
    del we
    stacks = []
    for c in range(3):
        wp = st.w_packed.view(e, n, -1)
        sc = st.scales.view(e, n, -1)
        bi = st.biases.view(e, n, -1)
        if c:
            wp, sc, bi = wp.clone(), sc.clone(), bi.clone()
        stacks.append(q.ExpertWeights(wp, sc, bi, n, k, gs, bits))
    rows = ec["rows"]
    gx = [synth.normal_x((rows, k), ec["dtype"], seed=ec["x_seed"] + c).to(dev) for c in range(3)]
    gi = [synth.permutation(e, ec["idx_seed"] + c)[:rows].contiguous().to(dev) for c in range(3)]
    gy = [torch.empty(rows, n, dtype=gx[0].dtype, device=dev) for _ in range(3)]
    expert_bytes = n * k * bits // 8 + 2 * n * (k // gs) * 2
    gbytes = rows * (expert_bytes + k * 2 + n * 2 + 4)
    tg = _time_steps(lambda i: q.gather_qmv(gx[i % 3], stacks[i % 3], gi[i % 3], out=gy[i % 3]),
                     nsteps, nwarm, torch, not args.no_graph)
    res["gather_qmv"] = _leg(
        "gathered qmv effective HBM GB/s", gbytes, tg, "hbm", "GB/s", HBM_PEAK_GBS, "qmv decode kernels",
        {"workload": "gathered qmv: 128 rows x [1,1408] bf16, each against its own expert of a "
                     "[128,704,1408] 8-bit group 32 bf16 stack (seeded permutation)",
         "algorithmic_bytes_per_call": gbytes})
    del stacks, gx, gi, gy, st

    # standalone dequantize of the prefill weight
    pc = synth.PREFILL
    pn, pk = pc["n"], pc["k"]
    pw = synth.normal_weight(pn, pk, pc["w_std"], seed=pc["w_seed"])
    pq0 = q.quantize(pw.to(dev), pc["group_size"], pc["bits"], pc["dtype"])
    del pw
    pqs = [pq0, q.QuantizedWeight(pq0.w_packed.clone(), pq0.scales.clone(), pq0.biases.clone(), pn, pk,
                                  pc["group_size"], pc["bits"])]
    douts = [torch.empty(pn, pk, dtype=pq0.dtype, device=dev) for _ in range(2)]
    dbytes = pn * pk * pc["bits"] // 8 + 2 * pn * (pk // pc["group_size"]) * 2 + pn * pk * 2
    td = _time_steps(lambda i: q.dequantize(pqs[i % 2], out=douts[i % 2]), nsteps, nwarm, torch,
                     not args.no_graph)
    res["dequantize"] = _leg(
        "dequantize effective HBM GB/s", dbytes, td, "hbm", "GB/s", HBM_PEAK_GBS, "dequant_rows_kernel",
        {"workload": "dequantize W [14336,4096] 4-bit group 128 bf16 -> dense [14336,4096] bf16",
         "algorithmic_bytes_per_call": dbytes})
    del pqs, douts, pq0

    # unaligned K: the prefill shape at K = 4096 + 32 (group 32), and its 32-row decode
    uc = synth.UNALIGNED
    un, uk = uc["n"], uc["k"]
    uw = synth.normal_weight(un, uk, uc["w_std"], seed=uc["w_seed"])
    uq = q.quantize(uw.to(dev), uc["group_size"], uc["bits"], uc["dtype"])
    del uw
    ux = synth.normal_x((uc["b"], uc["s"], uk), uc["dtype"], seed=uc["x_seed"]).to(dev)
    uy = torch.empty(uc["b"], uc["s"], un, dtype=ux.dtype, device=dev)
    flops = 2.0 * uc["b"] * uc["s"] * un * uk
    tu = _time_steps(lambda i: q.qmm_t(ux, uq, out=uy), max(50, nsteps // 2), max(10, nwarm), torch, not args.no_graph)
    res["unaligned_k"] = _leg(
        "unaligned-K qmm_t TFLOP/s", flops, tu, "mfma", "TFLOP/s", MFMA_BF16_PEAK_TFLOPS, "qmm_prefill_dma_kernel",
        {"workload": "prefill qmm_t at unaligned K: x [4,512,4128] bf16, W [14336,4128] 4-bit group 32 "
                     "bf16 (last k step of 32)", "flops_per_call": flops})
    dx = ux[0, :32].contiguous().view(32, 1, uk)
    dy = torch.empty(32, 1, un, dtype=ux.dtype, device=dev)
    tdd = _time_steps(lambda i: q.qmv(dx, uq, out=dy), nsteps, nwarm, torch, not args.no_graph)
    ubytes = un * uk * uc["bits"] // 8 + 2 * un * (uk // uc["group_size"]) * 2 + 32 * uk * 2 + 32 * un * 2
    res["unaligned_k"]["decode_32_rows"] = _leg(
        "unaligned-K qmv effective HBM GB/s", ubytes, tdd, "hbm", "GB/s", HBM_PEAK_GBS, "qmv_parts_kernel",
        {"workload": "decode qmv at unaligned K: x [32,1,4128] bf16 against the same W [14336,4128] 4-bit group 32 "
                     "(last slot masked, rows cut into parts along K, two 16-row blocks in one launch)",
         "algorithmic_bytes_per_call": ubytes})
    del uq, ux, uy, dx, dy


def _small_legs(args, q, torch, dev, synth, floor_ms):
    """The small decode configurations (probe, batched decode projections, odd N) and the
    lm_head weight at one activation row.  The small ones move 0.5-3.6 MB per call, less
    than a microsecond of HBM time, so they are reported with the launch floor beside them;
    64 weight copies are rotated so the weights do not stay in the L2."""
    out = {"launch_floor_us": round(floor_ms * 1e3, 2), "legs": []}
    steps = max(20, args.steps // 4)

    def leg(name, x, qw0, entry, nbytes, copies=64, flops=None):
        qws = [qw0] + [q.QuantizedWeight(qw0.w_packed.clone(), qw0.scales.clone(), qw0.biases.clone(), qw0.N, qw0.K,
                                         qw0.group_size, qw0.bits) for _ in range(copies - 1)]
        ys = [torch.empty(*x.shape[:-1], qw0.N, dtype=x.dtype, device=dev) for _ in range(4)]
        fn = (lambda i: q.qmv(x, qws[i % copies], out=ys[i % 4])) if entry == "qmv" else \
             (lambda i: q.qmm_t(x, qws[i % copies], out=ys[i % 4]))
        t = _time_steps(fn, steps, 3, torch, not args.no_graph)
        r = {"workload": name, "us_per_call": round(t["wall_ms"] * 1e3, 2),
             "kernel_us": round(t["kernel_ms"] * 1e3, 2), "algorithmic_bytes": nbytes,
             "GB/s": round(nbytes / (t["kernel_ms"] * 1e-3) / 1e9, 1),
             "frac_hbm_peak": round(nbytes / (t["kernel_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        out["legs"].append(r)
        del qws, ys

    def nbytes_of(n, k, bits, gs, m):
        return n * k * bits // 8 + 2 * n * (k // gs) * 2 + m * k * 2 + m * n * 2

    # the issue-47331 probe: W [1024, 2048] 4-bit group 64 bf16, x [2,K], [2,1,K], [2,4,K]
    qp = q.quantize(synth.probe_weight().to(dev), 64, 4, "bf16")
    for shape in ((2, 2048), (2, 1, 2048), (2, 4, 2048)):
        x = synth.normal_x(shape, "bf16", seed=1).to(dev)
        m = x.numel() // 2048
        leg("probe qmm_t x %s, W [1024,2048] 4-bit g64 bf16" % list(shape), x, qp, "qmm_t",
            nbytes_of(1024, 2048, 4, 64, m))
    del qp
    # batched decode projections, B = 1 and 32, 4- and 8-bit, group 64, bf16
    for i, (k, n) in enumerate(synth.DECODE_SHAPES):
        w = synth.normal_weight(n, k, 0.02, seed=100 + i).to(dev)
        for bits in (4, 8):
            qw = q.quantize(w, 64, bits, "bf16")
            for b in (1, 32):
                x = synth.normal_x((b, 1, k), "bf16", seed=200 + i).to(dev)
                leg("decode x [%d,1,%d], W [%d,%d] %d-bit g64 bf16" % (b, k, n, k, bits), x, qw, "qmv",
                    nbytes_of(n, k, bits, 64, b))
            del qw
        del w
    # odd N at K = 4096, x alternating 2048, 1
    for n in (1, 1001):
        for bits, gs, dt in ((6, 32, "fp16"), (3, 128, "bf16")):
            qw = q.quantize(synth.normal_weight(n, 4096, 0.02, seed=400 + n + bits).to(dev), gs, bits, dt)
            x = synth.alternating_x(4096, dt).to(dev)
            leg("odd N x [1,4096] alternating, W [%d,4096] %d-bit g%d %s" % (n, bits, gs, dt), x, qw, "qmv",
                nbytes_of(n, 4096, bits, gs, 1))
            del qw
    return out


def _paired_ratio(args, q, torch, fold, forced, rounds=8, steps=10):
    """Paired, A/A-calibrated comparison of the per-batch-element launch against the folded
    one: each round times the folded call (A), the forced call (B) and the folded call again
    (A'), each as one graph replay of `steps` calls; the geometric means of B/A and A'/A over
    the rounds are reported (MLX pull request 4516, "Performance": geometric mean of paired
    Baseline/Candidate ratios from A/A-calibrated runs)."""
    import math
    ab, aa, ta, tb = [], [], [], []
    for r in range(rounds):
        t_a = _time_steps(fold, steps, 2, torch, not args.no_graph)["kernel_ms"]
        t_b = _time_steps(forced, steps, 2, torch, not args.no_graph)["kernel_ms"]
        t_a2 = _time_steps(fold, steps, 2, torch, not args.no_graph)["kernel_ms"]
        ab.append(t_b / t_a)
        aa.append(t_a2 / t_a)
        ta.append(t_a)
        tb.append(t_b)
    gm = lambda v: math.exp(sum(math.log(x) for x in v) / len(v))
    return {"rounds": rounds, "steps_per_timing": steps,
            "forced_over_folded_geomean": round(gm(ab), 3),
            "forced_over_folded_range": [round(min(ab), 3), round(max(ab), 3)],
            "aa_geomean": round(gm(aa), 4), "aa_range": [round(min(aa), 4), round(max(aa), 4)],
            "folded_kernel_ms_median": round(sorted(ta)[len(ta) // 2], 5),
            "forced_kernel_ms_median": round(sorted(tb)[len(tb) // 2], 5),
            "pages_apple_m4max_ms": {"batched_grid_z": 60.0, "flattened": 2.2}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--copies", type=int, default=4, help="weight copies rotated per step")
    ap.add_argument("--cpu-budget", type=float, default=8.0, help="seconds of oracle timing per phase")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["qmv", "qmm_t", "next", "small", "forced", "all"], default="all",
                    help="legs besides the headline qmv: the prefill qmm_t, the next rows "
                         "(gathered qmv, fused argmax, dequantize, embedding, unaligned K), the small "
                         "configurations, the per-batch-element launch alone (for counters), or all")
    ap.add_argument("--no-graph", action="store_true",
                    help="time the steps eagerly instead of replaying them from a HIP graph")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 256 MiB device copy (counter calibration) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import bit_affine_quantized_qmv_amd as q
    import synth

    dev = torch.device("cuda:0")
    if args.calibrate_copy:
        src = torch.empty(64 << 20, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "device copy", "bytes_read": src.numel() * 4,
                          "bytes_written": dst.numel() * 4, "launches": 5}))
        return
    q.load()
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
    if args.only == "forced":
        # the per-batch-element launch alone (32 grid slices of one row each), for counters
        t = _time_steps(lambda i: q.qmv(xs[i % copies], qws[i % copies], q.QMM_FLAG_FORCE_STRIDED,
                                        out=ys[i % copies]), args.steps, args.warmup, torch, not args.no_graph)
        print(json.dumps({"metric": "forced per-batch-element lm_head decode", "kernel_ms": t["kernel_ms"],
                          "ms_per_step": t["wall_ms"], "steps": args.steps}))
        return
    t = _time_steps(lambda i: q.qmv(xs[i % copies], qws[i % copies], out=ys[i % copies]),
                    args.steps, args.warmup, torch, not args.no_graph)
    qmv_value = qmv_bytes / (t["wall_ms"] * 1e-3) / 1e9
    achieved = qmv_bytes / (t["kernel_ms"] * 1e-3) / 1e9
    line = {
        "metric": "qmv effective HBM GB/s (lm_head decode)",
        "value": round(qmv_value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t["wall_ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,0.02) weights quantized on the GPU, N(0,1) activations)",
        "config": {"workload": "lm_head decode qmv: x [32,1,1024] bf16, W [151936,1024] 4-bit "
                               "group 64 bf16 scales/biases, folded to one 2D call",
                   "algorithmic_bytes_per_call": qmv_bytes, "weight_copies_rotated": copies,
                   "timing": "K steps captured in one HIP graph, one replay bracketed by synchronize"
                             if t["graph"] else "K eager steps bracketed by synchronize",
                   "pct_hbm_peak": round(100 * qmv_value / HBM_PEAK_GBS, 2)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": _traffic("qmv_stream_kernel_lm_head_traffic.md", QMV_SOURCES),
                     "kernel": "qmv_stream_kernel",
                     "kernel_ms": round(t["kernel_ms"], 5),
                     "kernel_ms_source": "events on the launch stream around the timed graph replay, per step"},
        "context": {"eager_python_ms_per_step": round(t["eager_ms"], 5)},
    }
    out["qmv"] = line
    nsteps = max(10, args.steps // 4)
    nwarm = max(3, args.warmup // 4)
    if args.only in ("all", "qmv"):
        # the per-batch-element launch (32 grid slices, each re-reading W) against the folded call
        line["context"]["forced_vs_folded"] = _paired_ratio(
            args, q, torch, lambda i: q.qmv(xs[i % copies], qws[i % copies], out=ys[i % copies]),
            lambda i: q.qmv(xs[i % copies], qws[i % copies], q.QMM_FLAG_FORCE_STRIDED, out=ys[i % copies]))
        # its HBM reads from the committed FETCH_SIZE pass (null once the kernel source changed)
        line["context"]["forced_vs_folded"]["fetch_ratio_to_folded"] = _profile_field(
            "qmv_stream_kernel_forced_per_batch_element_fetch.md", "forced-json", QMV_SOURCES, "ratio_to_folded")
        # the same weight at one activation row
        x1 = [synth.normal_x((1, k), cfg["dtype"], seed=cfg["x_seed"]).to(dev) for _ in range(copies)]
        y1 = [torch.empty(1, n, dtype=x0.dtype, device=dev) for _ in range(copies)]
        b1 = n * k * bits // 8 + 2 * n * (k // gs) * 2 + k * 2 + n * 2
        t1 = _time_steps(lambda i: q.qmv(x1[i % copies], qws[i % copies], out=y1[i % copies]), args.steps,
                         args.warmup, torch, not args.no_graph)
        line["context"]["lm_head_one_row"] = _leg(
            "qmv effective HBM GB/s (lm_head decode, one row)", b1, t1, "hbm", "GB/s", HBM_PEAK_GBS,
            "qmv_stream_kernel",
            {"workload": "lm_head decode qmv: x [1,1024] bf16, W [151936,1024] 4-bit group 64 bf16",
             "algorithmic_bytes_per_call": b1})
        del x1, y1
    if args.only in ("all", "next"):
        out["next"] = {}
        # fused argmax on the lm_head logits, with and without storing them
        idx = torch.empty(m, dtype=torch.int32, device=dev)
        val = torch.empty(m, dtype=torch.float32, device=dev)
        ws = q.argmax_workspace(m, dev)
        arg_rows = {}
        for logits in (True, False):
            ta = _time_steps(lambda i: q.qmv_argmax(xs[i % copies], qws[i % copies], logits=logits, workspace=ws,
                                                    out=ys[i % copies] if logits else None, out_index=idx,
                                                    out_value=val),
                             nsteps, nwarm, torch, not args.no_graph)
            nbytes = qmv_bytes - (0 if logits else m * n * 2) + m * 8
            arg_rows["with_logits" if logits else "no_logits"] = _leg(
                "fused argmax effective HBM GB/s", nbytes, ta, "hbm", "GB/s", HBM_PEAK_GBS,
                "qmv_stream_kernel",
                {"workload": "lm_head decode qmv + per-row argmax: x [32,1,1024] bf16, W [151936,1024] "
                             "4-bit group 64; logits %s" % ("stored" if logits else "not stored"),
                 "algorithmic_bytes_per_call": nbytes})
        out["next"]["qmv_argmax"] = arg_rows
        # per-row top-k of the lm_head logits: decode then top-k, and the top-k pass alone
        tk = 50
        tidx = torch.empty(m, tk, dtype=torch.int32, device=dev)
        tval = torch.empty(m, tk, dtype=torch.float32, device=dev)
        tws = q.topk_workspace(m, dev)
        tt = _time_steps(lambda i: q.qmv_topk(xs[i % copies], qws[i % copies], tk, out=ys[i % copies],
                                              out_index=tidx, out_value=tval, workspace=tws),
                         nsteps, nwarm, torch, not args.no_graph)
        tbytes = qmv_bytes + m * n * 2 + m * tk * 8
        topk_rows = {"qmv_topk": _leg(
            "decode + top-k effective HBM GB/s", tbytes, tt, "hbm", "GB/s", HBM_PEAK_GBS,
            "qmv_stream_kernel + topk_select_kernel + topk_merge_kernel",
            {"workload": "lm_head decode qmv + per-row top-50: x [32,1,1024] bf16, W [151936,1024] 4-bit "
                         "group 64; logits stored, then read by the top-k pass",
             "algorithmic_bytes_per_call": tbytes})}
        lg = [y.view(m, n) for y in ys]
        to = _time_steps(lambda i: q.topk(lg[i % copies], tk, out_index=tidx, out_value=tval, workspace=tws),
                         nsteps, nwarm, torch, not args.no_graph)
        obytes = m * n * 2 + m * tk * 8
        topk_rows["topk_alone"] = _leg(
            "top-k effective HBM GB/s", obytes, to, "hbm", "GB/s", HBM_PEAK_GBS, "topk_select_kernel + topk_merge_kernel",
            {"workload": "per-row top-50 of [32,151936] bf16 logits (column chunks per row)",
             "algorithmic_bytes_per_call": obytes})
        out["next"]["topk"] = topk_rows
        # quantized embedding gather from the lm_head table
        ec = synth.EMBED
        idxs = [synth.token_indices(ec["count"], n, ec["idx_seed"] + c).to(dev) for c in range(copies)]
        eouts = [torch.empty(ec["count"], k, dtype=x0.dtype, device=dev) for _ in range(copies)]
        row_bytes = k * bits // 8 + 2 * (k // gs) * 2
        ebytes = ec["count"] * (row_bytes + k * 2 + 4)
        te = _time_steps(lambda i: q.embedding(qws[i % copies], idxs[i % copies], out=eouts[i % copies]),
                         nsteps, nwarm, torch, not args.no_graph)
        out["next"]["embedding"] = _leg(
            "quantized embedding gather effective HBM GB/s", ebytes, te, "hbm", "GB/s", HBM_PEAK_GBS,
            "dequant_rows_kernel",
            {"workload": "embedding: 2048 seeded token rows of the [151936,1024] 4-bit group 64 bf16 table "
                         "-> [2048,1024] bf16", "algorithmic_bytes_per_call": ebytes})
        del idxs, eouts
    del qws, xs, ys

    if args.only in ("all", "small"):
        # launch floor: graph replay of a one-tile decode call (N = 16, K = 128)
        qf = q.quantize(synth.normal_weight(16, 128, 1.0, seed=5).to(dev), 64, 4, "bf16")
        xf = synth.normal_x((1, 128), "bf16", seed=5).to(dev)
        yf = torch.empty(1, 16, dtype=torch.bfloat16, device=dev)
        tfl = _time_steps(lambda i: q.qmv(xf, qf, out=yf), args.steps, 5, torch, not args.no_graph)
        out["small"] = _small_legs(args, q, torch, dev, synth, tfl["kernel_ms"])
        out["small"]["launch_floor_workload"] = "one 16x128 4-bit tile, x [1,128]: device time per launch"
        del qf, xf, yf

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
        # at least 50 timed and 10 warm-up launches (about 12 ms of matrix-core work each way)
        # whatever --steps says: shorter runs time the device's clock ramp, not the kernel
        psteps = max(50, args.steps // 4)
        pt = _time_steps(lambda i: q.qmm_t(pxs[i % pcopies], pqs[i % pcopies], out=pys[i % pcopies]),
                         psteps, max(10, args.warmup // 4), torch, not args.no_graph)
        buf = synth.normal_x((bb, 2 * ss, pk), pc["dtype"], seed=pc["buf_seed"]).to(dev)
        view = buf[:, 0:ss, :]
        pv = _time_steps(lambda i: q.qmm_t(view, pqs[i % pcopies], out=pys[i % pcopies]),
                         max(5, psteps // 2), 2, torch, not args.no_graph)
        tflops = flops / (pt["wall_ms"] * 1e-3) / 1e12
        ach = flops / (pt["kernel_ms"] * 1e-3) / 1e12
        out["qmm_t"] = {
            "metric": "qmm_t TFLOP/s (prefill)", "value": round(tflops, 1), "unit": "TFLOP/s",
            "steps": psteps, "ms_per_step": round(pt["wall_ms"], 5), "dtype": "bf16",
            "config": {"workload": "prefill qmm_t: x [4,512,4096] bf16, W [14336,4096] 4-bit group 128 "
                                   "bf16 scales/biases, y [4,512,14336]",
                       "flops_per_call": flops, "pct_mfma_peak": round(100 * tflops / MFMA_BF16_PEAK_TFLOPS, 2),
                       "narrowed_view_kernel_ms": round(pv["kernel_ms"], 5)},
            "roofline": {"bound": "mfma", "achieved": round(ach, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(ach / MFMA_BF16_PEAK_TFLOPS, 4),
                         "traffic": _traffic("qmm_prefill_dma_kernel_prefill_traffic.md", QMM_T_SOURCES),
                         "kernel": "qmm_prefill_dma_kernel", "kernel_ms": round(pt["kernel_ms"], 5),
                         "kernel_ms_source": "events on the launch stream around the timed graph replay, per step",
                         # matrix-core busy fraction from the SQ_VALU_MFMA_BUSY_CYCLES counter
                         "mfma_util_counter": _profile_field("qmm_prefill_dma_kernel_prefill_mfma_util.md",
                                                             "mfma-util-json", QMM_T_SOURCES, "mfma_util")},
        }
        del pqs, pxs, pys, buf, pw

    if args.only in ("all", "next"):
        _next_legs(args, q, torch, dev, synth, out["next"], nsteps, nwarm)

    # ------------------------------------------------------------ CPU oracle baselines
    if not args.no_cpu_baseline:
        out["qmv"]["cpu_baseline"] = _cpu_baseline_qmv(args, np, torch, qw0, w, x0, cfg)
        if "qmm_t" in out:
            out["qmm_t"]["cpu_baseline"] = _cpu_baseline_qmm_t(args, np, torch, pq0, px0)

    line = out["qmv"]
    if "qmm_t" in out:
        line["qmm_t"] = out["qmm_t"]
    if "small" in out:
        line["small_configs"] = out["small"]
    if "next" in out:
        line["next_rows"] = out["next"]
    print(json.dumps(line))


def _cpu_baseline_qmv(args, np, torch, qw0, w, x0, cfg):
    """The oracle on the lm_head workload, on bounded samples of weight rows: the per-call
    path (unpack, dequantize, float64 product against all 32 rows) with every BLAS thread
    and with one, plus the one-time phases (quantize, unpack + dequantize) on their own."""
    import oracle as O
    from threadpoolctl import threadpool_limits
    n, k, m, bits, gs = cfg["n"], cfg["k"], cfg["m"], cfg["bits"], cfg["group_size"]
    qw_h = {"w": qw0.w_packed.cpu().numpy().view(np.uint32),
            "s": qw0.scales.cpu().view(torch.int16).numpy().view(np.uint16),
            "b": qw0.biases.cpu().view(torch.int16).numpy().view(np.uint16)}
    x_h = x0.float().cpu().numpy().astype(np.float64).reshape(m, k)
    w_h = w.numpy()
    chunk = 4096

    def call_sample(i):
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

    def phase_rate(fn, budget):
        spent, rows, i = 0.0, 0, 0
        while spent < budget:
            lo = (i * chunk) % n
            hi = min(n, lo + chunk)
            t0 = time.perf_counter()
            fn(lo, hi)
            spent += time.perf_counter() - t0
            rows += hi - lo
            i += 1
        return rows / spent

    rate, desc, nsamp = _oracle_rate(call_sample, args.cpu_budget)
    threads = _blas_threads()
    with threadpool_limits(limits=1):
        rate1, _, nsamp1 = _oracle_rate(call_sample, args.cpu_budget / 2)
    q_rows = phase_rate(lambda lo, hi: O.quantize(w_h[lo:hi], gs, bits, "bf16"), args.cpu_budget / 4)
    d_rows = phase_rate(lambda lo, hi: O.dequant(O.unpack(qw_h["w"][lo:hi], bits, k), qw_h["s"][lo:hi],
                                                 qw_h["b"][lo:hi], gs, "bf16"), args.cpu_budget / 4)
    return {"value": round(rate, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": "%s (%d slices: unpack, dequantize, float64 product, %d BLAS threads)"
                      % (desc, nsamp, threads),
            "one_thread": {"value": round(rate1, 4), "unit": "GB/s", "cores": 1, "samples": nsamp1},
            "phases_seconds_for_whole_weight": {"quantize": round(n / q_rows, 2),
                                                "unpack_dequantize": round(n / d_rows, 2)},
            "host": _host_info()}


def _cpu_baseline_qmm_t(args, np, torch, pq0, px0):
    """The oracle's product for the prefill workload: 64-row activation blocks against the
    first 2048 weight rows (unpack and dequantize once), every BLAS thread and one."""
    import oracle as O
    import synth
    from threadpoolctl import threadpool_limits
    pc = synth.PREFILL
    pq_h = {"w": pq0.w_packed.cpu().numpy().view(np.uint32),
            "s": pq0.scales.cpu().view(torch.int16).numpy().view(np.uint16),
            "b": pq0.biases.cpu().view(torch.int16).numpy().view(np.uint16)}
    px_h = px0.float().cpu().numpy().astype(np.float64).reshape(-1, pc["k"])
    wrows = 2048
    codes = O.unpack(pq_h["w"][:wrows], pc["bits"], pc["k"])
    wd = O.dequant(codes, pq_h["s"][:wrows], pq_h["b"][:wrows], pc["group_size"], "bf16")

    def block_sample(i):
        t0 = time.perf_counter()
        r0 = (i * 64) % px_h.shape[0]
        O.matmul_rows(px_h[r0:r0 + 64], wd)
        dt = time.perf_counter() - t0
        return 2.0 * 64 * wrows * pc["k"] / 1e12, dt, "64-row activation blocks against the first %d weight rows" % wrows

    prate, pdesc, pn_s = _oracle_rate(block_sample, args.cpu_budget)
    threads = _blas_threads()
    with threadpool_limits(limits=1):
        prate1, _, pn1 = _oracle_rate(block_sample, args.cpu_budget / 2)
    return {"value": round(prate, 5), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": "%s (%d blocks; unpack + dequantize once, float64 product, %d BLAS threads)"
                      % (pdesc, pn_s, threads),
            "one_thread": {"value": round(prate1, 5), "unit": "TFLOP/s", "cores": 1, "samples": pn1},
            "host": _host_info()}


if __name__ == "__main__":
    main()
