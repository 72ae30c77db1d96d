#!/usr/bin/env python3
"""Benchmark of the per-owner Muon step on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic
gradients already resident in HBM: momentum (+ Nesterov), Newton-Schulz of
every matrix (5 iterations of A = X X^T, B = bA + cA^2, X = aX + BX) and the
lr-scaled update, all in libdmuon's HIP kernels.  The default workload is
the largest single-GPU batch, the 70B-class MLP matrices (4 of 28672 x 8192,
2 of 8192 x 28672, bf16, Nesterov); ``--config 2`` runs the 4-layer TinyMLP
of DMuon's Quick Start (d=512, ff=2048), ``--config 3`` the Llama-8B
projections, ``--config 4`` the 512-matrix NS-only batch and ``--config 1``
the fp32 TinyMLP.  ``--ns-backend gram`` runs the Gram-space iteration
with restarts instead (fp32 operands, or fp16 with ``--ns-prec f16``); the
value stays the direct method's algorithmic flops per second, so the two
backends compare on the same work.

Prints ONE JSON line: NS TFLOP/s (algorithmic, symmetry-aware flops) as the
value and ms per step, both from a timed region with nothing but the steps
in it; the dominant kernel's roofline from a second timed region of the
same K steps in which HIP events on the kernel's stream bracket each of its
launches; and the fp64 oracle's throughput on a bounded sample of the same
workload on the host cores, per phase.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "Muon step ms & NS TFLOP/s (MFMA util %) per owned matrix batch, 1 GPU"
# MI355X published dense MFMA peaks (TFLOP/s) and HBM3E bandwidth (GB/s).
# Dense MFMA peaks of MI355X: bf16 and fp16 2.5 PFLOP/s, fp32 157.3 TFLOP/s.
PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0, "bf16+f16": 2500.0, "f32": 157.3}
PEAK_HBM_GBS = 8000.0


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def ns_flops(shapes, ns_steps):
    """Algorithmic NS flops: per iteration p(p+1)q (upper-triangle X X^T),
    p^2(p+1) (symmetric A A) and 2p^2q (B X)."""
    tot = 0.0
    for m, n in shapes:
        p, q = float(min(m, n)), float(max(m, n))
        tot += ns_steps * (p * (p + 1) * q + p * p * (p + 1) + 2 * p * p * q)
    return tot


def roofline(row, arith):
    """Roofline position of a kernel from its algorithmic flops and bytes
    (summed over its launches) and its measured time: the bound is whichever
    of the MFMA peak and the HBM peak allows less time for that work."""
    t_mfma = row["flops"] / (PEAK_TFLOPS[arith] * 1e12) if row["flops"] else 0.0
    t_hbm = row["bytes"] / (PEAK_HBM_GBS * 1e9)
    secs = row["ms"] * 1e-3
    out = {"intensity_flop_per_byte": round(row["flops"] / row["bytes"], 2) if row["bytes"] else None,
           "mfma_frac": round(t_mfma / secs, 4), "hbm_frac": round(t_hbm / secs, 4)}
    if t_mfma >= t_hbm:
        achieved, peak = row["flops"] / secs / 1e12, PEAK_TFLOPS[arith]
        out.update({"bound": "mfma", "unit": "TFLOP/s"})
    else:
        achieved, peak = row["bytes"] / secs / 1e9, PEAK_HBM_GBS
        out.update({"bound": "hbm", "unit": "GB/s"})
    out.update({"achieved": round(achieved, 2), "peak": peak, "frac": round(achieved / peak, 4)})
    return out


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--config", type=int, default=5, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--op", default="muon", choices=["muon", "clip", "adamw", "gram_local"],
                    help="muon: the Muon step (default); clip / adamw: the element-wise "
                         "companions (gradient clipping, AdamW) on their own workloads; "
                         "gram_local: Gram-space NS of one tensor-parallel rank's blocks")
    ap.add_argument("--ns-backend", default="direct", choices=["direct", "gram"],
                    help="direct: X <- aX + BX every iteration (default); gram: the "
                         "Gram-space iteration with restarts")
    ap.add_argument("--ns-prec", default=None,
                    choices=["f32", "bf16", "bf16_split", "bf16_split_a", "auto", "f16"],
                    help="operand precision of the NS products (default: the "
                         "configuration's own for the direct backend, f32 for gram; gram "
                         "takes f32 or f16)")
    ap.add_argument("--restarts", default=None, metavar="K,K,...",
                    help="Gram backend: iterations that start a new window (default: 2; "
                         "'' for none)")
    ap.add_argument("--cpu-seconds", type=float, default=20.0,
                    help="budget of the oracle's host timing (0 disables it)")
    ap.add_argument("--grads", default="workload", choices=["workload", "host", "gauss"],
                    help="workload: the configuration's gradient recipe drawn on the device "
                         "(default; its Haar factors call the device QR solver); host: the "
                         "same recipe drawn by the numpy generator on the host and copied "
                         "in, so the process runs no solver on the device -- for profiled "
                         "runs; gauss: iid N(0,1) gradients of the same shapes and dtype, "
                         "drawn on the device without a solver (kernel work does not depend "
                         "on the values)")
    ap.add_argument("--launch", default="graph", choices=["graph", "stream"],
                    help="graph: each gradient set's step is recorded once "
                         "(dmuon_muon_step_graph / dmuon_ns_orthogonalize_graph) and "
                         "replayed (default); stream: every step calls the entry point, "
                         "which launches its kernels one by one. The evented region "
                         "always launches one by one (its events sit between launches)")
    ap.add_argument("--calib-copy", type=int, default=0, metavar="MIB",
                    help="run one plain device copy of this many MiB first (a "
                         "known-size reference for rocprofv3 byte counters)")
    return ap.parse_args()


def _host_sets(cfg, n_sets, device, dtype):
    """The configuration's gradient recipe drawn by the numpy generator on
    the host (no device solver), copied to ``device``."""
    import torch
    import workloads
    bases = [None] * len(cfg.shapes)
    if cfg.grad_kind == "powerlaw_t3" and n_sets > 1:
        for i, (m, n) in enumerate(cfg.shapes):
            bases[i] = workloads.powerlaw_basis_np(m, n, cfg.cfg_id, i)
            log(f"host basis {i + 1}/{len(cfg.shapes)} ready")
    sets = []
    for s in range(n_sets):
        sets.append([torch.from_numpy(workloads.grad_np(cfg.grad_kind, m, n, cfg.cfg_id, s, i,
                                                        basis=bases[i])).to(device, dtype)
                     for i, (m, n) in enumerate(cfg.shapes)])
        log(f"host gradient set {s + 1}/{n_sets} ready")
    return sets


def make_inputs(cfg, n_sets, device, grad_kind=None):
    """params, zero momentum buffers and ``n_sets`` gradient sets of ``cfg``
    on ``device``. ``grad_kind``: a gradient recipe drawn on the device, or
    "host" for the configuration's recipe drawn by numpy on the host."""
    import torch
    import workloads
    from workloads.synth import powerlaw_basis_torch
    dt = {"f32": torch.float32, "bf16": torch.bfloat16}
    shapes = cfg.shapes
    grad_kind = grad_kind or cfg.grad_kind
    params = [workloads.param_torch(m, n, cfg.cfg_id, i, device, dt[cfg.param_dtype])
              for i, (m, n) in enumerate(shapes)]
    bufs = [torch.zeros(m, n, dtype=torch.float32, device=device) for m, n in shapes]
    if grad_kind == "host":
        sets = _host_sets(cfg, n_sets, device, dt[cfg.grad_dtype])
        torch.cuda.synchronize()
        return params, bufs, sets
    bases = [None] * len(shapes)
    if grad_kind == "powerlaw_t3":
        for i, (m, n) in enumerate(shapes):
            bases[i] = powerlaw_basis_torch(m, n, cfg.cfg_id, i, device)
            log(f"basis {i + 1}/{len(shapes)} ready")
    sets = []
    for s in range(n_sets):
        sets.append([workloads.grad_torch(grad_kind, m, n, cfg.cfg_id, s, i, device,
                                          dt[cfg.grad_dtype], basis=bases[i])
                     for i, (m, n) in enumerate(shapes)])
        log(f"gradient set {s + 1}/{n_sets} ready")
    del bases
    torch.cuda.synchronize()
    return params, bufs, sets


def kernel_sha():
    h = hashlib.sha256()
    for f in ("dmuon_kernels.hip", "dmuon_optim.hip", "dmuon_device.h", "dmuon_internal.h",
              "dmuon_host.cpp"):
        with open(os.path.join(ROOT, "newton_schulz_06_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def traffic_for(kind, workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if
    it was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        tab = json.load(f)
    e = tab.get(f"{kind}@{workload}")
    if not e or e.get("kernel_source_sha256") != kernel_sha():
        return None
    return e.get("hbm_bytes_per_launch")


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([d.get("num_threads", 1) for d in threadpool_info()
                    if d.get("user_api") == "blas"] or [1])
    except Exception:
        return len(os.sched_getaffinity(0))


def cpu_baseline(cfg, budget_s, backend="direct", restarts=None, grad_sets=None):
    """The fp64 oracle as it stands, on the host, over the same inputs, timed
    per phase: momentum (oracle.momentum_update), Newton-Schulz
    (oracle.direct_newton_schulz, or oracle.gram_newton_schulz for the Gram
    backend) and the update (oracle.update_param).  Matrices are taken in
    the workload's order, step after step (the gradient sets the GPU ran,
    copied to the host, or else the seeded numpy recipe; the momentum
    carried over), until the budget is spent.  A matrix whose whole NS would
    not fit in the remaining budget (the 70B MLP's) runs one of its NS
    iterations instead, which is one fifth of the NS flops with the same
    products; the sample says which."""
    import numpy as np
    import oracle
    import workloads
    quintic = [tuple(oracle.QUINTIC)]
    t_phase = {"momentum": 0.0, "ns": 0.0, "update": 0.0}
    elems = {"momentum": 0, "update": 0}
    ns_flops_done = 0.0
    rate = 0.4e12  # assumed until measured: algorithmic NS flop/s of the oracle
    bufs, params = {}, {}
    parts = []
    step, t_total = 0, 0.0
    while t_total < budget_s:
        for i, (m, n) in enumerate(cfg.shapes):
            if grad_sets is not None:
                g = grad_sets[step % len(grad_sets)][i].double().cpu().numpy()
            else:
                g = workloads.grad_np(cfg.grad_kind, m, n, cfg.cfg_id, step, i)
            if i not in params:
                params[i] = workloads.param_np(m, n, cfg.cfg_id, i)
                bufs[i] = np.zeros((m, n))
            full = ns_flops([(m, n)], cfg.ns_steps)
            iters = cfg.ns_steps
            if backend == "direct" and t_total + full / rate > budget_s:
                iters = 1
            u = g
            if not cfg.ns_only:
                t0 = time.perf_counter()
                bufs[i], u = oracle.momentum_update(bufs[i], g, cfg.momentum, cfg.nesterov)
                t_phase["momentum"] += time.perf_counter() - t0
                elems["momentum"] += m * n
            t0 = time.perf_counter()
            if backend == "gram":
                O = oracle.gram_newton_schulz(u, steps=cfg.ns_steps, restart_iterations=restarts)
            elif iters == cfg.ns_steps:
                O = oracle.direct_newton_schulz(u, steps=cfg.ns_steps)
            else:
                O = oracle.direct_newton_schulz(u, coefficients=quintic)
            dt = time.perf_counter() - t0
            t_phase["ns"] += dt
            if dt > 5:
                log(f"oracle: {m}x{n}, {iters} NS iteration(s) in {dt:.1f} s")
            done = full * iters / cfg.ns_steps
            ns_flops_done += done
            rate = ns_flops_done / t_phase["ns"]
            if not cfg.ns_only:
                t0 = time.perf_counter()
                params[i] = oracle.update_param(params[i], O, cfg.lr, cfg.weight_decay)
                t_phase["update"] += time.perf_counter() - t0
                elems["update"] += m * n
            parts.append(f"{m}x{n}" + ("" if iters == cfg.ns_steps else f" ({iters} of "
                                                                        f"{cfg.ns_steps} NS iterations)"))
            t_total = sum(t_phase.values())
            if t_total >= budget_s:
                break
        step += 1
    numel = sum(m * n for m, n in cfg.shapes)
    ns_step = ns_flops(cfg.shapes, cfg.ns_steps)
    est = {"ns": ns_step / rate}
    if not cfg.ns_only:
        est["momentum"] = t_phase["momentum"] / elems["momentum"] * numel
        est["update"] = t_phase["update"] / elems["update"] * numel
    counts = {}
    for p_ in parts:
        counts[p_] = counts.get(p_, 0) + 1
    desc = ", ".join(f"{c} x {k}" for k, c in counts.items())
    return {
        "value": rate / 1e12,
        "unit": "NS TFLOP/s",
        "cores": blas_threads(),
        "kind": "oracle",
        "cpu_model": cpu_model(),
        "sample": (f"{len(parts)} matrices of the workload in order ({len(parts) // len(cfg.shapes)} "
                   f"whole steps and {len(parts) % len(cfg.shapes)} of the next: {desc}); "
                   f"{t_total:.1f} s; numpy fp64 BLAS"
                   + ("; Gram-space NS" if backend == "gram" else "")),
        "phase_s": {k: round(v, 3) for k, v in t_phase.items()},
        "step_s_estimate": {k: round(v, 2) for k, v in est.items()},
        "ms_per_step_estimate": round(sum(est.values()) * 1e3, 1),
    }


def calib_copy(mib, device):
    """One plain device-to-device copy of `mib` MiB: a known-size reference
    for rocprofv3's byte counters."""
    if not mib:
        return
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device=device)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def gram_flops(p, q, ns_steps=5, restarts=None):
    """Flops of Gram-space NS on a p x q oriented block, counted like the
    library's profile: per window, p(p+1)q for A = X X^T, p^2(p+1) for each
    symmetric p x p product (P's A A, Q <- P Q, P A, P (P A)) and 2p^2q
    for X <- Q X."""
    cuts = sorted({0, ns_steps} | {r for r in ([2] if restarts is None else restarts)
                                   if 0 < r < ns_steps})
    sym = p * p * (p + 1.0)
    tot = 0.0
    for s, e in zip(cuts[:-1], cuts[1:]):
        k = e - s
        tot += p * (p + 1.0) * q + k * sym + 3 * (k - 1) * sym + 2.0 * p * p * q
    return tot


def run_gram_local(args):
    """Gram-space NS of one tensor-parallel rank's blocks (one batch per
    orientation), with the shard group's all-reduce stubbed as identity:
    K timed calls; value = flops per second (fp32 MFMA)."""
    import numpy as np
    import torch
    import workloads
    import newton_schulz_06_amd as dm

    oc = workloads.OP_CONFIGS["gram_local"]
    steps = args.steps if args.steps is not None else 10
    warmup = args.warmup if args.warmup is not None else 2
    device = torch.device("cuda", 0)
    torch.cuda.set_device(device)
    calib_copy(args.calib_copy, device)
    gen = torch.Generator(device=device).manual_seed(19)
    dt = {"f32": torch.float32, "bf16": torch.bfloat16}[oc.dtype]
    batches = []
    flops = 0.0
    for t in (0, 1):
        shapes = [s for s, tt in zip(oc.shapes, oc.transposed) if tt == t]
        if not shapes:
            continue
        gs = [torch.randn(s, device=device, generator=gen).to(dt) for s in shapes]
        outs = [torch.empty_like(g) for g in gs]
        batches.append(dm.GramLocal(gs, outs, transposed=t, prec="f32"))
        for m, n in shapes:
            p, q = (n, m) if t else (m, n)
            flops += gram_flops(p, q)
    log(f"gram_local on {oc.name}: {len(oc.shapes)} blocks in {len(batches)} batches")

    def run():
        for b in batches:
            b()

    for _ in range(max(warmup - 1, 0)):
        run()
    with dm.profile() as prof_all:
        run()
    torch.cuda.synchronize()
    dominant = max(prof_all.rows, key=lambda k: prof_all.rows[k]["ms"])
    charged = sum(v["flops"] for v in prof_all.rows.values())
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    with dm.profile(kinds=[dominant]) as prof:
        e0.record(stream)
        for _ in range(steps):
            run()
        e1.record(stream)
        torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / steps
    tflops = flops / (ms_step * 1e-3) / 1e12
    log(f"timed {steps} calls: {ms_step:.4f} ms/call, {tflops:.1f} TFLOP/s")
    row = prof.rows[dominant]
    roof = roofline(row, "f32")
    roof.update({"kernel": dominant,
                 "flops_per_launch": row["flops"] / row["launches"],
                 "bytes_per_launch": row["bytes"] / row["launches"],
                 "avg_launch_ms": round(row["ms"] / row["launches"], 5),
                 "launches": row["launches"],
                 "traffic": traffic_for(dominant, oc.name)})
    cpu = None
    if args.cpu_seconds > 0:
        cpu = gram_local_cpu_baseline(oc, min(args.cpu_seconds, 30.0))
    out = {
        "metric": OP_METRIC["gram_local"],
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": oc.name, "blocks": len(oc.shapes),
                   "shapes": sorted({f"{m}x{n}" for m, n in oc.shapes}),
                   "block_dtype": oc.dtype, "ns_steps": 5, "restarts": [2],
                   "group_sum": "identity (one GPU's share)",
                   "parallelism": "1 GPU (one rank of a TP-8 group)"},
        "tflop_per_step": round(flops / 1e12, 6),
        "kernel_tflop_one_step": round(charged / 1e12, 6),
        "kernel_ms_one_step": {k: round(v["ms"], 4) for k, v in prof_all.rows.items()},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def gram_local_cpu_baseline(oc, budget_s):
    """The fp64 oracle's shard NS on the host, block by block (one rank, the
    group sum a no-op) until the budget is used."""
    import numpy as np
    import oracle
    rng = np.random.default_rng(0)
    t_total, flops, done = 0.0, 0.0, 0
    for (m, n), t in zip(oc.shapes, oc.transposed):
        g = rng.standard_normal((m, n))
        t0 = time.perf_counter()
        oracle.gram_newton_schulz_distributed_local([g], bool(t))
        t_total += time.perf_counter() - t0
        p, q = (n, m) if t else (m, n)
        flops += gram_flops(p, q)
        done += 1
        if t_total >= budget_s:
            break
    return {"value": flops / t_total / 1e12, "unit": "TFLOP/s",
            "cores": len(os.sched_getaffinity(0)), "kind": "oracle",
            "sample": f"{done} of {len(oc.shapes)} blocks, {t_total:.1f} s; numpy fp64 BLAS"}


OP_METRIC = {
    "clip": "Muon gradient clipping (norm + scale) ms & HBM GB/s, 1 GPU",
    "adamw": "AdamW update of non-Muon params ms & HBM GB/s, 1 GPU",
    "gram_local": "Gram NS of one TP rank's blocks ms & TFLOP/s (fp32 MFMA), 1 GPU",
}


def run_op(args):
    """Gradient clipping or AdamW on its workload: K timed calls, HBM-bound,
    value = algorithmic bytes moved per second."""
    import numpy as np
    import torch
    import workloads
    import newton_schulz_06_amd as dm

    oc = workloads.OP_CONFIGS[args.op]
    steps = args.steps if args.steps is not None else 20
    warmup = args.warmup if args.warmup is not None else 3
    device = torch.device("cuda", 0)
    torch.cuda.set_device(device)
    calib_copy(args.calib_copy, device)
    gen = torch.Generator(device=device).manual_seed(17)
    dt = {"f32": torch.float32, "bf16": torch.bfloat16}[oc.dtype]
    esz = 4 if oc.dtype == "f32" else 2
    numel = sum(m * n for m, n in oc.shapes)
    log(f"{args.op} on {oc.name}: {len(oc.shapes)} tensors, {numel / 1e6:.1f}M elements")
    if args.op == "clip":
        gs = [torch.randn(s, device=device, generator=gen).to(dt) for s in oc.shapes]
        call = dm.PreparedClip(gs, oc.max_norm, buckets=list(oc.buckets))
        # Every call must really clip: measure the largest bucket norm once,
        # then halve max_norm from call to call (each call scales by ~1/2).
        probe = dm.PreparedClip(gs, None, buckets=list(oc.buckets))
        probe()
        m0 = 0.5 * min(s["total_norm"] for s in probe.stats())
        run = lambda t: call(m0 * 0.5 ** t)  # noqa: E731
        bytes_call = 3.0 * numel * esz  # read (norm), read + write (scale)
    else:
        ps = [(0.02 * torch.randn(s, device=device, generator=gen)).to(dt) for s in oc.shapes]
        gs = [(0.1 * torch.randn(s, device=device, generator=gen)).to(dt) for s in oc.shapes]
        ms = [torch.zeros(s, device=device) for s in oc.shapes]
        vs = [torch.zeros(s, device=device) for s in oc.shapes]
        call = dm.PreparedAdamW(ps, gs, ms, vs)
        run = call
        bytes_call = numel * (2.0 * esz + esz + 16.0)  # p r/w, g, m and v r/w
    torch.cuda.synchronize()
    for w in range(max(warmup - 1, 0)):
        run(w + 1)
    with dm.profile() as prof_all:
        run(warmup)
    torch.cuda.synchronize()
    dominant = max(prof_all.rows, key=lambda k: prof_all.rows[k]["ms"])
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    with dm.profile(kinds=[dominant]) as prof:
        e0.record(stream)
        for s in range(steps):
            run(warmup + 1 + s)
        e1.record(stream)
        torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / steps
    gbs = bytes_call / (ms_step * 1e-3) / 1e9
    log(f"timed {steps} calls: {ms_step:.4f} ms/call, {gbs:.1f} GB/s")
    row = prof.rows[dominant]
    roof = roofline(row, "f32")
    roof.update({"kernel": dominant,
                 "flops_per_launch": 0.0,
                 "bytes_per_launch": row["bytes"] / row["launches"],
                 "avg_launch_ms": round(row["ms"] / row["launches"], 5),
                 "launches": row["launches"],
                 "traffic": traffic_for(dominant, oc.name)})
    cpu = None
    if args.cpu_seconds > 0:
        cpu = op_cpu_baseline(args.op, oc, min(args.cpu_seconds, 10.0))
    out = {
        "metric": OP_METRIC[args.op],
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": oc.dtype,
        "data": "synthetic",
        "config": {"workload": oc.name, "tensors": len(oc.shapes), "elements": numel,
                   "shapes": sorted({f"{m}x{n}" for m, n in oc.shapes}),
                   "buckets": len(set(oc.buckets)) if oc.buckets else None,
                   "parallelism": "1 GPU"},
        "bytes_per_step": bytes_call,
        "kernel_ms_one_step": {k: round(v["ms"], 4) for k, v in prof_all.rows.items()},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def op_cpu_baseline(op, oc, budget_s):
    """The fp64 oracle on the host over 256-row blocks of the workload's
    tensors, cycling through them until the budget is used; reported as
    algorithmic GB/s of the same operation."""
    import numpy as np
    import oracle
    rng = np.random.default_rng(0)
    done, t_total, nbytes = 0, 0.0, 0.0
    esz = 4 if oc.dtype == "f32" else 2
    rows = 256
    while t_total < budget_s:
        for m, n in oc.shapes:
            r = min(rows, m)
            if op == "clip":
                g = rng.standard_normal((r, n))
                t0 = time.perf_counter()
                oracle.clip_grad_norm([g], oc.max_norm)
                t_total += time.perf_counter() - t0
                nbytes += 3.0 * g.size * esz
            else:
                p, g = 0.02 * rng.standard_normal((r, n)), 0.1 * rng.standard_normal((r, n))
                t0 = time.perf_counter()
                oracle.adamw_step(p, g, np.zeros_like(p), np.zeros_like(p), 1)
                t_total += time.perf_counter() - t0
                nbytes += g.size * (3.0 * esz + 16.0)
            done += r * n
            if t_total >= budget_s:
                break
    return {"value": nbytes / t_total / 1e9, "unit": "GB/s", "cores": len(os.sched_getaffinity(0)),
            "kind": "oracle",
            "sample": f"{done / 1e6:.1f}M elements in {rows}-row blocks of the workload's "
                      f"tensors, {t_total:.1f} s; numpy fp64"}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)
    if args.op == "gram_local":
        run_gram_local(args)
        return
    if args.op != "muon":
        run_op(args)
        return
    import torch
    import workloads
    import newton_schulz_06_amd as dm

    cfg = workloads.CONFIGS[args.config]
    steps = args.steps if args.steps is not None else (100 if args.config in (1, 2, 4) else 20)
    warmup = args.warmup if args.warmup is not None else 10 if args.config in (1, 2, 4) else 3
    device = torch.device("cuda", 0)
    torch.cuda.set_device(device)
    calib_copy(args.calib_copy, device)
    n_sets = 1 if cfg.ns_only else max(1, min(cfg.steps, steps + warmup))
    grad_kind = {"gauss": "gauss", "host": "host"}.get(args.grads, cfg.grad_kind)
    log(f"config {cfg.cfg_id} ({cfg.name}): {len(cfg.shapes)} matrices, {n_sets} gradient sets"
        f" ({grad_kind})")
    params, bufs, sets = make_inputs(cfg, n_sets, device, grad_kind)
    shapes = list(cfg.shapes)
    flops_step = ns_flops(shapes, cfg.ns_steps)
    backend = args.ns_backend
    restarts = None
    if args.restarts is not None:
        restarts = [int(v) for v in args.restarts.split(",") if v.strip()]
    # The Gram backend runs on fp32 operands unless fp16 is asked for.
    prec = args.ns_prec or ("f32" if backend == "gram" else cfg.ns_prec)
    # the products' operand type ("bf16+f16": bf16 on the first iteration,
    # fp16 after; fp32 accumulation everywhere).  The automatic mode takes
    # fp16 only for matrices below 256-wide tiles (min side < 1024, or
    # more than 1/8 padding at 256).
    def tile256(m, n):
        p = min(m, n)
        return p >= 1024 and -(-p // 256) * 256 * 8 <= 9 * p
    if prec == "auto":
        arith = "bf16" if all(tile256(m, n) for m, n in shapes) else "bf16+f16"
    elif backend == "gram":
        arith = prec  # f32, or f16 from the first product on
    else:
        arith = {"f32": "f32", "f16": "bf16+f16"}.get(prec, "bf16")
    ns_kw = dict(ns_steps=cfg.ns_steps, prec=prec, backend=backend, restart_iterations=restarts)

    graph = args.launch == "graph"
    if cfg.ns_only:
        outs = [torch.empty_like(g) for g in sets[0]]
        call = dm.PreparedNs(sets[0], outs, **ns_kw)
        run_stream = lambda i: call()  # noqa: E731
        gcall = dm.PreparedNs(sets[0], outs, workspace=call.ws, graph=True, **ns_kw) if graph \
            else None
        run = (lambda i: gcall()) if graph else run_stream  # noqa: E731
    else:
        step_kw = dict(lr=cfg.lr, momentum=cfg.momentum, weight_decay=cfg.weight_decay,
                       nesterov=cfg.nesterov, **ns_kw)
        call = dm.PreparedMuonStep(params, bufs, sets, **step_kw)
        run_stream = call
        run = dm.PreparedMuonStep(params, bufs, sets, workspace=call.ws, graph=True,
                                  **step_kw) if graph else run_stream

    # Warm-up (every gradient set at least once); the last warm-up step
    # times every kernel kind once to find the dominant one.
    builds0 = dm.plan_builds()
    for w in range(max(warmup - 1, n_sets - 1, 0)):
        run(w % n_sets)
    if graph:
        if not cfg.ns_only:
            run.record()  # every gradient set's graph, before any timed region
        run_stream(0)  # the stream path's own warm-up (the evented region uses it)
    with dm.profile() as prof_all:
        run_stream((warmup - 1) % n_sets if warmup else 0)
    torch.cuda.synchronize()
    dominant = max(prof_all.rows, key=lambda k: prof_all.rows[k]["ms"])
    log(f"warm-up done; per-kind ms of one step: "
        + ", ".join(f"{k}={v['ms']:.3f}" for k, v in prof_all.rows.items())
        + f"; dominant: {dominant}")
    builds_warm = dm.plan_builds()

    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)

    # Timed region 1: the K steps alone (value, ms_per_step).
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for s in range(steps):
        run((warmup + s) % n_sets)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = e0.elapsed_time(e1) / steps
    ns_tflops = flops_step / (ms_step * 1e-3) / 1e12
    log(f"timed {steps} steps: {ms_step:.4f} ms/step (wall {wall * 1e3 / steps:.4f} ms/step), "
        f"NS {ns_tflops:.1f} TFLOP/s")

    # Timed region 2: the same K steps with HIP events on the launch stream
    # around every launch of the dominant kernel (its roofline).
    torch.cuda.synchronize()
    with dm.profile(kinds=[dominant]) as prof:
        e0.record(stream)
        for s in range(steps):
            run_stream((warmup + s) % n_sets)
        e1.record(stream)
        torch.cuda.synchronize()
    ms_step_ev = e0.elapsed_time(e1) / steps
    builds_timed = dm.plan_builds() - builds_warm
    log(f"evented region: {ms_step_ev:.4f} ms/step; launch tables built: "
        f"{builds_warm - builds0} in warm-up, {builds_timed} in the timed regions")

    row = prof.rows[dominant]
    roof = roofline(row, arith)
    roof.update({"kernel": dominant,
                 "flops_per_launch": row["flops"] / row["launches"],
                 "bytes_per_launch": row["bytes"] / row["launches"],
                 "avg_launch_ms": round(row["ms"] / row["launches"], 5),
                 "launches": row["launches"],
                 "ms_per_step_evented": round(ms_step_ev, 5),
                 "traffic": traffic_for(dominant, cfg.name)})

    cpu = None
    if args.cpu_seconds > 0:
        log("timing the fp64 oracle on the host")
        cpu = cpu_baseline(cfg, args.cpu_seconds, backend, restarts, grad_sets=sets)

    out = {
        "metric": METRIC,
        "value": round(ns_tflops, 3),
        "unit": "NS TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": arith,
        "data": "synthetic",
        "config": {
            "workload": cfg.name,
            "matrices": len(shapes),
            "shapes": sorted({f"{m}x{n}" for m, n in shapes}) if len(shapes) <= 32 else "512 small",
            "ns_steps": cfg.ns_steps,
            "ns_precision": prec,
            "ns_backend": backend,
            "param_dtype": cfg.param_dtype,
            "grad_dtype": cfg.grad_dtype,
            "nesterov": cfg.nesterov,
            "ns_only": cfg.ns_only,
            "gradients": f"{cfg.grad_kind} (numpy, host)" if grad_kind == "host" else grad_kind,
            "launch": "hip_graph" if graph else "stream",
            "parallelism": "1 GPU (owner-local batch)",
        },
        "ns_tflop_per_step": round(flops_step / 1e12, 6),
        # flops the library's kernels were charged with in one step (for the
        # Gram backend these differ from the direct count the value is based on)
        "kernel_tflop_one_step": round(sum(v["flops"] for v in prof_all.rows.values()) / 1e12, 6),
        "ns_mfma_frac": round(ns_tflops / PEAK_TFLOPS[arith], 4),
        # every kernel kind of one profiled warm-up step (HIP events around
        # each launch): time, algorithmic rates and both roofline fractions
        "kernels_one_step": {
            k: {"ms": round(v["ms"], 4), "launches": v["launches"],
                "tflop_s": round(v["flops"] / (v["ms"] * 1e-3) / 1e12, 2) if v["ms"] else None,
                "gb_s": round(v["bytes"] / (v["ms"] * 1e-3) / 1e9, 1) if v["ms"] else None,
                **{f: roofline(v, arith)[f] for f in ("bound", "mfma_frac", "hbm_frac")}}
            for k, v in prof_all.rows.items() if v["ms"] > 0},
        "matrices_per_s": round(len(shapes) / (ms_step * 1e-3), 1),
        "launch_tables_built_in_timed_regions": builds_timed,
        "kernel_ms_one_step": {k: round(v["ms"], 4) for k, v in prof_all.rows.items()},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
