"""Summaries of rocprofv3 CSV output for libdmuon's kernels.

    python -m newton_schulz_06_amd.rocprof_summary trace  <dir>   # --kernel-trace --stats run
    python -m newton_schulz_06_amd.rocprof_summary counter <dir> [copy_mib]  # --pmc run
    python -m newton_schulz_06_amd.rocprof_summary traffic <fetch_dir> <write_dir> \
        <copy_mib> <kind> <kernel_prefix> <workload> <summary.md>

`trace` prints per-kernel dispatch counts and average durations from the
kernel trace; `counter` prints per-kernel averages of every collected
counter.  With `copy_mib`, the plain copy of that many MiB that
``bench.py --calib-copy`` runs (the largest dispatch of the runtime's copy
kernel) gives the ratio known / measured, printed as the scale factor for
FETCH_SIZE and WRITE_SIZE (KiB per dispatch).  `traffic` takes one
FETCH_SIZE run and one WRITE_SIZE run (each with the calibration copy),
averages both counters over the dispatches of the kernels whose short name
starts with `kernel_prefix`, scales them, and records the HBM bytes per
launch in profiles/traffic.json under "<kind>@<workload>", with the hash of
the kernel sources the counters were taken on.
"""
import collections
import csv
import glob
import os
import re
import sys

KINDS = {"3": "syrk", "4": "poly", "5": "update_x", "9": "gram_mul"}


def short_name(name: str) -> str:
    m = re.search(r"dmuon::\(anonymous namespace\)::(\w+)(<[^>]*>)?", name)
    if m:
        kern, targs = m.group(1), m.group(2) or ""
        if kern == "gemm_f32_small_kernel":  # <KIND>: 16 x 16 fp32 tiles
            k = re.match(r"<(\d+)", targs)
            return f"{KINDS.get(k.group(1), k.group(1))}[{kern}<T=16>]" if k else kern
        t = re.match(r"<(\d+), (\d+)(?:, (\d+))?(?:, (\d+), (\d+))?", targs)
        if t and kern.startswith("gemm"):
            bk = f",BK={t.group(3)}" if kern == "gemm_bf16_kernel" and t.group(3) not in (None, "64") else ""
            # 16-bit operand formats: inputs and the X copies written next
            fmt = {("1", "1"): ",f16", ("0", "1"): ",bf16>f16"}.get((t.group(4), t.group(5)), "")
            return f"{KINDS.get(t.group(1), t.group(1))}[{kern}<T={t.group(2)}{bk}{fmt}>]"
        return kern
    if "elementwise" in name and ("copy" in name.lower() or "direct_copy" in name):
        return "torch_copy"
    return name.split("(")[0][-60:]


def _csv(dirname, suffix):
    hits = glob.glob(os.path.join(dirname, "**", f"*{suffix}"), recursive=True)
    if not hits:
        raise SystemExit(f"no *{suffix} under {dirname}")
    return hits[0]


def trace(dirname):
    path = _csv(dirname, "kernel_trace.csv")
    agg = collections.OrderedDict()
    for r in csv.DictReader(open(path)):
        k = short_name(r["Kernel_Name"])
        d = agg.setdefault(k, [0, 0.0])
        d[0] += 1
        d[1] += (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3  # us
    print(f"{'kernel':42s} {'calls':>6s} {'total_us':>12s} {'avg_us':>10s}")
    for k, (n, tot) in sorted(agg.items(), key=lambda kv: -kv[1][1]):
        print(f"{k:42s} {n:6d} {tot:12.1f} {tot / n:10.2f}")


def counter(dirname, copy_mib=None):
    path = _csv(dirname, "counter_collection.csv")
    vals = collections.defaultdict(lambda: collections.defaultdict(list))
    raw = collections.defaultdict(dict)  # counter -> {(dispatch, kernel name): value}
    for r in csv.DictReader(open(path)):
        k = short_name(r["Kernel_Name"])
        vals[k][r["Counter_Name"]].append(float(r["Counter_Value"]))
        raw[r["Counter_Name"]][(r["Dispatch_Id"], r["Kernel_Name"])] = float(r["Counter_Value"])
    for k, cs in vals.items():
        parts = [f"{c}={sum(v) / len(v):.1f}" for c, v in sorted(cs.items())]
        print(f"{k:42s} n={len(next(iter(cs.values())))}  " + "  ".join(parts))
    if copy_mib:
        # The plain device copy of ``bench.py --calib-copy`` is the largest
        # dispatch of the runtime's copy kernel in the run.
        known_kib = float(copy_mib) * 1024.0
        for c in ("FETCH_SIZE", "WRITE_SIZE"):
            vs = [v for (k, name), v in raw.get(c, {}).items() if "copyBuffer" in name]
            if not vs:
                continue
            v = max(vs)
            print(f"calibration: {c}={v:.1f} KiB for a {copy_mib} MiB copy -> "
                  f"scale {known_kib / v:.4f}")


def _counter_avg(dirname, counter_name, prefix):
    """(average over the matching dispatches, the calibration copy's value)."""
    path = _csv(dirname, "counter_collection.csv")
    per = collections.defaultdict(float)  # dispatch -> summed value
    copy = 0.0
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter_name:
            continue
        v = float(r["Counter_Value"])
        if short_name(r["Kernel_Name"]).startswith(prefix):
            per[r["Dispatch_Id"]] += v
        elif "copyBuffer" in r["Kernel_Name"]:
            copy = max(copy, v)
    if not per or not copy:
        raise SystemExit(f"{counter_name}: no dispatch of {prefix} or no calibration copy in {dirname}")
    return sum(per.values()) / len(per), copy


def traffic(fetch_dir, write_dir, copy_mib, kind, prefix, workload, summary):
    import json
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    sys.path.insert(0, root)
    import bench
    known_kib = float(copy_mib) * 1024.0
    fetch, fcopy = _counter_avg(fetch_dir, "FETCH_SIZE", prefix)
    write, wcopy = _counter_avg(write_dir, "WRITE_SIZE", prefix)
    fs, ws = known_kib / fcopy, known_kib / wcopy
    entry = {"kernel": prefix, "kernel_source_sha256": bench.kernel_sha(),
             "fetch_kib_per_dispatch": round(fetch, 1), "write_kib_per_dispatch": round(write, 1),
             "fetch_scale": round(fs, 4), "write_scale": round(ws, 4),
             "hbm_bytes_per_launch": int(round((fetch * fs + write * ws) * 1024.0)),
             "source": summary}
    path = os.path.join(root, "profiles", "traffic.json")
    tab = json.load(open(path)) if os.path.exists(path) else {}
    tab[f"{kind}@{workload}"] = entry
    with open(path, "w") as f:
        json.dump(tab, f, indent=1)
        f.write("\n")
    print(json.dumps({f"{kind}@{workload}": entry}, indent=1))


if __name__ == "__main__":
    if len(sys.argv) >= 2 and sys.argv[1] == "traffic" and len(sys.argv) == 9:
        traffic(*sys.argv[2:9])
        sys.exit(0)
    if len(sys.argv) < 3 or sys.argv[1] not in ("trace", "counter"):
        print(__doc__)
        sys.exit(2)
    if sys.argv[1] == "trace":
        trace(sys.argv[2])
    else:
        counter(sys.argv[2], sys.argv[3] if len(sys.argv) > 3 else None)
