"""Summaries of rocprofv3 CSV output for libdmuon's kernels.

    python -m newton_schulz_06_amd.rocprof_summary trace  <dir>   # --kernel-trace --stats run
    python -m newton_schulz_06_amd.rocprof_summary counter <dir> [copy_mib]  # --pmc run

`trace` prints per-kernel dispatch counts and average durations from the
kernel trace; `counter` prints per-kernel averages of every collected
counter.  With `copy_mib`, the plain copy of that many MiB that
``bench.py --calib-copy`` runs is located by its size and the ratio
known / measured is printed as the scale factor for FETCH_SIZE and
WRITE_SIZE (KiB per dispatch).
"""
import collections
import csv
import glob
import os
import re
import sys

KINDS = {"3": "syrk", "4": "poly", "5": "update_x"}


def short_name(name: str) -> str:
    m = re.search(r"dmuon::\(anonymous namespace\)::(\w+)(<[^>]*>)?", name)
    if m:
        kern, targs = m.group(1), m.group(2) or ""
        t = re.match(r"<(\d+), (\d+)", targs)
        if t and kern.startswith("gemm"):
            return f"{KINDS.get(t.group(1), t.group(1))}[{kern}<T={t.group(2)}>]"
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
    sizes = {}
    for r in csv.DictReader(open(path)):
        k = short_name(r["Kernel_Name"])
        vals[k][r["Counter_Name"]].append(float(r["Counter_Value"]))
        sizes[(k, r["Dispatch_Id"])] = int(r["Grid_Size"])
    for k, cs in vals.items():
        parts = [f"{c}={sum(v) / len(v):.1f}" for c, v in sorted(cs.items())]
        print(f"{k:42s} n={len(next(iter(cs.values())))}  " + "  ".join(parts))
    if copy_mib:
        known_kib = float(copy_mib) * 1024.0
        best = None
        for k, cs in vals.items():
            for c in ("FETCH_SIZE", "WRITE_SIZE"):
                for v in cs.get(c, []):
                    if v > 0 and abs(v - known_kib) / known_kib < 0.25:
                        best = (k, c, v) if best is None else best
        if best:
            k, c, v = best
            print(f"calibration: {k} {c}={v:.1f} KiB for a {copy_mib} MiB copy -> "
                  f"scale {known_kib / v:.4f}")
        else:
            print("calibration: no dispatch near the copy size found")


if __name__ == "__main__":
    if len(sys.argv) < 3 or sys.argv[1] not in ("trace", "counter"):
        print(__doc__)
        sys.exit(2)
    if sys.argv[1] == "trace":
        trace(sys.argv[2])
    else:
        counter(sys.argv[2], sys.argv[3] if len(sys.argv) > 3 else None)
