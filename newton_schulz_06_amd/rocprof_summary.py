"""Summaries of rocprofv3 CSV output for libdmuon's kernels.

    python -m newton_schulz_06_amd.rocprof_summary trace  <dir>   # --kernel-trace --stats run
    python -m newton_schulz_06_amd.rocprof_summary counter <dir> [copy_mib]  # --pmc run

`trace` prints per-kernel dispatch counts and average durations from the
kernel trace; `counter` prints per-kernel averages of every collected
counter.  With `copy_mib`, the plain copy of that many MiB that
``bench.py --calib-copy`` runs (the largest dispatch of the runtime's copy
kernel) gives the ratio known / measured, printed as the scale factor for
FETCH_SIZE and WRITE_SIZE (KiB per dispatch).
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
        t = re.match(r"<(\d+), (\d+)(?:, (\d+))?", targs)
        if t and kern.startswith("gemm"):
            bk = f",BK={t.group(3)}" if kern == "gemm_bf16_kernel" and t.group(3) not in (None, "64") else ""
            return f"{KINDS.get(t.group(1), t.group(1))}[{kern}<T={t.group(2)}{bk}>]"
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


if __name__ == "__main__":
    if len(sys.argv) < 3 or sys.argv[1] not in ("trace", "counter"):
        print(__doc__)
        sys.exit(2)
    if sys.argv[1] == "trace":
        trace(sys.argv[2])
    else:
        counter(sys.argv[2], sys.argv[3] if len(sys.argv) > 3 else None)
