"""Turn rocprofv3 CSV output into the short text summaries kept under profiles/.

    python -m mixture_experts_ffn_softplus_amd.profiling summarize \\
        --trace DIR --fetch DIR --write DIR --copy-fetch DIR --copy-write DIR --copy-mib 1024 \\
        --kernel REGEX --workload NAME --command "..." --out profiles/NAME.txt

DIRs are rocprofv3 output directories (``--output-format csv``): ``--trace`` from a
``--kernel-trace --stats`` run, ``--fetch`` / ``--write`` from ``--pmc FETCH_SIZE`` /
``--pmc WRITE_SIZE`` runs, and the ``copy`` pair from the same counters on a plain device copy of
``--copy-mib`` MiB (``bench.py --copy-calibration``), whose known size scales the counters to
bytes.  The summary records a hash of the kernel sources so that a stale traffic figure is
never reported for a kernel that has changed since it was measured.

    python -m mixture_experts_ffn_softplus_amd.profiling counters --pmc DIR --counter NAME \
        --kernel LABEL=REGEX ... --workload NAME --command "..." --out profiles/NAME.txt

summarises one counter of a ``--pmc`` run (e.g. the derived MfmaUtil: MFMA-busy cycles over
GPU-active cycles of every SIMD, in percent) per kernel pattern.
"""
import argparse
import csv
import glob
import hashlib
import os
import re
import statistics

HERE = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCES = ["csrc/gemm.hip", "csrc/moe_common.h", "csrc/moe_internal.h"]


def source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(HERE, rel), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _csv(d: str, suffix: str):
    files = glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no *{suffix} under {d}")
    with open(files[0]) as fh:
        return list(csv.DictReader(fh))


def kernel_durations(trace_dir: str, pattern: str):
    """Per-dispatch durations (us) of kernels whose name matches `pattern`."""
    rows = _csv(trace_dir, "kernel_trace.csv")
    rx = re.compile(pattern)
    return [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rows
            if rx.search(r["Kernel_Name"])]


def counter_values(pmc_dir: str, counter: str, pattern: str):
    rows = _csv(pmc_dir, "counter_collection.csv")
    rx = re.compile(pattern)
    return [float(r["Counter_Value"]) for r in rows
            if r["Counter_Name"] == counter and rx.search(r["Kernel_Name"])]


def stats_table(trace_dir: str, top: int = 12):
    rows = _csv(trace_dir, "kernel_stats.csv")
    out = []
    for r in rows[:top]:
        out.append(f"  {r['Name'][:78]:78s} calls={r['Calls']:>5s} "
                   f"avg_us={float(r['AverageNs']) / 1e3:10.2f} pct={float(r['Percentage']):6.2f}")
    return out


def summarize(a):
    dur = kernel_durations(a.trace, a.kernel)
    fetch = counter_values(a.fetch, "FETCH_SIZE", a.kernel)
    write = counter_values(a.write, "WRITE_SIZE", a.kernel)
    cf = counter_values(a.copy_fetch, "FETCH_SIZE", "copyBuffer")
    cw = counter_values(a.copy_write, "WRITE_SIZE", "copyBuffer")
    copy_kib = a.copy_mib * 1024.0
    fetch_scale = copy_kib / statistics.mean(cf)
    write_scale = copy_kib / statistics.mean(cw)
    f_kib, w_kib = statistics.mean(fetch), statistics.mean(write)
    traffic = (f_kib * fetch_scale + w_kib * write_scale) * 1024.0
    lines = [
        f"# rocprofv3 summary: kernel /{a.kernel}/ on workload {a.workload}",
        f"# commands (from the repository root):",
        *[f"#   {c}" for c in a.command],
        f"# summarised by: python -m mixture_experts_ffn_softplus_amd.profiling summarize ...",
        f"source_sha256: {source_hash()}",
        f"workload: {a.workload}",
        f"kernel_regex: {a.kernel}",
        f"dispatches_traced: {len(dur)}",
        f"kernel_avg_us: {statistics.mean(dur):.2f}",
        f"kernel_median_us: {statistics.median(dur):.2f}",
        f"kernel_min_us: {min(dur):.2f}",
        f"FETCH_SIZE_KiB_per_dispatch: {f_kib:.1f}",
        f"WRITE_SIZE_KiB_per_dispatch: {w_kib:.1f}",
        f"copy_calibration_MiB: {a.copy_mib}",
        f"copy_FETCH_SIZE_KiB: {statistics.mean(cf):.1f}",
        f"copy_WRITE_SIZE_KiB: {statistics.mean(cw):.1f}",
        f"fetch_scale: {fetch_scale:.4f}",
        f"write_scale: {write_scale:.4f}",
        f"traffic_bytes_per_launch: {traffic:.0f}",
        "top kernels by total time (kernel-trace --stats):",
        *stats_table(a.trace),
    ]
    with open(a.out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def durations(a):
    """Kernel-trace durations of each kernel pattern (no counters): small kernels whose time,
    not their traffic, is the figure of interest."""
    lines = [
        f"# rocprofv3 kernel durations on workload {a.workload}",
        f"# commands (from the repository root):",
        *[f"#   {c}" for c in a.command],
        f"# summarised by: python -m mixture_experts_ffn_softplus_amd.profiling durations ...",
        f"workload: {a.workload}",
    ]
    for name, pattern in (kv.split("=", 1) for kv in a.kernel):
        dur = kernel_durations(a.trace, pattern)
        lines += [f"{name}_regex: {pattern}", f"{name}_dispatches: {len(dur)}",
                  f"{name}_avg_us: {statistics.mean(dur):.2f}",
                  f"{name}_median_us: {statistics.median(dur):.2f}",
                  f"{name}_min_us: {min(dur):.2f}"]
    lines += ["top kernels by total time (kernel-trace --stats):", *stats_table(a.trace)]
    with open(a.out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def counters(a):
    """One counter (a plain or derived rocprofv3 counter, e.g. MfmaUtil) per kernel pattern:
    its mean, median and minimum over the dispatches of a --pmc run."""
    lines = [
        f"# rocprofv3 counter {a.counter} on workload {a.workload}",
        f"# commands (from the repository root):",
        *[f"#   {c}" for c in a.command],
        f"# summarised by: python -m mixture_experts_ffn_softplus_amd.profiling counters ...",
        f"source_sha256: {source_hash()}",
        f"workload: {a.workload}",
        f"counter: {a.counter}",
    ]
    for name, pattern in (kv.split("=", 1) for kv in a.kernel):
        v = counter_values(a.pmc, a.counter, pattern)
        lines += [f"{name}_regex: {pattern}", f"{name}_dispatches: {len(v)}",
                  f"{name}_mean: {statistics.mean(v):.3f}",
                  f"{name}_median: {statistics.median(v):.3f}",
                  f"{name}_min: {min(v):.3f}"]
    with open(a.out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def read_summary(path: str) -> dict:
    """key: value lines of a summary file (comments and tables skipped)."""
    out = {}
    with open(path) as fh:
        for ln in fh:
            if ln.startswith("#") or ln.startswith(" ") or ":" not in ln:
                continue
            k, v = ln.split(":", 1)
            out[k.strip()] = v.strip()
    return out


def traffic_if_current(path: str):
    """The summary's traffic bytes per launch, or None if the file is missing or the kernel
    sources changed since it was measured."""
    if not os.path.exists(path):
        return None
    s = read_summary(path)
    if s.get("source_sha256") != source_hash():
        return None
    return float(s["traffic_bytes_per_launch"])


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    p = sub.add_parser("summarize")
    for k in ("trace", "fetch", "write", "copy_fetch", "copy_write", "kernel", "workload", "out"):
        p.add_argument("--" + k.replace("_", "-"), dest=k, required=True)
    p.add_argument("--copy-mib", dest="copy_mib", type=int, default=1024)
    p.add_argument("--command", action="append", default=[])
    d = sub.add_parser("durations")
    for k in ("trace", "workload", "out"):
        d.add_argument("--" + k, dest=k, required=True)
    d.add_argument("--kernel", action="append", default=[], metavar="NAME=REGEX")
    d.add_argument("--command", action="append", default=[])
    c = sub.add_parser("counters")
    for k in ("pmc", "counter", "workload", "out"):
        c.add_argument("--" + k, dest=k, required=True)
    c.add_argument("--kernel", action="append", default=[], metavar="NAME=REGEX")
    c.add_argument("--command", action="append", default=[])
    sub.add_parser("hash")
    a = ap.parse_args()
    if a.cmd == "hash":
        print(source_hash())
    elif a.cmd == "durations":
        durations(a)
    elif a.cmd == "counters":
        counters(a)
    else:
        summarize(a)


if __name__ == "__main__":
    main()
