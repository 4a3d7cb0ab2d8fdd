"""Summaries of rocprofv3 output for the measurement records kept in profiles/.

    python -m decoder_only_pretraining_amd.profiling stats KERNEL_STATS_CSV \
        --title TITLE --command CMD --steps K [--top 30] --out FILE
    python -m decoder_only_pretraining_amd.profiling pmc \
        --fetch FETCH_CSV --write WRITE_CSV --copy-fetch CSV --copy-write CSV \
        --copy-bytes BYTES --kernel SUBSTRING --command CMD --out FILE

`stats` turns a `rocprofv3 --kernel-trace --stats --output-format csv`
kernel_stats.csv into a per-kernel table (total, share, calls, average).
    python -m decoder_only_pretraining_amd.profiling counters PASS_CSV [PASS_CSV ...] \
        --stats KERNEL_STATS_CSV --title TITLE --command CMD --out FILE

`counters` sums the SQ counters of each kernel group of the d12 call over
its dispatches (one counter_collection.csv per rocprofv3 --pmc pass) and
prints them with their share of the wave cycles and the instructions of
each kind per MFMA instruction.
`pmc` averages FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of the kernels
whose name contains SUBSTRING, calibrates both counters with a plain device
copy of known size, and records the HBM bytes per launch together with a
hash of the GEMM sources, so a later change of the kernel invalidates the
figure (see `traffic_for`).
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import os

PKG = os.path.dirname(os.path.abspath(__file__))
GEMM_SOURCES = [os.path.join(PKG, "csrc", f) for f in ("gemm_core.h", "gemm.hip")]


def source_hash(paths=GEMM_SOURCES) -> str:
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def _short(name: str, n: int = 120) -> str:
    name = name.replace("void gk::", "").replace("gk::", "")
    cut = name.find("(")
    if cut > 0:
        name = name[:cut]
    return name[:n]


def stats_table(path: str, steps: int, top: int = 30):
    rows = list(csv.DictReader(open(path)))
    total = sum(float(r["TotalDurationNs"]) for r in rows)
    lines = [f"{'ms/step':>9} {'share':>6} {'calls/step':>10} {'avg us':>9}  kernel"]
    for r in rows[:top]:
        t = float(r["TotalDurationNs"])
        lines.append(f"{t / steps / 1e6:9.3f} {100 * t / total:5.1f}% "
                     f"{int(r['Calls']) / steps:10.1f} {float(r['AverageNs']) / 1e3:9.1f}  "
                     f"{_short(r['Name'])}")
    lines.append(f"{total / steps / 1e6:9.3f} total kernel time per step ({len(rows)} kernels)")
    return lines


def _counter_avg(path: str, counter: str, kernel_substr: str | None):
    """Average per dispatch of `counter` over dispatches whose kernel name
    contains `kernel_substr` (None: the dispatch with the largest value)."""
    vals, best = [], None
    for r in csv.DictReader(open(path)):
        if r.get("Counter_Name") != counter:
            continue
        v = float(r["Counter_Value"])
        name = r.get("Kernel_Name", "")
        if kernel_substr is None:
            if best is None or v > best[0]:
                best = (v, name)
        elif kernel_substr in name:
            vals.append(v)
    if kernel_substr is None:
        return best
    return (sum(vals) / len(vals) if vals else float("nan"), len(vals))


def traffic_for(summary_path: str):
    """HBM bytes per launch recorded in a pmc summary, or None if the file
    is missing or the GEMM sources changed since the counters were taken."""
    if not os.path.exists(summary_path):
        return None
    kv = {}
    for line in open(summary_path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_sha256") != source_hash():
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# Kernel groups of the d12 call: (label, substrings of which one must occur
# in the kernel name, substrings none of which may occur).
COUNTER_GROUPS = [
    ("attn_fwd (window layers: 128-query tiles)", ["attn_fwd_tiled_kernel<128, true, 128"], []),
    ("attn_fwd (full layers: 256-query tiles)", ["attn_fwd_tiled_kernel<128, true, 256"], []),
    ("attn_bwd_pair (dK/dV + dQ)", ["attn_bwd_pair_kernel"], []),
    ("gemm weight gradients, token-major K-major kernel", ["EpPart, 0, gk::NoDeq, true>",
                                                           "EpPart, 0, NoDeq, true>"], []),
    ("gemm lm_head weight gradient, token-major", ["EpF32, 0, gk::NoDeq, true>",
                                                   "EpF32, 0, NoDeq, true>"], []),
    ("gemm_kmaj EpStore", ["EpStore"], []),
    ("gemm_kmaj EpResid", ["EpResid"], []),
    ("gemm_kmaj EpF32", ["EpF32, 0, gk::NoDeq, false>", "EpF32, 0, NoDeq, false>"], []),
    ("gemm_kmaj EpRelu2", ["EpRelu2I", "EpRelu2<"], ["Bwd"]),
    ("gemm_kmaj EpRelu2Bwd", ["EpRelu2Bwd"], []),
    ("gemm_kmaj EpSoftcap", ["EpSoftcap"], []),
    ("norm_bwd", ["norm_bwd_kernel"], []),
    ("mix_norm", ["mix_norm_kernel"], []),
]
_CYCLE_SHARE = ("SQ_ACTIVE_INST_", "SQ_WAIT_", "SQ_BUSY_CYCLES")


def counter_table(pass_csvs, stats_csv, groups=COUNTER_GROUPS):
    """Per kernel group: counter sums over its dispatches, their share of
    SQ_WAVE_CYCLES, and instructions per MFMA."""
    def member(name, inc, exc):
        return any(i in name for i in inc) and not any(e in name for e in exc)

    avg = {}
    for r in csv.DictReader(open(stats_csv)):
        for label, inc, exc in groups:
            if member(r["Name"], inc, exc):
                n, t = avg.get(label, (0, 0.0))
                avg[label] = (n + int(r["Calls"]), t + float(r["TotalDurationNs"]))
    sums = {label: {} for label, _, _ in groups}
    disp = {label: 0 for label, _, _ in groups}  # dispatches per pass (the most of any pass)
    for path in pass_csvs:
        seen = {label: set() for label, _, _ in groups}
        for r in csv.DictReader(open(path)):
            for label, inc, exc in groups:
                if member(r["Kernel_Name"], inc, exc):
                    c = r["Counter_Name"]
                    sums[label][c] = sums[label].get(c, 0.0) + float(r["Counter_Value"])
                    seen[label].add(r["Dispatch_Id"])
        for label in seen:
            disp[label] = max(disp[label], len(seen[label]))
    lines = []
    for label, _, _ in groups:
        c = sums[label]
        if not c:
            continue
        n, t = avg.get(label, (0, 0.0))
        per = t / n / 1e3 if n else float("nan")
        lines.append(f"== {label}: {disp[label]} dispatches, {per:.1f} us avg")
        wc = c.get("SQ_WAVE_CYCLES", 0.0)
        for k in sorted(c):
            share = (f"  ({100 * c[k] / wc:5.1f}% of wave cycles)"
                     if wc and k.startswith(_CYCLE_SHARE) else "")
            lines.append(f"   {k:<36} {c[k]:>16.0f}{share}")
        mf = c.get("SQ_INSTS_MFMA", 0.0)
        if mf:
            def pm(k):
                return c.get(k, 0.0) / mf
            busy = c.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0)
            co = c.get("SQ_VALU_MFMA_COEXEC_CYCLES", 0.0) / busy if busy else float("nan")
            lines.append(f"   per MFMA: VALU {pm('SQ_INSTS_VALU'):.2f}  SALU {pm('SQ_INSTS_SALU'):.2f}  "
                         f"LDS {pm('SQ_INSTS_LDS'):.2f}  VMEM {pm('SQ_INSTS_VMEM_RD'):.2f}  "
                         f"trans {pm('SQ_INSTS_VALU_TRANS_F32'):.2f};  co-issue {co:.3f};  "
                         f"MFMA-busy cycles per MFMA {busy / mf:.1f}")
        lines.append("")
    return lines


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("--title", required=True)
    s.add_argument("--command", required=True)
    s.add_argument("--steps", type=int, required=True)
    s.add_argument("--top", type=int, default=30)
    s.add_argument("--out", required=True)
    p = sub.add_parser("pmc")
    for a in ("--fetch", "--write", "--copy-fetch", "--copy-write", "--kernel", "--command",
              "--out", "--title"):
        p.add_argument(a, required=True)
    p.add_argument("--copy-bytes", type=float, required=True)
    c = sub.add_parser("counters")
    c.add_argument("csvs", nargs="+")
    for a in ("--stats", "--title", "--command", "--out"):
        c.add_argument(a, required=True)
    args = ap.parse_args()
    if args.cmd == "counters":
        lines = [f"# {args.title}"] + [f"# {l}" for l in args.command.split("\n")] + [""]
        lines += counter_table(args.csvs, args.stats)
        open(args.out, "w").write("\n".join(lines) + "\n")
        return
    if args.cmd == "stats":
        lines = [f"# {args.title}", f"# command: {args.command}",
                 f"# per step = totals / {args.steps} profiled steps (warmup included)", ""]
        lines += stats_table(args.csv, args.steps, args.top)
        open(args.out, "w").write("\n".join(lines) + "\n")
    else:
        f_avg, f_n = _counter_avg(args.fetch, "FETCH_SIZE", args.kernel)
        w_avg, w_n = _counter_avg(args.write, "WRITE_SIZE", args.kernel)
        cf, cf_name = _counter_avg(args.copy_fetch, "FETCH_SIZE", None)
        cw, cw_name = _counter_avg(args.copy_write, "WRITE_SIZE", None)
        fs = args.copy_bytes / (cf * 1024.0)
        ws = args.copy_bytes / (cw * 1024.0)
        traffic = f_avg * 1024.0 * fs + w_avg * 1024.0 * ws
        lines = [f"# {args.title}",
                 f"# command: {args.command}",
                 f"kernel: {args.kernel}",
                 f"source_sha256: {source_hash()}",
                 f"FETCH_SIZE_kib_per_dispatch: {f_avg:.1f} (over {f_n} dispatches)",
                 f"WRITE_SIZE_kib_per_dispatch: {w_avg:.1f} (over {w_n} dispatches)",
                 f"copy_bytes: {args.copy_bytes:.0f}",
                 f"copy_FETCH_SIZE_kib: {cf:.1f} ({_short(cf_name, 60)})",
                 f"copy_WRITE_SIZE_kib: {cw:.1f} ({_short(cw_name, 60)})",
                 f"fetch_scale: {fs:.4f}",
                 f"write_scale: {ws:.4f}",
                 f"traffic_bytes_per_launch: {traffic:.0f}"]
        open(args.out, "w").write("\n".join(lines) + "\n")


if __name__ == "__main__":
    main()
