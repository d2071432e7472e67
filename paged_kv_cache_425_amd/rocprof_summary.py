"""Summaries of rocprofv3 result databases (the rocpd SQLite files).

    python -m paged_kv_cache_425_amd.rocprof_summary trace RESULTS.db --command CMD --out OUT.md
    python -m paged_kv_cache_425_amd.rocprof_summary traffic --fetch F.db --write W.db \
        --kernel paged_decode_kernel --copy-bytes N --algorithmic-bytes A --workload NAME \
        --command-fetch CMD --command-write CMD --out OUT.md --out-json OUT.json

``trace`` tabulates kernel durations (count, mean, median, min, max).

``counters`` tabulates the per-dispatch value of every counter of one or more
``--pmc`` runs for one kernel (median over a window of its launches) and, when
SQ_VALU_MFMA_BUSY_CYCLES and GRBM_GUI_ACTIVE were both collected, the MFMA
utilisation: busy cycles summed over all SIMDs / (GUI-active cycles of one XCD x
256 CUs x 4 SIMDs).

``traffic`` turns the FETCH_SIZE / WRITE_SIZE counters (KiB per dispatch)
into HBM bytes per launch of one kernel.  Each counter is scaled by what it
reads for a plain device copy of known size recorded in the same run: the
largest ``__amd_rocclr_copyBuffer`` dispatches (the copies that clone the K/V
pools) move ``--copy-bytes`` bytes each way, so the scale factor of a counter
is copy_bytes / (its reading x 1024).  The JSON record carries the SHA-256 of
the kernel source the counters were taken on (comments and whitespace
removed), so a later change to the kernel's code makes the benchmark drop
the figure.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sqlite3
import statistics

HERE = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCE = os.path.join(HERE, "csrc", "paged_attention.hip")
COPY_KERNEL = "__amd_rocclr_copyBuffer"


def kernel_source_digest(path: str = KERNEL_SOURCE) -> str:
    """SHA-256 of a kernel source with its comments and whitespace removed: it changes
    when the code changes, not when a comment does."""
    with open(path) as fh:
        text = fh.read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)       # block comments
    text = re.sub(r"//[^\n]*", " ", text)                     # line comments
    text = re.sub(r"\s+", " ", text).strip()
    return hashlib.sha256(text.encode()).hexdigest()


def short(name: str) -> str:
    """Kernel name without its parameter list."""
    return name.split("(")[0].replace("void ", "")


def counter_values(db: str, counter: str) -> list:
    """(kernel name, dispatch id, summed counter value) per dispatch."""
    con = sqlite3.connect(db)
    rows = con.execute("select name, dispatch_id, sum(counter_value) from pmc_events "
                       "where counter_name = ? group by dispatch_id order by dispatch_id",
                       (counter,))
    return [(n, d, float(v)) for n, d, v in rows]


def kernel_durations_ordered(db: str) -> dict:
    con = sqlite3.connect(db)
    out: dict = {}
    for name, dur in con.execute("select name, duration from kernels order by start"):
        out.setdefault(name, []).append(dur / 1000.0)
    return out


def trace_table(db: str, last: int = 0, slices: list | None = None) -> str:
    durs = kernel_durations_ordered(db)
    lines = ["| kernel | launches | mean us | median us | min us | max us |",
             "|---|---|---|---|---|---|"]
    for name, ds in sorted(durs.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"| `{short(name)}` | {len(ds)} | {statistics.fmean(ds):.2f} | "
                     f"{statistics.median(ds):.2f} | {min(ds):.2f} | {max(ds):.2f} |")
    if last:
        lines += ["", f"The last {last} launches of each kernel launched at least {last} times "
                  "(the benchmark's timed steps):", "",
                  "| kernel | launches | mean us | median us | min us | max us |",
                  "|---|---|---|---|---|---|"]
        for name, ds in sorted(durs.items(), key=lambda kv: -sum(kv[1])):
            if len(ds) < last:
                continue
            d = ds[-last:]
            lines.append(f"| `{short(name)}` | {len(d)} | {statistics.fmean(d):.2f} | "
                         f"{statistics.median(d):.2f} | {min(d):.2f} | {max(d):.2f} |")
    for spec in slices or []:
        # KERNEL_SUBSTRING:START:COUNT:LABEL -- launches START .. START+COUNT-1 of that kernel
        sub, start, count, label = spec.split(":", 3)
        start, count = int(start), int(count)
        for name, ds in durs.items():
            if sub not in name:
                continue
            d = ds[start:start + count]
            if not d:
                continue
            lines += ["", f"{label}: launches {start}..{start + len(d) - 1} of `{short(name)}`:", "",
                      "| launches | mean us | median us | min us | max us |", "|---|---|---|---|---|",
                      f"| {len(d)} | {statistics.fmean(d):.2f} | {statistics.median(d):.2f} | "
                      f"{min(d):.2f} | {max(d):.2f} |"]
    return "\n".join(lines)


N_CU = 256
SIMD_PER_CU = 4


def dispatch_counters(db: str, kernel: str) -> dict:
    """counter -> list over the kernel's dispatches (in order) of (sum, instances)."""
    con = sqlite3.connect(db)
    out: dict = {}
    for cname, _d, total, inst in con.execute(
            "select counter_name, dispatch_id, sum(counter_value), count(*) from pmc_events "
            "where name like ? group by dispatch_id, counter_name order by dispatch_id",
            (f"%{kernel}%",)):
        out.setdefault(cname, []).append((float(total), int(inst)))
    return out


def counters_table(dbs: list, kernel: str, start: int, count: int) -> tuple:
    merged: dict = {}
    for db in dbs:
        for cname, vals in dispatch_counters(db, kernel).items():
            end = start + count if count else None
            merged[cname] = vals[start:end]
    if not merged:
        raise SystemExit(f"kernel {kernel} not found in the counter runs")
    lines = ["| counter | dispatches | instances | median per dispatch (sum over instances) |",
             "|---|---|---|---|"]
    med = {}
    for cname in sorted(merged):
        vals = merged[cname]
        med[cname] = (statistics.median(v for v, _ in vals), vals[0][1])
        lines.append(f"| {cname} | {len(vals)} | {vals[0][1]} | {med[cname][0]:,.0f} |")
    derived = {}
    if "SQ_VALU_MFMA_BUSY_CYCLES" in med and "GRBM_GUI_ACTIVE" in med:
        gui, inst = med["GRBM_GUI_ACTIVE"]
        per_xcd = gui / inst
        derived["mfma_util"] = med["SQ_VALU_MFMA_BUSY_CYCLES"][0] / (per_xcd * N_CU * SIMD_PER_CU)
        lines += ["", f"MFMA utilisation = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / {inst} "
                  f"x {N_CU} CUs x {SIMD_PER_CU} SIMDs) = {derived['mfma_util']:.3f}"]
    return "\n".join(lines), derived


def copy_factor(rows: list, copy_bytes: int) -> tuple:
    """Scale factor from the largest copy dispatches (those within 5% of the largest)."""
    vals = [v for n, _, v in rows if n.startswith(COPY_KERNEL)]
    if not vals:
        raise SystemExit("no copy dispatch in the counter run to calibrate against")
    top = max(vals)
    sel = [v for v in vals if v >= 0.95 * top]
    reading = statistics.median(sel)
    return copy_bytes / (reading * 1024.0), reading, len(sel)


def kernel_counter(rows: list, kernel: str) -> list:
    return [v for n, _, v in rows if kernel in n]


def main() -> None:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("db")
    t.add_argument("--command", required=True)
    t.add_argument("--title", default="Kernel trace")
    t.add_argument("--last", type=int, default=0,
                   help="also tabulate the last N launches of each kernel")
    t.add_argument("--slice", action="append", default=[],
                   help="KERNEL_SUBSTRING:START:COUNT:LABEL, stats of a window of launches")
    t.add_argument("--out", required=True)
    c = sub.add_parser("counters")
    c.add_argument("dbs", nargs="+")
    c.add_argument("--kernel", required=True)
    c.add_argument("--title", required=True)
    c.add_argument("--command", action="append", required=True,
                   help="the command of each run, in the order of the databases")
    c.add_argument("--start", type=int, default=0)
    c.add_argument("--count", type=int, default=0)
    c.add_argument("--out", required=True)
    f = sub.add_parser("traffic")
    f.add_argument("--fetch", required=True)
    f.add_argument("--write", required=True)
    f.add_argument("--kernel", required=True,
                   help="substring of the kernel's name that selects its dispatches")
    f.add_argument("--label", default="",
                   help="name of the kernel in the summary (default: --kernel)")
    f.add_argument("--copy-bytes", type=int, required=True)
    f.add_argument("--algorithmic-bytes", type=int, required=True)
    f.add_argument("--workload", required=True)
    f.add_argument("--command-fetch", required=True)
    f.add_argument("--command-write", required=True)
    f.add_argument("--start", type=int, default=0, help="first launch of the kernel to use")
    f.add_argument("--count", type=int, default=0, help="launches to use (0: all from start)")
    f.add_argument("--out", required=True)
    f.add_argument("--out-json", required=True)
    a = ap.parse_args()

    if a.cmd == "trace":
        text = (f"# {a.title}\n\nCommand (from the repository root on the GPU box):\n\n"
                f"```\n{a.command}\n```\n\n{trace_table(a.db, a.last, a.slice)}\n")
        with open(a.out, "w") as fh:
            fh.write(text)
        print(text)
        return

    if a.cmd == "counters":
        table, _ = counters_table(a.dbs, a.kernel, a.start, a.count)
        cmds = "\n".join(a.command)
        end = f"{a.start + a.count - 1}" if a.count else "last"
        text = (f"# {a.title}\n\nCommands (from the repository root on the GPU box), one "
                f"counter set per run:\n\n```\n{cmds}\n```\n\nKernel `{a.kernel}`, launches "
                f"{a.start}..{end} of each run.\n\n{table}\n")
        with open(a.out, "w") as fh:
            fh.write(text)
        print(text)
        return

    fr = counter_values(a.fetch, "FETCH_SIZE")
    wr = counter_values(a.write, "WRITE_SIZE")
    ff, fread, fn = copy_factor(fr, a.copy_bytes)
    wf, wread, wn = copy_factor(wr, a.copy_bytes)
    end = a.start + a.count if a.count else None
    fk = kernel_counter(fr, a.kernel)[a.start:end]
    wk = kernel_counter(wr, a.kernel)[a.start:end]
    if not fk or not wk:
        raise SystemExit(f"kernel {a.kernel} not found in the counter runs")
    fetch_b = statistics.median(fk) * 1024.0 * ff
    write_b = statistics.median(wk) * 1024.0 * wf
    total = fetch_b + write_b
    sha = kernel_source_digest()
    rec = {"workload": a.workload, "kernel": a.kernel, "bytes_per_launch": int(round(total)),
           "fetch_bytes_per_launch": int(round(fetch_b)),
           "write_bytes_per_launch": int(round(write_b)),
           "algorithmic_bytes_per_launch": a.algorithmic_bytes,
           "fetch_scale": ff, "write_scale": wf, "source_sha256": sha}
    with open(a.out_json, "w") as fh:
        json.dump(rec, fh, indent=1)
        fh.write("\n")
    label = a.label or a.kernel
    text = f"""# HBM traffic of `{label}` ({a.workload})

Commands (from the repository root on the GPU box), one counter per run:

```
{a.command_fetch}
{a.command_write}
```

Calibration: the largest `{COPY_KERNEL}` dispatches of the same runs clone the
K/V pools, {a.copy_bytes} bytes each.  FETCH_SIZE reads {fread:.1f} KiB for them
(median of {fn}), so its scale is {ff:.4f}; WRITE_SIZE reads {wread:.1f} KiB
(median of {wn}), scale {wf:.4f}.

| per launch of `{label}` | bytes |
|---|---|
| FETCH_SIZE x scale (median of launches {a.start}..{a.start + len(fk) - 1}) | {fetch_b:,.0f} |
| WRITE_SIZE x scale (median of launches {a.start}..{a.start + len(wk) - 1}) | {write_b:,.0f} |
| measured HBM traffic | {total:,.0f} |
| algorithmic bytes per launch | {a.algorithmic_bytes:,} |
| measured / algorithmic | {total / a.algorithmic_bytes:.4f} |

Kernel source SHA-256 (comments and whitespace removed): `{sha}`.
"""
    with open(a.out, "w") as fh:
        fh.write(text)
    print(text)


if __name__ == "__main__":
    main()
