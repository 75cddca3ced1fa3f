"""Summaries of rocprofv3 output for the measurement records.

    python -m gpt_pretraining_step_amd.profiling stats <kernel_stats.csv> --command "<cmd>" [--title T]
    python -m gpt_pretraining_step_amd.profiling traffic <fetch_dir> <write_dir> --site S --copy-bytes N
        --command-fetch "<cmd>" --command-write "<cmd>"

`stats` turns a `rocprofv3 --kernel-trace --stats` kernel-statistics CSV
into a Markdown table.  `counters` joins a per-dispatch kernel trace and
any number of per-dispatch counter runs of the same program (`bench.py
--counter-probe`: one micro-step, one optimizer step, then the marker and a
calibration copy) dispatch by dispatch, and tabulates per kernel and grid:
duration, MfmaUtil and VALUBusy, HBM bytes from FETCH_SIZE / WRITE_SIZE
scaled by the copy's readings, and the resulting GB/s.  `traffic` reads two per-dispatch counter runs
(`--pmc FETCH_SIZE`, then `--pmc WRITE_SIZE`) of `bench.py --traffic-probe`:
in those runs the library launches its empty marker kernel before every
launch of the probed site, and once more before a plain device copy of
`copy_bytes` bytes read and as many written.  The dispatch after each marker
is attributed to the site; the copy's readings calibrate the counters (bytes
expected / KiB counted).  The result is a Markdown record whose `traffic:`
line holds the per-launch HBM bytes and a hash of the kernel's sources, so
that a reader can tell when the kernel has changed since.

Pure CSV parsing: no GPU, no library import.
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
MARKER = "site_marker_kernel"

# Sources that define the kernels of a launch site (by site-name prefix).
SITE_SOURCES = {
    "gemm.": ["gemm_kernel.h", "gemm.hip", "tile_io.h", "common.h"],
    "attn.": ["attention.hip", "tile_io.h", "common.h"],
    "ln.": ["layernorm.hip", "common.h"],
    "ce.": ["ce.hip", "common.h"],
}


def site_sources_hash(site: str) -> str | None:
    for pre, files in SITE_SOURCES.items():
        if site.startswith(pre):
            h = hashlib.sha256()
            for f in files:
                with open(os.path.join(CSRC, f), "rb") as fh:
                    h.update(f.encode() + b"\0" + fh.read())
            return h.hexdigest()[:16]
    return None


def _rows(path_or_dir: str, suffix: str):
    path = path_or_dir
    if os.path.isdir(path_or_dir):
        cands = sorted(glob.glob(os.path.join(path_or_dir, "**", "*" + suffix), recursive=True))
        if not cands:
            raise FileNotFoundError(f"no *{suffix} under {path_or_dir}")
        path = cands[0]
    with open(path, newline="") as fh:
        return list(csv.DictReader(fh))


# ----------------------------------------------------------------- stats

def stats_markdown(csv_path: str, command: str, title: str, top: int = 30) -> str:
    rows = _rows(csv_path, "kernel_stats.csv")
    total = sum(float(r["TotalDurationNs"]) for r in rows)
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    out = [f"# {title}", "", "Command (from the repository root, on one MI355X):", "", "    " + command, "",
           "Durations from the kernel trace; average in microseconds.", "",
           "| kernel | calls | total ms | avg us | % |", "|---|---|---|---|---|"]
    for r in rows[:top]:
        name = r["Name"].replace("|", "\\|")
        if len(name) > 150:
            name = name[:147] + "..."
        tot = float(r["TotalDurationNs"])
        out.append(f"| `{name}` | {r['Calls']} | {tot / 1e6:.1f} | {float(r['AverageNs']) / 1e3:.2f} | "
                   f"{100 * tot / total:.2f} |")
    out.append(f"| (all {len(rows)} kernels) | | {total / 1e6:.1f} | | 100 |")
    return "\n".join(out) + "\n"


# --------------------------------------------------------------- traffic

def _per_dispatch(rows, counter: str):
    """{dispatch_id: (kernel_name, value)} for one counter."""
    out = {}
    for r in rows:
        if r["Counter_Name"] != counter:
            continue
        d = int(r["Dispatch_Id"])
        name, v = r["Kernel_Name"], float(r["Counter_Value"])
        if d in out:  # one row per dimension instance: sum them
            out[d] = (name, out[d][1] + v)
        else:
            out[d] = (name, v)
    return out


def attribute(rows, counter: str):
    """(site kernel name, per-launch values of the site, copy value)."""
    per = _per_dispatch(rows, counter)
    ids = sorted(per)
    follow = [ids[i + 1] for i, d in enumerate(ids[:-1]) if MARKER in per[d][0]]
    if len(follow) < 2:
        raise ValueError(f"{counter}: fewer than two marked dispatches")
    site_ids, copy_id = follow[:-1], follow[-1]
    names = {per[d][0] for d in site_ids}
    if len(names) != 1:
        raise ValueError(f"{counter}: marked dispatches run different kernels: {sorted(names)}")
    return names.pop(), [per[d][1] for d in site_ids], per[copy_id][1]


def traffic_record(fetch_dir: str, write_dir: str, site: str, copy_bytes: int, cmd_f: str, cmd_w: str,
                   workload: str = "gpt2") -> str:
    kf, fetch, copy_f = attribute(_rows(fetch_dir, "counter_collection.csv"), "FETCH_SIZE")
    kw, write, copy_w = attribute(_rows(write_dir, "counter_collection.csv"), "WRITE_SIZE")
    if kf != kw:
        raise ValueError(f"different kernels in the two runs: {kf} / {kw}")
    scale_f = copy_bytes / 1024.0 / copy_f
    scale_w = copy_bytes / 1024.0 / copy_w
    f_kib = sum(fetch) / len(fetch)
    w_kib = sum(write) / len(write)
    tb = f_kib * 1024 * scale_f + w_kib * 1024 * scale_w
    rec = {"site": site, "kernel": kf, "bytes_per_launch": round(tb), "fetch_kib": round(f_kib, 1),
           "write_kib": round(w_kib, 1), "fetch_scale": round(scale_f, 4), "write_scale": round(scale_w, 4),
           "launches": len(fetch), "sources_sha256_16": site_sources_hash(site), "workload": workload}
    lines = [f"# HBM traffic per launch: {site}" + ("" if workload == "gpt2" else f" ({workload} workload)"), "",
             f"Kernel: `{kf}`", "",
             "Commands (from the repository root, on one MI355X):", "",
             "    " + cmd_f, "    " + cmd_w, "",
             f"Per launch ({len(fetch)} launches of one micro-step): FETCH_SIZE {f_kib:.1f} KiB, "
             f"WRITE_SIZE {w_kib:.1f} KiB.",
             f"Calibration: a device copy of {copy_bytes} bytes read as FETCH_SIZE {copy_f:.1f} KiB and "
             f"WRITE_SIZE {copy_w:.1f} KiB, so the readings are scaled by {scale_f:.4f} and {scale_w:.4f}.",
             f"HBM bytes per launch: {tb / 1e6:.1f} MB.", "",
             "traffic: " + json.dumps(rec), ""]
    return "\n".join(lines)


def load_traffic(profiles_dir: str, site: str, workload: str = "gpt2"):
    """Bytes per launch recorded for `site` of `workload` (records without a
    workload are the GPT-2 micro-step's), or None when there is no record or
    the site's kernel sources have changed since it was taken."""
    for path in sorted(glob.glob(os.path.join(profiles_dir, "*.md"))):
        with open(path) as fh:
            for line in fh:
                if not line.startswith("traffic: "):
                    continue
                try:
                    rec = json.loads(line[len("traffic: "):])
                except json.JSONDecodeError:
                    continue
                if (rec.get("site") == site and rec.get("workload", "gpt2") == workload
                        and rec.get("sources_sha256_16") == site_sources_hash(site)):
                    return int(rec["bytes_per_launch"])
    return None


# -------------------------------------------------------------- counters

def _grid(r):
    for k in ("Grid_Size", "Grid_Size_X", "grid_size"):
        if k in r and r[k] not in (None, ""):
            return r[k]
    return ""


def _dispatches(rows, counters=True):
    """Per-dispatch records in dispatch order: (kernel, grid, {counter: value})
    for a counter run, (kernel, grid, duration ns) for a kernel trace."""
    out = {}
    for r in rows:
        d = int(r.get("Dispatch_Id") or r.get("Correlation_Id"))
        if counters:
            rec = out.setdefault(d, [r["Kernel_Name"], _grid(r), {}])
            rec[2][r["Counter_Name"]] = rec[2].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        else:
            out[d] = [r["Kernel_Name"], _grid(r), float(r["End_Timestamp"]) - float(r["Start_Timestamp"])]
    return [out[k] for k in sorted(out)]


def counters_markdown(trace_dir: str, pmc_dirs, copy_bytes: int, command: str, title: str) -> str:
    trace = _dispatches(_rows(trace_dir, "kernel_trace.csv"), counters=False)
    runs = [_dispatches(_rows(d, "counter_collection.csv")) for d in pmc_dirs]
    for run in runs:
        if len(run) != len(trace) or any(a[0] != b[0] for a, b in zip(run, trace)):
            raise ValueError("the runs did not dispatch the same kernels in the same order")
    n = len(trace)
    vals = [{} for _ in range(n)]
    for run in runs:
        for i, (_, _, c) in enumerate(run):
            vals[i].update(c)
    marks = [i for i, t in enumerate(trace) if MARKER in t[0]]
    if not marks:
        raise ValueError("no marker before the calibration copy")
    last = marks[-1]
    # the copy may run as several dispatches: its readings are their sum
    cal = {}
    for i in range(last + 1, n):
        for c, v in vals[i].items():
            cal[c] = cal.get(c, 0.0) + v
    scale = {}
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        if c in cal and cal[c] > 0:
            scale[c] = copy_bytes / 1024.0 / cal[c]
    groups = {}
    for i in range(last):  # everything before the marker and the copy
        k, g, dur = trace[i]
        if MARKER in k:
            continue
        e = groups.setdefault((k, g), {"n": 0, "dur": 0.0, "c": {}})
        e["n"] += 1
        e["dur"] += dur
        for c, v in vals[i].items():
            e["c"][c] = e["c"].get(c, 0.0) + v
    cols = [c for c in ("MfmaUtil", "VALUBusy") if any(c in e["c"] for e in groups.values())]
    have_b = [c for c in ("FETCH_SIZE", "WRITE_SIZE") if c in scale]
    head = ["kernel", "grid", "calls", "avg us"] + [f"{c} %" for c in cols]
    if have_b:
        head += [f"{'read' if c == 'FETCH_SIZE' else 'written'} MB" for c in have_b] + ["HBM GB/s"]
    out = [f"# {title}", "", "Commands (from the repository root, on one MI355X):", ""]
    out += ["    " + line for line in command.split("\n")]
    out += ["", f"Calibration: a device copy of {copy_bytes} bytes read as "
            + ", ".join(f"{c} {cal.get(c, 0):.1f} KiB (scale {scale[c]:.4f})" for c in have_b) + ".", "",
            "| " + " | ".join(head) + " |", "|" + "---|" * len(head)]
    total = sum(e["dur"] for e in groups.values())
    for (k, g), e in sorted(groups.items(), key=lambda kv: -kv[1]["dur"]):
        name = k.replace("|", "\\|")
        if len(name) > 140:
            name = name[:137] + "..."
        avg = e["dur"] / e["n"]
        row = [f"`{name}`", str(g), str(e["n"]), f"{avg / 1e3:.2f}"]
        row += [f"{e['c'][c] / e['n']:.1f}" if c in e["c"] else "" for c in cols]
        if have_b:
            byts = [e["c"].get(c, 0.0) / e["n"] * 1024 * scale[c] for c in have_b]
            row += [f"{b / 1e6:.1f}" for b in byts] + [f"{sum(byts) / avg:.0f}"]
        out.append("| " + " | ".join(row) + " |")
    out.append(f"| (all) | | | {total / 1e3:.1f} total | |")
    return "\n".join(out) + "\n"


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("--command", required=True)
    s.add_argument("--title", default="Kernel time")
    t = sub.add_parser("traffic")
    t.add_argument("fetch_dir")
    t.add_argument("write_dir")
    t.add_argument("--site", required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--command-fetch", required=True)
    t.add_argument("--command-write", required=True)
    t.add_argument("--workload", default="gpt2")
    c = sub.add_parser("counters")
    c.add_argument("trace_dir")
    c.add_argument("pmc_dirs", nargs="+")
    c.add_argument("--copy-bytes", type=int, required=True)
    c.add_argument("--command", required=True, help="the commands, newline-separated")
    c.add_argument("--title", default="Per-kernel counters")
    a = ap.parse_args(argv)
    if a.cmd == "stats":
        sys.stdout.write(stats_markdown(a.csv, a.command, a.title))
    elif a.cmd == "counters":
        sys.stdout.write(counters_markdown(a.trace_dir, a.pmc_dirs, a.copy_bytes, a.command, a.title))
    else:
        sys.stdout.write(traffic_record(a.fetch_dir, a.write_dir, a.site, a.copy_bytes, a.command_fetch,
                                        a.command_write, a.workload))
    return 0


if __name__ == "__main__":
    sys.exit(main())
