"""Summaries of rocprofv3 output for the layer's kernels (CSV output of rocprofv3 --kernel-trace or --pmc).

    python -m mixture_experts_transformer_gemv_amd.rocprof_summary trace DIR [--split REGEX:US]
        per kernel and grid size: dispatches, average / min / max duration (us), share of GPU time (markdown);
        --split lists a kernel's dispatches up to and above a duration in two rows
    python -m mixture_experts_transformer_gemv_amd.rocprof_summary traffic --fetch DIR --write DIR --workload W
            --kernel REGEX [--kernel REGEX] --algorithmic-bytes B --source FILE... --out RECORD.json
        HBM-side bytes per launch of a projection (the sum over its kernels matched by the regexes): FETCH_SIZE and
        WRITE_SIZE in KiB per dispatch, each scaled so that the plain 1 GiB device copy of the same run reads 1 GiB
        and writes 1 GiB; the first dispatch of each kernel (warm-up) is excluded.
    python -m mixture_experts_transformer_gemv_amd.rocprof_summary counters DIR
        per kernel and grid size: the average of every counter per dispatch (markdown)
    python -m mixture_experts_transformer_gemv_amd.rocprof_summary busy DIR
        per kernel and grid size: clock and MFMA busy from GRBM_GUI_ACTIVE and SQ_VALU_MFMA_BUSY_CYCLES (markdown)

Only reads files that rocprofv3 wrote; no GPU work.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys
from collections import defaultdict

CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")
COPY_KERNEL = re.compile(r"copyBuffer|CopyBuffer|copy_kernel|elementwise_kernel.*copy", re.I)


def _rows(directory: str, suffix: str):
    files = sorted(glob.glob(os.path.join(directory, "**", f"*{suffix}"), recursive=True))
    if not files:
        raise SystemExit(f"no *{suffix} under {directory}")
    for fn in files:
        with open(fn, newline="") as fh:
            yield from csv.DictReader(fh)


def short_name(name: str) -> str:
    """Kernel name without argument lists and return types (template arguments kept)."""
    n = re.sub(r"^void\s+", "", name).replace("(anonymous namespace)::", "")
    depth, out = 0, []
    for ch in n:  # drop the parameter list: the first '(' at template depth 0
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            break
        out.append(ch)
    n = "".join(out)
    n = n.replace("(gm::tile::Rows)1", "Rows::Main").replace("(gm::tile::Rows)3", "Rows::Tail")
    return n.strip()


def trace(directory: str, split=()) -> str:
    """split: (regex, microseconds) pairs; dispatches of a matching kernel are listed in two rows, up to and above
    that duration (launches of one grid size by different workloads)."""
    per = defaultdict(list)
    for r in _rows(directory, "kernel_trace.csv"):
        dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        grid = r.get("Grid_Size") or r.get("Grid_Size_X") or ""
        name = short_name(r["Kernel_Name"])
        for rx, us in split:
            if re.search(rx, name):
                name += f" ({'<=' if dur <= us else '>'} {us:g} us)"
        per[(name, grid)].append(dur)
    total = sum(sum(v) for v in per.values())
    lines = ["| kernel | grid size | dispatches | average (us) | median (us) | min (us) | max (us) | share of GPU time |",
             "|---|---:|---:|---:|---:|---:|---:|---:|"]
    for (k, g), v in sorted(per.items(), key=lambda kv: -sum(kv[1])):
        med = sorted(v)[len(v) // 2]
        lines.append(f"| `{k}` | {g} | {len(v)} | {sum(v) / len(v):.1f} | {med:.1f} | {min(v):.1f} | {max(v):.1f} | "
                     f"{100 * sum(v) / total:.2f}% |")
    return "\n".join(lines)


def _counter_per_dispatch(directory: str, counter: str):
    """{kernel name: [value per dispatch in dispatch order]} of one counter (summed over its rows per dispatch)."""
    per = defaultdict(lambda: defaultdict(float))
    for r in _rows(directory, "counter_collection.csv"):
        if r["Counter_Name"] != counter:
            continue
        per[r["Kernel_Name"]][int(r["Dispatch_Id"])] += float(r["Counter_Value"])
    return {k: [v[d] for d in sorted(v)] for k, v in per.items()}


def _copy_value(per: dict) -> float:
    vals = [v for k, vs in per.items() if COPY_KERNEL.search(k) for v in vs]
    if not vals:
        raise SystemExit("no device copy dispatch found for the calibration (run bench.py with --copy-probe-mib)")
    return max(vals)  # the 1 GiB copy is the largest copy of the run


def _sum_kernels(per: dict, regexes) -> tuple[float, list[str]]:
    total, names = 0.0, []
    for rx in regexes:
        hit = [k for k in per if re.search(rx, short_name(k))]
        if len(hit) != 1:
            raise SystemExit(f"kernel regex {rx!r} matches {len(hit)} kernels: {[short_name(k) for k in hit]}")
        vals = per[hit[0]][1:] or per[hit[0]]  # the first dispatch is the warm-up
        total += sum(vals) / len(vals)
        names.append(short_name(hit[0]))
    return total, names


def code_only(text: str) -> str:
    """Source text without comments and blank lines, each line stripped: what a kernel is built from (string
    literals in these sources hold no comment markers)."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = (re.sub(r"//.*", "", line).strip() for line in text.splitlines())
    return "\n".join(line for line in lines if line)


def source_hash(files, directory: str = CSRC) -> str:
    """Hash of the code (comments and blank lines left out) of a kernel's source files: a counter record stays valid
    across edits of comments and becomes stale when the code changes."""
    h = hashlib.sha256()
    for n in files:
        with open(os.path.join(directory, n), encoding="utf-8") as fh:
            h.update(code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def traffic(a) -> dict:
    fetch, write = _counter_per_dispatch(a.fetch, "FETCH_SIZE"), _counter_per_dispatch(a.write, "WRITE_SIZE")
    copy_bytes = a.copy_mib << 20
    fs = copy_bytes / (_copy_value(fetch) * 1024)
    ws = copy_bytes / (_copy_value(write) * 1024)
    f_kib, names = _sum_kernels(fetch, a.kernel)
    w_kib, _ = _sum_kernels(write, a.kernel)
    b = f_kib * 1024 * fs + w_kib * 1024 * ws
    return {"kernel": " + ".join(names), "workload": a.workload, "fetch_size_kib_per_dispatch": f_kib,
            "write_size_kib_per_dispatch": w_kib,
            "calibration": {"copy_bytes": copy_bytes, "fetch_scale": fs, "write_scale": ws},
            "bytes_per_launch": b, "algorithmic_bytes_per_launch": a.algorithmic_bytes,
            "traffic_over_algorithmic": b / a.algorithmic_bytes if a.algorithmic_bytes else None,
            "source_files": a.source, "source_hash": source_hash(a.source), "command": a.command or [],
            "note": "HBM-side bytes per dispatch of the projection (all of its launches) = FETCH_SIZE * fetch_scale "
                    "+ WRITE_SIZE * write_scale; the scales make the plain device copy of the run read and write "
                    "its size; the first (warm-up) dispatch is excluded"}


def counters(directory: str) -> str:
    per = defaultdict(lambda: defaultdict(lambda: defaultdict(float)))
    grids = {}
    for r in _rows(directory, "counter_collection.csv"):
        k = short_name(r["Kernel_Name"])
        per[k][r["Counter_Name"]][int(r["Dispatch_Id"])] += float(r["Counter_Value"])
        grids[k] = r.get("Grid_Size", "")
    names = sorted({c for v in per.values() for c in v})
    lines = ["| kernel | grid size | " + " | ".join(names) + " |", "|---|---:|" + "---:|" * len(names)]
    for k, v in sorted(per.items()):
        cells = []
        for c in names:
            d = v.get(c, {})
            vals = [d[i] for i in sorted(d)][1:] or list(d.values())
            cells.append(f"{sum(vals) / len(vals):.4g}" if vals else "")
        lines.append(f"| `{k}` | {grids[k]} | " + " | ".join(cells) + " |")
    return "\n".join(lines)


def busy(directory: str, xcds: int = 8, simds: int = 1024) -> str:
    """Clock and MFMA busy per kernel and grid size from GRBM_GUI_ACTIVE (busy cycles, summed over the XCDs) and
    SQ_VALU_MFMA_BUSY_CYCLES (summed over the SIMDs; 32 per v_mfma_f32_32x32x16_bf16, 16 per 16x16x32):
    clock = GRBM_GUI_ACTIVE / XCDs / duration, MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (SIMDs x GRBM_GUI_ACTIVE / XCDs).
    The first dispatch of each kernel and grid is excluded."""
    per = defaultdict(lambda: defaultdict(lambda: defaultdict(float)))
    dur = defaultdict(dict)
    for r in _rows(directory, "counter_collection.csv"):
        key = (short_name(r["Kernel_Name"]), r.get("Grid_Size", ""))
        d = int(r["Dispatch_Id"])
        per[key][r["Counter_Name"]][d] += float(r["Counter_Value"])
        dur[key][d] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
    lines = ["| kernel | grid size | dispatches | duration (us) | clock (GHz) | MFMA busy |", "|---|---:|---:|---:|---:|---:|"]
    for key, v in sorted(per.items(), key=lambda kv: -sum(dur[kv[0]].values())):
        ids = sorted(dur[key])
        ids = ids[1:] or ids
        t = sum(dur[key][i] for i in ids)
        g = sum(v.get("GRBM_GUI_ACTIVE", {}).get(i, 0.0) for i in ids)
        m = sum(v.get("SQ_VALU_MFMA_BUSY_CYCLES", {}).get(i, 0.0) for i in ids)
        clk = g / xcds / t / 1e9 if t > 0 else float("nan")
        mb = m / (simds * g / xcds) if g > 0 else float("nan")
        lines.append(f"| `{key[0]}` | {key[1]} | {len(ids)} | {1e6 * t / len(ids):.1f} | {clk:.2f} | {100 * mb:.1f}% |")
    return "\n".join(lines)


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("dir")
    t.add_argument("--split", action="append", default=[], metavar="REGEX:US",
                   help="list the dispatches of the matching kernel up to and above US microseconds in two rows")
    c = sub.add_parser("counters")
    c.add_argument("dir")
    b = sub.add_parser("busy")
    b.add_argument("dir")
    f = sub.add_parser("traffic")
    f.add_argument("--fetch", required=True)
    f.add_argument("--write", required=True)
    f.add_argument("--workload", required=True)
    f.add_argument("--kernel", action="append", required=True)
    f.add_argument("--algorithmic-bytes", type=float, default=0.0)
    f.add_argument("--copy-mib", type=int, default=1024)
    f.add_argument("--source", nargs="+", required=True)
    f.add_argument("--command", action="append")
    f.add_argument("--out", required=True)
    a = ap.parse_args(argv)
    if a.cmd == "trace":
        print(trace(a.dir, [(x.rsplit(":", 1)[0], float(x.rsplit(":", 1)[1])) for x in a.split]))
    elif a.cmd == "counters":
        print(counters(a.dir))
    elif a.cmd == "busy":
        print(busy(a.dir))
    else:
        rec = traffic(a)
        with open(a.out, "w") as fh:
            json.dump(rec, fh, indent=1)
        print(f"{a.out}: {rec['bytes_per_launch'] / 1e9:.3f} GB per launch "
              f"({rec['traffic_over_algorithmic'] or float('nan'):.3f} x algorithmic)", file=sys.stderr)


if __name__ == "__main__":
    main()
