"""Summaries of rocprofv3 output for profiles/.

    python profile_report.py kernels DB.db [--title T] [--command C]
        Markdown table of a kernel trace (the rocpd SQLite file rocprofv3 writes):
        per kernel and grid, calls and average / min / max duration.

    python profile_report.py traffic --config NAME --fetch F.csv --write W.csv \
            --copy-fetch CF.csv --copy-write CW.csv --copy-bytes N [--command C ...]
        HBM bytes per launch of each kernel of the o_proj chain from two counter
        runs (FETCH_SIZE, then WRITE_SIZE: KiB per dispatch), each scaled by what
        the same counter reads for a plain device copy of N bytes.  Writes
        profiles/traffic_NAME.json (read by bench.py for roofline.traffic while
        the kernel sources are unchanged) and prints a Markdown summary.

    python profile_report.py pmc P.csv [--title T] [--command C]
        Mean of each collected counter per dispatch, for each launch of the chain.

    python profile_report.py chain DB.db [--title T] [--command C]
        µs per chain call from the kernel trace: quantize start to gemm end of each
        consecutive quantize -> einsum -> gemm triple, with the launches and gaps.

Kernels are told apart by name and output mode (the streaming kernel's second
template argument, the whole-K kernel's first, the tile kernel's third: 1 = BF16
out: fp8_gemm_nt, 2 = MXFP8 out: grouped_fp8_einsum); the quantize kernel is
mxfp8_quantize.  Only the grid that occurs most often is kept for
each, which drops the one-off launches of the set-up (weight quantization).
"""
from __future__ import annotations

import argparse
import collections
import csv
import json
import os
import re
import sqlite3
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))


def short_name(name: str) -> str:
    s = re.sub(r"\(.*", "", name)
    return s.replace("void mx::", "").replace("mx::", "").strip()


def template_args(n: str):
    """Top-level template arguments of `kernel<...>`, or None."""
    i = n.find("<")
    if i < 0 or not n.endswith(">"):
        return None
    args, depth, cur = [], 0, ""
    for ch in n[i + 1:-1]:
        if ch == "," and depth == 0:
            args.append(cur.strip())
            cur = ""
            continue
        depth += ch == "<"
        depth -= ch == ">"
        cur += ch
    args.append(cur.strip())
    return n[:i], args


def chain_role(name: str):
    """quantize / einsum (MXFP8 out) / gemm (BF16 out) from a kernel name: the output mode is the
    second template argument of the streaming kernel, the first of the whole-K kernels and the third
    of the tile kernel."""
    n = short_name(name)
    if n.startswith("quantize_kernel"):
        return "quantize"
    t = template_args(n)
    if not t:
        return None
    kern, args = t
    if kern == "stream_kernel" and len(args) >= 2:
        out = args[1]
    elif kern in ("whole_k_kernel", "whole_k_xb_kernel"):
        out = args[0]
    elif kern == "dl_gemm_kernel" and len(args) >= 3:
        out = args[2]
    else:
        return None
    return {"1": "gemm", "2": "einsum", "3": "einsum"}.get(out)


def cmd_kernels(a):
    db = sqlite3.connect(a.db)
    rows = db.execute(
        "select name, count(*), avg(duration), min(duration), max(duration), sum(duration), grid_x, workgroup_x, "
        "vgpr_count, accum_vgpr_count, lds_size from kernels group by name, grid_x order by sum(duration) desc"
    ).fetchall()
    tot = sum(r[5] for r in rows) or 1
    if a.title:
        print(f"# {a.title}\n")
    if a.command:
        print("Command (from the repository root, one MI355X):\n\n    " + a.command + "\n")
    print("| kernel | grid threads / WG | calls | avg µs | min µs | max µs | share | VGPR/AGPR | LDS B |")
    print("|---|---|---|---|---|---|---|---|---|")
    for name, n, avg, mn, mx, s, gx, wx, vg, ag, lds in rows:
        print(f"| `{short_name(name)[:100]}` | {gx} / {wx} | {n} | {avg / 1e3:.2f} | {mn / 1e3:.2f} | "
              f"{mx / 1e3:.2f} | {s / tot * 100:.1f}% | {vg}/{ag} | {lds} |")


def read_counter(path, counter):
    """{(role, grid): [values]} of one counter over the dispatches of a counter-collection CSV."""
    out = collections.defaultdict(list)
    other = collections.defaultdict(list)
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            role = chain_role(r["Kernel_Name"])
            key = (role, int(r["Grid_Size"]))
            (out if role else other)[key if role else (short_name(r["Kernel_Name"]), int(r["Grid_Size"]))].append(
                float(r["Counter_Value"]))
    return out, other


def main_grid(d, role):
    cands = {k: v for k, v in d.items() if k[0] == role}
    if not cands:
        return None, []
    k = max(cands, key=lambda k: len(cands[k]))
    return k[1], cands[k]


def cmd_traffic(a):
    sys.path.insert(0, ROOT)
    from bench import chain_bytes, kernel_source_hash
    import synth_inputs as si

    # the workload's shapes: a chain configuration, or one run at another token count (NAME_M<tokens>)
    base, _, tok = a.config.partition("_M")
    shape = si.CHAIN_CONFIGS[base].shape if base in si.CHAIN_CONFIGS else None
    algo = {}
    if shape is not None:
        M = int(tok) if tok else shape.M
        algo = chain_bytes(M, shape.G, shape.K, shape.N, shape.P)
    res = {"config": a.config, "kernel_source_hash": kernel_source_hash(), "commands": a.command or []}
    cal = {}
    for counter, path in (("FETCH_SIZE", a.copy_fetch), ("WRITE_SIZE", a.copy_write)):
        _, other = read_counter(path, counter)
        # the copy kernel: the largest per-dispatch value of the copy run
        vals = [max(v) for v in other.values()]
        if not vals:
            raise SystemExit(f"no dispatch with {counter} in {path}")
        kib = max(vals)
        cal[counter] = a.copy_bytes / (kib * 1024.0)
    res["calibration"] = {"copy_bytes": a.copy_bytes, "bytes_per_counted_byte": cal}
    lines = [f"# HBM traffic per launch, {a.config} configuration\n"]
    for c in a.command or []:
        lines.append("    " + c)
    lines.append("")
    lines.append(f"Calibration: a device copy of {a.copy_bytes} bytes reads as FETCH_SIZE x "
                 f"{cal['FETCH_SIZE']:.3f} and WRITE_SIZE x {cal['WRITE_SIZE']:.3f} bytes.\n")
    lines.append("| launch | grid | dispatches | FETCH bytes | WRITE bytes | HBM bytes per launch | algorithmic bytes "
                 "| ratio |")
    lines.append("|---|---|---|---|---|---|---|---|")
    fetch, _ = read_counter(a.fetch, "FETCH_SIZE")
    write, _ = read_counter(a.write, "WRITE_SIZE")
    for role in ("quantize", "einsum", "gemm"):
        gf, vf = main_grid(fetch, role)
        gw, vw = main_grid(write, role)
        if not vf or not vw:
            continue
        fb = sum(vf) / len(vf) * 1024 * cal["FETCH_SIZE"]
        wb = sum(vw) / len(vw) * 1024 * cal["WRITE_SIZE"]
        res[role] = {"grid": gf, "dispatches": len(vf), "fetch_bytes": fb, "write_bytes": wb,
                     "hbm_bytes_per_launch": fb + wb}
        if role in algo:
            res[role]["algorithmic_bytes"] = algo[role]
            extra = f" {algo[role]:.4g} | {(fb + wb) / algo[role]:.2f} |"
        else:
            extra = " | |"
        lines.append(f"| {role} | {gf} | {len(vf)} | {fb:.4g} | {wb:.4g} | {fb + wb:.4g} |" + extra)
    path = os.path.join(ROOT, "profiles", f"traffic_{a.config}.json")
    with open(path, "w") as f:
        json.dump(res, f, indent=1)
    print("\n".join(lines))


def cmd_pmc(a):
    """Mean of every counter per dispatch, per chain launch (most frequent grid)."""
    vals = collections.defaultdict(lambda: collections.defaultdict(list))
    with open(a.csv) as f:
        for r in csv.DictReader(f):
            role = chain_role(r["Kernel_Name"])
            if role:
                vals[(role, int(r["Grid_Size"]))][r["Counter_Name"]].append(float(r["Counter_Value"]))
    if a.title:
        print(f"# {a.title}\n")
    if a.command:
        print("Command (from the repository root, one MI355X):\n\n    " + a.command + "\n")
    counters = sorted({c for v in vals.values() for c in v})
    print("| launch | grid | dispatches | " + " | ".join(counters) + " |")
    print("|---|---|---|" + "---|" * len(counters))
    for role in ("quantize", "einsum", "gemm"):
        keys = [k for k in vals if k[0] == role]
        if not keys:
            continue
        k = max(keys, key=lambda k: len(next(iter(vals[k].values()))))
        n = len(next(iter(vals[k].values())))
        cells = [f"{sum(vals[k][c]) / len(vals[k][c]):.6g}" if vals[k].get(c) else "" for c in counters]
        print(f"| {role} | {k[1]} | {n} | " + " | ".join(cells) + " |")


def cmd_chain(a):
    """µs per chain call from kernel-trace timestamps: each quantize -> einsum -> gemm triple of consecutive
    dispatches (the headline chain), from the quantize's start to the gemm's end; plus each launch's
    duration and the gaps between them."""
    import statistics

    db = sqlite3.connect(a.db)
    rows = db.execute("select name, start, end, grid_x from kernels order by start").fetchall()
    seq = [(chain_role(n), s, e, g) for n, s, e, g in rows]
    # the chain's own quantize grid: the most frequent quantize grid
    qgrids = collections.Counter(g for r, _, _, g in seq if r == "quantize")
    if not qgrids:
        raise SystemExit("no quantize dispatch in the trace")
    qgrid = qgrids.most_common(1)[0][0]
    spans, parts = [], collections.defaultdict(list)
    for i in range(len(seq) - 2):
        q, e, g = seq[i], seq[i + 1], seq[i + 2]
        if q[0] == "quantize" and q[3] == qgrid and e[0] == "einsum" and g[0] == "gemm":
            spans.append((g[2] - q[1]) / 1e3)
            parts["quantize"].append((q[2] - q[1]) / 1e3)
            parts["gap quantize -> einsum"].append((e[1] - q[2]) / 1e3)
            parts["einsum"].append((e[2] - e[1]) / 1e3)
            parts["gap einsum -> gemm"].append((g[1] - e[2]) / 1e3)
            parts["gemm"].append((g[2] - g[1]) / 1e3)
    if not spans:
        raise SystemExit("no quantize -> einsum -> gemm sequence in the trace")
    if a.title:
        print(f"# {a.title}\n")
    if a.command:
        print("Command (from the repository root, one MI355X):\n\n    " + a.command + "\n")
    q = statistics.quantiles(spans, n=10)
    print(f"{len(spans)} chain calls (quantize start -> gemm end): median {statistics.median(spans):.2f} µs, "
          f"min {min(spans):.2f}, 10th percentile {q[0]:.2f}, 90th percentile {q[-1]:.2f}.\n")
    print("| part | median µs | min µs |")
    print("|---|---|---|")
    for k, v in parts.items():
        print(f"| {k} | {statistics.median(v):.2f} | {min(v):.2f} |")


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    pm = sub.add_parser("pmc")
    pm.add_argument("csv")
    pm.add_argument("--title", default="")
    pm.add_argument("--command", default="")
    k = sub.add_parser("kernels")
    k.add_argument("db")
    k.add_argument("--title", default="")
    k.add_argument("--command", default="")
    t = sub.add_parser("traffic")
    t.add_argument("--config", required=True)
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--copy-fetch", required=True)
    t.add_argument("--copy-write", required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--command", action="append")
    c = sub.add_parser("chain")
    c.add_argument("db")
    c.add_argument("--title", default="")
    c.add_argument("--command", default="")
    a = ap.parse_args()
    {"kernels": cmd_kernels, "traffic": cmd_traffic, "pmc": cmd_pmc, "chain": cmd_chain}[a.cmd](a)


if __name__ == "__main__":
    main()
