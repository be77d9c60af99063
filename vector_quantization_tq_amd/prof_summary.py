"""Summaries of rocprofv3 CSV output (kernel statistics and counter runs).

    python -m vector_quantization_tq_amd.prof_summary stats KERNEL_STATS_CSV
    python -m vector_quantization_tq_amd.prof_summary traffic --fetch FETCH_CSV --write WRITE_CSV \\
        --kernel scores_kernel --copy neg_kernel --copy-bytes 268435456 --sources FILE ...
    python -m vector_quantization_tq_amd.prof_summary counters --kernel attend_chunk_kernel COUNTER_CSV ...

`stats` prints one line per kernel (calls, average / min / max duration).
`traffic` turns the FETCH_SIZE and WRITE_SIZE counters (KiB per dispatch,
each from its own rocprofv3 --pmc run) of one kernel into bytes per launch,
each scaled by what the same counter reads for a copy kernel of known size,
and prints them with the sha256 of the kernel's sources.  `counters` prints
the mean per dispatch of every counter in the given runs for one kernel,
per wave (divided by SQ_WAVES), and the shares of the wave cycles spent
issuing (SQ_ACTIVE_INST_*) and waiting (SQ_WAIT_*).
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import os
import re
import sys


def _demangle_nested(s: str) -> str:
    """Nested name and integer / bool template arguments of an Itanium-mangled
    kernel name.  rocprofv3 leaves a name mangled when its demangler stops on a
    parameter type (``DF16_``, _Float16); the parameter list is dropped here."""
    i, parts = 3, []
    while i < len(s) and s[i].isdigit():
        j = i
        while s[j].isdigit():
            j += 1
        n = int(s[i:j])
        ident = s[j:j + n]
        i = j + n
        parts.append("anon" if ident.startswith("_GLOBAL__N") else ident)
    name = "::".join(parts)
    if i < len(s) and s[i] == "I":
        i += 1
        args = []
        while True:
            m = re.match(r"L([ibjlm])(n?\d+)E", s[i:])
            if not m:
                break
            v = m.group(2).replace("n", "-")
            args.append(("true" if v == "1" else "false") if m.group(1) == "b" else v)
            i += m.end()
        name += "<" + ", ".join(args) + ">"
    return name


def short_name(name: str) -> str:
    """Kernel name without its argument list and return type."""
    if name.startswith("_ZN"):
        return _demangle_nested(name)
    n = name.replace("(anonymous namespace)", "anon")
    depth = 0
    for i, ch in enumerate(n):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            n = n[:i]
            break
    n = re.sub(r"^void ", "", n)
    return n


def kernel_stats(path):
    rows = []
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            rows.append({"name": short_name(r["Name"]), "calls": int(r["Calls"]),
                         "avg_us": float(r["AverageNs"]) / 1e3, "min_us": float(r["MinNs"]) / 1e3,
                         "max_us": float(r["MaxNs"]) / 1e3, "pct": float(r["Percentage"])})
    return rows


def counter_means(path, counter):
    """{short kernel name: (mean value, dispatches)} for one counter."""
    acc = {}
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            full = r["Kernel_Name"]
            v = float(r["Counter_Value"])
            s, c = acc.get(full, (0.0, 0))
            acc[full] = (s + v, c + 1)
    return {k: (s / c, c) for k, (s, c) in acc.items()}


def pick(means, pattern):
    hits = [(k, v) for k, v in means.items() if pattern in k or pattern in short_name(k)]
    if len(hits) != 1:
        raise SystemExit(f"pattern {pattern!r} matches {len(hits)} kernels: {[short_name(k) for k, _ in hits]}")
    return hits[0]


def sources_sha256(paths, root):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(root, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--kernel", required=True)
    t.add_argument("--copy", required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--sources", nargs="+", required=True)
    t.add_argument("--root", default=os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    c = sub.add_parser("counters")
    c.add_argument("--kernel", required=True)
    c.add_argument("csv", nargs="+")
    a = ap.parse_args(argv)
    if a.cmd == "counters":
        means, name = {}, None
        for path in a.csv:
            with open(path, newline="") as f:
                counters = sorted({r["Counter_Name"] for r in csv.DictReader(f)})
            for ctr in counters:
                k, (v, n) = pick(counter_means(path, ctr), a.kernel)
                means[ctr], name = (v, n), k
        waves = means.get("SQ_WAVES", (1.0, 1))[0]
        print(f"kernel: {short_name(name)}")
        print(f"{'counter':30s} {'per dispatch':>16} {'per wave':>12} {'dispatches':>10}")
        for ctr in sorted(means):
            v, n = means[ctr]
            print(f"{ctr:30s} {v:16.0f} {v / waves:12.1f} {n:10d}")
        if "SQ_WAVE_CYCLES" in means:
            wc = means["SQ_WAVE_CYCLES"][0]
            for ctr in sorted(means):
                if ctr.startswith(("SQ_ACTIVE_INST", "SQ_WAIT")):
                    print(f"share of wave cycles, {ctr}: {means[ctr][0] / wc:.3f}")
        return 0
    if a.cmd == "stats":
        rows = kernel_stats(a.csv)
        print(f"{'calls':>6} {'avg_us':>10} {'min_us':>10} {'max_us':>10} {'pct':>6}  kernel")
        for r in rows:
            print(f"{r['calls']:>6} {r['avg_us']:>10.2f} {r['min_us']:>10.2f} {r['max_us']:>10.2f} {r['pct']:>6.2f}  "
                  f"{r['name']}")
        return 0
    fm, wm = counter_means(a.fetch, "FETCH_SIZE"), counter_means(a.write, "WRITE_SIZE")
    kf_name, (kf, nf) = pick(fm, a.kernel)
    _, (kw, nw) = pick(wm, a.kernel)
    _, (cf, _) = pick(fm, a.copy)
    _, (cw, _) = pick(wm, a.copy)
    ff = cf * 1024.0 / a.copy_bytes
    wf = cw * 1024.0 / a.copy_bytes
    fetch_b = kf * 1024.0 / ff
    write_b = kw * 1024.0 / wf
    print(f"kernel: {short_name(kf_name)}")
    print(f"dispatches: fetch run {nf}, write run {nw}")
    print(f"fetch_kib_per_dispatch: {kf:.2f}")
    print(f"write_kib_per_dispatch: {kw:.2f}")
    print(f"copy_bytes_each_way: {a.copy_bytes}")
    print(f"copy_fetch_kib: {cf:.2f}")
    print(f"copy_write_kib: {cw:.2f}")
    print(f"fetch_factor: {ff:.5f}")
    print(f"write_factor: {wf:.5f}")
    print(f"fetch_bytes_per_launch: {fetch_b:.0f}")
    print(f"write_bytes_per_launch: {write_b:.0f}")
    print(f"traffic_bytes_per_launch: {fetch_b + write_b:.0f}")
    print(f"sources: {' '.join(a.sources)}")
    print(f"source_sha256: {sources_sha256(a.sources, a.root)}")
    return 0


if __name__ == "__main__":
    sys.exit(main())
