"""Turn rocprofv3 CSV output of bench.py runs into short profile summaries.

Expects, under one directory, for every workload number N:
  trace_wN/t_kernel_stats.csv  + trace_wN.log   (--kernel-trace --stats run; the
                                                  log holds bench.py's JSON line)
  fetch_wN/f_counter_collection.csv               (--pmc FETCH_SIZE run)
  write_wN/w_counter_collection.csv               (--pmc WRITE_SIZE run)
and the copy calibration runs fetch_copy/ and write_copy/ (bench.py
--copy-calibration 1024: five 1 GiB device copies).

FETCH_SIZE and WRITE_SIZE are reported in KiB per dispatch.  Each is scaled by
the ratio of the bytes a plain 1 GiB copy moves to what the same counter
reports for it, so the figures are HBM bytes per launch.

Writes profiles/<kernel>__<workload>.md for the dominant kernel of every
workload and updates profiles/traffic.json (keyed by workload name), which
bench.py reads while the kernel's sources are unchanged.

Usage: python profsummary.py PROF_DIR [--workloads 2 3 4 5]
       [--out profiles]
"""
from __future__ import annotations

import argparse
import collections
import csv
import json
import os
import re
import statistics
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

COPY_BYTES = 1 << 30

TRACE_CMD = ("rocprofv3 --kernel-trace --stats --output-format csv -d $REPO/gpurun_out/prof/trace_w{n} "
             "-o t -- python3 $REPO/bench.py --workload {n} --steps 50 --warmup 200 --no-cpu-baseline")
PMC_CMD = ("rocprofv3 --pmc {ctr} --output-format csv -d $REPO/gpurun_out/prof/{tag}_w{n} -o {o} "
           "-- python3 $REPO/bench.py --workload {n} --steps 3 --warmup 1 --warmup-s 0 --no-cpu-baseline")
COPY_CMD = ("rocprofv3 --pmc {ctr} --output-format csv -d $REPO/gpurun_out/prof/{tag}_copy -o {o} "
            "-- python3 $REPO/bench.py --copy-calibration 1024")


# Itanium-mangled template arguments of this library's kernels, for names the
# profiler leaves mangled (it does not demangle _Float16, "DF16_").
_MANGLED_ARGS = [(r"Li(-?\d+)E", r"\1"), (r"Lb0E", "false"), (r"Lb1E", "true"),
                 (r"DF16_", "_Float16"), (r"^t", "unsigned short"), (r"^f", "float")]


def _demangle_pkv(name: str) -> str:
    """`_ZN3pkv12_GLOBAL__N_1<len><ident>I<args>EEvNS_8AttnArgsE` ->
    `<ident><args>`; other names are returned unchanged."""
    m = re.match(r"_ZN3pkv12_GLOBAL__N_1(\d+)", name)
    if not m:
        return name
    rest = name[m.end():]
    ident, rest = rest[:int(m.group(1))], rest[int(m.group(1)):]
    if not rest.startswith("I"):
        return ident
    rest, args = rest[1:], []
    while rest and not rest.startswith("E"):
        for pat, rep in _MANGLED_ARGS:
            a = re.match(pat if pat.startswith("^") else "^" + pat, rest)
            if a:
                args.append(a.expand(rep) if "\\" in rep else rep)
                rest = rest[a.end():]
                break
        else:
            return name
    return f"{ident}<{', '.join(args)}>"


def short(name: str) -> str:
    """`void pkv::(anonymous namespace)::attn_valu_kernel<...>(pkv::AttnArgs)` -> base name."""
    n = name.split("(pkv::")[0]
    n = n.replace("void ", "").replace("pkv::(anonymous namespace)::", "")
    return _demangle_pkv(n)


def base(name: str) -> str:
    return short(name).split("<")[0]


def counters(path: str):
    agg = collections.defaultdict(list)
    with open(path) as f:
        for r in csv.DictReader(f):
            agg[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return agg


def stats(path: str):
    out = []
    with open(path) as f:
        for r in csv.DictReader(f):
            out.append((r["Name"], int(r["Calls"]), float(r["TotalDurationNs"]),
                        float(r["AverageNs"]), float(r["Percentage"])))
    return out


def bench_line(path: str):
    with open(path) as f:
        for line in f:
            if line.startswith('{"metric"'):
                return json.loads(line)
    raise ValueError(f"no bench JSON line in {path}")


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("prof_dir")
    ap.add_argument("--workloads", type=int, nargs="+", default=[2, 3, 4, 5])
    ap.add_argument("--out", default=os.path.join(ROOT, "profiles"))
    args = ap.parse_args()
    import bench

    P = args.prof_dir
    fc = counters(os.path.join(P, "fetch_copy", "f_counter_collection.csv"))
    wc = counters(os.path.join(P, "write_copy", "w_counter_collection.csv"))
    copy_name = next(k for k in fc if "copyBuffer" in k)
    fetch_kib = statistics.mean(fc[copy_name])
    write_kib = statistics.mean(wc[copy_name])
    fscale = COPY_BYTES / (fetch_kib * 1024)
    wscale = COPY_BYTES / (write_kib * 1024)

    tj_path = os.path.join(args.out, "traffic.json")
    traffic = json.load(open(tj_path)) if os.path.exists(tj_path) else {}
    for n in args.workloads:
        rec = bench_line(os.path.join(P, f"trace_w{n}.log"))
        wl = rec["config"]["workload"]
        roof = rec["roofline"]
        st = stats(os.path.join(P, f"trace_w{n}", "t_kernel_stats.csv"))
        fk = counters(os.path.join(P, f"fetch_w{n}", "f_counter_collection.csv"))
        wk = counters(os.path.join(P, f"write_w{n}", "w_counter_collection.csv"))
        want = "attn_mfma_prefill_kernel" if roof["bound"] == "mfma" else None
        attn = [s for s in st if base(s[0]) in bench.KERNEL_SOURCES]
        dom = next((s for s in attn if base(s[0]) == want), None) if want else None
        if dom is None:
            dom = max(attn, key=lambda s: s[2])
        kname = base(dom[0])
        f_b = statistics.mean(fk[dom[0]]) * 1024 * fscale
        w_b = statistics.mean(wk[dom[0]]) * 1024 * wscale
        alg = roof["kernel_bytes"]
        traffic[wl] = {
            "kernel": kname,
            "kernel_instance": short(dom[0]),
            "source_hash": bench.kernel_source_hash(kname),
            "fetch_bytes_per_launch": int(round(f_b)),
            "write_bytes_per_launch": int(round(w_b)),
            "bytes_per_launch": int(round(f_b + w_b)),
            "fetch_scale": round(fscale, 5),
            "write_scale": round(wscale, 5),
            "algorithmic_bytes_per_launch": alg,
            "summary": f"profiles/{kname}__{wl}.md",
        }
        lines = [f"# {kname} — {wl}", "",
                 f"Workload: `bench.py --workload {n}`: {rec['config']['description']}.",
                 f"Algorithmic bytes per step {rec['config']['algorithmic_bytes']:,}; the "
                 f"dominant kernel is charged {alg:,} B per launch"
                 + (f" and {roof['kernel_flops']:,} flop" if "kernel_flops" in roof else "") + ".",
                 "", "## Kernel trace", "", "Command (from the repository root on a GPU host; "
                 "`REPO` = repository root):", "", "```", "cd /tmp && export TMPDIR=/tmp",
                 TRACE_CMD.format(n=n), "```", "",
                 "| kernel | calls | total µs | average µs | % |", "|---|---|---|---|---|"]
        for name, calls, tot, avg, pct in st:
            lines.append(f"| `{short(name)}` | {calls} | {tot / 1e3:.1f} | {avg / 1e3:.3f} | {pct:.2f} |")
        unit = roof["unit"]
        lines += ["", f"The same run's bench line: {rec['value']} GB/s per step "
                  f"({rec['pct_of_peak']} % of 8 TB/s), {rec['us_per_step']} µs per step; "
                  f"dominant kernel ({roof['kernel']}, launches {', '.join(rec['kernels_launched'])}) "
                  f"{roof['kernel_ms'] * 1e3:.2f} µs by the library's HIP events "
                  f"({roof['launches_timed']} timed launches; {roof['kernel_ms_method']}) = "
                  f"{roof['achieved']} {unit}, "
                  f"{100 * roof['frac']:.1f} % of {roof['peak']} {unit}; trace average "
                  f"{dom[3] / 1e3:.2f} µs.", "",
                  "## HBM traffic (separate counter runs, then a copy calibration)", "", "```",
                  PMC_CMD.format(ctr="FETCH_SIZE", tag="fetch", n=n, o="f"),
                  PMC_CMD.format(ctr="WRITE_SIZE", tag="write", n=n, o="w"),
                  COPY_CMD.format(ctr="FETCH_SIZE", tag="fetch", o="f"),
                  COPY_CMD.format(ctr="WRITE_SIZE", tag="write", o="w"), "```", "",
                  "| kernel | dispatches | FETCH_SIZE mean | WRITE_SIZE mean |", "|---|---|---|---|"]
        for k in fk:
            if "copyBuffer" in k:
                continue
            lines.append(f"| `{short(k)}` | {len(fk[k])} | {statistics.mean(fk[k]):,.1f} KiB | "
                         f"{statistics.mean(wk.get(k, [0])):,.1f} KiB |")
        lines.append(f"| `__amd_rocclr_copyBuffer` (1 GiB copy) | {len(fc[copy_name])} | "
                     f"{fetch_kib:,.1f} KiB | {write_kib:,.1f} KiB |")
        lines += ["", f"Calibration: the 1 GiB copy reads and writes {COPY_BYTES:,} B; FETCH_SIZE "
                  f"is scaled by {fscale:.5f}, WRITE_SIZE by {wscale:.5f}.", "",
                  f"Dominant kernel per launch: {f_b:,.0f} B fetched + {w_b:,.0f} B written = "
                  f"{f_b + w_b:,.0f} B, {(f_b + w_b) / alg:.3f} x its algorithmic bytes."]
        path = os.path.join(args.out, f"{kname}__{wl}.md")
        with open(path, "w") as f:
            f.write("\n".join(lines) + "\n")
        print(f"wrote {path}: {(f_b + w_b) / alg:.3f} x algorithmic bytes")
    with open(tj_path, "w") as f:
        json.dump(traffic, f, indent=1, sort_keys=True)
        f.write("\n")
    return 0


if __name__ == "__main__":
    sys.exit(main())
