"""Summarise rocprofv3 result databases into the short text files kept in profiles/.

    # kernel durations (from a --kernel-trace --stats run)
    python -m token_level_head_amd.rocprof_summary trace RUN_results.db --cmd "<rocprofv3 command>" \
        --workload dit_s2_256 > profiles/kernels_dit_s2_256.md

    # any counters of one --pmc run (e.g. the MFMA and SQ counters of the mixing kernel)
    python -m token_level_head_amd.rocprof_summary pmc RUN_results.db --workload dit_s2_4096 \
        --cmd "<command>" --kernel mix_ --out profiles/mfma_dit_s2_4096.json

    # HBM traffic (from one --pmc FETCH_SIZE run and one --pmc WRITE_SIZE run)
    python -m token_level_head_amd.rocprof_summary counters FETCH_results.db WRITE_results.db \
        --workload dit_s2_256 --cmd-fetch "<command>" --cmd-write "<command>" \
        --out profiles/counters_dit_s2_256.json

FETCH_SIZE and WRITE_SIZE are scaled by what the same counter reports for the
plain 1 GiB device copy that ``bench.py --copy-calibration`` runs: bytes =
counter_KiB * (copy bytes / copy counter KiB).  The counters file records the
digest of the source file of each kernel it measured (with the shared headers);
``bench.py`` reports a kernel's traffic only while that digest matches.
"""
import argparse
import json
import sqlite3
import sys

from .build import kernel_source_digest, source_digest

COPY_BYTES = 1 << 30  # bench.py --copy-calibration copies 2^28 float32 values


def short_name(name):
    base = name.replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "")
    return base.replace("mhla::", "")


def trace_rows(db):
    c = sqlite3.connect(db)
    rows = c.execute("select name, count(*), avg(duration), min(duration), max(duration), sum(duration) "
                     "from kernels group by name order by sum(duration) desc").fetchall()
    return [dict(name=r[0], calls=r[1], avg_ns=r[2], min_ns=r[3], max_ns=r[4], total_ns=r[5]) for r in rows]


def cmd_trace(args):
    rows = trace_rows(args.db)
    total = sum(r["total_ns"] for r in rows) or 1
    print(f"# rocprofv3 kernel trace: {args.workload}\n")
    print(f"Command: `{args.cmd}`\n")
    print(f"Kernel sources digest: `{source_digest()}`\n")
    print("| kernel | calls | avg us | min us | max us | % of GPU time | source digest |")
    print("|---|---|---|---|---|---|---|")
    for r in rows:
        name = short_name(r['name'])
        dig = kernel_source_digest(name) if "mhla::" in r['name'] else ""
        print(f"| `{name}` | {r['calls']} | {r['avg_ns'] / 1e3:.2f} | {r['min_ns'] / 1e3:.2f} | "
              f"{r['max_ns'] / 1e3:.2f} | {100 * r['total_ns'] / total:.1f} | {dig} |")


def counter_means(db, counter):
    c = sqlite3.connect(db)
    rows = c.execute("select kernel_name, count(*), avg(value), max(value) from counters_collection "
                     "where counter_name = ? group by kernel_name", (counter,)).fetchall()
    return {r[0]: {"dispatches": r[1], "avg_kib": r[2], "max_kib": r[3]} for r in rows}


def cmd_counters(args):
    fetch = counter_means(args.fetch_db, "FETCH_SIZE")
    write = counter_means(args.write_db, "WRITE_SIZE")
    copy_name = next(n for n in fetch if "copyBuffer" in n or "copy" in n.lower())
    f_scale = COPY_BYTES / (fetch[copy_name]["max_kib"])
    w_scale = COPY_BYTES / (write[copy_name]["max_kib"])
    kernels = {}
    for name in sorted(set(fetch) & set(write)):
        if not name.startswith("void mhla::") and "mhla::" not in name:
            continue
        fb = fetch[name]["avg_kib"] * f_scale
        wb = write[name]["avg_kib"] * w_scale
        kernels[short_name(name)] = {"fetch_kib": fetch[name]["avg_kib"], "write_kib": write[name]["avg_kib"],
                                     "fetch_bytes": fb, "write_bytes": wb, "traffic_bytes": fb + wb,
                                     "dispatches": fetch[name]["dispatches"],
                                     "source_digest": kernel_source_digest(short_name(name))}
    out = {"workload": args.workload, "source_digest": source_digest(),
           "copy_reference": {"kernel": copy_name, "bytes": COPY_BYTES, "fetch_kib": fetch[copy_name]["max_kib"],
                              "write_kib": write[copy_name]["max_kib"], "fetch_scale": f_scale,
                              "write_scale": w_scale},
           "commands": {"fetch": args.cmd_fetch, "write": args.cmd_write}, "kernels": kernels}
    with open(args.out, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out, indent=1))


def cmd_pmc(args):
    c = sqlite3.connect(args.db)
    rows = c.execute("select kernel_name, counter_name, avg(value), count(*) from counters_collection "
                     "group by kernel_name, counter_name").fetchall()
    kernels = {}
    for name, counter, avg, n in rows:
        if "mhla::" not in name or args.kernel not in name:
            continue
        k = kernels.setdefault(short_name(name), {"dispatches": n, "source_digest": kernel_source_digest(short_name(name))})
        k[counter] = avg
    for k in kernels.values():
        # SQ_VALU_MFMA_BUSY_CYCLES sums MFMA-busy cycles over all SIMDs; with the SQ busy
        # cycles (summed over the shader engines) it gives the MFMA-busy share of the SIMDs.
        if "SQ_VALU_MFMA_BUSY_CYCLES" in k and "SQ_BUSY_CYCLES" in k and args.simds_per_se:
            k["mfma_busy_frac"] = k["SQ_VALU_MFMA_BUSY_CYCLES"] / (k["SQ_BUSY_CYCLES"] * args.simds_per_se)
    out = {"workload": args.workload, "source_digest": source_digest(), "command": args.cmd, "kernels": kernels}
    with open(args.out, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out, indent=1))


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    t = sub.add_parser("trace")
    t.add_argument("db")
    t.add_argument("--cmd", required=True)
    t.add_argument("--workload", required=True)
    c = sub.add_parser("counters")
    c.add_argument("fetch_db")
    c.add_argument("write_db")
    c.add_argument("--workload", required=True)
    c.add_argument("--cmd-fetch", required=True)
    c.add_argument("--cmd-write", required=True)
    c.add_argument("--out", required=True)
    m = sub.add_parser("pmc")
    m.add_argument("db")
    m.add_argument("--workload", required=True)
    m.add_argument("--cmd", required=True)
    m.add_argument("--kernel", default="", help="substring of the kernel names to keep")
    m.add_argument("--simds-per-se", type=int, default=32, help="SIMDs per shader engine (MI355X: 8 CUs x 4)")
    m.add_argument("--out", required=True)
    args = ap.parse_args(argv)
    {"trace": cmd_trace, "counters": cmd_counters, "pmc": cmd_pmc}[args.what](args)


if __name__ == "__main__":
    sys.exit(main())
