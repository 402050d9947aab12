"""Short text summaries of rocprofv3 output for the ``profiles/`` folder.

Two subcommands:

``stats DIR --command CMD --title T``
    reads the results database a ``rocprofv3 --kernel-trace --stats`` run
    wrote under DIR and prints a markdown table of the top kernels (calls,
    total and mean duration).

``pmc DIR --counters C1 C2 .. --command CMD --title T``
    reads the counter CSV of one ``rocprofv3 --pmc C1 C2 ..`` pass and
    prints a markdown table of each counter's mean value per dispatch for
    the top kernels (by dispatch count times value of the first counter).

``counters --workload W --runs N --fetch DIR --write DIR --copy-fetch DIR --copy-write DIR``
    reads the ``--pmc FETCH_SIZE`` / ``--pmc WRITE_SIZE`` counter CSVs of the
    benchmark (N = pipeline steps the profiled run executed, warm-up
    included) and of the plain 1 GiB copy probe (``bench.py --copy-probe``),
    scales each counter by what it reads for the copy of known size, and
    prints (markdown) / writes (``--json``) the HBM bytes per launch of every
    kernel of the path, tagged with the hash of the kernel's source so that a
    stale figure is never reported for a changed kernel.
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import hashlib
import json
import os
import re
import sqlite3

PKG = os.path.dirname(os.path.abspath(__file__))

# benchmark kernel name -> (device kernel name prefixes, source file)
KERNELS = {
    "compress_dual": (("compress_dual_kernel",), "compress.hip"),
    "compress_csa": (("compress_kernel",), "compress.hip"),
    "compress_hca": (("compress_kernel",), "compress.hip"),
    "index_topk": (("index_",), "indexer.hip"),
    "attention": (("attn_fwd_kernel", "attn_combine_kernel"), "attention.hip"),
    "backward": (("bwd_",), "backward.hip"),
}
COPY_BYTES = 1 << 30  # bench.py --copy-probe copies 1 GiB per launch


def source_hash(fname: str) -> str:
    with open(os.path.join(PKG, "csrc", fname), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def short_name(n: str) -> str:
    n = n.replace("shattn::(anonymous namespace)::", "").replace("void ", "")
    n = re.sub(r"\((shattn|unsigned short const\*|float const\*).*", "", n)
    return n[:100]


def stats_table(d: str, command: str, title: str, top: int = 8) -> str:
    dbs = glob.glob(os.path.join(d, "**", "*.db"), recursive=True)
    if not dbs:
        raise SystemExit(f"no rocprofv3 database under {d}")
    con = sqlite3.connect(dbs[0])
    rows = list(con.execute("select name, total_calls, total_duration, average, percentage from top_kernels"))
    out = [f"# {title}", "", "Command:", "", "```", command, "```", "",
           "| kernel | calls | total us | avg us | % |", "|---|---|---|---|---|"]
    for n, c, t, a, p in rows[:top]:
        # the view reports microseconds
        out.append(f"| `{short_name(n)}` | {c} | {t:.1f} | {a:.2f} | {p:.1f} |")
    return "\n".join(out) + "\n"


def load_counter(d: str, counter: str) -> dict:
    """device kernel short name -> list of per-dispatch values (KiB)."""
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter CSV under {d}")
    agg = collections.defaultdict(list)
    for path in files:
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] == counter:
                    agg[short_name(r["Kernel_Name"])].append(float(r["Counter_Value"]))
    return agg


def pmc_table(d: str, names, command: str, title: str, top: int = 8) -> str:
    per = {c: load_counter(d, c) for c in names}
    kernels = sorted(per[names[0]], key=lambda k: -sum(per[names[0]][k]))[:top]
    out = [f"# {title}", "", "Command:", "", "```", command, "```", "",
           "Mean value per dispatch (counter units as rocprofv3 reports them).", "",
           "| kernel | dispatches | " + " | ".join(names) + " |", "|---|---|" + "---|" * len(names)]
    for k in kernels:
        n = len(per[names[0]][k])
        vals = []
        for c in names:
            v = per[c].get(k, [])
            vals.append(f"{sum(v) / len(v):.4g}" if v else "-")
        out.append(f"| `{k}` | {n} | " + " | ".join(vals) + " |")
    return "\n".join(out) + "\n"


def copy_factor(d: str, counter: str) -> float:
    agg = load_counter(d, counter)
    vals = [v for k, vs in agg.items() if "copy" in k.lower() for v in vs]
    if not vals:
        raise SystemExit(f"no copy kernel in {d}")
    kib = sorted(vals)[len(vals) // 2]
    return COPY_BYTES / (kib * 1024.0)


def counters(args) -> tuple[str, dict]:
    fr = copy_factor(args.copy_fetch, "FETCH_SIZE")
    fw = copy_factor(args.copy_write, "WRITE_SIZE")
    fetch = load_counter(args.fetch, "FETCH_SIZE")
    write = load_counter(args.write, "WRITE_SIZE")
    res = {}
    lines = [f"# HBM traffic per launch from rocprofv3 counters: {args.workload}", "",
             "Commands (each pass its own run):", "", "```", *args.command, "```", "",
             f"Copy-probe scale factors (1 GiB device copy): FETCH_SIZE x{fr:.3f}, WRITE_SIZE x{fw:.3f}.", "",
             "| kernel | device kernels | FETCH KiB/launch | WRITE KiB/launch | HBM MB/launch (scaled) |",
             "|---|---|---|---|---|"]
    for name in args.kernels:
        prefixes, src = KERNELS[name]
        dev = sorted({k for k in list(fetch) + list(write) if k.startswith(prefixes)})
        if not dev:
            continue
        f_kib = sum(sum(fetch.get(k, [])) for k in dev) / args.runs
        w_kib = sum(sum(write.get(k, [])) for k in dev) / args.runs
        hbm = f_kib * 1024 * fr + w_kib * 1024 * fw
        res[name] = {"source_sha": source_hash(src), "fetch_kib": round(f_kib, 1), "write_kib": round(w_kib, 1),
                     "hbm_bytes_per_launch": round(hbm)}
        lines.append(f"| {name} | {', '.join('`' + k + '`' for k in dev)} | {f_kib:.1f} | {w_kib:.1f} | "
                     f"{hbm / 1e6:.2f} |")
    return "\n".join(lines) + "\n", res


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("dir")
    s.add_argument("--command", required=True)
    s.add_argument("--title", required=True)
    q = sub.add_parser("pmc")
    q.add_argument("dir")
    q.add_argument("--counters", nargs="+", required=True)
    q.add_argument("--command", required=True)
    q.add_argument("--title", required=True)
    c = sub.add_parser("counters")
    c.add_argument("--workload", required=True)
    c.add_argument("--runs", type=int, required=True, help="pipeline steps in the profiled run")
    c.add_argument("--fetch", required=True)
    c.add_argument("--write", required=True)
    c.add_argument("--copy-fetch", required=True)
    c.add_argument("--copy-write", required=True)
    c.add_argument("--kernels", nargs="+", default=["compress_dual", "index_topk", "attention"])
    c.add_argument("--command", nargs="+", default=[], help="the rocprofv3 command lines, for the record")
    c.add_argument("--json", help="merge the figures into this JSON file under the workload")
    a = ap.parse_args()
    if a.cmd == "stats":
        print(stats_table(a.dir, a.command, a.title), end="")
        return
    if a.cmd == "pmc":
        print(pmc_table(a.dir, a.counters, a.command, a.title), end="")
        return
    text, res = counters(a)
    print(text, end="")
    if a.json:
        data = {}
        if os.path.exists(a.json):
            with open(a.json) as f:
                data = json.load(f)
        data.setdefault(a.workload, {}).update(res)
        with open(a.json, "w") as f:
            json.dump(data, f, indent=1, sort_keys=True)
            f.write("\n")


if __name__ == "__main__":
    main()
