"""Short text summaries of rocprofv3 output (CSV), for the profiles folder.

  python -m compressed_attention_fwht_amd.profsummary stats KERNEL_STATS_CSV \\
      --title T --cmd "the rocprofv3 command" --out FILE.md
      per-kernel calls / average / min / max duration and share of GPU time.

  python -m compressed_attention_fwht_amd.profsummary coverage KERNEL_STATS_CSV \\
      --title T --cmd "the rocprofv3 command" --out FILE.md
      every instance of the library's kernels the run launched (name with its
      template arguments, the parameter list dropped) and its call count.

  python -m compressed_attention_fwht_amd.profsummary counters COUNTER_CSV \\
      --kernels "NAME[;NAME...]" --title T --cmd "..." --out FILE.md
      mean per-dispatch value of every counter of the run for each kernel.

  python -m compressed_attention_fwht_amd.profsummary traffic \\
      --fetch FETCH_COUNTER_CSV --write WRITE_COUNTER_CSV --kernel "NAME[;NAME...]" \\
      --source "FILE[;FILE...]" --copy-bytes N --cmd-fetch "..." --cmd-write "..." \\
      --out FILE.md
      FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of kernel NAME, each scaled
      by what the same counter reads for a plain device copy of N bytes (the
      largest __amd_rocclr_copyBuffer dispatches of the run), giving HBM bytes
      per launch; with several names, the sum of their per-dispatch means (the
      kernels of one call, each launched once per call).  The result goes into
      a JSON block with the SHA-256 of every source file the kernels are built
      from, so a reader can tell whether it still applies.

Host-side text processing only; nothing here touches the GPU.
"""
import argparse
import collections
import csv
import hashlib
import json
import os
import sys

CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")


def _short(name, n=90):
    return name if len(name) <= n else name[: n - 3] + "..."


def stats(args):
    rows = list(csv.DictReader(open(args.csv)))
    total = sum(float(r["TotalDurationNs"]) for r in rows) or 1.0
    lines = [f"# {args.title}", "", "Command:", "", "```", args.cmd, "```", "",
             "| kernel | calls | avg us | min us | max us | share of GPU time |",
             "|---|---|---|---|---|---|"]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        lines.append(f"| `{_short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                     f"{100 * float(r['TotalDurationNs']) / total:.1f} % |")
    open(args.out, "w").write("\n".join(lines) + "\n")


def _instance(name):
    """'void kvq::k<1, 2>(int, ...)' -> 'k<1, 2>'; None outside the library."""
    name = name.replace("void ", "", 1)
    if not name.startswith("kvq::"):
        return None
    name = name[len("kvq::"):]
    depth = 0
    for i, ch in enumerate(name):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            return name[:i]
    return name


def coverage(args):
    rows = list(csv.DictReader(open(args.csv)))
    calls = collections.Counter()
    for r in rows:
        inst = _instance(r["Name"])
        if inst is not None:
            calls[inst] += int(r["Calls"])
    lines = [f"# {args.title}", "", "Command:", "", "```", args.cmd, "```", "",
             f"{len(calls)} kernel instances launched.", "",
             "| kernel instance | calls |", "|---|---|"]
    for k in sorted(calls):
        lines.append(f"| `{k}` | {calls[k]} |")
    open(args.out, "w").write("\n".join(lines) + "\n")


def _per_dispatch(path, counter):
    vals = collections.defaultdict(dict)   # kernel -> dispatch -> value
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        vals[r["Kernel_Name"]][r["Dispatch_Id"]] = float(r["Counter_Value"])
    return vals


def _kernel_mean(vals, key):
    hits = [v for name, d in vals.items() if key in name for v in d.values()]
    if not hits:
        raise SystemExit(f"no dispatch of a kernel named like {key!r}")
    return sum(hits) / len(hits), len(hits)


def _copy_kib(vals):
    copies = [v for name, d in vals.items() if "copyBuffer" in name for v in d.values()]
    if not copies:
        raise SystemExit("no __amd_rocclr_copyBuffer dispatch (run with the calibration copy)")
    top = max(copies)
    big = [v for v in copies if v >= 0.5 * top]
    return sum(big) / len(big), len(big)


def traffic(args):
    fv = _per_dispatch(args.fetch, "FETCH_SIZE")
    wv = _per_dispatch(args.write, "WRITE_SIZE")
    keys = args.kernel.split(";")
    per_f = [_kernel_mean(fv, k) for k in keys]
    per_w = [_kernel_mean(wv, k) for k in keys]
    f_k, nf = sum(m for m, _ in per_f), [n for _, n in per_f]
    w_k, nw = sum(m for m, _ in per_w), [n for _, n in per_w]
    f_c, ncf = _copy_kib(fv)
    w_c, ncw = _copy_kib(wv)
    ff = args.copy_bytes / (f_c * 1024.0)
    fw = args.copy_bytes / (w_c * 1024.0)
    fetch_b = f_k * 1024.0 * ff
    write_b = w_k * 1024.0 * fw
    shas = {src: hashlib.sha256(open(os.path.join(CSRC, src), "rb").read()).hexdigest()
            for src in args.source.split(";")}
    d = {"kernel": args.kernel, "sources_sha256": shas,
         "fetch_kib_per_dispatch": round(f_k, 1), "write_kib_per_dispatch": round(w_k, 1),
         "per_kernel_kib": {k: [round(f, 1), round(w, 1)]
                            for k, (f, _), (w, _) in zip(keys, per_f, per_w)},
         "dispatches": {"fetch_run": nf, "write_run": nw},
         "copy_bytes": args.copy_bytes,
         "copy_fetch_kib": round(f_c, 1), "copy_write_kib": round(w_c, 1),
         "fetch_scale": round(ff, 4), "write_scale": round(fw, 4),
         "fetch_bytes_per_launch": round(fetch_b), "write_bytes_per_launch": round(write_b),
         "traffic_bytes_per_launch": round(fetch_b + write_b)}
    if args.algorithmic_bytes:
        d["algorithmic_bytes_per_launch"] = args.algorithmic_bytes
        d["traffic_over_algorithmic"] = round((fetch_b + write_b) / args.algorithmic_bytes, 3)
    lines = [f"# {args.title}", "",
             "HBM traffic per launch from two counter passes, each scaled by the same counter",
             f"read for a plain device copy of {args.copy_bytes} bytes in the same run.", "",
             "FETCH_SIZE pass:", "", "```", args.cmd_fetch, "```", "",
             "WRITE_SIZE pass:", "", "```", args.cmd_write, "```", "",
             "| | kernel KiB/dispatch | copy KiB/dispatch | scale | bytes/launch |",
             "|---|---|---|---|---|",
             f"| FETCH_SIZE | {f_k:.1f} | {f_c:.1f} | {ff:.4f} | {fetch_b:.0f} |",
             f"| WRITE_SIZE | {w_k:.1f} | {w_c:.1f} | {fw:.4f} | {write_b:.0f} |", "",
             "```json", json.dumps(d, indent=1), "```"]
    open(args.out, "w").write("\n".join(lines) + "\n")


def counters(args):
    keys = args.kernels.split(";")   # kernel names hold commas
    vals = collections.defaultdict(lambda: collections.defaultdict(list))
    names = {}
    for r in csv.DictReader(open(args.csv)):
        for k in keys:
            if k in r["Kernel_Name"]:
                vals[k][r["Counter_Name"]].append(float(r["Counter_Value"]))
                names[k] = r["Kernel_Name"]
    cnames = sorted({c for k in keys for c in vals[k]})
    lines = [f"# {args.title}", "", "Command:", "", "```", args.cmd, "```", "",
             "Mean per dispatch (dispatches in parentheses).", "",
             "| counter | " + " | ".join(f"`{_short(names.get(k, k), 40)}`" for k in keys) + " |",
             "|---|" + "---|" * len(keys)]
    for c in cnames:
        cells = []
        for k in keys:
            v = vals[k].get(c, [])
            cells.append(f"{sum(v) / len(v):.4g} ({len(v)})" if v else "-")
        lines.append(f"| {c} | " + " | ".join(cells) + " |")
    open(args.out, "w").write("\n".join(lines) + "\n")


def main(argv=None):
    p = argparse.ArgumentParser(prog="profsummary")
    sub = p.add_subparsers(dest="cmd_name", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("--title", required=True)
    s.add_argument("--cmd", required=True)
    s.add_argument("--out", required=True)
    v = sub.add_parser("coverage")
    v.add_argument("csv")
    v.add_argument("--title", required=True)
    v.add_argument("--cmd", required=True)
    v.add_argument("--out", required=True)
    c = sub.add_parser("counters")
    c.add_argument("csv")
    c.add_argument("--kernels", required=True)
    c.add_argument("--title", required=True)
    c.add_argument("--cmd", required=True)
    c.add_argument("--out", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--kernel", required=True)
    t.add_argument("--source", required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--algorithmic-bytes", type=int, default=0)
    t.add_argument("--title", required=True)
    t.add_argument("--cmd-fetch", required=True)
    t.add_argument("--cmd-write", required=True)
    t.add_argument("--out", required=True)
    a = p.parse_args(argv)
    {"stats": stats, "coverage": coverage, "counters": counters, "traffic": traffic}[a.cmd_name](a)


if __name__ == "__main__":
    main(sys.argv[1:])
