"""Summarise a rocprofv3 kernel trace of the batched decoder as per-kernel statistics.

    python trace_summary.py <kernel_trace.csv> [--from-step S] [--title TEXT] [--command TEXT] > out.md
    python trace_summary.py --stats <kernel_stats.csv> [--title TEXT] [--command TEXT] [--note TEXT] > out.md

The second form renders the `--stats` table rocprofv3 writes (kernel_stats.csv) as markdown.

The batched decoder ends every step with one final_norm_ssp_k (or final_norm_k) dispatch, so
--from-step S keeps only the dispatches after the S-th of those: the steps S+1 .. of the
replay that was traced.  The weight-streaming products (wsn_k) are split by their role in the
layer, read from the kernel order: the projection before the window attention (qkv) or before
the cross-attention (qx); the residual product after the window attention (wo), after the
cross-attention (wox) or after the FFN input product (ffn_out); the FFN input product (ffn_in)
and the gated merge (merge).
"""
from __future__ import annotations

import argparse
import collections
import csv
import sys


def short_name(n: str) -> str:
    n = n.replace("rlt::(anonymous namespace)::", "").replace("void ", "")
    return n.split("(")[0].strip()


def roles(seq):
    """(role, duration ns) for every dispatch of `seq` = [(name, start, end)] in start order."""
    out = []
    for i, (n, s, e) in enumerate(seq):
        role = n
        if n.startswith("wsn_k"):
            args = n[len("wsn_k<"):-1].replace(" ", "").split(",")
            epi = int(args[1]) if len(args) >= 2 else -1
            prev = seq[i - 1][0] if i else ""
            nxt = seq[i + 1][0] if i + 1 < len(seq) else ""
            if epi == 0:
                role = "wsn_k qkv" if nxt.startswith("swa") else ("wsn_k qx" if nxt.startswith("cross") else n)
            elif epi == 1:
                role = ("wsn_k wo" if prev.startswith("swa") else "wsn_k wox" if prev.startswith("cross")
                        else "wsn_k ffn_out" if prev.startswith("wsn_k") else n)
            elif epi in (2, 3):
                role = "wsn_k ffn_in"
            elif epi == 4:
                role = "wsn_k merge"
        out.append((role, e - s))
    return out


def header(w, title, command, note=""):
    w(f"# {title}\n\n")
    if command:
        w("Command (on the GPU box, `cd /tmp && export TMPDIR=/tmp` first):\n\n")
        for line in command.split(";"):
            w(f"    {line.strip()}\n")
        w("\n")
    if note:
        w(note.strip() + "\n\n")


def stats_table(path, title, command, note):
    rows = list(csv.DictReader(open(path)))
    w = sys.stdout.write
    header(w, title, command, note)
    w("| kernel | calls | avg us | total ms | % |\n|---|---:|---:|---:|---:|\n")
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        name = short_name(r["Name"])
        if len(name) > 90:
            name = name[:87] + "..."
        w(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
          f"{float(r['TotalDurationNs']) / 1e6:.3f} | {float(r['Percentage']):.2f} |\n")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("trace", nargs="?")
    ap.add_argument("--stats", help="a rocprofv3 kernel_stats.csv to render instead of a trace")
    ap.add_argument("--from-step", type=int, default=0)
    ap.add_argument("--title", default="Kernel trace statistics")
    ap.add_argument("--command", default="")
    ap.add_argument("--note", default="")
    args = ap.parse_args()
    if args.stats:
        return stats_table(args.stats, args.title, args.command, args.note)
    seq = []
    with open(args.trace) as f:
        for r in csv.DictReader(f):
            seq.append((short_name(r["Kernel_Name"]), int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
    seq.sort(key=lambda x: x[1])
    steps_seen = 0
    if args.from_step > 0:
        for i, (n, _, _) in enumerate(seq):
            if n.startswith("final_norm"):
                steps_seen += 1
                if steps_seen == args.from_step:
                    seq = seq[i + 1:]
                    break
        else:
            raise SystemExit(f"the trace has only {steps_seen} decoder steps")
    steps = sum(1 for n, _, _ in seq if n.startswith("final_norm"))
    stats = collections.defaultdict(list)
    for role, d in roles(seq):
        stats[role].append(d)
    total = sum(sum(v) for v in stats.values())
    span = (seq[-1][2] - seq[0][1]) if seq else 0
    w = sys.stdout.write
    header(w, args.title, args.command, args.note)
    w(f"Dispatches after decoder step {args.from_step}: {len(seq)} kernels over {steps} decoder steps; "
      f"sum of kernel durations {total / 1e9:.3f} s, first start to last end {span / 1e9:.3f} s "
      f"({total / max(span, 1) * 100:.1f} % busy).\n\n")
    w("| kernel (role) | calls | avg us | total s | % |\n|---|---:|---:|---:|---:|\n")
    for k, v in sorted(stats.items(), key=lambda kv: -sum(kv[1])):
        w(f"| `{k}` | {len(v)} | {sum(v) / len(v) / 1e3:.2f} | {sum(v) / 1e9:.3f} | {100 * sum(v) / total:.2f} |\n")


if __name__ == "__main__":
    main()
