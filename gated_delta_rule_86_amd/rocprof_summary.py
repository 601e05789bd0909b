"""Turn rocprofv3 outputs of the benchmark into the short text summaries kept
under profiles/.

    python -m gated_delta_rule_86_amd.rocprof_summary stats  <kernel_stats.csv> <out.md> --command "..."
    python -m gated_delta_rule_86_amd.rocprof_summary traffic <fetch_dir> <write_dir> <out.md> --command "..."
    python -m gated_delta_rule_86_amd.rocprof_summary counters <pmc_dir> <out.md> --command "..."

`stats` summarises a --kernel-trace --stats run (calls, average and total
duration per kernel).  `traffic` takes two --pmc runs (FETCH_SIZE, then
WRITE_SIZE; KiB per dispatch) of ``bench.py --calibrate-copy``, scales each
counter by what it reads for the plain device copy of known size the
benchmark runs, and reports HBM bytes per launch for each kernel.  The
summary records a hash of the kernel sources it was measured on; bench.py
reports the traffic only while the sources still hash the same.  `counters`
tabulates the per-kernel medians of any other --pmc run (MFMA and VALU
utilisation, LDS bank conflicts).
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import os
import re
import statistics

PKG = os.path.dirname(os.path.abspath(__file__))

# Kernel-name fragments -> short names used in the summaries and bench.py.
KERNELS = (("chunk_prep_kernel", "gdr2_chunk_prep"), ("chunk_fused_kernel", "gdr2_chunk_fused"),
           ("chunk_state_kernel", "gdr2_chunk_state"), ("bwd_gate_sum_kernel", "gdr2_bwd_gate_sum"),
           ("chunk_span_kernel", "gdr2_chunk_span"), ("span_fold_kernel", "gdr2_span_fold"),
           ("decode_step_kernel", "gdr2_decode_step"), ("bwd_prep_kernel", "gdr2_bwd_prep"),
           ("bwd_dout_kernel", "gdr2_bwd_dout"), ("bwd_frag_kernel", "gdr2_bwd_frag"),
           ("bwd_scan_kernel", "gdr2_bwd_scan"), ("bwd_span_kernel", "gdr2_bwd_span"), ("bwd_sgrad", "gdr2_bwd_sgrad"),
           ("bwd_xgrad", "gdr2_bwd_xgrad"), ("bwd_norm_kernel", "gdr2_bwd_norm"),
           ("bwd_decay_kernel", "gdr2_bwd_decay"), ("zero_kernel", "gdr2_zero_fill"), ("copy", "plain_copy"))
COPY_BYTES_MARK = "calibration copy bytes:"


def source_hash() -> str:
    """sha256 over the HIP sources of the library (what the counters measure)."""
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(PKG, "csrc", "*"))):
        with open(p, "rb") as f:
            h.update(os.path.basename(p).encode())
            h.update(f.read())
    return h.hexdigest()[:16]


_PREP_VARIANT = re.compile(r"chunk_(?:prep|fused)_kernel(?:ILi(\d+)ELi(\d+)ELi(\d+)ELb(\d)|<(\d+), (\d+), (\d+), (true|false))")
_SHAPE = re.compile(r"chunk_(?:prep|fused)_kernel(?:I.*?E(DF16b|f)Li(\d+)ELi(\d+)E|<[^>]*?, (__bf16|float), (\d+), (\d+)>)")


def short_name(kernel: str) -> str | None:
    for frag, name in KERNELS:
        if frag in kernel:
            if name in ("gdr2_chunk_prep", "gdr2_chunk_fused"):
                # one kernel per gate-width mix (0 = widths read at run time)
                m = _PREP_VARIANT.search(kernel)
                if m:
                    g = m.groups()
                    wb, ww, wg, pro = g[0:4] if g[0] is not None else g[4:8]
                    tag = ",".join("x" if x == "0" else ("1" if x == "1" else "d") for x in (wb, ww, wg))
                    name += f"[b,w,g={tag}" + (",prologue]" if pro in ("1", "true") else "]")
                # other shapes than bf16, d = 128, chunk 64 are named
                m = _SHAPE.search(kernel)
                if m:
                    g = m.groups()
                    dt, d, c = g[0:3] if g[0] is not None else g[3:6]
                    dt = "bf16" if dt in ("DF16b", "__bf16") else "f32"
                    if (dt, d, c) != ("bf16", "128", "64"):
                        name += f"[{dt},d{d},c{c}]"
            return name
    return None


def _find(path, pattern):
    if os.path.isfile(path):
        return path
    hits = glob.glob(os.path.join(path, "**", pattern), recursive=True)
    if not hits:
        raise FileNotFoundError(f"no {pattern} under {path}")
    return hits[0]


def stats(args):
    f = _find(args.csv, "*kernel_stats.csv")
    rows = list(csv.DictReader(open(f)))
    out = [f"# rocprofv3 kernel statistics: {args.title}", "",
           f"Command (from the repository root on the MI355X machine):", "", f"    {args.command}", "",
           f"Kernel sources hash: `{source_hash()}`", "",
           "| kernel | calls | average (us) | total (us) |", "|---|---|---|---|"]
    for r in rows:
        name = short_name(r["Name"]) or r["Name"][:60]
        out.append(f"| {name} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                   f"{float(r['TotalDurationNs']) / 1e3:.1f} |")
    open(args.out, "w").write("\n".join(out) + "\n")
    print("\n".join(out))


def _counter_per_kernel(path, counter):
    f = _find(path, "*counter_collection.csv")
    vals = {}
    for r in csv.DictReader(open(f)):
        if r["Counter_Name"] != counter:
            continue
        name = short_name(r["Kernel_Name"])
        if name:
            vals.setdefault(name, []).append(float(r["Counter_Value"]))
    return {k: statistics.median(v) for k, v in vals.items()}, {k: max(v) for k, v in vals.items()}


def traffic(args):
    copy_bytes = args.copy_bytes
    fetch, fetch_max = _counter_per_kernel(args.fetch_dir, "FETCH_SIZE")
    write, write_max = _counter_per_kernel(args.write_dir, "WRITE_SIZE")
    fetch["plain_copy"], write["plain_copy"] = fetch_max["plain_copy"], write_max["plain_copy"]
    if "plain_copy" not in fetch or "plain_copy" not in write:
        raise SystemExit("the plain copy kernel is missing from the counter runs")
    # a copy of N bytes reads N and writes N bytes; the calibration copy is
    # the largest copy dispatch of the run
    kf = copy_bytes / fetch_max["plain_copy"]
    kw = copy_bytes / write_max["plain_copy"]
    out = [f"# HBM traffic per launch (rocprofv3 --pmc): {args.title}", "",
           "Commands (from the repository root on the MI355X machine), one counter per run:", "",
           f"    {args.command_fetch}", f"    {args.command_write}", "",
           f"Counters are KiB per dispatch.  Each is scaled by what it reads for the "
           f"plain device copy of {copy_bytes} bytes that the benchmark runs "
           f"(bytes per counter unit: FETCH {kf:.1f}, WRITE {kw:.1f}).", "",
           f"Kernel sources hash: `{source_hash()}`", "",
           "| kernel | FETCH_SIZE (KiB) | WRITE_SIZE (KiB) | read bytes | written bytes | total bytes |",
           "|---|---|---|---|---|---|"]
    machine = []
    for name in sorted(set(fetch) & set(write)):
        rb, wb = fetch[name] * kf, write[name] * kw
        out.append(f"| {name} | {fetch[name]:.0f} | {write[name]:.0f} | {rb:.4g} | {wb:.4g} | {rb + wb:.4g} |")
        machine.append(f"traffic {name} {rb + wb:.0f}")
    out += ["", "Machine-readable (bytes per launch):", "", "```"] + machine + \
           [f"source_hash {source_hash()}", "```"]
    open(args.out, "w").write("\n".join(out) + "\n")
    print("\n".join(out))


def counters(args):
    """Per-kernel medians of every counter (or derived metric) of one --pmc
    run, one row per kernel."""
    f = _find(args.pmc_dir, "*counter_collection.csv")
    vals = {}
    names = []
    for r in csv.DictReader(open(f)):
        kn = short_name(r["Kernel_Name"])
        if not kn:
            continue
        c = r["Counter_Name"]
        if c not in names:
            names.append(c)
        vals.setdefault(kn, {}).setdefault(c, []).append(float(r["Counter_Value"]))
    out = [f"# rocprofv3 counters per launch: {args.title}", "",
           "Command (from the repository root on the MI355X machine):", "", f"    {args.command}", "",
           f"Kernel sources hash: `{source_hash()}`", "", args.note, "",
           "| kernel | launches | " + " | ".join(names) + " |", "|---|---|" + "---|" * len(names)]
    for kn in sorted(vals):
        row = [f"{statistics.median(vals[kn][c]):.4g}" if c in vals[kn] else "" for c in names]
        n = max(len(v) for v in vals[kn].values())
        out.append(f"| {kn} | {n} | " + " | ".join(row) + " |")
    open(args.out, "w").write("\n".join(out) + "\n")
    print("\n".join(out))


def read_traffic(path: str) -> dict | None:
    """Bytes per launch by kernel from a traffic summary, if it was measured on
    the current sources; else None."""
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"^source_hash (\w+)$", text, re.M)
    if not m or m.group(1) != source_hash():
        return None
    return {k: float(v) for k, v in re.findall(r"^traffic (\S+) ([0-9.eE+]+)$", text, re.M)}


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("out")
    s.add_argument("--command", required=True)
    s.add_argument("--title", default="benchmark")
    t = sub.add_parser("traffic")
    t.add_argument("fetch_dir")
    t.add_argument("write_dir")
    t.add_argument("out")
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--command-fetch", required=True)
    t.add_argument("--command-write", required=True)
    t.add_argument("--title", default="benchmark")
    c = sub.add_parser("counters")
    c.add_argument("pmc_dir")
    c.add_argument("out")
    c.add_argument("--command", required=True)
    c.add_argument("--title", default="benchmark")
    c.add_argument("--note", default="")
    a = ap.parse_args()
    {"stats": stats, "traffic": traffic, "counters": counters}[a.cmd](a)


if __name__ == "__main__":
    main()
