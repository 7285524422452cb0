"""Summaries of rocprofv3 runs of bench.py, as committed under profiles/.

    python profile_summary.py times   --run TAG:DIR ... --cmd CMD --md OUT.md [--bench-log LOG]
    python profile_summary.py traffic --fetch TAG:DIR ... --write TAG:DIR ... --cmd CMD --json OUT.json --md OUT.md
    python profile_summary.py pmc     --run TAG:DIR ... --cmd CMD --json OUT.json --md OUT.md

Each DIR is a rocprofv3 output directory (``-d DIR --output-format csv``);
TAG says which bench legs the run held: ``headline`` (``--legs prefill,copy``),
``long`` (``--legs long,copy``) or ``legs`` (the other legs, ``copy``
included).  Kernels are named by what they compute for a workload
(``gdn_out_kernel`` is the 2 x 16 x 8192 prefill's; the gated-delta kernels
of a ``long`` run, the 1 x 16 x 262144 prefill, get the suffix ``_long``, and
those of a ``legs`` run belong to the packed batch and get ``_varlen_16seq``).

* times: per-kernel call counts and durations from the kernel trace.
* traffic: HBM bytes per dispatch = FETCH_SIZE x f + WRITE_SIZE x w (KiB),
  f and w chosen so that the same counters on the 256 MiB device copy of the
  run read 256 MiB each; written with the SHA-256 of each kernel's source, so
  bench.py can tell when a figure no longer describes the code.
* pmc: MfmaUtil, MfmaFlopsBF16, LdsUtil, LdsBankConflict per dispatch (the
  derived counters of rocprofv3 for gfx950) and the mean duration from the
  kernel trace of the same run.
"""

import argparse
import csv
import glob
import hashlib
import json
import os
import statistics
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
CSRC = "gated_delta_rule_causal_amd/csrc/"
SOURCES = {
    "gdn_": CSRC + "gdn_mfma.hip",
    "la_": CSRC + "la_mfma.hip",
    "gla_": CSRC + "la_mfma.hip",
    "recurrent_kernel": CSRC + "recurrent.hip",
    "kda_": CSRC + "kda_chunk.hip",
    "gdn_preprocess": CSRC + "preops.hip",
}
COPY_BYTES = 256 << 20
SETTLE_WORKGROUPS = 64 * 32 * 2   # bench.py settle(): 64 x 32 heads, two workgroups per head


def short_name(name):
    """Kernel name without namespaces and argument list, template arguments kept."""
    name = name.replace("(anonymous namespace)::", "").replace("la::", "").replace("void ", "")
    return name.split("(")[0].strip()


def kernel_key(name, tag, wg=None):
    """Name of a dispatch in the summaries; None for kernels not summarised,
    among them the bench's clock-settling decode steps (64 sequences x 32
    heads, 4096 workgroups: `wg`), which are not a measured leg."""
    s = short_name(name)
    base = s.split("<")[0]
    targs = [a.strip() for a in s[len(base) + 1:-1].split(",")] if "<" in s else []
    if base in ("gdn_map_kernel", "gdn_lead_map_kernel", "gdn_combine_kernel", "gdn_out_kernel",
                "gdn_varlen_plan_kernel"):
        return base + {"legs": "_varlen_16seq", "long": "_long"}.get(tag, "")
    if base == "la_chunked_mfma_kernel" and len(targs) == 3:   # <GATED, OUT, PACKED>
        return (("gla" if targs[0] == "true" else "la") + "_chunked_mfma_kernel_" +
                ("out" if targs[1] == "true" else "state") + ("_varlen" if targs[2] == "true" else ""))
    if base == "la_combine_kernel" and targs:
        return "gla_combine_kernel" if targs[0] == "true" else "la_combine_kernel"
    if base == "recurrent_kernel" and len(targs) == 6:
        kind = {"0": "normalized", "1": "gated_delta", "2": "gated", "3": "kda"}.get(targs[0], targs[0])
        if targs[5] != "true":
            return f"recurrent_kernel_{kind}_recurrent_prefill"
        return None if wg == SETTLE_WORKGROUPS else f"recurrent_kernel_{kind}_decode"
    if base == "gdn_preprocess_kernel":
        return base + ("_varlen" if targs and targs[-1] == "true" else "")
    if base in ("kda_tile_kernel", "kda_scan_kernel"):
        return base
    if "copyBuffer" in base:
        return "copy"
    return None


def source_of(key):
    for prefix in sorted(SOURCES, key=len, reverse=True):
        if key.startswith(prefix):
            return SOURCES[prefix]
    return None


def sha256(path):
    return hashlib.sha256(open(os.path.join(ROOT, path), "rb").read()).hexdigest()


def runs(specs):
    for spec in specs:
        tag, _, d = spec.partition(":")
        if tag not in ("headline", "long", "legs") or not d:
            sys.exit(f"bad run spec {spec!r}: expected headline:DIR, long:DIR or legs:DIR")
        yield tag, d


def read_csvs(d, suffix):
    files = sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True))
    if not files:
        sys.exit(f"no *{suffix} under {d}")
    rows = []
    for f in files:
        with open(f, newline="") as fh:
            rows.extend(csv.DictReader(fh))
    return rows


def col(row, *names):
    for n in names:
        if n in row and row[n] != "":
            return row[n]
    raise KeyError(f"none of {names} in {sorted(row)}")


def workgroups(row):
    g = int(float(col(row, "Grid_Size_X", "Grid_Size")))
    w = int(float(col(row, "Workgroup_Size_X", "Workgroup_Size")))
    return g // max(w, 1)


def trace_durations(d, tag):
    """{key: [duration_us, ...]} and {short name: [(workgroups, us), ...]} from a kernel trace."""
    by_key, by_name = {}, {}
    for r in read_csvs(d, "kernel_trace.csv"):
        us = (int(col(r, "End_Timestamp")) - int(col(r, "Start_Timestamp"))) / 1e3
        name = col(r, "Kernel_Name")
        by_name.setdefault(short_name(name), []).append((workgroups(r), us))
        k = kernel_key(name, tag, workgroups(r))
        if k:
            by_key.setdefault(k, []).append(us)
    return by_key, by_name


def counters(d, tag):
    """{key: {counter: [value per dispatch, ...]}} from counter_collection.csv."""
    per = {}
    for r in read_csvs(d, "counter_collection.csv"):
        k = kernel_key(col(r, "Kernel_Name"), tag, workgroups(r))
        if not k:
            continue
        disp = col(r, "Dispatch_Id", "Correlation_Id")
        per.setdefault(k, {}).setdefault(col(r, "Counter_Name"), {})
        cur = per[k][col(r, "Counter_Name")]
        cur[disp] = cur.get(disp, 0.0) + float(col(r, "Counter_Value"))
    return {k: {c: list(v.values()) for c, v in cs.items()} for k, cs in per.items()}


def header(title, cmds):
    out = [f"# {title}", "", "Commands (from the repository root on one MI355X, gfx950):", "", "```"]
    out += cmds
    out += ["```", ""]
    return out


def do_times(a):
    lines = header("Kernel times (rocprofv3 --kernel-trace)", a.cmd)
    lines += ["| kernel | workgroups | calls | avg µs | min µs | max µs |", "|---|---:|---:|---:|---:|---:|"]
    for tag, d in runs(a.run):
        _, by_name = trace_durations(d, tag)
        rows = []
        for name, xs in by_name.items():
            for wg in sorted({w for w, _ in xs}):
                if kernel_key(name, tag, wg) in (None, "copy"):
                    continue   # torch's own kernels (uploads, input draws), copies, clock settling: not the path
                us = [u for w, u in xs if w == wg]
                rows.append((sum(us), name, wg, us))
        for _, name, wg, us in sorted(rows, reverse=True):
            lines.append(f"| `{name}` ({tag}) | {wg} | {len(us)} | {statistics.mean(us):.2f} | {min(us):.2f} | "
                         f"{max(us):.2f} |")
    if a.bench_log:
        js = [l for l in open(a.bench_log) if l.startswith("{")]
        if js:
            rec = json.loads(js[-1])
            keep = {k: rec.get(k) for k in ("value", "unit", "steps", "warmup", "ms_per_step", "roofline")}
            lines += ["", "bench.py line printed by the same run (its HIP-event timings):", "", "```json",
                      json.dumps(keep), "```"]
    open(a.md, "w").write("\n".join(lines) + "\n")


def do_traffic(a):
    fetch, write = {}, {}
    for tag, d in runs(a.fetch):
        for k, cs in counters(d, tag).items():
            fetch.setdefault(k, []).extend(cs.get("FETCH_SIZE", []))
    for tag, d in runs(a.write):
        for k, cs in counters(d, tag).items():
            write.setdefault(k, []).extend(cs.get("WRITE_SIZE", []))
    # the copy dispatches that moved the 256 MiB buffer: the largest ones
    f_copy = max(fetch.get("copy", [0]))
    w_copy = max(write.get("copy", [0]))
    if f_copy <= 0 or w_copy <= 0:
        sys.exit("no device copy in the runs: run bench.py with the 'copy' leg")
    fs, ws = COPY_BYTES / (f_copy * 1024), COPY_BYTES / (w_copy * 1024)
    out = {"note": f"HBM bytes per dispatch: FETCH_SIZE x {fs:.4f} + WRITE_SIZE x {ws:.4f} (KiB -> bytes), factors "
                   "from a 256 MiB device copy in the same runs", "fetch_scale": fs, "write_scale": ws, "kernels": {}}
    lines = header("HBM traffic per dispatch (rocprofv3 --pmc FETCH_SIZE, WRITE_SIZE)", a.cmd)
    lines += [f"Scale factors from the 256 MiB device copy: FETCH_SIZE x {fs:.4f}, WRITE_SIZE x {ws:.4f}.", "",
              "| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM MiB read | HBM MiB written |",
              "|---|---:|---:|---:|---:|---:|"]
    for k in sorted(set(fetch) & set(write)):
        src = source_of(k)
        if src is None:
            continue
        fk, wk = statistics.median(fetch[k]), statistics.median(write[k])
        rb, wb = fk * 1024 * fs, wk * 1024 * ws
        out["kernels"][k] = {"bytes_per_dispatch": rb + wb, "read_bytes": rb, "write_bytes": wb, "source": src,
                             "source_sha256": sha256(src)}
        lines.append(f"| `{k}` | {len(fetch[k])} | {fk:.0f} | {wk:.0f} | {rb / 2**20:.1f} | {wb / 2**20:.1f} |")
    json.dump(out, open(a.json, "w"), indent=1)
    open(a.md, "w").write("\n".join(lines) + "\n")


def do_pmc(a):
    names = ("MfmaUtil", "MfmaFlopsBF16", "LdsUtil", "LdsBankConflict")
    out = {"note": "rocprofv3 --pmc " + " ".join(names) + " (derived counters of gfx950), median per dispatch; avg_us "
                   "from the kernel trace of the same run", "kernels": {}}
    lines = header("MFMA and LDS counters per dispatch (rocprofv3 --pmc)", a.cmd)
    lines += ["MfmaUtil: MFMA busy cycles / (GPU busy cycles x SIMDs); LdsUtil: LDS busy cycles / (GPU busy cycles x "
              "CUs); LdsBankConflict: bank-conflict cycles per conflict-free LDS cycle; MFMA TFLOP/s: MfmaFlopsBF16 / "
              "avg µs (dense tile flops as issued).", "",
              "| kernel | dispatches | avg µs | MfmaUtil % | MFMA TFLOP/s | LdsUtil % | LdsBankConflict |",
              "|---|---:|---:|---:|---:|---:|---:|"]
    for tag, d in runs(a.run):
        cs = counters(d, tag)
        dur, _ = trace_durations(d, tag)
        for k in sorted(cs):
            src = source_of(k)
            if src is None or not all(n in cs[k] for n in names) or k not in dur:
                continue
            rec = {n: statistics.median(cs[k][n]) for n in names}
            rec["avg_us"] = statistics.mean(dur[k])
            rec["dispatches"] = len(cs[k]["MfmaUtil"])
            rec["source"], rec["source_sha256"] = src, sha256(src)
            out["kernels"][k] = rec
            tf = rec["MfmaFlopsBF16"] / (rec["avg_us"] * 1e-6) / 1e12
            lines.append(f"| `{k}` | {rec['dispatches']} | {rec['avg_us']:.2f} | {rec['MfmaUtil']:.1f} | {tf:.1f} | "
                         f"{rec['LdsUtil']:.1f} | {rec['LdsBankConflict']:.3f} |")
    json.dump(out, open(a.json, "w"), indent=1)
    open(a.md, "w").write("\n".join(lines) + "\n")


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    t = sub.add_parser("times")
    t.add_argument("--run", nargs="+", required=True)
    t.add_argument("--bench-log")
    tr = sub.add_parser("traffic")
    tr.add_argument("--fetch", nargs="+", required=True)
    tr.add_argument("--write", nargs="+", required=True)
    tr.add_argument("--json", required=True)
    p = sub.add_parser("pmc")
    p.add_argument("--run", nargs="+", required=True)
    p.add_argument("--json", required=True)
    for s in (t, tr, p):
        s.add_argument("--cmd", action="append", required=True, help="a command that made the runs (repeatable)")
        s.add_argument("--md", required=True)
    a = ap.parse_args()
    {"times": do_times, "traffic": do_traffic, "pmc": do_pmc}[a.what](a)


if __name__ == "__main__":
    main()
