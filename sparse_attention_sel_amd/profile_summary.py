"""Summaries of rocprofv3 runs of the benchmark, as the text tables kept under
profiles/.  Reads rocprofv3's CSV output (``--output-format csv``) and writes
Markdown (and, for the traffic of the main stage, a JSON record that bench.py
reads back).  Three kinds:

  kernels  ``--kernel-trace --stats``: calls and average / min / max duration
           per kernel.
  traffic  two ``--pmc`` runs (FETCH_SIZE, WRITE_SIZE) of the benchmark and
           the same two of ``bench.py --copy-calibration`` (a plain 1 GiB
           device copy): each kernel's KiB per dispatch, scaled to bytes by
           what the counters read for the copy's known bytes, and GB/s over
           the kernel's average duration from a kernel-trace run.
  mfma     ``--pmc MfmaFlopsBF16 MfmaFlopsF16 MfmaUtil`` runs: MFMA FLOPs the
           matrix units executed per dispatch, their rate over the dispatch's
           duration, and the busy fraction.

    python -m sparse_attention_sel_amd.profile_summary kernels --trace DIR --title T --command C --out F.md
    python -m sparse_attention_sel_amd.profile_summary traffic --fetch DIR --write DIR --copy-fetch DIR \\
        --copy-write DIR --trace DIR --workload W --command C [--command C ...] --out F.md [--json F.json]
    python -m sparse_attention_sel_amd.profile_summary mfma --run W=DIR [--run W=DIR ...] --title T \\
        --command C --out F.md

Each output names the commands that produced its inputs and the command that
produced it.
"""

from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import re
import sys
from collections import defaultdict

PEAK_HBM_GBS = 8000.0
PEAK_MFMA_TFLOPS = 2500.0
COPY_BYTES = 1 << 30  # bytes read and written by one calibration copy

_TYPES = {"__bf16": "bf16", "_Float16": "fp16", "float": "fp32", "__hip_bfloat16": "bf16"}


# ---------------------------------------------------------------------------
# names
# ---------------------------------------------------------------------------
def _template_args(name: str, kernel: str):
    m = re.search(r"\b" + kernel + r"<([^>]*)>", name)
    if not m:
        return None
    return [a.strip() for a in m.group(1).split(",")]


_ARG = re.compile(r"DF16b|DF16_|f|Li(-?\d+)E|Lb([01])E")


def demangle(name: str) -> str:
    """The library's template kernels as rocprofv3 reports them (Itanium
    mangled, with bf16 / fp16 arguments its demangler leaves as they are),
    e.g. _ZN3fsa12_GLOBAL__N_16k_mainIDF16bLi128ELi64EDF16bLb0EE... ->
    fsa::(anonymous namespace)::k_main<__bf16, 128, 64, __bf16, false>.
    Other names are returned unchanged."""
    m = re.match(r"_ZN3fsa12_GLOBAL__N_1(\d+)", name)
    if not m:
        return name
    n = int(m.group(1))
    pos = m.end()
    kernel = name[pos : pos + n]
    pos += n
    if not name.startswith("I", pos):
        return f"fsa::(anonymous namespace)::{kernel}"
    pos += 1
    args = []
    while pos < len(name) and name[pos] != "E":
        a = _ARG.match(name, pos)
        if not a:
            return name
        tok = a.group(0)
        if tok == "DF16b":
            args.append("__bf16")
        elif tok == "DF16_":
            args.append("_Float16")
        elif tok == "f":
            args.append("float")
        elif a.group(1) is not None:
            args.append(a.group(1))
        else:
            args.append("true" if a.group(2) == "1" else "false")
        pos = a.end()
    return f"fsa::(anonymous namespace)::{kernel}<{', '.join(args)}>"


def pretty(name: str) -> str:
    """Readable kernel name: the library's kernels with their template
    arguments spelled out, other kernels shortened."""
    name = demangle(name)
    t = lambda x: _TYPES.get(x, x)  # noqa: E731
    for k in ("k_main_local", "k_main"):
        a = _template_args(name, k)
        if a and len(a) in (5, 6):
            split = ", two 64-key halves" if len(a) == 6 and a[5] == "true" else ""
            return (f"`{k}<{t(a[0])}, d={a[1]}, B_K={a[2]}, partial={t(a[3])}"
                    f"{', one-pass' if a[4] == 'true' else ''}{split}>`")
    a = _template_args(name, "k_main16")
    if a and len(a) == 5:
        split = ", two 64-key halves" if a[4] == "true" else ""
        return f"`k_main16<{t(a[0])}, d={a[1]}, B_K={a[2]}, partial={t(a[3])}{split}>`"
    a = _template_args(name, "k_main_mixed16")
    if a and len(a) == 2:
        return f"`k_main_mixed16<{t(a[0])}, d=256, B_K=64, partial={t(a[1])}>`"
    a = _template_args(name, "k_main_mixed")
    if a and len(a) == 4:
        return f"`k_main_mixed<{t(a[0])}, d={a[1]}, B_K={a[2]}, partial={t(a[3])}>`"
    a = _template_args(name, "k_main_local16")
    if a and len(a) == 2:
        return f"`k_main_local16<{t(a[0])}, d=256, B_K=64, partial={t(a[1])}>`"
    for k in ("k_stats_local", "k_stats", "k_nsa", "k_bwd_kv_reduce"):
        a = _template_args(name, k)
        if a and len(a) == 3:
            return f"`{k}<{t(a[0])}, d={a[1]}, B_K={a[2]}>`"
    a = _template_args(name, "k_bwd_main")
    if a and len(a) == 4:
        return f"`k_bwd_main<{t(a[0])}, d={a[1]}, B_K={a[2]}, partial={t(a[3])}>`"
    a = _template_args(name, "k_bwd_delta")
    if a and len(a) == 2:
        return f"`k_bwd_delta<{t(a[0])}, d={a[1]}>`"
    a = _template_args(name, "k_reduce")
    if a and len(a) in (4, 5):
        kind = "local" if a[2] == "true" else "all slots"
        split = ", two 64-key halves" if len(a) == 5 and a[4] == "true" else ""
        return f"`k_reduce<{t(a[0])}, partial={t(a[1])}, {kind}{', one-pass' if a[3] == 'true' else ''}{split}>`"
    a = _template_args(name, "k_select")
    if a and len(a) == 1:
        return f"`k_select<{'rows in registers' if a[0] == 'true' else 'rows from memory'}>`"
    a = _template_args(name, "k_mfma_loop")
    if a and len(a) == 1:
        return f"`k_mfma_loop<{t(a[0])}>`"
    m = re.search(r"\b(k_[a-z_]+)\b", name)
    if m and "fsa::" in name:
        return f"`{m.group(1)}`"
    if name.startswith("Cijk_"):
        return "`Cijk_...` (hipBLASLt GEMM)"
    short = re.sub(r"\(.*", "", name.replace("(anonymous namespace)::", "")).replace("void ", "").strip()
    if len(short) > 70:
        short = short[:67] + "..."
    return f"`{short}`"


# ---------------------------------------------------------------------------
# CSV inputs
# ---------------------------------------------------------------------------
def _one(directory: str, suffix: str) -> str:
    hits = sorted(glob.glob(os.path.join(directory, "**", "*" + suffix), recursive=True))
    if not hits:
        raise FileNotFoundError(f"no *{suffix} under {directory}")
    return max(hits, key=os.path.getsize)


def _rows(path: str):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def kernel_stats(directory: str):
    """{kernel name: (calls, avg ns, min ns, max ns, total ns)} of a
    --kernel-trace --stats run."""
    out = {}
    for r in _rows(_one(directory, "kernel_stats.csv")):
        out[r["Name"]] = (int(r["Calls"]), float(r["AverageNs"]), float(r["MinNs"]), float(r["MaxNs"]),
                          float(r["TotalDurationNs"]))
    return out


def counters(directory: str):
    """{kernel name: {counter: [value per dispatch]}} and {kernel name:
    [duration ns per dispatch]} of a --pmc run."""
    vals = defaultdict(lambda: defaultdict(dict))
    dur = defaultdict(dict)
    for r in _rows(_one(directory, "counter_collection.csv")):
        k = r["Kernel_Name"]
        d = r.get("Dispatch_Id") or r.get("Correlation_Id")
        vals[k][r["Counter_Name"]][d] = float(r["Counter_Value"])
        if r.get("Start_Timestamp") and r.get("End_Timestamp"):
            dur[k][d] = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
    return ({k: {c: list(v.values()) for c, v in cs.items()} for k, cs in vals.items()},
            {k: list(v.values()) for k, v in dur.items()})


def _mean(xs):
    return sum(xs) / len(xs) if xs else 0.0


# ---------------------------------------------------------------------------
# kinds
# ---------------------------------------------------------------------------
def write_kernels(a):
    st = kernel_stats(a.trace)
    total = sum(v[4] for v in st.values()) or 1.0
    lines = [f"# Kernel durations: {a.title}", ""]
    if a.note:
        lines += [a.note, ""]
    lines += ["Commands (repository root, MI355X):", ""]
    lines += [f"    {c}" for c in a.command] + [f"    {summary_command()}", ""]
    lines += ["| kernel | calls | avg us | min us | max us | share |", "|---|---|---|---|---|---|"]
    for name, (calls, avg, mn, mx, tot) in sorted(st.items(), key=lambda kv: -kv[1][4]):
        lines.append(f"| {pretty(name)} | {calls} | {avg / 1e3:.1f} | {mn / 1e3:.1f} | {mx / 1e3:.1f} | "
                     f"{100 * tot / total:.1f}% |")
    _write(a.out, lines)


def _copy_scale(directory: str, counter: str, nbytes: int) -> float:
    vals, _ = counters(directory)
    best = None
    for k, cs in vals.items():
        if "copyBuffer" in k and counter in cs:
            v = max(cs[counter])
            best = v if best is None else max(best, v)
    if not best:
        raise RuntimeError(f"no copy kernel with {counter} in {directory}")
    return nbytes / (best * 1024.0)


def write_traffic(a):
    fetch, _ = counters(a.fetch)
    write, _ = counters(a.write)
    fs = _copy_scale(a.copy_fetch, "FETCH_SIZE", COPY_BYTES)
    ws = _copy_scale(a.copy_write, "WRITE_SIZE", COPY_BYTES)
    st = kernel_stats(a.trace)
    rows = []
    for k in set(fetch) | set(write):
        fk = _mean(fetch.get(k, {}).get("FETCH_SIZE", []))
        wk = _mean(write.get(k, {}).get("WRITE_SIZE", []))
        n = max(len(fetch.get(k, {}).get("FETCH_SIZE", [])), len(write.get(k, {}).get("WRITE_SIZE", [])))
        avg = st.get(k, (0, 0.0))[1]
        fb, wb = fk * 1024 * fs, wk * 1024 * ws
        gbs = (fb + wb) / (avg * 1e-9) / 1e9 if avg else 0.0
        rows.append((k, n, fb, wb, fk, wk, avg, gbs))
    rows.sort(key=lambda r: -(r[2] + r[3]))
    lines = [f"# HBM traffic per launch: {a.workload}", ""]
    lines += [f"FETCH_SIZE and WRITE_SIZE (KiB per dispatch, averaged over each kernel's dispatches), scaled by what "
              f"the same counters read for a plain 1 GiB device-to-device copy (FETCH_SIZE x {fs:.4f}, "
              f"WRITE_SIZE x {ws:.4f} give the copy's bytes).  GB/s = (fetch + write bytes) / the kernel's "
              f"average duration in the kernel-trace run; % is of the 8 TB/s HBM peak (bytes served by the MALL "
              f"count too).", ""]
    if a.note:
        lines += [a.note, ""]
    lines += ["Commands (repository root, MI355X):", ""] + [f"    {c}" for c in a.command]
    lines += [f"    {summary_command()}", ""]
    lines += ["| kernel | dispatches | fetch GB | write GB | fetch KiB (raw) | write KiB (raw) | avg us | GB/s | "
              "% of 8 TB/s |", "|---|---|---|---|---|---|---|---|---|"]
    for k, n, fb, wb, fk, wk, avg, gbs in rows:
        lines.append(f"| {pretty(k)} | {n} | {fb / 1e9:.3f} | {wb / 1e9:.3f} | {fk:.0f} | {wk:.0f} | "
                     f"{avg / 1e3:.1f} | {gbs:.0f} | {100 * gbs / PEAK_HBM_GBS:.1f}% |")
    # the three-pass forward's main stage: k_main_mixed, or k_main / k_main16 and k_main_local /
    # k_main_local16, not the one-pass variants
    main = [r for r in rows
            if re.match(r"`k_main(_local|_mixed)?(16)?<", pretty(r[0])) and "one-pass" not in pretty(r[0])]
    if main:
        fb, wb = sum(r[2] for r in main), sum(r[3] for r in main)
        names = " + ".join(pretty(r[0]).strip("`") for r in main)
        lines += ["", f"Main stage = {names}: fetch {fb / 1e9:.3f} GB, write {wb / 1e9:.3f} GB per call."]
    _write(a.out, lines)
    if a.json and main:
        rec = {
            "kernel": " + ".join(pretty(r[0]).strip("`") for r in main),
            "fetch_bytes": sum(r[2] for r in main),
            "write_bytes": sum(r[3] for r in main),
            "fetch_kib_raw": sum(r[4] for r in main),
            "write_kib_raw": sum(r[5] for r in main),
            "source_sha256": a.source_sha256,
            "source_hash_note": "sha256 of the forward kernel sources without comments or blank lines "
                                "(bench.kernel_source_hash)",
            "workload": a.workload,
            "fetch_scale": fs,
            "write_scale": ws,
            "commands": list(a.command) + [summary_command()],
        }
        with open(a.json, "w") as f:
            json.dump(rec, f, indent=1)
            f.write("\n")


def write_mfma(a):
    lines = [f"# MFMA counters: {a.title}", ""]
    lines += ["Derived rocprofv3 counters per dispatch, averaged over every dispatch of each kernel in the run: "
              "`MfmaFlopsBF16` / `MfmaFlopsF16` (FLOPs the MFMA units executed, padding included) and "
              "`MfmaUtil` (MFMA busy cycles over active cycles x SIMDs, percent).  Durations are those of the same "
              "dispatches under counter collection; TFLOP/s = MFMA FLOPs / duration, against the 2.5 PFLOP/s "
              "dense bf16/fp16 peak.", ""]
    if a.note:
        lines += [a.note, ""]
    lines += ["Commands (repository root, MI355X):", ""] + [f"    {c}" for c in a.command]
    lines += [f"    {summary_command()}", ""]
    for spec in a.run:
        wname, directory = spec.split("=", 1)
        vals, dur = counters(directory)
        lines += [f"## {wname}", "", "| kernel | dispatches | MFMA GFLOP / dispatch | us / dispatch | MFMA TFLOP/s | "
                  "of 2.5 PF | MfmaUtil % |", "|---|---|---|---|---|---|---|"]
        rows = []
        for k, cs in vals.items():
            fl = [x + y for x, y in zip(cs.get("MfmaFlopsBF16", []), cs.get("MfmaFlopsF16", []))] or \
                 cs.get("MfmaFlopsBF16", []) or cs.get("MfmaFlopsF16", [])
            if not fl or max(fl) <= 0:
                continue
            flops, us = _mean(fl), _mean(dur.get(k, [])) / 1e3
            tf = flops / (us * 1e-6) / 1e12 if us else 0.0
            rows.append((k, len(fl), flops, us, tf, _mean(cs.get("MfmaUtil", []))))
        for k, n, flops, us, tf, util in sorted(rows, key=lambda r: pretty(r[0])):
            lines.append(f"| {pretty(k)} | {n} | {flops / 1e9:.1f} | {us:.0f} | {tf:.0f} | "
                         f"{100 * tf / PEAK_MFMA_TFLOPS:.1f}% | {util:.1f} |")
        lines.append("")
    _write(a.out, lines)


def _write(path, lines):
    with open(path, "w") as f:
        f.write("\n".join(lines).rstrip() + "\n")


def summary_command() -> str:
    return "python3 -m sparse_attention_sel_amd.profile_summary " + " ".join(
        a if " " not in a else repr(a) for a in sys.argv[1:])


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    sub = ap.add_subparsers(dest="kind", required=True)
    k = sub.add_parser("kernels")
    k.add_argument("--trace", required=True)
    k.add_argument("--title", required=True)
    k.add_argument("--note", default="")
    k.add_argument("--command", action="append", default=[])
    k.add_argument("--out", required=True)
    t = sub.add_parser("traffic")
    for n in ("--fetch", "--write", "--copy-fetch", "--copy-write", "--trace", "--workload", "--out"):
        t.add_argument(n, required=True)
    t.add_argument("--json", default=None)
    t.add_argument("--source-sha256", default=None)
    t.add_argument("--note", default="")
    t.add_argument("--command", action="append", default=[])
    m = sub.add_parser("mfma")
    m.add_argument("--run", action="append", required=True, help="WORKLOAD=DIR of a --pmc run")
    m.add_argument("--title", required=True)
    m.add_argument("--note", default="")
    m.add_argument("--command", action="append", default=[])
    m.add_argument("--out", required=True)
    a = ap.parse_args(argv)
    if a.kind == "kernels":
        write_kernels(a)
    elif a.kind == "traffic":
        if a.json and a.source_sha256 is None:
            root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
            sys.path.insert(0, root)
            import bench

            a.source_sha256 = bench.kernel_source_hash(root)
        write_traffic(a)
    else:
        write_mfma(a)


if __name__ == "__main__":
    main()
