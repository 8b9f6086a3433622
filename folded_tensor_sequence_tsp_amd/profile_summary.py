"""Short text summaries of rocprofv3 runs of the benchmark, for ``profiles/``.

Reads the CSV output of three rocprofv3 runs of the same ``bench.py`` command:

* ``--kernel-trace --stats`` (``*_kernel_stats.csv``): calls and average
  duration per kernel;
* ``--pmc FETCH_SIZE`` and ``--pmc WRITE_SIZE`` (``*_counter_collection.csv``):
  KiB per dispatch.

A summary covers one unit: an entry point's kernels (``tsp_attn_core``
launches ``attn_kernel``, and for short sequences ``attn_combine_kernel``),
whose per-launch durations and bytes are summed.  With ``--first N --skip K`` the durations come from the
per-dispatch kernel trace (``*_kernel_trace.csv``) instead: the first N
dispatches of each of the unit's kernels, in dispatch order, less the first K
of them (the benchmark makes its unit-scale roofline launches of the attention
core before any other attention work, one untimed launch and then the timed
ones).

The counter runs also hold a plain device copy of known size (``bench.py
--copy-probe-mib``); the ratio of its true bytes to what each counter reads for
it is the calibration factor applied to the other kernels' counts (on gfx950
FETCH_SIZE reads about half of the bytes a copy moves, WRITE_SIZE all of them).

The summary ends with machine-readable lines that ``bench.py`` reads:
``avg_ms_per_launch`` and ``traffic_bytes_per_launch`` of the chosen unit and
``source_sha256`` of the sources it was built from, so that the figures are
dropped (null) as soon as the kernels' sources change.

    python -m folded_tensor_sequence_tsp_amd.profile_summary --trace DIR --fetch DIR --write DIR \\
        --kernel tsp_attn_core --copy-mib 1024 --command "..." --out profiles/NAME.md
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import os

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")

# Units a summary can cover: an entry point's kernels (matched by name prefix)
# and the sources they are built from (hashed into the summary).
# unit -> (kernel name prefixes, sources).  "kernels.h:Name" stands for the
# definition of struct Name in kernels.h only (the arguments the kernels read),
# so that unrelated declarations added there leave a summary valid.
UNITS = {
    "tsp_attn_core": (["attn_kernel", "attn_combine_kernel"],
                      ["attention.hip", "device_common.h", "kernels.h:AttnArgs"]),
    "attn_kernel": (["attn_kernel"], ["attention.hip", "device_common.h", "kernels.h:AttnArgs"]),
    "gemm_kernel": (["gemm_kernel"], ["gemm.hip", "device_common.h", "kernels.h:GemmArgs"]),
    # backward of the attention core (its transposed-tile pre-passes share the
    # forward's vt_prep_kernel and are listed in the table, not in the unit)
    "tsp_attn_core_backward": (["bwd_stats_kernel", "dkv_kernel", "dq_kernel"],
                               ["attn_backward.hip", "device_common.h", "kernels.h:AttnBwdArgs"]),
    # one whole forward layer (tsp_attn_project + tsp_attn_core + tsp_layer_post)
    "tsp_layer_forward": (["gemm_kernel", "attn_kernel", "attn_combine_kernel", "row_prep_kernel",
                           "bf16_to_f16_kernel"],
                          ["gemm.hip", "attention.hip", "prep.hip", "device_common.h", "kernels.h:GemmArgs",
                           "kernels.h:AttnArgs"]),
}
KERNEL_SOURCES = {k: v[1] for k, v in UNITS.items()}
# Units whose kernels launch several times per call, in different forms: their
# figures are totals over all matching dispatches divided by the dispatch count
# of the named kernel, which runs once per call (a layer has one attention
# launch, four GEMMs and two weight conversions).
PER_CALL = {"tsp_layer_forward": "attn_kernel"}


def _source_text(name: str) -> bytes:
    fname, _, struct = name.partition(":")
    with open(os.path.join(CSRC, fname), "rb") as f:
        text = f.read()
    if not struct:
        return text
    start = text.index(b"struct " + struct.encode() + b" {")
    return text[start:text.index(b"\n};", start) + 3]


def source_sha256(kernel: str) -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        h.update(name.encode() + b"\0" + _source_text(name))
    return h.hexdigest()


def _one(pattern: str) -> str:
    found = sorted(glob.glob(pattern))
    if not found:
        raise FileNotFoundError(pattern)
    return found[0]


def _short(name: str) -> str:
    name = name.replace("void ", "").replace("tsp::(anonymous namespace)::", "")
    return name.split("(")[0] if "tsp::" in name or "gemm_kernel" in name or "attn_kernel" in name else name[:60]


def kernel_stats(trace_dir: str):
    rows = list(csv.DictReader(open(_one(os.path.join(trace_dir, "*kernel_stats.csv")))))
    return [(_short(r["Name"]), int(r["Calls"]), float(r["AverageNs"]) / 1e6, float(r["Percentage"])) for r in rows]


def first_dispatch_ms(trace_dir: str, kernels, first: int, skip: int):
    """Per-call ms of a unit from the kernel trace: for each kernel prefix, the
    mean duration of its dispatches [skip, first) in dispatch order; summed over
    the unit's kernels (each launches once per call).  Returns (ms, calls)."""
    rows = list(csv.DictReader(open(_one(os.path.join(trace_dir, "*kernel_trace.csv")))))
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    total, calls = 0.0, None
    for k in kernels:
        durs = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e6 for r in rows
                if _short(r["Kernel_Name"]).startswith(k)][:first][skip:]
        if not durs:
            continue
        total += sum(durs) / len(durs)
        calls = len(durs) if calls is None else min(calls, len(durs))
    return total, calls or 0


def counters(pmc_dir: str):
    """{dispatch id: (kernel name, counter value KiB)}"""
    rows = list(csv.DictReader(open(_one(os.path.join(pmc_dir, "*counter_collection.csv")))))
    return {int(r["Dispatch_Id"]): (r["Kernel_Name"], float(r["Counter_Value"])) for r in rows}


def _copy_factor(cnt, copy_bytes: int) -> tuple:
    vals = [v for n, v in cnt.values() if "copyBuffer" in n]
    if len(vals) != 1:
        raise RuntimeError(f"expected one copy probe dispatch, found {len(vals)}")
    return copy_bytes / (vals[0] * 1024.0), vals[0]


def summarise(trace, fetch, write, unit, copy_mib, command, workload, first=None, skip=0):
    """Markdown summary of a kernel-trace run and, when fetch and write are
    given, of its two counter runs (traffic of the unit's kernels)."""
    stats = kernel_stats(trace)
    kernels = UNITS[unit][0]
    per = PER_CALL.get(unit)
    avg_ms = 0.0
    first_note = None
    if first:
        avg_ms, n_calls = first_dispatch_ms(trace, kernels, first, skip)
        first_note = (f"avg_ms_per_launch is the mean over dispatches {skip + 1}..{first} (in dispatch order, "
                      f"{n_calls} calls) of each of the unit's kernels, from the per-dispatch kernel trace: "
                      f"{avg_ms:.4f} ms per call.")
    elif per:
        calls = sum(c for n, c, _, _ in stats if n.startswith(per))
        avg_ms = sum(c * ms for n, c, ms, _ in stats if n.startswith(tuple(kernels))) / calls
    else:
        for k in kernels:
            avg_ms += sum(ms for n, _, ms, _ in stats if n.startswith(k))
    if fetch and write:
        f, w = counters(fetch), counters(write)
        copy_bytes = copy_mib << 20
        ff, f_copy = _copy_factor(f, copy_bytes)
        wf, w_copy = _copy_factor(w, copy_bytes)
        fetch_b = write_b = 0.0
        if per:
            mine = lambda n: "tsp::" in n and any(k in n for k in kernels)
            fetch_b = sum(v for n, v in f.values() if mine(n)) * 1024.0 * ff / sum(per in n for n, _ in f.values())
            write_b = sum(v for n, v in w.values() if mine(n)) * 1024.0 * wf / sum(per in n for n, _ in w.values())
        for k in kernels if not per else []:
            fk = [v for n, v in f.values() if k in n]
            wk = [v for n, v in w.values() if k in n]
            if not fk or not wk:  # a kernel of the unit that this workload does not launch
                continue
            fetch_b += sum(fk) / len(fk) * 1024.0 * ff
            write_b += sum(wk) / len(wk) * 1024.0 * wf
    lines = [f"# rocprofv3 summary: {unit} ({' + '.join(kernels)}), {workload}", "",
             "Commands (run from the repository root on the GPU; `-d`/`-o` name the output folders):", "",
             "```", *command.split(" ;; "), "```", "",
             "## Kernel time (--kernel-trace --stats)", "",
             "| kernel | calls | avg ms | % of GPU time |", "|---|---|---|---|"]
    lines += [f"| {n} | {c} | {ms:.4f} | {p:.2f} |" for n, c, ms, p in stats if "at::native" not in n]
    if first_note:
        lines += ["", first_note]
    if not (fetch and write):
        lines += ["", "## Machine-readable", "",
                  f"kernel: {unit}",
                  f"kernels: {', '.join(kernels)}",
                  f"avg_ms_per_launch: {avg_ms:.4f}",
                  "traffic_bytes_per_launch: none (no counter runs)",
                  f"source_sha256: {source_sha256(unit)}", ""]
        return "\n".join(lines)
    lines += ["", "## HBM traffic (--pmc FETCH_SIZE, --pmc WRITE_SIZE; KiB per dispatch)", "",
              f"Calibration: a plain {copy_mib} MiB device copy reads FETCH_SIZE = {f_copy:.0f} KiB and "
              f"WRITE_SIZE = {w_copy:.0f} KiB, so fetch counts are scaled by {ff:.4f} and write counts by {wf:.4f}.",
              "", "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | fetched bytes (scaled) | written bytes (scaled) |",
              "|---|---|---|---|---|"]
    seen = set()
    for d in sorted(f):
        n, v = f[d]
        if "tsp::" not in n or d not in w:
            continue
        key = _short(n)
        if key in seen:
            continue
        seen.add(key)
        lines.append(f"| {key} | {v:.0f} | {w[d][1]:.0f} | {v * 1024 * ff:.4e} | {w[d][1] * 1024 * wf:.4e} |")
    lines += ["", "## Machine-readable (read by bench.py)", "",
              f"kernel: {unit}",
              f"kernels: {', '.join(kernels)}",
              f"avg_ms_per_launch: {avg_ms:.4f}",
              f"traffic_bytes_per_launch: {fetch_b + write_b:.0f}",
              f"fetch_bytes_per_launch: {fetch_b:.0f}",
              f"write_bytes_per_launch: {write_b:.0f}",
              f"source_sha256: {source_sha256(unit)}", ""]
    return "\n".join(lines)


def _machine_values(path: str) -> dict:
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith(("#", "|", " ")):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    return vals


def read_avg_ms(path: str, unit: str):
    """avg_ms_per_launch of a summary (None when missing or taken from other sources)."""
    if not os.path.exists(path):
        return None
    vals = _machine_values(path)
    if vals.get("kernel") != unit or vals.get("source_sha256") != source_sha256(unit):
        return None
    try:
        return float(vals["avg_ms_per_launch"])
    except (KeyError, ValueError):
        return None


def read_traffic(path: str, unit: str):
    """traffic_bytes_per_launch from a summary, or None when it is missing or
    was taken from other sources of the kernels than the current ones."""
    if not os.path.exists(path):
        return None
    vals = _machine_values(path)
    if vals.get("kernel") != unit or vals.get("source_sha256") != source_sha256(unit):
        return None
    try:
        return float(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--trace", required=True)
    ap.add_argument("--fetch", default=None, help="FETCH_SIZE counter run (optional, with --write)")
    ap.add_argument("--write", default=None, help="WRITE_SIZE counter run (optional, with --fetch)")
    ap.add_argument("--kernel", default="tsp_attn_core", choices=sorted(UNITS))
    ap.add_argument("--copy-mib", type=int, default=1024)
    ap.add_argument("--command", required=True, help="the profiling commands, separated by ' ;; '")
    ap.add_argument("--workload", required=True)
    ap.add_argument("--out", required=True)
    ap.add_argument("--first", type=int, default=None,
                    help="per-call time from the first N dispatches of the unit's kernels (kernel trace)")
    ap.add_argument("--skip", type=int, default=0, help="of those, leave out the first K (untimed warmup)")
    a = ap.parse_args()
    text = summarise(a.trace, a.fetch, a.write, a.kernel, a.copy_mib, a.command, a.workload, a.first, a.skip)
    with open(a.out, "w") as fh:
        fh.write(text)
    print(text)


if __name__ == "__main__":
    main()
