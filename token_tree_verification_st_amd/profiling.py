"""Summaries of rocprofv3 output for profiles/ (host-side text processing).

    python -m token_tree_verification_st_amd.profiling stats   STATS_CSV OUT.md TITLE COMMAND \\
        [TRACE_CSV KERNEL_PREFIX]
    python -m token_tree_verification_st_amd.profiling linear_traffic FETCH_CSV WRITE_CSV \\
        COPY_BYTES LM_GRID OUT.md CMD_F CMD_W
    python -m token_tree_verification_st_amd.profiling traffic FETCH_CSV WRITE_CSV COPY_BYTES \\
        WORKLOAD OUT.md COMMAND_FETCH COMMAND_WRITE
    python -m token_tree_verification_st_amd.profiling kernels_traffic FETCH_CSV WRITE_CSV \\
        COPY_BYTES OUT.md TITLE COMMAND_FETCH COMMAND_WRITE KERNEL_PREFIX...
    python -m token_tree_verification_st_amd.profiling sq OUT.md KERNEL TITLE CSV... -- COMMAND...

`traffic` reads two --pmc runs of the same bench command (FETCH_SIZE, then
WRITE_SIZE, KiB per dispatch).  Each counter is scaled by what it reads for
the plain device copy of COPY_BYTES that `bench.py --copy-calibration` runs in
the same process, and the per-call HBM bytes of st_tree_attention (streaming
kernel + split merge) are written with the hash of the attention sources, so
bench.py can tell whether the figure still describes the built kernel.
"""

from __future__ import annotations

import csv
import hashlib
import os
import re
import sys
from collections import defaultdict

PKG = os.path.dirname(os.path.abspath(__file__))
ATTENTION_SOURCES = ("csrc/attention.hip", "csrc/st_internal.h", "csrc/step_internal.h",
                     "csrc/kv_compact_dev.h", "csrc/greedy_walk_dev.h", "csrc/stoch_walk_dev.h",
                     "build.py")
ATTENTION_KERNELS = ("attn_stream_kernel", "attn_valu_kernel", "attn_combine_kernel<")
COPY_KERNEL = "__amd_rocclr_copyBuffer"


def attention_source_hash() -> str:
    h = hashlib.sha256()
    for rel in ATTENTION_SOURCES:
        with open(os.path.join(PKG, rel), "rb") as f:
            h.update(rel.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def _short(name: str) -> str:
    n = name.replace("(anonymous namespace)::", "")
    n = re.sub(r"^void ", "", n)
    return n.split("(")[0]


def stats_md(stats_csv: str, title: str, command: str) -> str:
    rows = list(csv.DictReader(open(stats_csv)))
    out = [f"# {title}", "", "Command (run from /tmp with TMPDIR=/tmp; $R = repository root):", "",
           "```", command, "```", "",
           "| kernel | calls | avg us | min us | max us | share |", "|---|---|---|---|---|---|"]
    for r in rows:
        out.append(f"| {_short(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                   f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                   f"{float(r['Percentage']):.1f}% |")
    return "\n".join(out) + "\n"


LINEAR_SOURCES = ("csrc/layer.hip", "csrc/st_internal.h", "build.py")


def linear_source_hash() -> str:
    h = hashlib.sha256()
    for rel in LINEAR_SOURCES:
        with open(os.path.join(PKG, rel), "rb") as f:
            h.update(rel.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def grid_table(trace_csv: str, prefix: str) -> str:
    """Durations of the kernels whose short name starts with ``prefix``, per
    launch shape (grid size), from a --kernel-trace csv."""
    d = defaultdict(list)
    for r in csv.DictReader(open(trace_csv)):
        if _short(r["Kernel_Name"]).startswith(prefix):
            d[int(r["Grid_Size_X"])].append(
                (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    out = ["", f"{prefix} by launch shape:", "", "| grid (threads) | calls | avg us | min us |"
           " max us |", "|---|---|---|---|---|"]
    for g in sorted(d):
        v = d[g]
        out.append(f"| {g} | {len(v)} | {sum(v) / len(v):.2f} | {min(v):.2f} | {max(v):.2f} |")
    return "\n".join(out) + "\n"


def attention_calls_table(trace_csv: str) -> str:
    """The streaming attention kernel's launches split by what follows them on
    the same hardware queue: the split merge (a plain st_tree_attention call)
    or the merge + compaction launch (the one-call step, whose acceptance
    kernel may run beside it on another queue), with the plain calls'
    duration from the streaming kernel's start to the merge's end."""
    rows = sorted(csv.DictReader(open(trace_csv)), key=lambda r: int(r["Start_Timestamp"]))
    by_queue = defaultdict(list)
    for r in rows:
        by_queue[r["Queue_Id"]].append(r)
    plain, single, step, call = [], [], [], []
    for q in by_queue.values():
        for i, r in enumerate(q[:-1]):
            if not _short(r["Kernel_Name"]).startswith("attn_stream_kernel"):
                continue
            nxt = _short(q[i + 1]["Kernel_Name"])
            dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
            if nxt.startswith("attn_combine_kernel"):
                plain.append(dur)
                call.append((int(q[i + 1]["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
            elif nxt.startswith("attn_combine_compact_kernel"):
                step.append(dur)
            else:
                single.append(dur)
    out = ["", "attn_stream_kernel by caller (the launch that follows it on its queue):", "",
           "| launches | count | avg us | min us | max us |", "|---|---|---|---|---|"]
    for name, v in (("st_tree_attention (then the split merge)", plain),
                    ("st_tree_attention, one split a request (no merge)", single),
                    ("verification step (then merge + compaction)", step),
                    ("st_tree_attention call, stream start to merge end", call)):
        if v:
            out.append(f"| {name} | {len(v)} | {sum(v) / len(v):.2f} | {min(v):.2f} | "
                       f"{max(v):.2f} |")
    return "\n".join(out) + "\n"


def _per_grid(counter_csv: str, counter: str, prefix: str):
    """Per grid size of the kernels whose short name starts with ``prefix``:
    mean counter value (KiB) and dispatch count."""
    vals = defaultdict(list)
    for r in csv.DictReader(open(counter_csv)):
        if r["Counter_Name"] == counter and _short(r["Kernel_Name"]).startswith(prefix):
            vals[int(r["Grid_Size"])].append(float(r["Counter_Value"]))
    return {g: (sum(v) / len(v), len(v)) for g, v in vals.items()}


def linear_traffic_md(fetch_csv, write_csv, copy_bytes, lm_grid, cmd_f, cmd_w):
    """HBM bytes of the projection kernel per dispatch shape (grid size), scaled
    by the same run's calibration copy."""
    f = _per_dispatch(fetch_csv, "FETCH_SIZE")
    w = _per_dispatch(write_csv, "WRITE_SIZE")
    f_scale = copy_bytes / (f[COPY_KERNEL][2] * 1024.0)
    w_scale = copy_bytes / (w[COPY_KERNEL][2] * 1024.0)
    fg = _per_grid(fetch_csv, "FETCH_SIZE", "linear_kernel")
    wg = _per_grid(write_csv, "WRITE_SIZE", "linear_kernel")
    out = ["# st_linear HBM traffic, workload llama7b_layer", "",
           "Commands (run from /tmp with TMPDIR=/tmp; $R = repository root):", "",
           "```", cmd_f, cmd_w, "```", "",
           f"Calibration: a device copy of {copy_bytes} bytes in the same process reads "
           f"FETCH_SIZE x {f_scale:.3f} and WRITE_SIZE x {w_scale:.3f} of its true bytes.", "",
           "| linear_kernel grid (threads) | dispatches | fetch bytes | write bytes |",
           "|---|---|---|---|"]
    lm = None
    for g in sorted(set(fg) | set(wg)):
        fb = fg.get(g, (0.0, 0))[0] * 1024.0 * f_scale
        wb = wg.get(g, (0.0, 0))[0] * 1024.0 * w_scale
        out.append(f"| {g} | {fg.get(g, (0, 0))[1]} | {fb:.0f} | {wb:.0f} |")
        if g == lm_grid:
            lm = fb + wb
    out += ["", f"The vocabulary projection (32000 x 4096, 64 rows) is the grid of {lm_grid} "
            "threads.", "", "Machine-readable (read by bench.py):", "",
            f"source_sha256: {linear_source_hash()}",
            f"bytes_per_launch: {lm:.0f}", ""]
    return "\n".join(out)


def read_linear_traffic(path: str):
    if not os.path.exists(path):
        return None
    text = open(path).read()
    h = re.search(r"^source_sha256: (\w+)", text, re.M)
    b = re.search(r"^bytes_per_launch: (\d+)", text, re.M)
    if not h or not b or h.group(1) != linear_source_hash():
        return None
    return int(b.group(1))


def _per_dispatch(counter_csv: str, counter: str):
    """Per kernel name: (mean counter value in KiB over its dispatches, number
    of dispatches, largest single value)."""
    vals = defaultdict(list)
    for r in csv.DictReader(open(counter_csv)):
        if r["Counter_Name"] == counter:
            vals[_short(r["Kernel_Name"])].append(float(r["Counter_Value"]))
    return {k: (sum(v) / len(v), len(v), max(v)) for k, v in vals.items()}


def traffic(fetch_csv: str, write_csv: str, copy_bytes: int):
    f = _per_dispatch(fetch_csv, "FETCH_SIZE")
    w = _per_dispatch(write_csv, "WRITE_SIZE")
    if COPY_KERNEL not in f or COPY_KERNEL not in w:
        raise SystemExit("the calibration copy is missing from the counter runs")
    # the calibration copy is the largest copy dispatch of the run
    f_scale = copy_bytes / (f[COPY_KERNEL][2] * 1024.0)
    w_scale = copy_bytes / (w[COPY_KERNEL][2] * 1024.0)
    per_kernel = {}
    for k in sorted(set(f) | set(w)):
        if any(k.startswith(p.rstrip("<")) for p in ATTENTION_KERNELS) and \
                ("combine_compact" not in k):
            fb = f.get(k, (0.0, 0, 0.0))[0] * 1024.0 * f_scale
            wb = w.get(k, (0.0, 0, 0.0))[0] * 1024.0 * w_scale
            per_kernel[k] = (fb, wb, f.get(k, (0, 0, 0))[1])
    return f_scale, w_scale, per_kernel


def traffic_md(fetch_csv, write_csv, copy_bytes, workload, cmd_f, cmd_w):
    f_scale, w_scale, per_kernel = traffic(fetch_csv, write_csv, copy_bytes)
    total = sum(fb + wb for fb, wb, _ in per_kernel.values())
    out = [f"# st_tree_attention HBM traffic, workload {workload}", "",
           "Commands (run from /tmp with TMPDIR=/tmp; $R = repository root):", "",
           "```", cmd_f, cmd_w, "```", "",
           f"Calibration: a device copy of {copy_bytes} bytes in the same process reads "
           f"FETCH_SIZE x {f_scale:.3f} and WRITE_SIZE x {w_scale:.3f} of its true bytes.", "",
           "| kernel | dispatches | fetch bytes | write bytes |", "|---|---|---|---|"]
    for k, (fb, wb, n) in per_kernel.items():
        out.append(f"| {k} | {n} | {fb:.0f} | {wb:.0f} |")
    # the split partials: written by the streaming kernel, read back by the merge
    partials = sum(wb for k, (fb, wb, n) in per_kernel.items() if k.startswith("attn_stream")) + \
        sum(fb for k, (fb, wb, n) in per_kernel.items() if k.startswith("attn_combine"))
    merges = any(k.startswith("attn_combine") for k in per_kernel)
    out += ["", f"Split partials (the streaming kernel's writes{' and the merge reading them back' if merges else ''}): "
            f"{partials:.0f} bytes per call." if merges else
            "", "Machine-readable (read by bench.py):", "",
            f"source_sha256: {attention_source_hash()}",
            f"bytes_per_launch: {total:.0f}",
            f"split_partial_bytes: {partials if merges else 0:.0f}", ""]
    return "\n".join(out)


def read_traffic(path: str, field: str = "bytes_per_launch"):
    """bytes_per_launch (or another figure, e.g. split_partial_bytes) from a
    traffic summary, or None when the summary is missing or was taken from
    different attention sources."""
    if not os.path.exists(path):
        return None
    text = open(path).read()
    h = re.search(r"^source_sha256: (\w+)", text, re.M)
    b = re.search(rf"^{field}: (\d+)", text, re.M)
    if not h or not b or h.group(1) != attention_source_hash():
        return None
    return int(b.group(1))


def kernels_traffic_md(fetch_csv, write_csv, copy_bytes, title, cmd_f, cmd_w, prefixes):
    """HBM bytes per dispatch of every kernel whose short name starts with one
    of ``prefixes``, scaled by the same run's calibration copy."""
    f = _per_dispatch(fetch_csv, "FETCH_SIZE")
    w = _per_dispatch(write_csv, "WRITE_SIZE")
    if COPY_KERNEL not in f or COPY_KERNEL not in w:
        raise SystemExit("the calibration copy is missing from the counter runs")
    f_scale = copy_bytes / (f[COPY_KERNEL][2] * 1024.0)
    w_scale = copy_bytes / (w[COPY_KERNEL][2] * 1024.0)
    out = [f"# {title}", "", "Commands (run from /tmp with TMPDIR=/tmp; $R = repository root):",
           "", "```", cmd_f, cmd_w, "```", "",
           f"Calibration: a device copy of {copy_bytes} bytes in the same process reads "
           f"FETCH_SIZE x {f_scale:.3f} and WRITE_SIZE x {w_scale:.3f} of its true bytes.", "",
           "| kernel | dispatches | fetch bytes | write bytes |", "|---|---|---|---|"]
    for k in sorted(set(f) | set(w)):
        if any(k.startswith(p) for p in prefixes):
            fb = f.get(k, (0.0, 0, 0.0))[0] * 1024.0 * f_scale
            wb = w.get(k, (0.0, 0, 0.0))[0] * 1024.0 * w_scale
            out.append(f"| {k} | {f.get(k, (0, 0, 0))[1]} | {fb:.0f} | {wb:.0f} |")
    return "\n".join(out) + "\n"


def sq_md(csvs, kernel: str, title: str, commands) -> str:
    """SQ counters of one kernel from rocprofv3 --pmc passes: the average per
    dispatch over the kernel's dispatches, and per wavefront (SQ_WAVES)."""
    sums, counts = {}, {}
    for path in csvs:
        with open(path, newline="") as f:
            for r in csv.DictReader(f):
                if _short(r["Kernel_Name"]) != kernel:
                    continue
                c = r["Counter_Name"]
                sums[c] = sums.get(c, 0.0) + float(r["Counter_Value"])
                counts[c] = counts.get(c, 0) + 1
    avg = {c: sums[c] / counts[c] for c in sums}
    waves = avg.get("SQ_WAVES", 1.0) or 1.0
    n = max(counts.values()) if counts else 0
    out = [f"# {title}", "", "Commands (run from /tmp with TMPDIR=/tmp; $R = repository root), "
           "one pass each:", "", "```", *commands, "```", "",
           f"Average per dispatch over the {n} dispatches of `{kernel}` "
           f"({waves:.0f} wavefronts each):", "", "| counter | per dispatch | per wavefront |",
           "|---|---|---|"]
    for c in sorted(avg):
        out.append(f"| {c} | {avg[c]:.0f} | {avg[c] / waves:.1f} |")
    if "SQ_WAVE_CYCLES" in avg:
        wc = avg["SQ_WAVE_CYCLES"]
        parts = [f"{k} / SQ_WAVE_CYCLES = {100 * avg[k] / wc:.0f}%"
                 for k in ("SQ_WAIT_ANY", "SQ_ACTIVE_INST_ANY", "SQ_WAIT_INST_ANY") if k in avg]
        out += ["", "Shares of wavefront time: " + ", ".join(parts) + "."]
    return "\n".join(out) + "\n"


def main(argv):
    if argv[0] == "stats":
        stats_csv, out, title, command = argv[1:5]
        text = stats_md(stats_csv, title, command)
        if len(argv) > 6:   # TRACE_CSV KERNEL_PREFIX: add a per-launch-shape table
            text += grid_table(argv[5], argv[6])
            if argv[6] == "attn_stream_kernel":
                text += attention_calls_table(argv[5])
        open(out, "w").write(text)
    elif argv[0] == "linear_traffic":
        fcsv, wcsv, copy_bytes, lm_grid, out, cmd_f, cmd_w = argv[1:8]
        open(out, "w").write(linear_traffic_md(fcsv, wcsv, int(copy_bytes), int(lm_grid), cmd_f,
                                               cmd_w))
    elif argv[0] == "sq":   # OUT KERNEL TITLE CSV... -- COMMAND...
        out, kernel, title = argv[1:4]
        i = argv.index("--")
        open(out, "w").write(sq_md(argv[4:i], kernel, title, argv[i + 1:]))
    elif argv[0] == "kernels_traffic":   # FETCH WRITE COPY OUT TITLE CMD_F CMD_W PREFIX...
        fcsv, wcsv, copy_bytes, out, title, cmd_f, cmd_w = argv[1:8]
        open(out, "w").write(kernels_traffic_md(fcsv, wcsv, int(copy_bytes), title, cmd_f, cmd_w,
                                                argv[8:]))
    elif argv[0] == "traffic":
        fcsv, wcsv, copy_bytes, workload, out, cmd_f, cmd_w = argv[1:8]
        open(out, "w").write(traffic_md(fcsv, wcsv, int(copy_bytes), workload, cmd_f, cmd_w))
    else:
        raise SystemExit(__doc__)


if __name__ == "__main__":
    main(sys.argv[1:])
