"""rocprofv3 helpers for the measurement summaries (measurement tooling that
sits beside bench.py; not part of the library).

``python profiling.py copy`` runs a plain
device-to-device copy of 256 MiB three times: the reference workload whose
FETCH_SIZE / WRITE_SIZE readings calibrate the HBM traffic counters.

``... profiling stats <kernel_stats.csv> <out.md> <command> [<kernel_trace.csv> [<skip_last> [<step-end kernel>]]]`` and
``... profiling traffic <kernel regex> <fetch.csv> <write.csv> <copy_fetch.csv>
<copy_write.csv> <out.json> <out.md> <commands...>`` turn rocprofv3 CSV output
into the short text summaries kept with the sources.
"""
import csv
import hashlib
import json
import os
import re
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(ROOT, "block_diffusion_drafter_softmax_amd", "csrc")

# Sources the streaming GEMM kernels are compiled from: a traffic summary is
# valid only for the sources it was taken on.
GEMM_SOURCES = [os.path.join(CSRC, f) for f in ("gemm.hip", "stream.h", "common.h", "kernels.h")]
COPY_BYTES = 256 << 20


def source_hash(paths=GEMM_SOURCES):
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def copy_probe():
    import torch
    a = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda").fill_(1)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(f"copied {COPY_BYTES} bytes x3", flush=True)


def _rows(path):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def counter_per_dispatch(path, name_re, counter):
    """Mean counter value (KiB) over the dispatches whose kernel name matches."""
    vals = [float(r["Counter_Value"]) for r in _rows(path)
            if r["Counter_Name"] == counter and re.search(name_re, r["Kernel_Name"])]
    if not vals:
        raise SystemExit(f"no {counter} rows for /{name_re}/ in {path}")
    return sum(vals) / len(vals), len(vals)


def copy_factor(path, counter):
    """Known bytes / counted bytes for the largest copy dispatch."""
    vals = [float(r["Counter_Value"]) for r in _rows(path)
            if r["Counter_Name"] == counter and "copy" in r["Kernel_Name"].lower()]
    counted_kib = max(vals)
    return (COPY_BYTES / 1024) / counted_kib, counted_kib


def write_stats(stats_csv, out_md, command, trace_csv=None, skip_last=0, last_kernel="verify_rows", top=24):
    rows = _rows(stats_csv)
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    lines = ["# Kernel time, rocprofv3 --kernel-trace --stats", "", "Command:", "", "```", command, "```", "",
             "| kernel | calls | total ms | avg us | min us | max us | % |", "|---|---|---|---|---|---|---|"]
    for r in rows[:top]:
        name = r["Name"].replace("|", "/")
        if len(name) > 90:
            name = name[:87] + "..."
        lines.append(f"| `{name}` | {r['Calls']} | {float(r['TotalDurationNs']) / 1e6:.3f} | "
                     f"{float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                     f"{float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.2f} |")
    if trace_csv:
        lines += ["", "## One decode step", ""] + step_breakdown(trace_csv, last_kernel=last_kernel,
                                                                 skip_last=skip_last)
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")


def step_breakdown(trace_csv, last_kernel="verify_rows", steps=10, skip_last=0):
    """Per-kernel time of one decode step, averaged over `steps` steps of a
    kernel trace (a step ends with the verification kernel), leaving out the
    final `skip_last` steps (e.g. a pass run with a kernel timer attached).
    Kernels between the dual-pass drafter's selection and assembly kernels
    are listed as its second pass."""
    rows = _rows(trace_csv)
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    ends = [i for i, r in enumerate(rows) if r["Kernel_Name"].replace("void ", "", 1).startswith(last_kernel)]
    if skip_last:
        ends = ends[:-skip_last]
    steps = min(steps, len(ends) - 1)
    agg, span, busy = {}, 0.0, 0.0
    for a, b in zip(ends[-steps - 1:-1], ends[-steps:]):
        seg = rows[a + 1: b + 1]
        span += (int(seg[-1]["End_Timestamp"]) - int(seg[0]["Start_Timestamp"])) / 1e3
        second = False
        for r in seg:
            k = r["Kernel_Name"].split("(")[0].replace("void ", "")
            if k.startswith("d2sd_select"):
                second = True
            elif k.startswith("d2sd_assemble"):
                second = False
            elif second:
                k += " (second pass)"
            dt = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
            n, t = agg.get(k, (0, 0.0))
            agg[k] = (n + 1, t + dt)
            busy += dt
    out = [f"Per step, mean of {steps} steps (the last {skip_last} of the trace left out): "
           f"first kernel start to last kernel end "
           f"{span / steps:.1f} us, kernels busy {busy / steps:.1f} us.", "",
           "| kernel | launches/step | us/step | avg us |", "|---|---|---|---|"]
    for k, (n, t) in sorted(agg.items(), key=lambda x: -x[1][1]):
        out.append(f"| `{k}` | {n / steps:g} | {t / steps:.1f} | {t / n:.2f} |")
    return out


def write_traffic(name_re, fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, out_json, out_md, commands):
    ff, ff_counted = copy_factor(copy_fetch_csv, "FETCH_SIZE")
    wf, wf_counted = copy_factor(copy_write_csv, "WRITE_SIZE")
    fetch_kib, n_f = counter_per_dispatch(fetch_csv, name_re, "FETCH_SIZE")
    write_kib, n_w = counter_per_dispatch(write_csv, name_re, "WRITE_SIZE")
    fetch_b = fetch_kib * 1024 * ff
    write_b = write_kib * 1024 * wf
    d = {"kernel_regex": name_re, "source_sha256_16": source_hash(),
         "fetch_kib_per_dispatch": fetch_kib, "write_kib_per_dispatch": write_kib,
         "dispatches": [n_f, n_w], "fetch_factor": ff, "write_factor": wf,
         "copy_counted_kib": {"FETCH_SIZE": ff_counted, "WRITE_SIZE": wf_counted},
         "bytes_per_launch": round(fetch_b + write_b)}
    with open(out_json, "w") as f:
        json.dump(d, f, indent=1)
        f.write("\n")
    lines = ["# HBM traffic per launch, rocprofv3 --pmc", "",
             f"Kernel: `{name_re}` ({n_f} dispatches), sources sha256[:16] {d['source_sha256_16']}.", "",
             "Calibration: a plain 256 MiB device copy reads "
             f"FETCH_SIZE {ff_counted:.0f} KiB and WRITE_SIZE {wf_counted:.0f} KiB for 262144 KiB moved, "
             f"so FETCH_SIZE is scaled by {ff:.4f} and WRITE_SIZE by {wf:.4f}.", "",
             "| counter | KiB/dispatch (raw) | factor | bytes/launch |", "|---|---|---|---|",
             f"| FETCH_SIZE | {fetch_kib:.1f} | {ff:.4f} | {fetch_b:.0f} |",
             f"| WRITE_SIZE | {write_kib:.1f} | {wf:.4f} | {write_b:.0f} |",
             f"| total | | | {fetch_b + write_b:.0f} |", "", "Commands:", "", "```"] + list(commands) + ["```"]
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    return d


def main(argv):
    if not argv:
        raise SystemExit(__doc__)
    if argv[0] == "copy":
        copy_probe()
    elif argv[0] == "stats":
        write_stats(argv[1], argv[2], argv[3], argv[4] if len(argv) > 4 else None,
                    int(argv[5]) if len(argv) > 5 else 0, argv[6] if len(argv) > 6 else "verify_rows")
    elif argv[0] == "traffic":
        print(json.dumps(write_traffic(*argv[1:8], argv[8:])))
    else:
        raise SystemExit(__doc__)


if __name__ == "__main__":
    main(sys.argv[1:])
