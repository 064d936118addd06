"""rocprofv3 helpers for the measurement summaries (measurement tooling that
sits beside bench.py; not part of the library).

``python profiling.py copy`` runs a plain
device-to-device copy of 256 MiB three times: the reference workload whose
FETCH_SIZE / WRITE_SIZE readings calibrate the HBM traffic counters.

``... profiling stats <kernel_stats.csv> <out.md> <command> [<kernel_trace.csv> [<skip_last> [<step-end kernel>]]]`` and
``... profiling traffic <kernel regex> <fetch.csv> <write.csv> <copy_fetch.csv>
<copy_write.csv> <out.json> <out.md> <commands...>`` and
``... profiling counters <workload> <dir> <out.md> <commands...>`` (per-kernel
FETCH_SIZE / WRITE_SIZE and MFMA utilisation of one bench workload, from the
runs under <dir>/pmc_{fetch,write,mfma,copy_fetch,copy_write}) turn rocprofv3
CSV output into the short text summaries kept with the sources.
"""
import csv
import hashlib
import json
import os
import re
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(ROOT, "block_diffusion_drafter_softmax_amd", "csrc")

# Sources each measured kernel is compiled from: a traffic summary is valid
# only for the sources it was taken on.
GEMM_SOURCES = [os.path.join(CSRC, f) for f in ("gemm.hip", "stream.h", "common.h", "kernels.h")]
KERNEL_SOURCES = {
    "gate_up": GEMM_SOURCES,
    "attention": [os.path.join(CSRC, f) for f in ("attention.hip", "common.h", "kernels.h")],
    "lm_head": [os.path.join(CSRC, f) for f in ("mm.hip", "lmhead.hip", "stream.h", "common.h", "kernels.h")],
}
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
    """Mean counter value (KiB) over the dispatches whose kernel name matches
    (`regex#grid` also requires that grid size, in threads)."""
    name_re, _, grid = name_re.partition("#")
    vals = [float(r["Counter_Value"]) for r in _rows(path)
            if r["Counter_Name"] == counter and re.search(name_re, r["Kernel_Name"])
            and (not grid or r["Grid_Size"] == grid)]
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
    kernel trace (a step ends with the verification kernel `last_kernel` and
    holds an LM head launch), leaving out the final `skip_last` steps (e.g. a
    pass run with a kernel timer attached).
    Kernels between the dual-pass drafter's selection and assembly kernels
    are listed as its second pass."""
    rows = _rows(trace_csv)
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    name = [r["Kernel_Name"].replace("void ", "", 1) for r in rows]
    ends = [i for i, k in enumerate(name) if k.startswith(last_kernel)]
    # a step holds an LM head launch: verification passes run after the
    # timed steps (acceptance draws) end with the same kernel but are no step
    segs = [(a + 1, b + 1) for a, b in zip(ends[:-1], ends[1:])
            if any(k.startswith(("lmhead", "mm_lmhead")) for k in name[a + 1:b + 1])]
    if skip_last:
        segs = segs[:-skip_last]
    steps = min(steps, len(segs))
    agg, span, busy = {}, 0.0, 0.0
    for a, b in segs[-steps:]:
        seg = rows[a:b]
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


def write_traffic(name_re, fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, out_json, out_md, commands,
                  sources=GEMM_SOURCES):
    ff, ff_counted = copy_factor(copy_fetch_csv, "FETCH_SIZE")
    wf, wf_counted = copy_factor(copy_write_csv, "WRITE_SIZE")
    fetch_kib, n_f = counter_per_dispatch(fetch_csv, name_re, "FETCH_SIZE")
    write_kib, n_w = counter_per_dispatch(write_csv, name_re, "WRITE_SIZE")
    fetch_b = fetch_kib * 1024 * ff
    write_b = write_kib * 1024 * wf
    d = {"kernel_regex": name_re, "source_sha256_16": source_hash(sources),
         "fetch_kib_per_dispatch": fetch_kib, "write_kib_per_dispatch": write_kib,
         "dispatches": [n_f, n_w], "fetch_factor": ff, "write_factor": wf,
         "copy_counted_kib": {"FETCH_SIZE": ff_counted, "WRITE_SIZE": wf_counted},
         "bytes_per_launch": round(fetch_b + write_b)}
    with open(out_json, "w") as f:
        json.dump(d, f, indent=1)
        f.write("\n")
    lines = ["# HBM traffic per launch, rocprofv3 --pmc", "",
             f"Kernel: `{name_re}` ({n_f} dispatches; `#n`: grid size n only), sources sha256[:16] "
             f"{d['source_sha256_16']} ({', '.join(os.path.basename(p) for p in sources)}).", "",
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


def _dispatches(path):
    """{dispatch id: (kernel label, grid size, {counter: value}, duration ns)} of a counter run."""
    d = {}
    for r in _rows(path):
        k = int(r["Dispatch_Id"])
        name = r["Kernel_Name"].replace("void ", "").split("(")[0]
        e = d.setdefault(k, [name, int(r["Grid_Size"]), {}, int(r["End_Timestamp"]) - int(r["Start_Timestamp"])])
        e[2][r["Counter_Name"]] = float(r["Counter_Value"])
    return d


def _label(name, grid, last):
    """Tell the streaming GEMM's launches of the Qwen3-8B-shaped step apart
    by grid size (O and down share one: by their order); the tiled GEMM's by
    grid size (threads)."""
    if name.startswith("mm_kernel"):
        return f"{name} (grid {grid})", last
    if name != "ws_kernel<1, 4, 0>":
        return name, last
    n = {98304: "QKV", 114688: "append K/V"}.get(grid, "")
    if grid == 65536:
        n = "O" if last != "O" else "down"
        last = n
    return f"{name} ({n})" if n else name, last


def write_counters(workload, d, out_md, commands):
    """Per-kernel HBM bytes (FETCH_SIZE, WRITE_SIZE scaled by the copy probe's
    factors) and MFMA utilisation (MfmaUtil: the summed SQ_VALU_MFMA_BUSY_CYCLES
    over GRBM_GUI_ACTIVE of one XCC times the 1024 SIMDs) per dispatch."""
    ff, _ = copy_factor(os.path.join(d, "pmc_copy_fetch", "run_counter_collection.csv"), "FETCH_SIZE")
    wf, _ = copy_factor(os.path.join(d, "pmc_copy_write", "run_counter_collection.csv"), "WRITE_SIZE")
    agg = {}
    for kind in ("fetch", "write", "mfma"):
        p = os.path.join(d, f"pmc_{kind}", "run_counter_collection.csv")
        if not os.path.exists(p):
            continue
        last = None
        for k, (name, grid, c, dur) in sorted(_dispatches(p).items()):
            lab, last = _label(name, grid, last)
            a = agg.setdefault(lab, {})
            for cn, v in c.items():
                a.setdefault(cn, []).append(v)
            a.setdefault("dur_" + kind, []).append(dur)
    mean = lambda v: sum(v) / len(v)
    lines = [f"# Per-kernel counters, rocprofv3 --pmc: workload `{workload}`", "",
             f"FETCH_SIZE scaled by {ff:.4f}, WRITE_SIZE by {wf:.4f} (a plain 256 MiB device copy); "
             "MfmaUtil = sum of SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE of one XCC x 1024 SIMDs), "
             "the profiler's own formula (GRBM_GUI_ACTIVE is summed over the 8 XCCs in the CSV, so "
             "divided by 8). Kernels with no MFMA work show 0.", "",
             "| kernel | dispatches | FETCH bytes / dispatch | WRITE bytes / dispatch | MfmaUtil % |", "|---|---|---|---|---|"]
    rows = []
    for lab, a in agg.items():
        f = mean(a["FETCH_SIZE"]) * 1024 * ff if "FETCH_SIZE" in a else float("nan")
        w = mean(a["WRITE_SIZE"]) * 1024 * wf if "WRITE_SIZE" in a else float("nan")
        busy, gui = a.get("SQ_VALU_MFMA_BUSY_CYCLES"), a.get("GRBM_GUI_ACTIVE")
        util = 100 * sum(busy) / (sum(gui) / 8 * 1024) if busy and gui and sum(gui) else 0.0
        n = len(a.get("FETCH_SIZE", a.get("SQ_VALU_MFMA_BUSY_CYCLES", [0])))
        rows.append((f, lab, n, w, util))
    for f, lab, n, w, util in sorted(rows, key=lambda r: -(r[0] if r[0] == r[0] else 0)):
        if f != f or f < 1e5:
            continue
        lines.append(f"| `{lab}` | {n} | {f:,.0f} | {w:,.0f} | {util:.1f} |")
    lines += ["", "Commands:", "", "```"] + list(commands) + ["```"]
    with open(out_md, "w") as fo:
        fo.write("\n".join(lines) + "\n")


def main(argv):
    if not argv:
        raise SystemExit(__doc__)
    if argv[0] == "copy":
        copy_probe()
    elif argv[0] == "stats":
        write_stats(argv[1], argv[2], argv[3], argv[4] if len(argv) > 4 else None,
                    int(argv[5]) if len(argv) > 5 else 0, argv[6] if len(argv) > 6 else "verify_rows")
    elif argv[0] == "traffic":  # traffic [--sources gate_up|attention|lm_head] <regex> <csvs...> <json> <md> <cmds>
        srcs = GEMM_SOURCES
        if argv[1] == "--sources":
            srcs = KERNEL_SOURCES[argv[2]]
            argv = argv[2:]
        print(json.dumps(write_traffic(*argv[1:8], argv[8:], sources=srcs)))
    elif argv[0] == "counters":
        write_counters(argv[1], argv[2], argv[3], argv[4:])
    else:
        raise SystemExit(__doc__)


if __name__ == "__main__":
    main(sys.argv[1:])
