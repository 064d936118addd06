"""Host logic of the profile summaries: how a kernel trace is cut into decode
steps (CPU only, synthetic trace rows)."""
import csv

import profiling


def _trace(path, names):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        t = 0
        for n in names:
            w.writerow({"Kernel_Name": n, "Start_Timestamp": t, "End_Timestamp": t + 1000})
            t += 2000


def test_steps_hold_an_lm_head_and_skip_trailing_passes(tmp_path):
    step = ["ws_kernel<1, 4, 0>(WsArgs)", "lmhead_kernel<1, 4>(LmArgs)", "verify_rows_kernel<0>(VerifyArgs)",
            "verify_greedy_kernel(VerifyArgs)"]
    draw = ["verify_rows_kernel<0>(VerifyArgs)", "verify_greedy_kernel(VerifyArgs)"]
    timed = ["ws_kernel<1, 4, 0>(WsArgs)"] * 3 + step[1:]  # a second, event-timed pass: 3 launches
    names = step * 4 + timed * 2 + draw * 5
    p = tmp_path / "trace.csv"
    _trace(p, names)
    out = profiling.step_breakdown(str(p), last_kernel="verify_greedy", steps=10, skip_last=2)
    # segments: 4 steps (the first one has no predecessor delimiter), 2 timed
    # ones (skipped), 5 draws (no LM head); 3 steps remain
    assert out[0].startswith("Per step, mean of 3 steps")
    rows = {r.split("`")[1]: r.split("|")[2].strip() for r in out if r.startswith("| `")}
    assert rows == {"ws_kernel<1, 4, 0>": "1", "lmhead_kernel<1, 4>": "1", "verify_rows_kernel<0>": "1",
                    "verify_greedy_kernel": "1"}
    # each step: 4 kernels of 1 us, 2 us apart -> 7 us start to end
    assert "end 7.0 us, kernels busy 4.0 us" in out[0]


def test_second_pass_kernels_are_labelled(tmp_path):
    step = ["mm_lmhead_kernel", "d2sd_select_kernel", "mm_kernel<0, 4>", "mm_lmhead_kernel",
            "d2sd_assemble_kernel", "verify_greedy_kernel"]
    p = tmp_path / "trace.csv"
    _trace(p, step * 3)
    out = profiling.step_breakdown(str(p), last_kernel="verify_greedy", steps=10)
    names = {r.split("`")[1] for r in out if r.startswith("| `")}
    assert names == {"mm_lmhead_kernel", "d2sd_select_kernel", "mm_kernel<0, 4> (second pass)",
                     "mm_lmhead_kernel (second pass)", "d2sd_assemble_kernel", "verify_greedy_kernel"}
    assert out[0].startswith("Per step, mean of 2 steps")
