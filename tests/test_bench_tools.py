"""CPU tests of the benchmark's trace summary: a synthetic rocprofv3 kernel
trace laid out the way bench.py dispatches its passes (per part: warmup, the
three steps that time a part's step, the wall-clock pass, then the event pass
in chunks, each chunk's untimed settle steps before its timed steps) must
come back with only the timed calls of each part, each part's store matched
to its own steps."""
import contextlib
import csv
import io
import os
import re

import bench

STEP_KERNELS = {
    "decode": ["pkv::store_kvcache_kernel(pkv::StoreArgs)", "void pkv::decode_sk_kernel<4>(pkv::DecodeArgs)",
               "void pkv::decode_sk_reduce_kernel<4>(pkv::DecodeArgs)"],
    "prefill": ["pkv::store_kvcache_kernel(pkv::StoreArgs)",
                "void pkv::prefill_mfma_kernel<1, 4, 1, 2, false, 1>(pkv::PrefillArgs)"],
}
PASS_US = {"warmup": 0, "settle": 900, "timed": 100, "events": 200}


def _dur_us(part_index, kernel, pas):
    # attention kernels: 1000 per part + the pass code; stores: 10 per part + the pass code
    base = 10 * (part_index + 1) if "store" in kernel else 1000 * (part_index + 1)
    return base + PASS_US[pas]


def _synthetic_trace(path, workload, steps, warmup, settle):
    parts = bench.WORKLOADS[workload]
    seq = []   # (part index, pass) of every step in dispatch order
    for pi in range(len(parts)):
        seq += [(pi, "warmup")] * (warmup + min(3, warmup + steps))
    for pi in range(len(parts)):
        seq += [(pi, "timed")] * steps
    for pi in range(len(parts)):
        for c0 in range(0, steps, bench.EVENT_CHUNK_STEPS):
            seq += [(pi, "settle")] * settle[pi]
            seq += [(pi, "events")] * (min(c0 + bench.EVENT_CHUNK_STEPS, steps) - c0)
    rows, t = [], 0
    for pi, pas in seq:
        for k in STEP_KERNELS[parts[pi][0]]:
            d = int(_dur_us(pi, k, pas) * 1000)
            rows.append({"Kernel_Name": k, "Start_Timestamp": t, "End_Timestamp": t + d})
            t += d + 5000
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_kernel_trace.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        w.writerows(rows)


def test_trace_summary_keeps_only_the_timed_calls_of_each_part(tmp_path):
    workload, steps, warmup, settle = "default", 20, 3, [2, 7, 5, 3]
    _synthetic_trace(str(tmp_path), workload, steps, warmup, settle)
    buf = io.StringIO()
    with contextlib.redirect_stdout(buf):
        bench.summarize_trace(str(tmp_path), workload, steps, warmup, "cmd", settle)
    table = [ln for ln in buf.getvalue().splitlines() if ln.startswith("| ") and "preset" in ln]
    parts = bench.WORKLOADS[workload]
    seen = 0
    for ln in table:
        cells = [c.strip() for c in ln.strip("|").split("|")]
        kernel, wl, n, mean = cells[0], cells[1], int(cells[2]), float(cells[3])
        preset = int(re.search(r"preset (\d+)", wl).group(1))
        pi = next(i for i, (ph, p) in enumerate(parts) if p == preset)
        assert n == 2 * steps, ln                       # wall-clock and event passes, no settle steps
        name = next(k for k in STEP_KERNELS[parts[pi][0]] if kernel in k)
        want = (_dur_us(pi, name, "timed") + _dur_us(pi, name, "events")) / 2
        assert abs(mean - want) < 0.05, (ln, want)
        seen += 1
    # every part's attention kernel(s) and store
    assert seen == sum(len(STEP_KERNELS[ph]) for ph, _ in parts), buf.getvalue()


def test_trace_summary_rejects_a_settle_count_that_does_not_match(tmp_path):
    _synthetic_trace(str(tmp_path), "default", 20, 3, [2, 7, 5, 3])
    buf = io.StringIO()
    try:
        with contextlib.redirect_stdout(buf):
            bench.summarize_trace(str(tmp_path), "default", 20, 3, "cmd", [2, 7, 5, 4])
    except SystemExit as e:
        assert "dispatches, expected" in str(e)
    else:
        raise AssertionError("a wrong settle count went unnoticed")
