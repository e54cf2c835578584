"""bench.py's command-line contract, checked without a GPU: more than one GPU
is refused with a message (the library runs on one GPU), and every workload
is listed."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_help_lists_the_workloads():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--help"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0
    for w in ("c2048_p2048_f32", "c4096_p28672_bf16", "c1_p16383_f32_splitkv", "c1_p131071_f32_splitkv",
              "c2048_p2048_f32_paged16"):
        assert w in r.stdout


def _write_counter_csv(path, rows):
    import csv
    os.makedirs(os.path.dirname(path), exist_ok=True)
    cols = ["Correlation_Id", "Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp",
            "End_Timestamp"]
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=cols)
        w.writeheader()
        for i, (kernel, counter, value, dur_ns) in enumerate(rows):
            w.writerow({"Correlation_Id": i, "Dispatch_Id": i, "Kernel_Name": kernel, "Counter_Name": counter,
                        "Counter_Value": value, "Start_Timestamp": 1000, "End_Timestamp": 1000 + dur_ns})


def test_rocprof_summary_scales_traffic_by_the_copy_calibration(tmp_path):
    """The harness's CSV -> summary step on synthetic rocprofv3 output: two
    calls of the prefill kernel, a copy kernel whose FETCH_SIZE reads half
    its known 512 MiB, so the kernel's fetched KiB are doubled, written KiB
    taken as they are."""
    sys.path.insert(0, ROOT)
    import bench
    prof = tmp_path / "prof"
    kern = ("void (anonymous namespace)::attn_prefill_kernel<float, 4, 4, 0>(float const*, float const*, "
            "float const*, float*, int, int, int, int, (anonymous namespace)::PagedCache, "
            "(anonymous namespace)::KeySplit)")
    copy = "void at::native::vectorized_elementwise_kernel<4, at::native::MulFunctor<float>>(int, ...)"
    half = (512 << 20) // 1024 // 2
    _write_counter_csv(str(prof / "fetch" / "fetch_counter_collection.csv"),
                       [(kern, "FETCH_SIZE", 8000.0, 400000), (kern, "FETCH_SIZE", 8400.0, 400000),
                        (copy, "FETCH_SIZE", half, 90000), (copy, "FETCH_SIZE", 12.0, 1000)])
    _write_counter_csv(str(prof / "write" / "write_counter_collection.csv"),
                       [(kern, "WRITE_SIZE", 16384.0, 400000), (kern, "WRITE_SIZE", 16384.0, 400000),
                        (copy, "WRITE_SIZE", 2 * half, 90000)])
    out = tmp_path / "profiles"
    out.mkdir()
    written = bench.summarize_rocprof("c2048_p2048_f32", str(prof), profiles_dir=str(out))
    assert len(written) == 2
    import json
    e = json.load(open(out / "traffic.json"))["c2048_p2048_f32"]
    assert e["fetch_scale"] == 2.0 and e["write_scale"] == 1.0
    assert e["bytes_per_launch"] == int(8200.0 * 1024 * 2 + 16384.0 * 1024)
    assert e["algorithmic_bytes"] == 48 << 20
    assert e["kernel_source_sha256_16"] == bench.kernel_source_hash()
    text = open(out / "attn_prefill_c2048_p2048_f32_counters.md").read()
    assert "rocprofv3 --pmc FETCH_SIZE" in text and "ratio" in text


def test_clock_from_log_on_a_synthetic_log():
    """The benchmark's reading of the clock log, on a hand-made one: two
    workgroups at exactly 2000 and 2400 MHz (shader-clock cycles over 100 MHz
    ticks), the second with a second work item; medians, busy-time average,
    phase spans in microseconds at each workgroup's own clock, kernel span
    and start spread from the 100 MHz counter."""
    sys.path.insert(0, ROOT)
    import bench
    import numpy as np
    import torch

    def wg(mhz, t0_tick, ticks, marks_us, second_us=None):
        cyc_per_us = mhz                       # cycles per microsecond at `mhz` MHz
        c0 = 1_000_000
        row = [c0, t0_tick, c0 + int(ticks / 100.0 * cyc_per_us), t0_tick + ticks]
        row += [c0 + int(u * cyc_per_us) for u in marks_us]
        row += [0 if second_us is None else c0 + int(second_us * cyc_per_us)]
        return row

    log = torch.tensor([wg(2000.0, 500, 1000, [1.0, 6.0, 7.0]),                  # 10 us at 2000 MHz
                        wg(2400.0, 520, 2000, [2.0, 8.0, 9.0], second_us=10.0)],  # 20 us at 2400 MHz
                       dtype=torch.int64)
    c = bench.clock_from_log(log)
    assert c["median_mhz"] == 2400.0 and c["min_mhz"] == 2000.0 and c["max_mhz"] == 2400.0
    # busy-time average: all cycles over all ticks = (20000 + 48000) / 3000 ticks * 100
    assert abs(c["busy_average_mhz"] - (20000 + 48000) / 3000 * 100) < 0.2
    ph = c["phases_us"]
    assert ph["workgroups_with_two_items"] == 1
    assert ph["first_item_prologue"] == 1.5 and ph["first_item_key_loop"] == 5.5
    assert ph["first_item_epilogue"] == 1.0
    assert ph["second_item_prologue"] == 1.0 and ph["second_item_rest"] == 10.0
    assert ph["workgroup"] == 15.0
    assert ph["kernel_span"] == round((2520 - 500) / 100.0, 2) and ph["start_spread"] == 0.2
    assert np.isfinite(list(v for v in ph.values() if v is not None)).all()
