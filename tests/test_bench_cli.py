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
