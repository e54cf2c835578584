"""The library's host code (launch planner, workspace sizing, argument
validation) under UndefinedBehaviorSanitizer: an instrumented build (host
side only; the device code is built as usual) is called over extreme and
random chunk and cache sizes by host_fuzz.py, and any report (integer
overflow, out-of-range enum, shift, ...) fails the test.  CPU only."""
import glob
import os
import subprocess
import sys

import pytest

from chunked_prefill_flash_amd import build

HERE = os.path.dirname(os.path.abspath(__file__))


def ubsan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.ubsan_standalone-x86_64.so"))
    return hits[-1] if hits else None


@pytest.mark.timeout(600)
def test_host_entry_points_have_no_undefined_behaviour(tmp_path):
    rt = ubsan_runtime()
    if rt is None:
        pytest.skip("no UBSan runtime in this ROCm installation")
    so = str(tmp_path / "libattn_ubsan.so")
    flags = [f for f in build.flags() if f not in ("-O3",)]
    cmd = [build.hipcc(), *flags, "-O1", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-shared-libsan", build.SRC, "-o", so]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, LD_PRELOAD=rt, UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, os.path.join(HERE, "host_fuzz.py"), so, "120"], capture_output=True,
                       text=True, env=env, timeout=500)
    assert r.returncode == 0 and "runtime error" not in r.stderr, (r.stdout[-2000:], r.stderr[-4000:])
    assert "host_fuzz:" in r.stdout
