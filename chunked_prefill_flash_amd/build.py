"""Build the HIP library libattn_prefill.so in-tree with hipcc for gfx950.

    python -m chunked_prefill_flash_amd.build

The library exposes the C ABI declared in include/attn_prefill.h; the Python
binding in this package loads it with ctypes.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "attn_prefill.hip")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libattn_prefill.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (looked in $HIPCC, /opt/rocm/bin, PATH)")


def flags(extra=()) -> list:
    return [
        "--offload-arch=" + ARCH,
        "-O3",
        "-std=c++20",
        "-fPIC",
        "-shared",
        "-Wall",
        "-I", INCLUDE,
        # Keep the compiler from forming packed fp32 (v_pk_*_f32) instructions.
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        *extra,
    ]


def build(verbose: bool = False, extra=()) -> str:
    """Compile the library; always recompiles.  Returns the .so path."""
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), *flags(extra), SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = ("packed-fp32-ops", "is not a recognized feature for this target")
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if not any(s in ln for s in noise)]
    if r.returncode != 0:
        sys.stderr.write("\n".join(msgs) + "\n")
        raise RuntimeError("hipcc failed (%d): %s" % (r.returncode, " ".join(cmd)))
    if verbose and msgs:
        sys.stderr.write("\n".join(msgs) + "\n")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
