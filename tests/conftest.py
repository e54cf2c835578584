import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_sessionstart(session):
    # A fresh checkout has no built library: compile it (hipcc cross-compiles
    # for gfx950 without a GPU) so the host-side ABI tests can load it.  GPU
    # runs use the library built beforehand and never reach this.
    from chunked_prefill_flash_amd import build as hip_build
    if not os.path.exists(hip_build.LIB):
        try:
            hip_build.build()
        except Exception as exc:  # the ABI tests then report the missing library
            sys.stderr.write("could not build the HIP library: %s\n" % exc)


def pytest_collection_modifyitems(config, items):
    # GPU tests are collected everywhere but skipped when no GPU is visible, so a
    # plain `pytest` on a CPU-only machine stays green.  On a GPU machine they run.
    try:
        import torch
        have_gpu = torch.cuda.is_available()
    except Exception:
        have_gpu = False
    if have_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)
