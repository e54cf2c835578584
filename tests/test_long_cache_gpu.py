"""GPU parity on a cache past 2 GiB: 1,100,000 fp32 positions, so K/V rows
from position 2^20 on start at byte offsets of 2^31 and beyond (2 KiB per
position, all 8 KV heads).  The prefill entry point runs a ragged 40-row chunk
at the end of the cache and the split-KV entry point its last row as a single
token, so both the staged-tile kernel and the decode kernel address the whole
range.  Bands of i.i.d. positions with strongly scaled keys sit at both ends
and across the 2^31-byte boundary; see synth.case_long_cache.

The oracle computes sampled rows one by one (all 32 heads of the chunk's
first, a middle and its last row); tolerance as in test_parity_gpu.py.
"""
import functools

import numpy as np
import pytest
import torch

import chunked_prefill_flash_amd as cpf
import oracle
import synth

pytestmark = pytest.mark.gpu

T = 1_100_000
C = 40
P = T - C
ROWS = (0, 17, C - 1)


@functools.lru_cache(maxsize=1)
def inputs():
    q, k, v, bands = synth.case_long_cache(C, P, 1100)
    rows = np.repeat(np.array(ROWS, dtype=np.int32), 32)
    heads = np.tile(np.arange(32, dtype=np.int32), len(ROWS))
    ref = oracle.attn_rows(q, k, v, P, rows, heads).reshape(len(ROWS), 32, 64)
    return q, k, v, bands, ref


def close_f32(got, ref, what):
    err = np.abs(got.astype(np.float64) - ref.astype(np.float64))
    bad = ~(err <= 1e-4 + 1e-3 * np.abs(ref.astype(np.float64)))
    assert not bad.any(), "%s: %d bad, max err %g" % (what, bad.sum(), np.nanmax(err))


def test_bands_cross_the_2gib_offset():
    _, k, _, bands, _ = inputs()
    row_bytes = k.shape[1] * k.shape[2] * 4
    lo, hi = bands[1]
    assert lo * row_bytes < 2 ** 31 < hi * row_bytes
    assert T * row_bytes > 2 ** 31


def test_prefill_past_2gib():
    q, k, v, _, ref = inputs()
    dev = torch.device("cuda", 0)
    kd = torch.from_numpy(k).to(dev)
    vd = torch.from_numpy(v).to(dev)
    out = torch.full((C, 32, 64), float("nan"), device=dev)
    cpf.attn_prefill(torch.from_numpy(q).to(dev), kd, vd, out=out, P=P)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.isfinite(got).all()
    close_f32(got[list(ROWS)], ref, "prefill C=%d P=%d" % (C, P))


def test_decode_past_2gib():
    q, k, v, _, ref = inputs()
    dev = torch.device("cuda", 0)
    q1 = torch.from_numpy(np.ascontiguousarray(q[C - 1:])).to(dev)
    need, splits = cpf.splitkv_workspace(1, T - 1, torch.float32)
    ws = torch.full((need // 4 + 4,), float("nan"), device=dev)
    out = torch.full((1, 32, 64), float("nan"), device=dev)
    cpf.attn_prefill_splitkv(q1, torch.from_numpy(k).to(dev), torch.from_numpy(v).to(dev), out=out, P=T - 1,
                             workspace=ws)
    torch.cuda.synchronize()
    assert splits > 1
    close_f32(out.cpu().numpy(), ref[-1:], "decode P=%d" % (T - 1))
