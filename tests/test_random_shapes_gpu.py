"""GPU parity over a seeded sweep of shapes, every output element against the
oracle, through the contiguous, paged and split-KV entry points.

The launch planner picks the work-item height, the key-split count, the
pairing of row tiles and the number of splits from (C, P, dtype); the sweep
covers the chunk lengths where the bf16 shape changes (256, 2048, 4096) on
both sides, and random (C, P, dtype, entry point, page size) drawn from
SplitMix64 with log-uniform C in [1, 1500] and P in [0, 3000] (P = 0 one time
in four).  Inputs carry three 4.0 plants in the chunk, which must come out
as exactly 4.0.  Tolerances as in test_parity_gpu.py.
"""
import math
import os

import numpy as np
import pytest
import torch

import chunked_prefill_flash_amd as cpf
import oracle
import synth

pytestmark = pytest.mark.gpu

HQ, D = 32, 64
PAGE_SIZES = (1, 3, 16, 31, 64, 128)


def _draw_cases(n, seed=0x5EED):
    r = synth.uniform53(seed, 8 * n)
    cases = []
    for t in range(n):
        u = r[8 * t: 8 * t + 8]
        entry = ("prefill", "paged", "splitkv")[int(u[0] * 3) % 3]
        dtype = "bf16" if u[1] < 0.5 else "f32"
        C = max(1, int(round(math.exp(u[2] * math.log(1500)))))
        P = 0 if u[3] < 0.25 else int(round(math.exp(u[4] * math.log(3000))))
        page = PAGE_SIZES[int(u[5] * len(PAGE_SIZES)) % len(PAGE_SIZES)]
        cases.append((entry, dtype, C, P, page))
    return cases


THRESHOLDS = [("prefill", "bf16", C, P, 0) for C, P in
              [(255, 5), (256, 0), (257, 5), (2047, 0), (2048, 5), (2049, 0), (4095, 5), (4096, 0), (4097, 5)]]
CASES = THRESHOLDS + _draw_cases(24)


def _gpu(x, dtype):
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(x)).cuda()
    return torch.from_numpy(synth.to_bf16_bits(x).view(np.int16)).view(torch.bfloat16).cuda()


def _widen(x, dtype):
    return x if dtype == "f32" else synth.bf16_bits_to_f32(synth.to_bf16_bits(x))


@pytest.mark.parametrize("entry,dtype,C,P,page", CASES,
                         ids=["%s-%s-C%d-P%d%s" % (e, d, c, p, "-pg%d" % g if e == "paged" else "")
                              for e, d, c, p, g in CASES])
def test_shape(entry, dtype, C, P, page):
    seed = 20000 + 7 * C + 13 * P + (1 if dtype == "bf16" else 0)
    q, k, v, plants = synth.case_planted_chunk(C, P, seed, 3)
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    out = torch.full((C, HQ, D), float("nan"), device="cuda")
    if entry == "prefill":
        cpf.attn_prefill(_gpu(q, dtype), _gpu(k, dtype), _gpu(v, dtype), out=out, P=P)
    elif entry == "paged":
        kp, vp, table = synth.to_pages(k, v, page, seed + 5)
        cpf.attn_prefill_paged(_gpu(q, dtype), _gpu(kp, dtype), _gpu(vp, dtype), torch.from_numpy(table).cuda(), P,
                               out=out)
    else:
        need, _ = cpf.splitkv_workspace(C, P, tdt)
        ws = torch.full((need // 4 + 4,), float("nan"), device="cuda")
        cpf.attn_prefill_splitkv(_gpu(q, dtype), _gpu(k, dtype), _gpu(v, dtype), out=out, P=P, workspace=ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    qo, ko, vo = _widen(q, dtype), _widen(k, dtype), _widen(v, dtype)
    ref = oracle.attn_prefill(qo, ko, vo, P).astype(np.float64)
    if dtype == "f32":
        tol = 1e-4 + 1e-3 * np.abs(ref)
    else:
        tol = 1e-5 + 2.0 ** -8 * oracle.attn_prefill(qo, ko, np.abs(vo), P).astype(np.float64)
    err = np.abs(got - ref)
    bad = ~(err <= tol)
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        pytest.fail("%d of %d out of tolerance; first %s got %r ref %r" % (bad.sum(), bad.size, i, got[i], ref[i]))
    for p in plants:
        assert np.all(got[p - P, 0] == 4.0), "planted row %d" % (p - P)


def test_wide_sweep_sampled_rows():
    """A wider seeded sweep checked on sampled rows (first, last, six drawn, the
    planted ones; all 32 heads): entry point among contiguous, paged (pages of
    1-256 positions), split-KV, paged split-KV, split-KV without a workspace
    and per-row; C log-uniform in [1, 2500], P in [0, 6000] (0 one time in
    five).  CPF_SWEEP_CASES sets the number of cases (default 200, a few
    seconds; 3000 take under two minutes), CPF_SWEEP_MAX_C and CPF_SWEEP_MAX_P
    the ranges' upper ends (the planner's multi-round rules for 1025+ rows
    against prefixes of 8C need a wider P)."""
    n = int(os.environ.get("CPF_SWEEP_CASES", "200"))
    max_c = int(os.environ.get("CPF_SWEEP_MAX_C", "2500"))
    max_p = int(os.environ.get("CPF_SWEEP_MAX_P", "6000"))
    r = synth.uniform53(778, 8 * n)
    bad = []
    for t in range(n):
        u = r[8 * t: 8 * t + 8]
        entry = ("prefill", "paged", "splitkv", "rowwise", "paged_splitkv", "noalloc")[int(u[0] * 6) % 6]
        dtype = "bf16" if u[1] < 0.5 else "f32"
        C = max(1, int(round(math.exp(u[2] * math.log(max_c)))))
        P = 0 if u[3] < 0.2 else int(round(math.exp(u[4] * math.log(max_p))))
        page = (1, 2, 7, 16, 31, 64, 100, 128, 256)[int(u[5] * 9) % 9]
        if entry == "rowwise" and C * (P + C) > 3e6:
            entry = "prefill"   # the per-row baseline is slow on big shapes
        seed = 50000 + t
        q, k, v, plants = synth.case_planted_chunk(C, P, seed, 3)
        tdt = torch.float32 if dtype == "f32" else torch.bfloat16
        if entry == "noalloc" and cpf.splitkv_workspace(C, P, tdt)[0] > cpf.NOALLOC_SCRATCH_BYTES:
            entry = "splitkv"   # beyond the fixed scratch array
        out = torch.full((C, HQ, D), float("nan"), device="cuda")
        if entry == "prefill":
            cpf.attn_prefill(_gpu(q, dtype), _gpu(k, dtype), _gpu(v, dtype), out=out, P=P)
        elif entry == "rowwise":
            cpf.attn_prefill_rowwise(_gpu(q, dtype), _gpu(k, dtype), _gpu(v, dtype), out=out, P=P)
        elif entry == "paged":
            kp, vp, table = synth.to_pages(k, v, page, seed + 5)
            cpf.attn_prefill_paged(_gpu(q, dtype), _gpu(kp, dtype), _gpu(vp, dtype),
                                   torch.from_numpy(table).cuda(), P, out=out)
        elif entry == "paged_splitkv":
            kp, vp, table = synth.to_pages(k, v, page, seed + 5)
            need, _ = cpf.splitkv_workspace(C, P, tdt)
            ws = torch.full((need // 4 + 4,), float("nan"), device="cuda")
            cpf.attn_prefill_paged_splitkv(_gpu(q, dtype), _gpu(kp, dtype), _gpu(vp, dtype),
                                           torch.from_numpy(table).cuda(), P, out=out, workspace=ws)
        elif entry == "noalloc":
            cpf.attn_prefill_splitkv_noalloc(_gpu(q, dtype), _gpu(k, dtype), _gpu(v, dtype), out, P=P)
        else:
            need, _ = cpf.splitkv_workspace(C, P, tdt)
            ws = torch.full((need // 4 + 4,), float("nan"), device="cuda")
            cpf.attn_prefill_splitkv(_gpu(q, dtype), _gpu(k, dtype), _gpu(v, dtype), out=out, P=P, workspace=ws)
        torch.cuda.synchronize()
        got = out.cpu().numpy().astype(np.float64)
        rows = sorted(set([0, C - 1] + [int(x * C) % C for x in synth.uniform53(seed + 9, 6)] + [p - P for p in plants]))
        rr = np.repeat(np.array(rows, dtype=np.int32), HQ)
        hh = np.tile(np.arange(HQ, dtype=np.int32), len(rows))
        qo, ko, vo = _widen(q, dtype), _widen(k, dtype), _widen(v, dtype)
        ref = oracle.attn_rows(qo, ko, vo, P, rr, hh).astype(np.float64)
        if dtype == "f32":
            tol = 1e-4 + 1e-3 * np.abs(ref)
        else:
            tol = 1e-5 + 2.0 ** -8 * oracle.attn_rows(qo, ko, np.abs(vo), P, rr, hh).astype(np.float64)
        ok = bool(np.all(np.abs(got[rr, hh] - ref) <= tol)) and bool(np.isfinite(got).all())
        ok = ok and all(bool(np.all(got[p - P, 0] == 4.0)) for p in plants)
        if not ok:
            bad.append((t, entry, dtype, C, P, page))
        if (t + 1) % 50 == 0:   # progress for long sweeps (visible with -s)
            print("sweep: %d of %d cases, %d failed" % (t + 1, n, len(bad)), flush=True)
    assert not bad, "%d of %d cases failed, first %s" % (len(bad), n, bad[:5])
